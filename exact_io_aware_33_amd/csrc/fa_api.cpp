// C ABI entry points of libfa (declared in include/fa.h): argument checks on
// the host, then one launch sequence on the caller's stream.  Every argument
// error is reported before the first HIP call; nothing here allocates,
// synchronises or keeps state between calls (apart from the calling thread's
// last error message).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <algorithm>

#include "fa.h"
#include "fa_internal.hpp"

namespace {

thread_local char g_err[512] = "";

fa_status_t fail(fa_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Rows past the end of a (batch, head) slice that a tile may address (the
// largest tile is 128 rows); they read as zeros through the buffer range
// check.
constexpr int64_t kRowSlack = 256;

int elem_size(int32_t dt) { return dt == FA_DTYPE_F32 ? 4 : 2; }

int32_t keys_of(const fa_problem_t *p) { return p->seqlen_k ? p->seqlen_k : p->seqlen; }

bool k_strides_default(const fa_problem_t *p) {
  return p->k_stride_b == 0 && p->k_stride_h == 0 && p->k_stride_n == 0;
}

// Checks shared by every entry point.
fa_status_t check_problem(const fa_problem_t *p) {
  if (!p) return fail(FA_ERR_INVALID, "problem pointer is NULL");
  if (p->batch <= 0 || p->heads <= 0 || p->seqlen <= 0)
    return fail(FA_ERR_INVALID, "batch, heads and seqlen must be >= 1 (got %d, %d, %d)", p->batch,
                p->heads, p->seqlen);
  if (p->seqlen_k < 0) return fail(FA_ERR_INVALID, "seqlen_k must be >= 0 (got %d)", p->seqlen_k);
  if (p->fwd_query_tile != 0 && p->fwd_query_tile != 64 && p->fwd_query_tile != 128 &&
      p->fwd_query_tile != 256)
    return fail(FA_ERR_INVALID, "fwd_query_tile must be 0, 64, 128 or 256 (got %d)", p->fwd_query_tile);
  if (p->dtype != FA_DTYPE_F32 && p->dtype != FA_DTYPE_F16 && p->dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_INVALID, "unknown dtype %d", p->dtype);
  if (p->head_dim <= 0) return fail(FA_ERR_INVALID, "head_dim must be >= 1 (got %d)", p->head_dim);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", p->head_dim);
  if (!std::isfinite(p->scale) || p->scale < 0.f)
    return fail(FA_ERR_INVALID, "scale must be finite and >= 0");
  const int64_t bh = (int64_t)p->batch * p->heads;
  for (int64_t n : {(int64_t)p->seqlen, (int64_t)keys_of(p)})
    if (bh * n * p->head_dim >= (int64_t(1) << 31))
      return fail(FA_ERR_UNSUPPORTED, "B*H*N*d exceeds the 32-bit index range");
  const int es = elem_size(p->dtype);
  const bool kdef = k_strides_default(p);
  const int64_t st[2][3] = {{p->stride_b, p->stride_h, p->stride_n},
                            {kdef ? p->stride_b : p->k_stride_b, kdef ? p->stride_h : p->k_stride_h,
                             kdef ? p->stride_n : p->k_stride_n}};
  const int64_t rows_of[2] = {p->seqlen, keys_of(p)};
  for (int t = 0; t < 2; ++t) {
    const char *nm = t ? "k_stride_n" : "stride_n";
    if (st[t][0] < 0 || st[t][1] < 0 || st[t][2] < 0)
      return fail(FA_ERR_INVALID, "strides must be non-negative");
    if (st[t][2] < p->head_dim)
      return fail(FA_ERR_INVALID, "%s (%lld) smaller than head_dim", nm, (long long)st[t][2]);
    if ((st[t][0] * es) % 16 || (st[t][1] * es) % 16 || (st[t][2] * es) % 16)
      return fail(FA_ERR_UNSUPPORTED, "strides must be multiples of 16 bytes (16-byte vector path)");
    // The kernels address the rows of one (batch, head) slice -- including
    // up to kRowSlack rows past its end, which a tile may overrun and the
    // buffer range check turns into zeros -- with 32-bit byte offsets from
    // the slice's start (buffer record count, tile offsets).
    if ((rows_of[t] + kRowSlack) * st[t][2] * es >= (int64_t(1) << 31))
      return fail(FA_ERR_UNSUPPORTED,
                  "(%s + %d) * %s * element size = %lld bytes reaches 2^31 (32-bit row offsets)",
                  t ? "N_k" : "N_q", (int)kRowSlack, nm,
                  (long long)((rows_of[t] + kRowSlack) * st[t][2] * es));
  }
  if (p->key_lens && !aligned16(p->key_lens))
    return fail(FA_ERR_UNSUPPORTED, "key_lens must be 16-byte aligned");
  if (!std::isfinite(p->dropout_p) || p->dropout_p < 0.f || p->dropout_p >= 1.f)
    return fail(FA_ERR_INVALID, "dropout_p must be in [0, 1)");
  return FA_OK;
}

// Dropout threshold t = round-half-even(256 p) clamped to [0, 255]; t = 0
// keeps every element (no dropout).
uint32_t drop_threshold(float p) {
  const double t = std::nearbyint((double)p * 256.0);
  return (uint32_t)(t < 0.0 ? 0.0 : (t > 255.0 ? 255.0 : t));
}

fa_status_t check_tensor(const void *ptr, const char *name) {
  if (!ptr) return fail(FA_ERR_INVALID, "%s is NULL", name);
  if (!aligned16(ptr))
    return fail(FA_ERR_UNSUPPORTED, "%s is not 16-byte aligned (16-byte vector path)", name);
  return FA_OK;
}

fa_status_t check_mask(const fa_problem_t *p, const uint8_t *mask, int32_t mb, int64_t hstride) {
  if (!mask) return fail(FA_ERR_INVALID, "block_mask is NULL");
  if (mb <= 0) return fail(FA_ERR_INVALID, "mask_block must be >= 1 (got %d)", mb);
  if (p->seqlen % mb || keys_of(p) % mb)
    return fail(FA_ERR_INVALID, "mask_block %d does not divide N_q = %d and N_k = %d", mb, p->seqlen,
                keys_of(p));
  if (mb % 128) return fail(FA_ERR_UNSUPPORTED, "mask_block %d is not a multiple of 128", mb);
  if (p->seqlen / mb > 1024 || keys_of(p) / mb > 1024)
    return fail(FA_ERR_UNSUPPORTED, "N / mask_block exceeds 1024");
  if (hstride < 0) return fail(FA_ERR_INVALID, "mask_head_stride must be >= 0");
  return FA_OK;
}

fa::AttnParams make_params(const fa_problem_t *p) {
  fa::AttnParams a{};
  a.B = p->batch;
  a.H = p->heads;
  a.Nq = p->seqlen;
  a.Nk = keys_of(p);
  a.d = p->head_dim;
  a.sb = p->stride_b;
  a.sh = p->stride_h;
  a.sn = p->stride_n;
  const bool same = k_strides_default(p);
  a.ksb = same ? p->stride_b : p->k_stride_b;
  a.ksh = same ? p->stride_h : p->k_stride_h;
  a.ksn = same ? p->stride_n : p->k_stride_n;
  a.cshift = a.Nk - a.Nq;
  a.scale = p->scale;
  a.scale_log2 = p->scale * fa::kLog2eHost;
  a.causal = p->causal != 0;
  a.key_lens = p->key_lens;
  a.drop_thr = drop_threshold(p->dropout_p);
  a.drop_scale = a.drop_thr ? (float)(256.0 / (256.0 - a.drop_thr)) : 1.f;
  a.drop_key0 = (uint32_t)(p->dropout_seed & 0xFFFFFFFFu);
  a.drop_key1 = (uint32_t)(p->dropout_seed >> 32);
  a.drop_offset = p->dropout_offset;
  a.qtile = 128;
  return a;
}

fa_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
}

fa_status_t fwd_impl(const fa_problem_t *p, const uint8_t *mask, int32_t mb, int64_t hstride,
                     bool sparse, const void *q, const void *k, const void *v, void *o, float *lse,
                     void *stream) {
  g_err[0] = 0;
  fa_status_t st;
  if ((st = check_problem(p)) != FA_OK) return st;
  if ((st = check_tensor(q, "q")) != FA_OK || (st = check_tensor(k, "k")) != FA_OK ||
      (st = check_tensor(v, "v")) != FA_OK || (st = check_tensor(o, "o")) != FA_OK ||
      (st = check_tensor(lse, "lse")) != FA_OK)
    return st;
  if (sparse && (st = check_mask(p, mask, mb, hstride)) != FA_OK) return st;
  fa::AttnParams a = make_params(p);
  a.qtile = p->fwd_query_tile ? p->fwd_query_tile : 128;
  if (a.qtile != 128 && (p->dtype == FA_DTYPE_F32 || a.drop_thr != 0))
    return fail(FA_ERR_UNSUPPORTED, "fwd_query_tile %d is built for fp16 / bf16 without dropout", a.qtile);
  if (a.qtile == 256 && sparse)
    return fail(FA_ERR_UNSUPPORTED, "fwd_query_tile 256 is not built for block masks");
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  if (sparse) {
    a.mask = mask;
    a.mb = mb;
    a.nblk_q = p->seqlen / mb;
    a.nblk_k = keys_of(p) / mb;
    a.mask_hstride = hstride;
  }
  return hip_status(fa::launch_fwd(a, (fa_dtype_t)p->dtype, sparse, (hipStream_t)stream));
}

// Split count the library picks: about two workgroups per CU over 256 CUs
// (a sweep over decoding shapes, 8K-128K keys, d = 64 and 128, put 512
// workgroups within 2% of the best count everywhere), at least four key tiles
// per range, at most 128 ranges.
int32_t auto_splits(const fa_problem_t *p) {
  const int64_t nqt = (p->seqlen + 127) / 128;
  const int64_t base = (int64_t)p->batch * p->heads * nqt;
  const int kt = fa::fwd_key_tile((fa_dtype_t)p->dtype);
  const int64_t tiles = (keys_of(p) + kt - 1) / kt;
  int64_t sp = (512 + base - 1) / base;
  sp = std::min<int64_t>(sp, std::max<int64_t>(1, tiles / 4));
  sp = std::min<int64_t>(sp, 128);
  return (int32_t)std::max<int64_t>(1, sp);
}

}  // namespace

namespace fa {

fa_status_t set_error(fa_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

// The backward entry points.  With `scratch` set, the workspace is not an
// argument: once every argument has passed its checks, scratch(need, &ws,
// &ws_bytes) supplies it (and may refuse).
fa_status_t bwd_impl(const fa_problem_t *p, const uint8_t *mask, int32_t mb, int64_t hstride,
                     bool sparse, const void *q, const void *k, const void *v, const void *o,
                     const float *lse, const void *dout, void *dq, void *dk, void *dv, void *ws,
                     size_t ws_bytes, unsigned stages, void *stream, ScratchFn scratch) {
  g_err[0] = 0;
  if (stages == 0 || (stages & ~(unsigned)FA_BWD_ALL))
    return fail(FA_ERR_INVALID, "stages must be a nonzero subset of FA_BWD_ALL (got %u)", stages);
  fa_status_t st;
  if ((st = check_problem(p)) != FA_OK) return st;
  if ((st = check_tensor(q, "q")) != FA_OK || (st = check_tensor(k, "k")) != FA_OK ||
      (st = check_tensor(v, "v")) != FA_OK || (st = check_tensor(o, "o")) != FA_OK ||
      (st = check_tensor(lse, "lse")) != FA_OK || (st = check_tensor(dout, "dout")) != FA_OK ||
      (st = check_tensor(dq, "dq")) != FA_OK || (st = check_tensor(dk, "dk")) != FA_OK ||
      (st = check_tensor(dv, "dv")) != FA_OK)
    return st;
  if (!scratch && (st = check_tensor(ws, "workspace")) != FA_OK) return st;
  if (sparse && (st = check_mask(p, mask, mb, hstride)) != FA_OK) return st;
  const int64_t rows = (int64_t)p->batch * p->heads * p->seqlen;
  const size_t need = fa::ws_total_bytes(rows);
  if (scratch && (st = scratch(need, &ws, &ws_bytes)) != FA_OK) return st;
  if (ws_bytes < need)
    return fail(FA_ERR_INVALID, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, need);
  fa::AttnParams a = make_params(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o_in = o;
  a.lse = const_cast<float *>(lse);
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws_negd = static_cast<float *>(ws);
  a.ws_lse2 = reinterpret_cast<float *>(static_cast<char *>(ws) + fa::ws_array_bytes(rows));
  if (sparse) {
    a.mask = mask;
    a.mb = mb;
    a.nblk_q = p->seqlen / mb;
    a.nblk_k = keys_of(p) / mb;
    a.mask_hstride = hstride;
  }
  return hip_status(fa::launch_bwd(a, (fa_dtype_t)p->dtype, sparse, stages, (hipStream_t)stream));
}

}  // namespace fa

using fa::bwd_impl;

extern "C" {

fa_status_t fa_fwd(const fa_problem_t *p, const void *q, const void *k, const void *v, void *o,
                   float *lse, void *stream) {
  return fwd_impl(p, nullptr, 0, 0, false, q, k, v, o, lse, stream);
}

fa_status_t fa_fwd_blocksparse(const fa_problem_t *p, const uint8_t *block_mask, int32_t mask_block,
                               int64_t mask_head_stride, const void *q, const void *k, const void *v,
                               void *o, float *lse, void *stream) {
  return fwd_impl(p, block_mask, mask_block, mask_head_stride, true, q, k, v, o, lse, stream);
}

size_t fa_bwd_workspace_bytes(const fa_problem_t *p) {
  g_err[0] = 0;
  if (check_problem(p) != FA_OK) return 0;
  const int64_t rows = (int64_t)p->batch * p->heads * p->seqlen;
  return fa::ws_total_bytes(rows);
}

fa_status_t fa_bwd(const fa_problem_t *p, const void *q, const void *k, const void *v, const void *o,
                   const float *lse, const void *dout, void *dq, void *dk, void *dv, void *workspace,
                   size_t workspace_bytes, void *stream) {
  return bwd_impl(p, nullptr, 0, 0, false, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                  workspace_bytes, FA_BWD_ALL, stream, nullptr);
}

fa_status_t fa_bwd_blocksparse(const fa_problem_t *p, const uint8_t *block_mask, int32_t mask_block,
                               int64_t mask_head_stride, const void *q, const void *k, const void *v,
                               const void *o, const float *lse, const void *dout, void *dq, void *dk,
                               void *dv, void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl(p, block_mask, mask_block, mask_head_stride, true, q, k, v, o, lse, dout, dq, dk, dv,
                  workspace, workspace_bytes, FA_BWD_ALL, stream, nullptr);
}

fa_status_t fa_bwd_ex(const fa_problem_t *p, const uint8_t *block_mask, int32_t mask_block,
                      int64_t mask_head_stride, const void *q, const void *k, const void *v,
                      const void *o, const float *lse, const void *dout, void *dq, void *dk, void *dv,
                      void *workspace, size_t workspace_bytes, uint32_t stages, void *stream) {
  return bwd_impl(p, block_mask, mask_block, mask_head_stride, block_mask != nullptr, q, k, v, o, lse,
                  dout, dq, dk, dv, workspace, workspace_bytes, stages, stream, nullptr);
}

fa_status_t fa_merge_partials(const fa_problem_t *p, int32_t num_parts, const void *const *o_parts,
                              const float *const *lse_parts, void *o, float *lse, void *stream) {
  g_err[0] = 0;
  fa_status_t st;
  if ((st = check_problem(p)) != FA_OK) return st;
  if (num_parts < 1 || num_parts > FA_MERGE_MAX_PARTS)
    return fail(FA_ERR_INVALID, "num_parts must be in [1, %d] (got %d)", FA_MERGE_MAX_PARTS, num_parts);
  if (!o_parts || !lse_parts) return fail(FA_ERR_INVALID, "o_parts and lse_parts must not be NULL");
  fa::MergeParams a{};
  for (int s = 0; s < num_parts; ++s) {
    char name[32];
    snprintf(name, sizeof name, "o_parts[%d]", s);
    if ((st = check_tensor(o_parts[s], name)) != FA_OK) return st;
    snprintf(name, sizeof name, "lse_parts[%d]", s);
    if ((st = check_tensor(lse_parts[s], name)) != FA_OK) return st;
    a.o_parts[s] = o_parts[s];
    a.lse_parts[s] = lse_parts[s];
  }
  if ((st = check_tensor(o, "o")) != FA_OK || (st = check_tensor(lse, "lse")) != FA_OK) return st;
  a.o = o;
  a.lse = lse;
  a.B = p->batch;
  a.H = p->heads;
  a.Nq = p->seqlen;
  a.d = p->head_dim;
  a.S = num_parts;
  a.sb = p->stride_b;
  a.sh = p->stride_h;
  a.sn = p->stride_n;
  return hip_status(fa::launch_merge(a, (fa_dtype_t)p->dtype, (hipStream_t)stream));
}

int32_t fa_fwd_splitkv_num_splits(const fa_problem_t *p) {
  g_err[0] = 0;
  if (check_problem(p) != FA_OK) return 0;
  return auto_splits(p);
}

size_t fa_fwd_splitkv_workspace_bytes(const fa_problem_t *p, int32_t num_splits) {
  g_err[0] = 0;
  if (check_problem(p) != FA_OK) return 0;
  if (num_splits > 1024) {
    fail(FA_ERR_INVALID, "num_splits must be <= 1024 (got %d)", num_splits);
    return 0;
  }
  const int32_t sp = num_splits > 0 ? num_splits : auto_splits(p);
  return fa::splitkv_total_bytes((int64_t)p->batch * p->heads * p->seqlen, p->head_dim, sp);
}

fa_status_t fa_fwd_splitkv(const fa_problem_t *p, const uint8_t *block_mask, int32_t mask_block,
                           int64_t mask_head_stride, int32_t num_splits, const void *q, const void *k,
                           const void *v, void *o, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  fa_status_t st;
  if ((st = check_problem(p)) != FA_OK) return st;
  if ((st = check_tensor(q, "q")) != FA_OK || (st = check_tensor(k, "k")) != FA_OK ||
      (st = check_tensor(v, "v")) != FA_OK || (st = check_tensor(o, "o")) != FA_OK ||
      (st = check_tensor(lse, "lse")) != FA_OK || (st = check_tensor(workspace, "workspace")) != FA_OK)
    return st;
  const bool sparse = block_mask != nullptr;
  if (sparse && (st = check_mask(p, block_mask, mask_block, mask_head_stride)) != FA_OK) return st;
  if (num_splits > 1024) return fail(FA_ERR_INVALID, "num_splits must be <= 1024 (got %d)", num_splits);
  if (drop_threshold(p->dropout_p) != 0)
    return fail(FA_ERR_UNSUPPORTED, "dropout is not built for the split-KV forward");
  const int32_t sp = num_splits > 0 ? num_splits : auto_splits(p);
  const int64_t rows = (int64_t)p->batch * p->heads * p->seqlen;
  const size_t need = fa::splitkv_total_bytes(rows, p->head_dim, sp);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes,
                need);
  fa::AttnParams a = make_params(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.nsplit = sp;
  a.part_o = static_cast<float *>(workspace);
  a.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                         fa::splitkv_o_bytes(rows, p->head_dim, sp));
  if (sparse) {
    a.mask = block_mask;
    a.mb = mask_block;
    a.nblk_q = p->seqlen / mask_block;
    a.nblk_k = keys_of(p) / mask_block;
    a.mask_hstride = mask_head_stride;
  }
  return hip_status(fa::launch_fwd_splitkv(a, (fa_dtype_t)p->dtype, sparse, (hipStream_t)stream));
}

}  // extern "C"

namespace {

fa_status_t check_rows(int32_t dtype, int64_t rows, int64_t cols, const void *x, int64_t ld_x,
                       void *y, int64_t ld_y) {
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_INVALID, "unknown dtype %d", dtype);
  if (rows <= 0 || cols <= 0)
    return fail(FA_ERR_INVALID, "rows and cols must be >= 1 (got %lld, %lld)", (long long)rows,
                (long long)cols);
  if (rows >= (int64_t(1) << 31) || cols >= (int64_t(1) << 31))
    return fail(FA_ERR_UNSUPPORTED, "rows and cols must be < 2^31");
  const uintptr_t es = (uintptr_t)elem_size(dtype);
  if (ld_x < cols || ld_y < cols) return fail(FA_ERR_INVALID, "ld_x and ld_y must be >= cols");
  if (!x || !y) return fail(FA_ERR_INVALID, "x and y must not be NULL");
  if (reinterpret_cast<uintptr_t>(x) % es || reinterpret_cast<uintptr_t>(y) % es)
    return fail(FA_ERR_INVALID, "x and y must be aligned to their element size");
  return FA_OK;
}

// Whether every row of x and y starts 16-byte aligned (16-byte accesses).
bool rows_vec(int32_t dtype, const void *x, int64_t ld_x, const void *y, int64_t ld_y) {
  const int64_t es = elem_size(dtype);
  return aligned16(x) && aligned16(y) && (ld_x * es) % 16 == 0 && (ld_y * es) % 16 == 0;
}

bool aligned4(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 3u) == 0; }

}  // namespace

extern "C" {

fa_status_t fa_softmax_rows(int32_t dtype, int64_t rows, int64_t cols, const void *x, int64_t ld_x,
                            void *y, int64_t ld_y, float *lse, void *stream) {
  g_err[0] = 0;
  fa_status_t st;
  if ((st = check_rows(dtype, rows, cols, x, ld_x, y, ld_y)) != FA_OK) return st;
  if (lse && !aligned4(lse)) return fail(FA_ERR_INVALID, "lse is not 4-byte aligned");
  fa::RedParams a{};
  a.vec = rows_vec(dtype, x, ld_x, y, ld_y);
  a.x = x;
  a.y = y;
  a.lse = lse;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ld_x;
  a.ldy = ld_y;
  a.groups = 1;
  a.inner = 1;
  a.cpg = cols;
  return hip_status(fa::launch_softmax_rows(a, (fa_dtype_t)dtype, (hipStream_t)stream));
}

fa_status_t fa_layernorm_rows(int32_t dtype, int64_t rows, int64_t cols, const void *x, int64_t ld_x,
                              const void *gamma, const void *beta, float eps, int32_t groups,
                              int64_t inner, void *y, int64_t ld_y, float *mean, float *rstd,
                              void *stream) {
  g_err[0] = 0;
  fa_status_t st;
  if ((st = check_rows(dtype, rows, cols, x, ld_x, y, ld_y)) != FA_OK) return st;
  if (!std::isfinite(eps) || eps < 0.f) return fail(FA_ERR_INVALID, "eps must be finite and >= 0");
  if (groups < 1 || inner < 1) return fail(FA_ERR_INVALID, "groups and inner must be >= 1");
  if (cols % inner) return fail(FA_ERR_INVALID, "inner (%lld) must divide cols (%lld)", (long long)inner,
                                (long long)cols);
  if ((int64_t)groups * (cols / inner) >= (int64_t(1) << 31))
    return fail(FA_ERR_UNSUPPORTED, "groups * cols / inner (the channel count) must be < 2^31");
  const uintptr_t es = (uintptr_t)elem_size(dtype);
  if ((gamma && (reinterpret_cast<uintptr_t>(gamma) % es)) ||
      (beta && (reinterpret_cast<uintptr_t>(beta) % es)))
    return fail(FA_ERR_INVALID, "gamma and beta must be aligned to their element size");
  if ((mean && !aligned4(mean)) || (rstd && !aligned4(rstd)))
    return fail(FA_ERR_INVALID, "mean and rstd must be 4-byte aligned");
  fa::RedParams a{};
  a.vec = rows_vec(dtype, x, ld_x, y, ld_y);
  a.gvec = (!gamma || aligned16(gamma)) && (!beta || aligned16(beta));
  a.x = x;
  a.y = y;
  a.gamma = gamma;
  a.beta = beta;
  a.mean = mean;
  a.rstd = rstd;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ld_x;
  a.ldy = ld_y;
  a.eps = eps;
  a.groups = groups;
  a.inner = inner;
  a.cpg = cols / inner;
  return hip_status(fa::launch_layernorm_rows(a, (fa_dtype_t)dtype, (hipStream_t)stream));
}

const char *fa_status_string(fa_status_t status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID: return "FA_ERR_INVALID: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: configuration not built";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
  }
  return "unknown fa_status_t";
}

const char *fa_last_error(void) { return g_err; }

int32_t fa_abi_version(void) { return FA_ABI_VERSION; }

}  // extern "C"
