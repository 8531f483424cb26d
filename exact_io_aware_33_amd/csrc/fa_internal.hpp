// Host/device parameter blocks and the launcher interface between the C ABI
// (fa_api.cpp) and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

constexpr float kLog2eHost = 1.4426950408889634f;

// Everything a kernel needs, by value (one kernel argument).
struct AttnParams {
  const void *q, *k, *v;
  void *o;
  float *lse;
  // backward only
  const void *o_in;   // forward output, read by the preprocess kernel
  const void *dout;
  void *dq, *dk, *dv;
  float *ws_negd;     // [B*H*N]  -D = -rowsum(dO * O)
  float *ws_lse2;     // [B*H*N]  LSE * log2(e); +inf for rows that see no key
  // problem
  int32_t B, H, Nq, Nk, d;   // N_q queries, N_k keys
  int64_t sb, sh, sn;        // element strides of Q, O, dO, dQ ([B,H,N_q,d])
  int64_t ksb, ksh, ksn;     // element strides of K, V, dK, dV ([B,H,N_k,d])
  int32_t cshift;            // N_k - N_q: causal rule j <= i + cshift
  float scale;               // softmax scale
  float scale_log2;          // scale * log2(e)
  int32_t causal;
  const int32_t *key_lens;   // device [B] or nullptr
  // block sparsity
  const uint8_t *mask;       // device [N_q/mb, N_k/mb] (+ head stride) or nullptr
  int32_t mb;                // block size (multiple of 128)
  int32_t nblk_q, nblk_k;    // N_q / mb, N_k / mb
  int64_t mask_hstride;      // bytes between heads' masks (0 = shared)
  // dropout (Philox4x32-10 keep decisions); drop_thr == 0: none
  uint32_t drop_thr;         // t: an element whose decision byte is < t is dropped
  float drop_scale;          // 256 / (256 - t), the factor of kept elements
  uint32_t drop_key0, drop_key1;  // Philox key (seed low, high word)
  uint32_t drop_offset;      // fourth counter word
  // split-KV forward: nsplit > 0 ranges of key tiles per query tile, each
  // writing an fp32 partial (O_s normalised by its own sum, LSE_s)
  int32_t nsplit;
  float *part_o;             // [nsplit][B*H*N_q][d]
  float *part_lse;           // [nsplit][B*H*N_q]
  // forward: queries per workgroup (64, 128 or 256); 128 for the other kernels
  int32_t qtile;
  // backward: the dQ pass computes -D and LSE*log2(e) of its own queries (in
  // the preprocessing kernel's arithmetic) and writes them to the workspace,
  // instead of reading what the preprocessing kernel wrote
  int32_t dq_pre;
  // workgroups of the launched kernel resident on one CU at a time (set by
  // the launcher from the occupancy query): tile_of deals the first that many
  // passes of each XCD's tile list in alternating direction
  int32_t cu_fill;
};

// Workgroups of kernel `fn` (`threads` per workgroup, static LDS only) that one
// CU holds at a time, queried once per kernel; 1 if the query fails.
inline int resident_per_cu(const void *fn, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

// Merge of partial results over disjoint key sets (fa_merge.hip): part s is
// (o_parts[s], lse_parts[s]); O and every O_s share the strides (sb, sh, sn).
struct MergeParams {
  const void *o_parts[FA_MERGE_MAX_PARTS];
  const float *lse_parts[FA_MERGE_MAX_PARTS];
  void *o;
  float *lse;
  int32_t B, H, Nq, d, S;
  int64_t sb, sh, sn;
};
hipError_t launch_merge(const MergeParams &p, fa_dtype_t dt, hipStream_t s);

// Row reductions (fa_reduce.hip): softmax, LayerNorm / GroupNorm.
struct RedParams {
  const void *x;
  void *y;
  const void *gamma, *beta;  // dtype [channels] or nullptr
  float *lse, *mean, *rstd;  // fp32 [rows] outputs or nullptr
  int64_t rows, cols, ldx, ldy;
  float eps;
  int64_t groups, inner, cpg;  // channel of element e of row r: (r % groups) * cpg + e / inner
  bool vec;   // x and y rows start 16-byte aligned: 16-byte accesses
  bool gvec;  // gamma and beta start 16-byte aligned
};
hipError_t launch_softmax_rows(const RedParams &p, fa_dtype_t dt, hipStream_t s);
hipError_t launch_layernorm_rows(const RedParams &p, fa_dtype_t dt, hipStream_t s);

// Launchers (defined in fa_fwd.hip / fa_bwd.hip).  They assume validated
// arguments and return hipSuccess or the launch error.
hipError_t launch_fwd(const AttnParams &p, fa_dtype_t dt, bool sparse, hipStream_t s);
// Split-KV forward: p.nsplit ranges per query tile into p.part_o / p.part_lse,
// then the merge into p.o / p.lse.
hipError_t launch_fwd_splitkv(const AttnParams &p, fa_dtype_t dt, bool sparse, hipStream_t s);
// Key tiles per forward tile for a dtype (the unit a split range is made of).
int fwd_key_tile(fa_dtype_t dt);
// `stages`: bit set of FA_BWD_PRE / FA_BWD_MAIN / FA_BWD_DQ, run in that order.
hipError_t launch_bwd(const AttnParams &p, fa_dtype_t dt, bool sparse, unsigned stages,
                      hipStream_t s);

// Records a message for fa_last_error() and returns `st`.
fa_status_t set_error(fa_status_t st, const char *fmt, ...);

// Supplies the backward workspace of at least `need` bytes when the caller
// passes none (the allocation-free entry point): sets *ws and *bytes or
// returns an error status (with set_error).
typedef fa_status_t (*ScratchFn)(size_t need, void **ws, size_t *bytes);

// Argument checks and the backward launch sequence shared by every backward
// entry point (fa_api.cpp).  With `scratch` non-null, `ws` / `ws_bytes` are
// ignored and the workspace comes from scratch() after all other checks.
fa_status_t bwd_impl(const fa_problem_t *p, const uint8_t *mask, int32_t mb, int64_t hstride,
                     bool sparse, const void *q, const void *k, const void *v, const void *o,
                     const float *lse, const void *dout, void *dq, void *dk, void *dv, void *ws,
                     size_t ws_bytes, unsigned stages, void *stream, ScratchFn scratch);

// Backward workspace: two floats per query row, each array 256-byte aligned:
// -D = -rowsum(dO * O), then LSE in the base-2 domain.
inline size_t ws_array_bytes(int64_t rows) { return (size_t)((rows * 4 + 255) / 256 * 256); }
inline size_t ws_total_bytes(int64_t rows) { return 2 * ws_array_bytes(rows); }

// Split-KV workspace: fp32 partial outputs [S][rows][d], then partial LSE
// [S][rows], each 256-byte aligned.
inline size_t splitkv_o_bytes(int64_t rows, int d, int splits) {
  return (size_t)(((int64_t)splits * rows * d * 4 + 255) / 256 * 256);
}
inline size_t splitkv_total_bytes(int64_t rows, int d, int splits) {
  return splitkv_o_bytes(rows, d, splits) + (size_t)(((int64_t)splits * rows * 4 + 255) / 256 * 256);
}

}  // namespace fa
