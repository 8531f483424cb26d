/*
 * fa.h -- C ABI of libfa: exact, tiled scaled-dot-product attention for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (FlashAttention summary page, paper 2205.14135, section
 * "Problem and motivation"): for every batch b and head h,
 *     S = scale * Q K^T,   P = softmax(S) row by row,   O = P V,
 * with Q, O in R^{N_q x d} and K, V in R^{N_k x d} (N_q = N_k for
 * self-attention; N_q != N_k for cross-attention and decoding).  The score matrix S and the probabilities P
 * never reach device memory: they live in registers one tile at a time
 * (same page, "Key ideas": tiling and recomputation; section "Incremental
 * softmax tracking": the running max / running sum update).
 *
 * Masking (same page, "Key ideas", kernel-fusion bullet names masking; section
 * "Block-Sparse FlashAttention" defines the block mask).  Key j is visible to
 * query i iff every active rule allows it:
 *   causal      : j <= i + N_k - N_q           (fa_problem_t.causal != 0; the
 *                                               queries are the last N_q
 *                                               positions of the key sequence,
 *                                               so j <= i when N_q = N_k)
 *   key padding : j < key_lens[b]              (fa_problem_t.key_lens != NULL;
 *                                               values are clamped to [0, N_k])
 *   block mask  : M[i / mb][j / mb] != 0        (the *_blocksparse entry points)
 * A query row with no visible key gets O = 0, LSE = -inf and zero gradients.
 *
 * Dropout (same page, "Key ideas", kernel-fusion bullet: dropout is one of
 * the steps fused into the attention kernel; the page fixes no generator).
 * With dropout_p > 0 the forward computes O = (P o Z) V, where Z_ij is 0
 * (dropped) or 1 / (1 - t/256) (kept) and t = round-half-even(256 p),
 * clamped to [0, 255], computed in double from the float field.  The keep
 * decisions come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC'11) with
 *     key     = (dropout_seed mod 2^32, dropout_seed div 2^32),
 *     counter = (i / 4, j / 4, b * H + h, dropout_offset):
 * output word w of that call decides query 4 (i / 4) + w, its byte k
 * (bits 8k .. 8k+7) key 4 (j / 4) + k, and the element is kept iff that
 * byte >= t.  The decisions are a function of (seed, offset, b, h, i, j)
 * only: the backward pass regenerates them instead of storing Z, and its
 * gradients are those of <dO, (P o Z) V> with Z held fixed.  LSE is the
 * statistics of P, unaffected by dropout.
 *
 * Saved statistics: the forward pass writes LSE_i = m_i + ln(l_i), the natural
 * log-sum-exp of the scaled, masked score row i (the summary page keeps (l, m)
 * for the backward pass; LSE carries the same information, P = exp(S - LSE)).
 *
 * Backward: the gradients of <dO, O> with respect to Q, K and V, computed by
 * recomputing S and P tile by tile from Q, K, V, O and LSE (summary page,
 * "Key ideas", recomputation bullet).  The gradient formulas themselves are
 * the analytic derivatives of the definition above.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Q, O, dO, dQ are [B, H, N_q, d] arrays of the problem's dtype with
 *   element strides (stride_b, stride_h, stride_n); K, V, dK, dV are
 *   [B, H, N_k, d] arrays with strides (k_stride_b, k_stride_h, k_stride_n)
 *   (all three 0: the Q strides); unit stride along d.  LSE is a contiguous
 *   float32 [B, H, N_q].  A contiguous [B, H, N, d] array has strides
 *   (H*N*d, N*d, d); a [B, N, H, d] array has (N*H*d, d, H*d).
 * Memory.  Every data pointer is a DEVICE pointer owned by the caller; the
 *   library never allocates, frees or keeps device memory between calls and
 *   holds no state, so concurrent calls on different streams are safe.  (The
 *   first launch of each kernel variant in a process also asks the runtime,
 *   once, how many of its workgroups one CU holds: a host-side query that
 *   enqueues nothing, used only to order the tiles.)
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *   enqueue work and return; the caller synchronises before reading results
 *   and keeps every buffer alive until then.
 * Alignment.  Q, K, V, O, dO, dQ, dK, dV must be 16-byte aligned and all six
 *   strides multiples of 16 bytes; LSE, key_lens and the workspace 16-byte
 *   aligned (the kernels move 16-byte vectors).  A NULL pointer is
 *   FA_ERR_INVALID; a misaligned pointer or stride is FA_ERR_UNSUPPORTED.
 * Errors.  Argument errors are detected on the host before any HIP call and
 *   returned synchronously (FA_ERR_INVALID, FA_ERR_UNSUPPORTED); a failed
 *   launch returns FA_ERR_HIP.  Faults during execution surface at the
 *   caller's next synchronisation, as usual for HIP.  Nothing aborts or throws
 *   across this boundary.  fa_last_error() gives a message for the last failed
 *   call on the calling thread.
 * Supported shapes.  dtype FP16 or BF16 with d in {64, 128}; dtype FP32 with
 *   d in {64, 128}.  N_q, N_k >= 1 (any values, not only multiples of the
 *   tile), B >= 1, H >= 1, B*H*N*d < 2^31 for N = N_q and N = N_k.  scale
 *   finite and >= 0.  The kernels address the rows of one (batch, head)
 *   slice with 32-bit byte offsets from its first row, tiles overrunning the
 *   end by up to 256 rows (read as zeros), so
 *       (N_q + 256) * stride_n * element size   < 2^31  and
 *       (N_k + 256) * k_stride_n * element size < 2^31
 *   (FA_ERR_UNSUPPORTED otherwise; e.g. [B, N, H, d] storage with
 *   N * H * d * element size near 2 GiB).
 */
#ifndef EXACT_IO_AWARE_FA_H
#define EXACT_IO_AWARE_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 4

typedef enum fa_dtype {
  FA_DTYPE_F32 = 0,   /* IEEE float32 storage, float32 arithmetic            */
  FA_DTYPE_F16 = 1,   /* IEEE float16 storage, float32 accumulation          */
  FA_DTYPE_BF16 = 2   /* bfloat16 storage, float32 accumulation              */
} fa_dtype_t;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID = 1,      /* bad argument: NULL pointer, size <= 0, non-finite
                              or negative scale, dropout_p outside [0, 1),
                              workspace too small, block size that does not
                              divide N_q and N_k, row stride below head_dim,
                              fwd_query_tile not 0, 64, 128 or 256           */
  FA_ERR_UNSUPPORTED = 2,  /* well-formed but not built: head_dim / dtype pair,
                              block size not a multiple of 128, a query tile
                              not built for the dtype / mask, a pointer or
                              stride that is not 16-byte aligned, sizes over
                              the 32-bit index / byte-offset ranges           */
  FA_ERR_HIP = 3           /* the HIP runtime refused a launch                 */
} fa_status_t;

/* One attention problem.  Shared by the forward and backward entry points. */
typedef struct fa_problem {
  int32_t batch;            /* B >= 1                                          */
  int32_t heads;            /* H >= 1                                          */
  int32_t seqlen;           /* N_q >= 1: number of queries (and of keys unless
                               seqlen_k is set)                               */
  int32_t head_dim;         /* d: 64 or 128                                    */
  int64_t stride_b;         /* Q, O, dO, dQ: element stride between batches    */
  int64_t stride_h;         /*   ... between heads                            */
  int64_t stride_n;         /*   ... between rows (tokens)                    */
  float scale;              /* S = scale * Q K^T; finite, >= 0 (1/sqrt(d) usual) */
  int32_t causal;           /* nonzero: key j visible to query i only if j <= i */
  int32_t dtype;            /* fa_dtype_t                                      */
  const int32_t *key_lens;  /* device int32 [B] or NULL (no padding): keys
                               j >= key_lens[b] are masked for every query and
                               head of batch b; clamped to [0, N_k] on device  */
  float dropout_p;          /* probability of dropping an element of P, in
                               [0, 1); 0 = no dropout (then the two fields
                               below are ignored)                             */
  uint32_t dropout_offset;  /* fourth Philox counter word (e.g. a step count) */
  uint64_t dropout_seed;    /* Philox key                                     */
  int32_t seqlen_k;         /* N_k: number of keys; 0 = N_q                    */
  int32_t fwd_query_tile;   /* queries per forward workgroup, B_r: 0 = the
                               library's choice (128), or 64, 128 or 256 (64
                               and 256 for FP16 / BF16 without dropout; 256
                               not with a block mask).  Read by fa_fwd and
                               fa_fwd_blocksparse (the K / V tiles streamed
                               through on-chip memory serve B_r queries, so
                               re-reads of K and V scale as 1 / B_r); every
                               other entry point requires 0 or ignores it    */
  int64_t k_stride_b;       /* K, V, dK, dV: element stride between batches;
                               all three k_stride_* 0 = the Q strides         */
  int64_t k_stride_h;       /*   ... between heads                            */
  int64_t k_stride_n;       /*   ... between rows (keys)                      */
} fa_problem_t;

/* Forward pass (summary page, "Incremental softmax tracking", steps 1-4).
 *   q       : device [B,H,N_q,d] input (dtype), read only.
 *   k, v    : device [B,H,N_k,d] inputs (dtype), read only.
 *   o       : device [B,H,N_q,d] output (dtype), written in full (rows of
 *             fully masked queries are written as zeros).
 *   lse     : device float32 [B,H,N_q] output, contiguous, written in full.
 * Returns FA_OK once the work is enqueued on `stream`. */
fa_status_t fa_fwd(const fa_problem_t *p, const void *q, const void *k,
                   const void *v, void *o, float *lse, void *stream);

/* Block-sparse forward (summary page, section "Block-Sparse FlashAttention":
 * only the nonzero blocks of M in {0,1}^{N_q/mb x N_k/mb} are evaluated).
 *   block_mask       : device uint8 [N_q/mb, N_k/mb], row-major (row = query
 *                      block, column = key block); nonzero = evaluate.
 *   mask_block       : mb, a positive multiple of 128 that divides N_q and N_k.
 *   mask_head_stride : bytes between the masks of consecutive heads, or 0 for
 *                      one mask shared by all heads (the mask of head h is at
 *                      block_mask + h * mask_head_stride; one per head, shared
 *                      by all batches).
 * The other arguments and the causal / key_lens fields act as in fa_fwd; all
 * active masks are combined with AND.  N_q / mb and N_k / mb must not exceed
 * 1024. */
fa_status_t fa_fwd_blocksparse(const fa_problem_t *p, const uint8_t *block_mask,
                               int32_t mask_block, int64_t mask_head_stride,
                               const void *q, const void *k, const void *v,
                               void *o, float *lse, void *stream);

/* Split-KV forward, for decoding and other shapes with few query tiles per
 * (batch, head) and many keys: the key tiles each 128-query tile sees are cut
 * into num_splits contiguous ranges, one workgroup each, so that the launch
 * fills the GPU; every range leaves a partial output (divided by its own
 * exponential sum) and a partial LSE in fp32, and a merge kernel combines
 * them with the summary page's merge equation (section "Incremental softmax
 * tracking") in log-sum-exp form:
 *     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 * The result is the one fa_fwd / fa_fwd_blocksparse computes (up to rounding).
 *   block_mask       : NULL for the dense path, else as for fa_fwd_blocksparse
 *                      (mask_block, mask_head_stride as there).
 *   num_splits       : 1..1024, or <= 0 for the library's choice
 *                      (fa_fwd_splitkv_num_splits); more ranges than key tiles
 *                      leave some ranges empty (they weigh 0 in the merge).
 *   workspace        : device scratch of at least
 *                      fa_fwd_splitkv_workspace_bytes(p, num_splits) bytes,
 *                      caller-owned, contents on entry ignored, not shared with
 *                      a concurrent call.
 * Other arguments as for fa_fwd.  Dropout is not built for this path
 * (dropout_p that rounds to t > 0 gives FA_ERR_UNSUPPORTED). */
int32_t fa_fwd_splitkv_num_splits(const fa_problem_t *p);  /* >= 1; 0 if p is invalid */
size_t fa_fwd_splitkv_workspace_bytes(const fa_problem_t *p, int32_t num_splits); /* 0 if invalid */
fa_status_t fa_fwd_splitkv(const fa_problem_t *p, const uint8_t *block_mask, int32_t mask_block,
                           int64_t mask_head_stride, int32_t num_splits, const void *q,
                           const void *k, const void *v, void *o, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Merge of partial results over disjoint key sets (summary page, section
 * "Incremental softmax tracking": the merge equation, here in log-sum-exp
 * form, since each part's output is already divided by its own sum):
 *     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 * Part s is what fa_fwd / fa_fwd_blocksparse return for the queries against
 * the s-th of S disjoint subsets of the keys -- the per-hop result of
 * context-parallel (ring) attention, where K / V shards visit each query
 * shard in turn (same page, "Limitations and open questions": attention
 * across devices is left open there).  The merged (O, LSE) is the forward
 * result over the union of the key sets, and is what fa_bwd needs, per
 * shard, for that shard's exact dK, dV and its share of dQ (the shares sum
 * to dQ).
 *   p          : the problem of the queries; batch, heads, seqlen (N_q),
 *                head_dim, stride_b / _h / _n and dtype are used (all other
 *                fields are checked as for fa_fwd and otherwise ignored).
 *   num_parts  : S, 1 <= S <= FA_MERGE_MAX_PARTS.
 *   o_parts    : HOST array of S device pointers; o_parts[s] is an
 *                [B,H,N_q,d] array of dtype with p's strides (read only).
 *   lse_parts  : HOST array of S device pointers; lse_parts[s] is a
 *                contiguous float32 [B,H,N_q] array (read only).  A part with
 *                LSE_s = -inf (it saw no key) weighs 0, whatever its O_s.
 *   o, lse     : outputs, laid out as the parts; o may be the same memory as
 *                any o_parts[s], lse as any lse_parts[s] (in-place merge).
 *                A row no part saw gets O = 0, LSE = -inf.
 * Arithmetic in fp32; O is rounded to dtype once.  Nothing is allocated:
 * the S pointers travel in the kernel's arguments. */
#define FA_MERGE_MAX_PARTS 64
fa_status_t fa_merge_partials(const fa_problem_t *p, int32_t num_parts,
                              const void *const *o_parts,
                              const float *const *lse_parts, void *o,
                              float *lse, void *stream);

/* Size in bytes of the device workspace fa_bwd needs for problem p (0 if p is
 * invalid).  It holds two float32 per query row (B*H*N_q rows): rowsum(dO * O)
 * and the saved LSE rescaled to base 2, O(N) extra memory (summary page,
 * "Complexity analysis": O(N) beyond inputs and outputs). */
size_t fa_bwd_workspace_bytes(const fa_problem_t *p);

/* Backward pass: gradients of <dO, O> (summary page, "Key ideas",
 * recomputation bullet: S and P are rebuilt per tile from Q, K, V, O, LSE).
 *   q, k, v, o : the forward's inputs and output (dtype), read only.
 *   lse        : the forward's float32 [B,H,N_q] statistics, read only.
 *   dout       : device [B,H,N_q,d] upstream gradient dO (dtype), read only.
 *   dq         : device [B,H,N_q,d] output (dtype), written in full.
 *   dk, dv     : device [B,H,N_k,d] outputs (dtype), written in full.
 *   workspace  : device scratch of at least fa_bwd_workspace_bytes(p) bytes,
 *                owned by the caller, contents on entry ignored; it must not
 *                be shared with a concurrently running call.
 * The mask and dropout fields of p must equal those used for the forward
 * pass. */
fa_status_t fa_bwd(const fa_problem_t *p, const void *q, const void *k,
                   const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Block-sparse backward: fa_bwd restricted to the nonzero blocks of the mask,
 * whose arguments mean what they mean for fa_fwd_blocksparse.  Keys that no
 * query sees get dK = dV = 0. */
fa_status_t fa_bwd_blocksparse(const fa_problem_t *p, const uint8_t *block_mask,
                               int32_t mask_block, int64_t mask_head_stride,
                               const void *q, const void *k, const void *v,
                               const void *o, const float *lse,
                               const void *dout, void *dq, void *dk, void *dv,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/* Stages of the backward launch sequence (bit set for fa_bwd_ex). */
typedef enum fa_bwd_stage {
  FA_BWD_PRE = 1,    /* D = rowsum(dO * O) and LSE*log2(e) into the workspace */
  FA_BWD_MAIN = 2,   /* key-stationary pass: recompute S, P per tile; write
                        dK, dV (reads the workspace)                         */
  FA_BWD_DQ = 4,     /* query-stationary pass: recompute S, P per tile; write
                        dQ (reads the workspace, or fills it when PRE is in
                        the same call; independent of FA_BWD_MAIN)           */
  FA_BWD_ALL = 7
} fa_bwd_stage_t;

/* fa_bwd / fa_bwd_blocksparse with the launch sequence split into stages, so
 * a caller can time a stage on its own or put other work between stages.
 * block_mask == NULL selects the dense path (mask_block, mask_head_stride
 * ignored); otherwise the arguments mean what they mean for
 * fa_bwd_blocksparse.  `stages` is a nonzero subset of FA_BWD_ALL.  When it
 * holds both PRE and DQ, the dQ pass does the preprocessing of its own
 * queries (bitwise the values the PRE stage writes) and fills the workspace,
 * with no separate preprocessing launch, and MAIN, if named, runs after it;
 * otherwise the named stages run in the order PRE, MAIN, DQ.  So FA_BWD_ALL
 * launches two kernels (dQ, then dK/dV), and PRE | DQ followed by MAIN is
 * the same sequence in two calls.  Calling with PRE, then MAIN, then DQ (or
 * DQ before MAIN) on one stream, with the same workspace, gives exactly the
 * result of one call with FA_BWD_ALL; MAIN and DQ may also run concurrently
 * (on two streams) once PRE has completed.  Arguments a stage does not read
 * are still checked. */
fa_status_t fa_bwd_ex(const fa_problem_t *p, const uint8_t *block_mask,
                      int32_t mask_block, int64_t mask_head_stride,
                      const void *q, const void *k, const void *v,
                      const void *o, const float *lse, const void *dout,
                      void *dq, void *dk, void *dv, void *workspace,
                      size_t workspace_bytes, uint32_t stages, void *stream);

/* Allocation-free backward, for callers that cannot allocate device memory
 * or be handed a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Computes exactly what fa_bwd_ex
 * with FA_BWD_ALL computes (same kernels, same results; block_mask NULL = the
 * dense path, otherwise as for fa_bwd_blocksparse), but its workspace is a
 * fixed device array inside the library, of
 * FA_BWD_NOALLOC_MAX_WORKSPACE_BYTES, which every GPU the library runs on
 * holds from its first call until the process ends.  The call allocates,
 * frees and memsets nothing (the workspace needs no clearing: the first
 * backward kernel writes all of it that the others read).
 *   - The device is the one current on the calling thread; `stream` must
 *     belong to it.  The first call on a device looks up the array's address
 *     there (hipGetSymbolAddress), later calls reuse it.
 *   - Problems whose workspace (fa_bwd_workspace_bytes: two floats per query
 *     row, B*H*N_q rows) exceeds the array get FA_ERR_UNSUPPORTED before
 *     any HIP call.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on the same GPU (on other streams, from other threads) race and
 *     give wrong gradients.  Calls ordered on one stream are safe.
 * Other arguments and errors as for fa_bwd_ex. */
#define FA_BWD_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)16 << 20)
fa_status_t fa_bwd_noalloc(const fa_problem_t *p, const uint8_t *block_mask,
                           int32_t mask_block, int64_t mask_head_stride,
                           const void *q, const void *k, const void *v,
                           const void *o, const float *lse, const void *dout,
                           void *dq, void *dk, void *dv, void *stream);

/* ---------------------------------------------------------------------------
 * Other streaming reductions (math-properties page, section 8: softmax-based
 * routing and gating, LayerNorm and GroupNorm have attention's structure, a
 * finite state updated block by block).  Row-wise over a [rows, cols] matrix
 * of the given dtype whose rows start ld elements apart (ld >= cols; pointers
 * aligned to the element size; rows that start 16-byte aligned are read and
 * written 16 bytes at a time, others element by element); y may equal x.
 * Device pointers, caller-owned; errors as for the attention entry points. */

/* y = softmax(x) per row: y_j = exp(x_j - m) / l, m = max_j x_j,
 * l = sum_j exp(x_j - m); lse (fp32 [rows], may be NULL) = m + ln l.  A row
 * whose entries are all -inf gets y = 0 and lse = -inf.  The per-thread state
 * (m, l) is merged across threads with the summary page's merge equation. */
fa_status_t fa_softmax_rows(int32_t dtype, int64_t rows, int64_t cols, const void *x,
                            int64_t ld_x, void *y, int64_t ld_y, float *lse, void *stream);

/* LayerNorm / GroupNorm per row: mean = sum x / n, var = sum (x - mean)^2 / n,
 * rstd = 1 / sqrt(var + eps), y_e = (x_e - mean) rstd gamma[c] + beta[c] with
 * channel c = (row % groups) * (cols / inner) + e / inner.  LayerNorm:
 * groups = 1, inner = 1 (c = e, gamma / beta of cols entries).  GroupNorm of
 * an [N, C, S] input with G groups: rows = N G, cols = (C / G) S, groups = G,
 * inner = S, gamma / beta of C entries.  gamma, beta: dtype, may be NULL
 * (scale 1, shift 0); mean, rstd: fp32 [rows] outputs, may be NULL.  eps
 * finite and >= 0; inner must divide cols; the channel count groups * cols /
 * inner must be < 2^31 (FA_ERR_UNSUPPORTED otherwise).  The per-thread state
 * (n, mean, M2) is merged with the Chan-Golub-LeVeque pairwise update. */
fa_status_t fa_layernorm_rows(int32_t dtype, int64_t rows, int64_t cols, const void *x,
                              int64_t ld_x, const void *gamma, const void *beta, float eps,
                              int32_t groups, int64_t inner, void *y, int64_t ld_y, float *mean,
                              float *rstd, void *stream);

/* Static description of a status code (never NULL). */
const char *fa_status_string(fa_status_t status);

/* Message describing the last failed call made by the calling thread ("" if
 * none).  The pointer stays valid until that thread's next library call. */
const char *fa_last_error(void);

/* FA_ABI_VERSION of the loaded library. */
int32_t fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_FA_H */
