// Dropout keep decisions, generated inside the attention kernels.
//
// The FlashAttention summary page (paper 2205.14135), section "Key ideas",
// kernel-fusion bullet, counts dropout among the steps fused into the one
// attention kernel; the page fixes no generator.  Here the decisions are a
// pure function of (seed, offset, batch*H + head, query, key), so the backward
// pass regenerates exactly the forward's mask instead of storing it.  The
// generator is Philox4x32-10 as defined by Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3" (SC'11): a four-word counter,
// a two-word key, ten rounds of two 32x32->64-bit products, the key bumped by
// two Weyl constants between rounds.  One call covers an aligned 4x4 block of
// the (query, key) plane: counter (i/4, j/4, head, offset), word w <-> query
// 4(i/4) + w, byte k of a word <-> key 4(j/4) + k; an element is kept iff its
// byte is >= t (t = round(256 p)).
//
// Lane mapping.  A 32x32 MFMA accumulator gives each lane one column (the
// lane's query in the forward and dQ kernels, the lane's key in the dK/dV
// kernel) and, for g = 0..3, the four consecutive rows 8g + 4h + 0..3 (h =
// half-wave).  So one 4x4 Philox block is spread over the four lanes of a quad
// (lanes 4a..4a+3), one column each, and every lane needs four blocks per
// 32x32 tile.  Each lane of the quad generates a different one of the quad's
// four blocks and a transpose across the quad (three DPP moves) gives every
// lane its own column of all four: one Philox call per lane per 32x32 tile.
#pragma once

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

// Round r (or rounds R0 .. R1-1) of Philox4x32-10 on the counter c, (k0, k1)
// being the key of round 0 (round r uses it bumped r times by the Weyl
// constants).  Split so that a kernel can spread one generator call over
// several groups of matrix instructions.
// (r is a constant wherever the caller's loop is unrolled, and so are the
// round keys' increments.)
__device__ __forceinline__ void philox_round(uint32_t (&c)[4], uint32_t k0, uint32_t k1, int r) {
  k0 += (uint32_t)r * 0x9E3779B9u;
  k1 += (uint32_t)r * 0xBB67AE85u;
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
  const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
  c[1] = (uint32_t)p1;
  c[3] = (uint32_t)p0;
  c[0] = n0;
  c[2] = n2;
}
template <int R0, int R1>
__device__ __forceinline__ void philox_rounds(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = R0; r < R1; ++r) philox_round(c, k0, k1, r);
}
constexpr int kPhiloxRounds = 10;

// Philox4x32-10 on the counter c under key (k0, k1); c is replaced by the
// four output words.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
  philox_rounds<0, kPhiloxRounds>(c, k0, k1);
}

// Value of x held by quad lane (own ^ X), X = 1, 2, 3 (DPP quad_perm).
template <int X>
__device__ __forceinline__ uint32_t quad_xor(uint32_t x) {
  constexpr int ctrl = X == 1 ? 0xB1 : (X == 2 ? 0x4E : 0x1B);  // [1,0,3,2] [2,3,0,1] [3,2,1,0]
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, ctrl, 0xF, 0xF, false);
}

// y[k] = x[k ^ w] for this lane's quad index w (two conditional pair swaps).
__device__ __forceinline__ void xor_permute(uint32_t (&x)[4], int w) {
  const bool b0 = w & 1, b1 = w & 2;
  const uint32_t t0 = b0 ? x[1] : x[0], t1 = b0 ? x[0] : x[1];
  const uint32_t t2 = b0 ? x[3] : x[2], t3 = b0 ? x[2] : x[3];
  x[0] = b1 ? t2 : t0;
  x[1] = b1 ? t3 : t1;
  x[2] = b1 ? t0 : t2;
  x[3] = b1 ? t1 : t3;
}

// Transpose across the quad: quad lane w enters with x = the four words of
// block w and leaves with x[g] = word w of block g.  (After xor_permute, lane
// g sends its word (g ^ k) to lane g ^ k in exchange k; a second xor_permute
// puts the received words back in block order.)
__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int lane) {
  const int w = lane & 3;
  xor_permute(x, w);
  x[1] = quad_xor<1>(x[1]);
  x[2] = quad_xor<2>(x[2]);
  x[3] = quad_xor<3>(x[3]);
  xor_permute(x, w);
}

// Byte transpose of four words: byte u of the result x[k] is byte k of x[u].
__device__ __forceinline__ void byte_transpose(uint32_t (&x)[4]) {
  const uint32_t lo01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
  const uint32_t hi01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
  const uint32_t lo23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  x[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
  x[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  x[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  x[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// Decision bytes of a 32x32 tile whose column (lane) is query qi and whose
// rows are the keys kb + reg_row(r, h) (forward, dQ kernels; kb a multiple of
// 32, qi = lane mod 4): on return byte k of x[g] decides register 4g + k.
// In stages: the counter (keep_ctr_query_col), the ten rounds
// (philox_rounds), the exchange across the quad (keep_finish_query_col).
__device__ __forceinline__ void keep_ctr_query_col(uint32_t (&x)[4], const AttnParams &p, int bh, int qi,
                                                   int kb, int lane) {
  const int w = lane & 3, h = (lane >> 5) & 1;
  x[0] = (uint32_t)qi >> 2;
  x[1] = (uint32_t)((kb >> 2) + 2 * w + h);  // quad lane w: keys kb + 8w + 4h + 0..3
  x[2] = (uint32_t)bh;
  x[3] = p.drop_offset;
}
__device__ __forceinline__ void keep_finish_query_col(uint32_t (&x)[4], int lane) { quad_transpose(x, lane); }
__device__ __forceinline__ void keep_bytes_query_col(uint32_t (&x)[4], const AttnParams &p, int bh,
                                                     int qi, int kb, int lane) {
  keep_ctr_query_col(x, p, bh, qi, kb, lane);
  philox4x32_10(x, p.drop_key0, p.drop_key1);
  keep_finish_query_col(x, lane);
}

// Decision bytes of a 32x32 tile whose column (lane) is key `key` and whose
// rows are the queries q0 + reg_row(r, h) (dK/dV kernel; q0 a multiple of 32,
// key = lane mod 4): on return byte k of x[g] decides register 4g + k.
// Stages as for keep_bytes_query_col.
__device__ __forceinline__ void keep_ctr_key_col(uint32_t (&x)[4], const AttnParams &p, int bh, int q0,
                                                 int key, int lane) {
  const int w = lane & 3, h = (lane >> 5) & 1;
  x[0] = (uint32_t)((q0 >> 2) + 2 * w + h);  // quad lane w: queries q0 + 8w + 4h + 0..3
  x[1] = (uint32_t)key >> 2;
  x[2] = (uint32_t)bh;
  x[3] = p.drop_offset;
}
__device__ __forceinline__ void keep_finish_key_col(uint32_t (&x)[4], int lane) {
  byte_transpose(x);  // x[k] byte u: query 4 G + u, key 4 (key / 4) + k
  quad_transpose(x, lane);
}
__device__ __forceinline__ void keep_bytes_key_col(uint32_t (&x)[4], const AttnParams &p, int bh,
                                                   int q0, int key, int lane) {
  keep_ctr_key_col(x, p, bh, q0, key, lane);
  philox4x32_10(x, p.drop_key0, p.drop_key1);
  keep_finish_key_col(x, lane);
}

// Whether register r of the tile is kept.
__device__ __forceinline__ bool kept(const uint32_t (&x)[4], int r, uint32_t thr) {
  return ((x[r >> 2] >> (8 * (r & 3))) & 0xFFu) >= thr;
}

// Keep mask of the packed 16-bit pair (registers r, r + 1; r even): 0xFFFF in
// each half whose element is kept.  add = (0x8000 - t) * 0x10001: the two
// decision bytes, spread to the two halves, reach bit 15 / 31 iff >= t, and
// v_perm's sign-replicating selectors (8, 9) widen those bits to the halves.
__device__ __forceinline__ uint32_t keep_mask_pair(const uint32_t (&x)[4], int r, uint32_t add) {
  const uint32_t e = __builtin_amdgcn_perm(0u, x[r >> 2], (r & 2) ? 0x0c030c02u : 0x0c010c00u);
  return __builtin_amdgcn_perm(0u, e + add, 0x09090808u);
}

__host__ __device__ constexpr uint32_t keep_pair_add(uint32_t thr) { return (0x8000u - thr) * 0x10001u; }

// MFMA operand `f` (registers first .. first + KPL - 1 of the tile) with the
// dropped elements zeroed.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag drop_frag(typename Mma<T>::frag f, const uint32_t (&x)[4],
                                                           int first, uint32_t thr, uint32_t add) {
  if constexpr (Mma<T>::KPL == 1) {
    return kept(x, first, thr) ? f : 0.f;
  } else {
    u32x4 u = __builtin_bit_cast(u32x4, f);
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] &= keep_mask_pair(x, first + 2 * q, add);
    return __builtin_bit_cast(typename Mma<T>::frag, u);
  }
}

}  // namespace fa
