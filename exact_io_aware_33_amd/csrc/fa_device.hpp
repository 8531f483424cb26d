// Device-side building blocks shared by the forward and backward kernels:
// MFMA wrappers per storage type, LDS fragment reads, cross-half-wave
// exchange, and the workgroup -> tile mapping.
//
// Matrix-core conventions used throughout (CDNA3/CDNA4 MFMA lane layouts,
// checked on gfx950 by an in-bounds probe):
//   32x32 MFMA with K = 2*KPL: lane l holds A[m = l%32][k = KPL*(l/32) + e] and
//     B[k = KPL*(l/32) + e][n = l%32], e < KPL; the 16 accumulator registers
//     hold C[8*(r/4) + 4*(l/32) + r%4][l%32], r < 16.
//   16x16 MFMA with K = 4*KPL: lane l holds A[m = l%16][k = KPL*(l/16) + e],
//     B[k = KPL*(l/16) + e][n = l%16]; accumulators C[4*(l/16) + r][l%16].
// KPL = 8 for 16-bit types (v_mfma_f32_32x32x16_{f16,bf16},
// v_mfma_f32_16x16x32_{f16,bf16}) and KPL = 1 for fp32 (32x32x2, 16x16x4).
//
// "Register order": the 32x32 accumulator register r of a lane in half h
// holds row 8*(r/4) + 4*h + r%4.  A product that contracts over those rows can
// feed the accumulator registers (converted) straight back as an MFMA operand,
// as long as its other operand enumerates the contraction index in the same
// order: step t, element e <-> register KPL*t + e.  reg_row() gives that row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Row held by accumulator register r of a lane in half-wave h (32x32 layout).
__device__ __forceinline__ constexpr int reg_row(int r, int h) {
  return 8 * (r >> 2) + 4 * h + (r & 3);
}

template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  static constexpr int KPL = 8;
  using frag = bf16x8;
  __device__ static __forceinline__ f32x16 mma32(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mma16(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<_Float16> {
  static constexpr int KPL = 8;
  using frag = f16x8;
  __device__ static __forceinline__ f32x16 mma32(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mma16(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KPL = 1;
  using frag = float;
  __device__ static __forceinline__ f32x16 mma32(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mma16(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// ---- conversions -----------------------------------------------------------
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }
template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

// Pack KPL consecutive fp32 registers (starting at element `first` of a
// 16-register accumulator) into an MFMA operand of type T.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag pack_frag(const f32x16 &acc, int first) {
  if constexpr (Mma<T>::KPL == 1) {
    return acc[first];
  } else {
    typename Mma<T>::frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (T)acc[first + e];
    return f;
  }
}

// Sum of the KPL elements of an MFMA operand, added to `acc` (v_dot2 with ones
// for 16-bit types: the sum of exactly the rounded values the MFMA consumes).
template <typename T>
__device__ __forceinline__ float frag_sum(typename Mma<T>::frag f, float acc) {
  if constexpr (Mma<T>::KPL == 1) {
    return acc + f;
  } else if constexpr (__is_same(T, __bf16)) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 v = {f[e], f[e + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(v, one, acc, false);
    }
    return acc;
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const f16x2 v = {f[e], f[e + 1]};
      acc = __builtin_amdgcn_fdot2(v, one, acc, false);
    }
    return acc;
  }
}

// ---- global memory -----------------------------------------------------------
__device__ __forceinline__ u32x4 ldg16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void stg16(void *p, u32x4 v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}

// Buffer resource over `bytes` bytes from `base` (raw buffer, stride 0):
// loads past the end return zeros, which is how rows >= N are zero-filled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes at byte offset voffset + soffset (soffset wave-uniform).
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       r, voffset, __builtin_amdgcn_readfirstlane(soffset), 0));
}

// Buffer descriptor words (base, stride 0, `bytes` records, raw addressing)
// for the LDS-DMA load below, which takes the descriptor as SGPR operands.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), (int)bytes, 0x00020000};
}
// LDS-DMA: lane i loads 16 bytes at voffset + soffset of the buffer and the
// hardware writes them to LDS byte address lds_addr + 16 i (gfx950
// buffer_load_dwordx4 with the lds bit; lds_addr goes in M0 and must be
// wave-uniform, as must soffset).  Out-of-range lanes deliver zeros.  Written
// as inline assembly so that the compiler does not make every later LDS read
// wait for it: the caller waits for the vector-memory counter (and
// synchronises the workgroup) before reading the destination.  The compiler
// does not see inside the statement, so it carries its own wait states: an
// SGPR operand may have just been written by a VALU instruction
// (v_readfirstlane), which needs 5 before a vector-memory read of it, and M0
// needs 1 before the LDS-DMA read of it.
__device__ __forceinline__ void buf_load16_lds(i32x4 rsrc, uint32_t lds_addr, int voffset, int soffset) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(soffset), "{m0}"(lds_addr)
               : "memory");
}
// The same with 4 bytes per lane (lane i -> lds_addr + 4 i).
__device__ __forceinline__ void buf_load4_lds(i32x4 rsrc, uint32_t lds_addr, int voffset, int soffset) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(soffset), "{m0}"(lds_addr)
               : "memory");
}
// s_waitcnt immediate that waits until at most n vector-memory operations of
// the wave are outstanding (other counters not waited on).
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// ---- LDS reads ---------------------------------------------------------------
// KPL contiguous elements of type T at byte offset `off` of LDS.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag lds_frag(const char *lds, int off) {
  return *reinterpret_cast<const typename Mma<T>::frag *>(lds + off);
}

// Transposed fragment read for 16-bit types (ds_read_b64_tr_b16).  Within each
// group of 16 lanes the instruction returns to lane i, element e, the element
// (i % 4) of the 8 bytes read by source lane 4*e + i/4.  So if every lane of a
// group addresses  base + row(s/4) * pitch + (col0 + 4*(s%4)) * 2,  s = lane%16,
// lane i receives M[row(e)][col0 + i] for e = 0..3: four rows of one column.
__device__ __forceinline__ i16x4 lds_tr4(const char *lds, int byte_off) {
  // `lds` points into a __shared__ array: the cast is an address-space cast
  // from the generic to the LDS address space.
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)(lds + byte_off));
}

// Byte offset of (row, byte-in-row) in an LDS matrix with row pitch PITCH
// whose 16-byte chunks are permuted within each row by XOR with swz(row).
// For 16-bit data the permutations are chosen (and checked on gfx950 with the
// LDS bank-conflict counter) so that the kernels' access patterns hit distinct
// banks:
//   ROWB = 128 (8 chunks): swz = 4*((r>>1)&1) + ((r>>2)&3) -- 16 consecutive
//     rows at one chunk fall in 16 distinct 16-byte slots of 256 bytes, and 4
//     consecutive rows (aligned to 4) at an aligned 4-chunk group fall in the
//     4 distinct 64-byte quarters;
//   ROWB = 256 (16 chunks): swz = 4*(r&3) + ((r>>2)&3), same two properties;
//   ROWB = 64 (dS^T, 4 chunks): swz = 2*((r>>3)&1) + ((r>>2)&1) -- rows
//     {0..3, 8..11} (+4) read as aligned 2-chunk pairs fall in 8 distinct
//     32-byte slots.
// SWZ = false: plain rows (fp32 data, padded pitch).
template <int PITCH, int ROWB, bool SWZ>
struct Layout {
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (!SWZ) return 0;
    else if constexpr (ROWB == 128) return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    else if constexpr (ROWB == 256) return 4 * (r & 3) + ((r >> 2) & 3);
    else return 2 * ((r >> 3) & 1) + ((r >> 2) & 1);
  }
  static __device__ __forceinline__ int off(int row, int byte) {
    return row * PITCH + (byte ^ (swz(row) << 4));
  }
};

// Element e of MFMA step t in register order, from an LDS matrix with rows =
// contraction index: M[row0 + reg_row(KPL*t + e, h)][col0 + l32].
template <typename T, typename L>
__device__ __forceinline__ typename Mma<T>::frag regorder_frag(const char *lds, int row0, int t, int col0,
                                                              int lane = threadIdx.x & 63) {
  if constexpr (Mma<T>::KPL == 1) {
    const int row = row0 + reg_row(t, lane >> 5);
    return *reinterpret_cast<const float *>(lds + L::off(row, (col0 + (lane & 31)) * 4));
  } else {
    const int g = lane >> 4, s16 = lane & 15;
    const int r = row0 + 16 * t + 4 * (g >> 1) + (s16 >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (s16 & 3);
    const i16x4 lo = lds_tr4(lds, L::off(r, col * 2));
    const i16x4 hi = lds_tr4(lds, L::off(r + 8, col * 2));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(typename Mma<T>::frag, v);
  }
}

// 16x16 operand in natural order from an LDS matrix whose rows are the
// contraction index: lane (g = lane/16, i = lane%16) gets
// M[row0 + KPL*g + e][col0 + i], e < KPL.
template <typename T, typename L>
__device__ __forceinline__ typename Mma<T>::frag colfrag16(const char *lds, int row0, int col0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  if constexpr (Mma<T>::KPL == 1) {
    return *reinterpret_cast<const float *>(lds + L::off(row0 + g, (col0 + (lane & 15)) * 4));
  } else {
    const int s16 = lane & 15;
    const int r = row0 + 8 * g + (s16 >> 2);
    const int col = col0 + 4 * (s16 & 3);
    const i16x4 lo = lds_tr4(lds, L::off(r, col * 2));
    const i16x4 hi = lds_tr4(lds, L::off(r + 4, col * 2));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(typename Mma<T>::frag, v);
  }
}

// Cross half-wave exchange: value held by lane l ^ 32.
__device__ __forceinline__ float xor32(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes < 32 get (own, partner) ; lanes >= 32 get (partner, own)
  return (threadIdx.x & 32) ? __uint_as_float(s[0]) : __uint_as_float(s[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- workgroup -> tile mapping ----------------------------------------------
// Workgroups are handed to the 8 XCDs round-robin by id.  Remap so that each
// XCD receives a contiguous range of logical ids (consecutive tiles of the same
// (batch, head), which then share K/V in that XCD's L2).  Bijective for any
// grid size; correctness does not depend on the dispatch order.
__host__ __device__ __forceinline__ int xcd_remap(int id, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd, rem = total % kXcd;
  const int xcd = id % kXcd, slot = id / kXcd;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
}

// (batch*head, tile rank) of workgroup `id` in a launch of `total` = BH x
// ntile workgroups.  Workgroups go to the 8 XCDs round-robin by id; each XCD
// takes whole heads (all their tiles), so a head's K/V re-reads stay in one
// L2.  When the heads split evenly over the XCDs, XCD x takes heads x, x + 8,
// x + 16, ...: every XCD then gets heads of every batch, and with key padding
// (work per head proportional to its batch's key length) the XCDs stay
// evenly loaded, which a contiguous range of heads (a few whole batches per
// XCD) does not.  Otherwise each XCD takes a contiguous range (xcd_remap).
// Within an XCD: head by head; or, for causal launches (rank 0 = the longest
// tile) of up to 64 tiles per head, rank-major: every head of the XCD gets
// its rank-0 tile before any gets its rank-1 tile, so the longest tiles of
// all heads start first and the short ones fill the end of the launch.
// Rank-major keeps all of the XCD's heads active at once: at 128 tiles per
// head (16K keys, d = 64) their K and V no longer fit the XCD's 4 MB L2
// together, HBM reads grew 1.6-2x for a 1.4% faster step, so long sequences
// stay head by head.
//
// The first `fill` passes of kCuPerXcd slots (fill = workgroups resident per
// CU) deal the longest-first list in alternating direction; later slots keep
// it in order.  An XCD places its first workgroups one per CU and then a
// second, third ... on each CU in the same order, so CU c starts with list
// positions c, 2 kCuPerXcd - 1 - c, 2 kCuPerXcd + c, ...: a long tile beside
// a short one.  A CU issues its oldest wavefronts first, so the workgroups
// sharing it run nearly one after another, and when the whole launch is
// resident at once (small problems) it ends with the CU whose tiles add up to
// the most work.  Later workgroups start as slots free up, longest first.
// Any order is correct; this one only balances the CUs.
constexpr int kCuPerXcd = 32;
__host__ __device__ __forceinline__ void tile_of(int id, int total, int ntile, bool rank_major,
                                                 int fill, int &bh, int &rank) {
  constexpr int kXcd = 8;
  const int nbh = total / ntile;
  if (nbh % kXcd == 0) {
    const int hpx = nbh / kXcd;  // heads per XCD; total / 8 = hpx * ntile exactly
    const int xcd = id % kXcd, slot = id / kXcd;
    int j;
    if (rank_major && ntile <= 64) {
      const int n = hpx * ntile;  // this XCD's slots
      const int pass = slot / kCuPerXcd, pos = slot - pass * kCuPerXcd;
      const int len = n - pass * kCuPerXcd < kCuPerXcd ? n - pass * kCuPerXcd : kCuPerXcd;
      const int q = pass * kCuPerXcd + ((pass & 1) && pass < fill ? len - 1 - pos : pos);
      j = q % hpx;
      rank = q / hpx;
    } else {
      j = slot / ntile;
      rank = slot - j * ntile;
    }
    bh = xcd + kXcd * j;
  } else {
    const int logical = xcd_remap(id, total);
    bh = logical / ntile;
    rank = logical - bh * ntile;
  }
}

}  // namespace fa
