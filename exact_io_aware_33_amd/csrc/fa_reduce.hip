// Row softmax and LayerNorm / GroupNorm as streaming reductions on gfx950.
//
// The math-properties page, section 8 ("Generalization"), lists softmax
// routing / gating, LayerNorm and GroupNorm as operations with attention's
// structure: a finite state updated block by block (its section 2) and merged
// across blocks.  Here a group of TPR threads owns one row; every thread
// builds the state of the 16-byte vectors it visits, the states of the group
// are merged (lane shuffles, then LDS across the waves of a row), and a
// second pass writes the output from the merged state:
//  * softmax: the state is (m, l), running max and exponential sum, merged by
//    the FlashAttention summary page's merge equation (section "Incremental
//    softmax tracking"): m = max(m_a, m_b), l = l_a e^(m_a - m) + l_b e^(m_b - m);
//    y = e^(x - m) / l, lse = m + ln l.  Kept in base 2 (x log2 e).
//  * LayerNorm / GroupNorm: the state is (n, mean, M2), merged by the pairwise
//    update of Chan, Golub and LeVeque (1979): n = n_a + n_b,
//    d = mean_b - mean_a, mean = mean_a + d n_b / n,
//    M2 = M2_a + M2_b + d^2 n_a n_b / n;  y = (x - mean) rstd gamma + beta with
//    rstd = 1 / sqrt(M2 / n + eps).
//
// These kernels are bound by HBM bandwidth: the floor is one read of x and
// one write of y.  A row of up to 16 vectors per thread (TPR x 16 x 16 bytes:
// 2 KB at TPR = 8 up to 256 KB at TPR = 1024; LayerNorm up to 128 KB, 8 per
// thread, at TPR = 1024) stays in registers, packed as loaded, between the
// two passes, so x is read from HBM exactly once and every thread has all its
// loads in flight at once.  Longer rows are streamed twice
// (the second read mostly from L2 / MALL).  Short rows share a wavefront
// (TPR = 8: eight rows per wave), so no lane idles on a 64-element row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <typename T>
struct RowVec {
  static constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte vector
  // Vector c of a row (elements c*EPV .. c*EPV+EPV-1) as loaded; elements
  // past `cols` read as `fill`.  `vec`: the row start is 16-byte aligned (one
  // 16-byte access), else element accesses.
  static __device__ __forceinline__ u32x4 load(const T *row, int64_t cols, int64_t c, float fill,
                                               bool vec) {
    const int64_t e0 = c * EPV;
    if (vec && e0 + EPV <= cols) return *reinterpret_cast<const u32x4 *>(row + e0);
    u32x4 raw;
    T *t = reinterpret_cast<T *>(&raw);
#pragma unroll
    for (int i = 0; i < EPV; ++i) t[i] = e0 + i < cols ? row[e0 + i] : (T)fill;
    return raw;
  }
  static __device__ __forceinline__ void unpack(u32x4 raw, float (&v)[EPV]) {
    const T *t = reinterpret_cast<const T *>(&raw);
#pragma unroll
    for (int i = 0; i < EPV; ++i) v[i] = (float)t[i];
  }
  static __device__ __forceinline__ void store(T *row, int64_t cols, int64_t c, const float (&v)[EPV],
                                               bool vec) {
    const int64_t e0 = c * EPV;
    if (vec && e0 + EPV <= cols) {
      u32x4 raw;
      T *t = reinterpret_cast<T *>(&raw);
#pragma unroll
      for (int i = 0; i < EPV; ++i) t[i] = (T)v[i];
      *reinterpret_cast<u32x4 *>(row + e0) = raw;
    } else {
#pragma unroll
      for (int i = 0; i < EPV; ++i)
        if (e0 + i < cols) row[e0 + i] = (T)v[i];
    }
  }
};

// Make the held vectors opaque to the compiler between passes, so that it
// converts them again in the next pass instead of keeping every converted
// element alive (which would double or triple the registers a row needs).
// An empty statement: no instruction is emitted.
template <int NV>
__device__ __forceinline__ void opaque(u32x4 (&r)[NV]) {
#pragma unroll
  for (int k = 0; k < NV; ++k) asm volatile("" : "+v"(r[k]));
}

// ---- softmax state (base-2 units)
struct SmState {
  float m, l;
};
__device__ __forceinline__ SmState sm_merge(SmState a, SmState b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return {m, 0.f};
  return {m, a.l * fast_exp2(a.m - m) + b.l * fast_exp2(b.m - m)};
}

// ---- moment state
struct MoState {
  float n, mean, m2;
};
__device__ __forceinline__ MoState mo_merge(MoState a, MoState b) {
  const float n = a.n + b.n;
  if (n == 0.f) return {0.f, 0.f, 0.f};
  const float d = b.mean - a.mean, fb = b.n / n;
  return {n, fmaf(d, fb, a.mean), a.m2 + b.m2 + d * d * a.n * fb};
}

// Merge the states of the TPR threads of one row: xor shuffles inside the
// wave (groups are aligned, so every partner is in the same row), then for
// rows wider than a wave the per-wave states through LDS, in wave order, so
// every thread of the row ends with the same state.
template <int TPR, typename S, typename F>
__device__ __forceinline__ S row_merge(S s, F merge, S *lds) {
  constexpr int LANES = TPR < 64 ? TPR : 64;
#pragma unroll
  for (int off = LANES / 2; off >= 1; off >>= 1) {
    S o;
    float *po = reinterpret_cast<float *>(&o);
    const float *ps = reinterpret_cast<const float *>(&s);
#pragma unroll
    for (int k = 0; k < (int)(sizeof(S) / 4); ++k) po[k] = __shfl_xor(ps[k], off);
    s = merge(s, o);
  }
  if constexpr (TPR > 64) {
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = s;
    __syncthreads();
    s = lds[0];
#pragma unroll
    for (int w = 1; w < TPR / 64; ++w) s = merge(s, lds[w]);
  }
  return s;
}

// Launch geometry shared by both kernels: TPR threads per row, NV > 0 vectors
// per thread held in registers (NV = 0: the row is streamed twice).  A
// workgroup has max(TPR, 256) threads and holds that many / TPR rows.
template <int TPR>
struct RowGroup {
  static constexpr int NT = TPR > 256 ? TPR : 256;
  static constexpr int RPW = NT / TPR;

  int t;        // thread index within the row
  int64_t row;  // row of this thread's group
  __device__ __forceinline__ RowGroup()
      : t((int)(threadIdx.x % TPR)), row((int64_t)blockIdx.x * RPW + threadIdx.x / TPR) {
    // One row per wave or per workgroup: say so, so that row addresses live
    // in scalar registers and each held vector needs one 32-bit offset.
    if constexpr (TPR >= 64) row = __builtin_amdgcn_readfirstlane((int)row);
  }
};

template <typename T, int TPR, int NV>
__global__ void __launch_bounds__(RowGroup<TPR>::NT)
    softmax_rows_kernel(RedParams p) {
  using IO = RowVec<T>;
  constexpr int EPV = IO::EPV;
  __shared__ SmState lds[TPR > 64 ? TPR / 64 : 1];
  const RowGroup<TPR> g;
  // Groups are whole waves (TPR >= 64) or parts of one; a group past the last
  // row leaves together, and no shuffle of another group reads its lanes.
  // For TPR > 64 the group is the workgroup, so the exit is uniform before
  // the barrier.
  if (g.row >= p.rows) return;
  const T *x = static_cast<const T *>(p.x) + g.row * p.ldx;
  T *y = static_cast<T *>(p.y) + g.row * p.ldy;
  const int64_t cols = p.cols, nvec = (cols + EPV - 1) / EPV;

  SmState s = {-INFINITY, 0.f};
  auto absorb = [&](u32x4 raw) {  // one vector as a (max, sum) state, merged in
    float v[EPV];
    IO::unpack(raw, v);
    float mx = v[0];
#pragma unroll
    for (int i = 1; i < EPV; ++i) mx = fmaxf(mx, v[i]);
    const float mb = mx * kLog2e;
    if (mb == -INFINITY) return;
    float lb = 0.f;
#pragma unroll
    for (int i = 0; i < EPV; ++i) lb += fast_exp2(fmaf(v[i], kLog2e, -mb));
    s = sm_merge(s, {mb, lb});
  };
  u32x4 keep[NV > 0 ? NV : 1];
  if constexpr (NV > 0) {
    // All loads first (every one in flight), then the thread's own state: the
    // maximum over its elements, then one exponential sum against it.  A
    // slot past the row end reloads the row's last vector (same cache line,
    // no branch) and is masked out, so the code has no per-slot control flow.
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t c = g.t + (int64_t)k * TPR;
      keep[k] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(x) +
                                                 (uint32_t)((c < nvec ? c : nvec - 1) * 16));
    }
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const bool ok = g.t + (int64_t)k * TPR < nvec;
      float v[EPV];
      IO::unpack(keep[k], v);
#pragma unroll
      for (int i = 0; i < EPV; ++i) mx = fmaxf(mx, ok ? v[i] : -INFINITY);
    }
    const float mb = mx * kLog2e;
    opaque(keep);
    if (mb != -INFINITY) {
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const bool ok = g.t + (int64_t)k * TPR < nvec;
        float v[EPV];
        IO::unpack(keep[k], v);
#pragma unroll
        for (int i = 0; i < EPV; i += 2) {
          const float e0 = fast_exp2(fmaf(v[i], kLog2e, -mb));
          const float e1 = fast_exp2(fmaf(v[i + 1], kLog2e, -mb));
          l0 += ok ? e0 : 0.f;
          l1 += ok ? e1 : 0.f;
        }
      }
      s = {mb, l0 + l1};
    }
    opaque(keep);
  } else {
    int64_t c = g.t;
    for (; c + 3 * TPR < nvec; c += 4 * TPR) {
      u32x4 r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = IO::load(x, cols, c + k * TPR, -INFINITY, p.vec);
#pragma unroll
      for (int k = 0; k < 4; ++k) absorb(r[k]);
    }
    for (; c < nvec; c += TPR) absorb(IO::load(x, cols, c, -INFINITY, p.vec));
  }
  s = row_merge<TPR>(s, sm_merge, lds);
  const bool empty = s.m == -INFINITY;  // every entry -inf: y = 0, lse = -inf
  const float inv = empty ? 0.f : 1.f / s.l;
  auto emit = [&](int64_t c, u32x4 raw) {
    float v[EPV];
    IO::unpack(raw, v);
#pragma unroll
    for (int i = 0; i < EPV; ++i) v[i] = empty ? 0.f : fast_exp2(fmaf(v[i], kLog2e, -s.m)) * inv;
    IO::store(y, cols, c, v, NV > 0 || p.vec);
  };
  if constexpr (NV > 0) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t c = g.t + (int64_t)k * TPR;
      if (c < nvec) emit(c, keep[k]);
    }
  } else {
    for (int64_t c = g.t; c < nvec; c += TPR) emit(c, IO::load(x, cols, c, -INFINITY, p.vec));
  }
  if (p.lse && g.t == 0) p.lse[g.row] = empty ? -INFINITY : (s.m + log2f(s.l)) * kLn2;
}

template <typename T, int TPR, int NV>
__global__ void __launch_bounds__(RowGroup<TPR>::NT)
    layernorm_rows_kernel(RedParams p) {
  using IO = RowVec<T>;
  constexpr int EPV = IO::EPV;
  __shared__ MoState lds[TPR > 64 ? TPR / 64 : 1];
  const RowGroup<TPR> g;
  if (g.row >= p.rows) return;  // as in the softmax kernel
  const T *x = static_cast<const T *>(p.x) + g.row * p.ldx;
  T *y = static_cast<T *>(p.y) + g.row * p.ldy;
  const int64_t cols = p.cols, nvec = (cols + EPV - 1) / EPV;
  // elements of vector c inside the row (only the last vector can be short)
  auto count = [&](int64_t c) {
    const int64_t left = cols - c * EPV;
    return left < EPV ? (int)left : EPV;
  };

  MoState s = {0.f, 0.f, 0.f};
  u32x4 keep[NV > 0 ? NV : 1];
  if constexpr (NV > 0) {
    // The thread's own moments from its registers: mean, then M2 about it
    // (the two-pass form, exact for the few values one thread holds).  Slots
    // past the row end reload the last vector and are masked, as in the
    // softmax kernel; every held vector is whole (EPV elements).
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t c = g.t + (int64_t)k * TPR;
      keep[k] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(x) +
                                                 (uint32_t)((c < nvec ? c : nvec - 1) * 16));
    }
    float sum = 0.f, n = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const bool ok = g.t + (int64_t)k * TPR < nvec;
      float v[EPV];
      IO::unpack(keep[k], v);
#pragma unroll
      for (int i = 0; i < EPV; ++i) sum += ok ? v[i] : 0.f;
      n += ok ? (float)EPV : 0.f;
    }
    opaque(keep);
    if (n > 0.f) {
      const float mean = sum / n;
      float m2 = 0.f;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const bool ok = g.t + (int64_t)k * TPR < nvec;
        float v[EPV];
        IO::unpack(keep[k], v);
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
          const float d = v[i] - mean;
          m2 += ok ? d * d : 0.f;
        }
      }
      s = {n, mean, m2};
    }
    opaque(keep);
  } else {
    for (int64_t c = g.t; c < nvec; c += TPR) {
      float v[EPV];
      IO::unpack(IO::load(x, cols, c, 0.f, p.vec), v);
      const int cnt = count(c);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < EPV; ++i) sum += v[i];
      const float mb = sum / (float)cnt;
      float m2 = 0.f;
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        const float d = v[i] - mb;
        m2 += i < cnt ? d * d : 0.f;
      }
      s = mo_merge(s, {(float)cnt, mb, m2});
    }
  }
  s = row_merge<TPR>(s, mo_merge, lds);
  const float mean = s.mean, rstd = 1.f / sqrtf(s.m2 / s.n + p.eps);
  const T *gamma = static_cast<const T *>(p.gamma), *beta = static_cast<const T *>(p.beta);
  // Channel arithmetic in 32 bits: cols, inner and the channel count are
  // below 2^31 (checked on the host).
  const uint32_t inner = (uint32_t)p.inner;
  const uint32_t cbase = (uint32_t)(g.row % p.groups) * (uint32_t)p.cpg;  // first channel of the row
  const bool plain = p.groups == 1 && inner == 1;  // LayerNorm: channel = element
  const bool whole = inner % EPV == 0;  // every vector lies in one channel
  // The affine step in three compile-time forms, chosen once per row:
  // 0 LayerNorm (gamma / beta vectors at the element's own position), 1 every
  // vector inside one channel (one gamma / beta value), 2 element by element.
  auto emit = [&](auto form, int64_t c, u32x4 raw) {
    constexpr int F = decltype(form)::value;
    float v[EPV];
    IO::unpack(raw, v);
    const int64_t e0 = c * EPV;
#pragma unroll
    for (int i = 0; i < EPV; ++i) v[i] = (v[i] - mean) * rstd;
    if constexpr (F == 0) {
      if (gamma || beta) {
        float gv[EPV], bv[EPV];
        if (gamma) IO::unpack(IO::load(gamma, cols, c, 1.f, p.gvec), gv);
        if (beta) IO::unpack(IO::load(beta, cols, c, 0.f, p.gvec), bv);
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
          if (gamma) v[i] *= gv[i];
          if (beta) v[i] += bv[i];
        }
      }
    } else if constexpr (F == 1) {
      const uint32_t ch = cbase + (uint32_t)e0 / inner;
      const float gs = gamma ? (float)gamma[ch] : 1.f, bs = beta ? (float)beta[ch] : 0.f;
#pragma unroll
      for (int i = 0; i < EPV; ++i) v[i] = fmaf(v[i], gs, bs);
    } else {
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        if (e0 + i < cols) {
          const uint32_t ch = cbase + (uint32_t)(e0 + i) / inner;
          if (gamma) v[i] *= (float)gamma[ch];
          if (beta) v[i] += (float)beta[ch];
        }
      }
    }
    IO::store(y, cols, c, v, NV > 0 || p.vec);
  };
  auto run = [&](auto form) {
    if constexpr (NV > 0) {
      // Four vectors at a time: the compiler barrier keeps the gamma / beta
      // loads of the next four below this group's stores, so at most four
      // vectors' worth of them are live beside the held row.
#pragma unroll
      for (int k0 = 0; k0 < NV; k0 += 4) {
#pragma unroll
        for (int k = k0; k < k0 + 4; ++k) {
          const int64_t c = g.t + (int64_t)k * TPR;
          if (c < nvec) emit(form, c, keep[k]);
        }
        asm volatile("" ::: "memory");
      }
    } else {
      for (int64_t c = g.t; c < nvec; c += TPR) emit(form, c, IO::load(x, cols, c, 0.f, p.vec));
    }
  };
  if (plain)
    run(std::integral_constant<int, 0>{});
  else if (whole)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 2>{});
  if (g.t == 0) {
    if (p.mean) p.mean[g.row] = mean;
    if (p.rstd) p.rstd[g.row] = rstd;
  }
}

// Shape choice.  Rows that do not start 16-byte aligned, or whose length is
// not a whole number of 16-byte vectors, are streamed twice (64 threads per
// row, or 1024 for long rows), with element accesses where a vector is not
// whole.  Else the smallest TPR in {8, 64, 256, 1024} whose threads hold
// the row in at most 16 vectors each; while the launch would have fewer than
// 64K threads and a wider group still leaves each thread at least 4 vectors,
// the next wider TPR (more of the GPU on few rows).  NV, the registers held,
// is the smallest of {4, 8, 16} that covers the row.  Longer rows (more than
// 1024 x `cap` vectors; cap = 16 for softmax, 8 for LayerNorm, whose 1024-
// thread instance would spill at 16) are streamed twice by 1024 threads.
struct RowShape {
  int tpr, nv;  // nv = 0: streamed
  int64_t grid;
};
template <typename T>
static RowShape row_shape(const RedParams &p, int cap) {
  constexpr int EPV = RowVec<T>::EPV;
  const int64_t nvec = (p.cols + EPV - 1) / EPV;
  static const int kTpr[4] = {8, 64, 256, 1024};
  if (!p.vec || p.cols % EPV) {  // element accesses at least at the row ends: streamed twice
    if (nvec <= 64 * 16) return {64, 0, (p.rows + 3) / 4};
    return {1024, 0, p.rows};
  }
  int i = 0;
  while (i < 3 && nvec > (int64_t)kTpr[i] * 16) ++i;
  if (nvec > (int64_t)kTpr[3] * 16) return {1024, 0, p.rows};
  while (i < 3 && p.rows * kTpr[i] < 65536 && nvec >= (int64_t)kTpr[i + 1] * 4) ++i;
  const int tpr = kTpr[i];
  const int64_t per = (nvec + tpr - 1) / tpr;
  const int nv = per <= 4 ? 4 : per <= 8 ? 8 : 16;
  if (tpr == 1024 && nv > cap) return {1024, 0, p.rows};
  const int rpw = (tpr > 256 ? tpr : 256) / tpr;
  return {tpr, nv, (p.rows + rpw - 1) / rpw};
}

// Every instance is named here, so each is compiled for the device.
#define FA_RED_TABLE(KERNEL, CAP)                                                             \
  template <typename T>                                                                       \
  static const void *KERNEL##_fn(int tpr, int nv) {                                           \
    switch (tpr) {                                                                            \
      case 8:                                                                                 \
        return nv == 4 ? (const void *)&KERNEL<T, 8, 4>                                       \
             : nv == 8 ? (const void *)&KERNEL<T, 8, 8> : (const void *)&KERNEL<T, 8, 16>;    \
      case 64:                                                                                \
        return nv == 0 ? (const void *)&KERNEL<T, 64, 0>                                      \
             : nv == 4 ? (const void *)&KERNEL<T, 64, 4>                                      \
             : nv == 8 ? (const void *)&KERNEL<T, 64, 8> : (const void *)&KERNEL<T, 64, 16>;  \
      case 256:                                                                               \
        return nv == 4 ? (const void *)&KERNEL<T, 256, 4>                                     \
             : nv == 8 ? (const void *)&KERNEL<T, 256, 8> : (const void *)&KERNEL<T, 256, 16>; \
      default:                                                                                \
        return nv == 0 ? (const void *)&KERNEL<T, 1024, 0>                                    \
             : nv == 4 ? (const void *)&KERNEL<T, 1024, 4>                                    \
             : nv == 8 ? (const void *)&KERNEL<T, 1024, 8> : (const void *)&KERNEL<T, 1024, CAP>; \
    }                                                                                         \
  }
FA_RED_TABLE(softmax_rows_kernel, 16)
FA_RED_TABLE(layernorm_rows_kernel, 8)
#undef FA_RED_TABLE

static hipError_t launch1(const void *fn, const RedParams &p, const RowShape &r, hipStream_t s) {
  RedParams a = p;
  void *args[] = {&a};
  const int nt = r.tpr > 256 ? r.tpr : 256;
  if (r.grid > 0x7fffffff) return hipErrorInvalidValue;
  return hipLaunchKernel(fn, dim3((unsigned)r.grid), dim3(nt), args, 0, s);
}

template <typename T>
static hipError_t softmax_t(const RedParams &p, hipStream_t s) {
  const RowShape r = row_shape<T>(p, 16);
  return launch1(softmax_rows_kernel_fn<T>(r.tpr, r.nv), p, r, s);
}

template <typename T>
static hipError_t layernorm_t(const RedParams &p, hipStream_t s) {
  const RowShape r = row_shape<T>(p, 8);
  return launch1(layernorm_rows_kernel_fn<T>(r.tpr, r.nv), p, r, s);
}

hipError_t launch_softmax_rows(const RedParams &p, fa_dtype_t dt, hipStream_t s) {
  switch (dt) {
    case FA_DTYPE_F32: return softmax_t<float>(p, s);
    case FA_DTYPE_F16: return softmax_t<_Float16>(p, s);
    case FA_DTYPE_BF16: return softmax_t<__bf16>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_layernorm_rows(const RedParams &p, fa_dtype_t dt, hipStream_t s) {
  switch (dt) {
    case FA_DTYPE_F32: return layernorm_t<float>(p, s);
    case FA_DTYPE_F16: return layernorm_t<_Float16>(p, s);
    case FA_DTYPE_BF16: return layernorm_t<__bf16>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
