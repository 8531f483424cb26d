// Row softmax and LayerNorm / GroupNorm as streaming reductions on gfx950.
//
// The math-properties page, section 8 ("Generalization"), lists softmax
// routing / gating, LayerNorm and GroupNorm as operations with attention's
// structure: a finite state updated block by block (its section 2) and merged
// across blocks.  Here every thread carries such a state over the 16-byte
// vectors of a row that it visits, the states of the lanes and of the waves
// of a row are merged, and a second pass writes the output from the merged
// state:
//  * softmax: the state is (m, l), running max and exponential sum, merged by
//    the FlashAttention summary page's merge equation (section "Incremental
//    softmax tracking"): m = max(m_a, m_b), l = l_a e^(m_a - m) + l_b e^(m_b - m);
//    y = e^(x - m) / l, lse = m + ln l.  Kept in base 2 (x log2 e).
//  * LayerNorm / GroupNorm: the state is (n, mean, M2), merged by the pairwise
//    update of Chan, Golub and LeVeque (1979): n = n_a + n_b,
//    d = mean_b - mean_a, mean = mean_a + d n_b / n,
//    M2 = M2_a + M2_b + d^2 n_a n_b / n;  y = (x - mean) rstd gamma + beta with
//    rstd = 1 / sqrt(M2 / n + eps).
// These kernels are bound by HBM bandwidth.  Rows that fit (RES) stay in
// registers between the two passes, so the input is read once; longer rows
// are read again in the second pass (mostly from L2 / MALL).  WPR = 1: one
// wavefront per row, four rows per workgroup (many rows); WPR = 4: one
// workgroup per row (few, long rows).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

constexpr int kResVecs = 8;  // 16-byte vectors per thread held in registers (RES)

template <typename T>
struct RowIO {
  static constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte vector
  // Vector c of a row: elements c*EPV .. c*EPV+EPV-1; past `cols` read as
  // `fill`.  `vec`: the row start is 16-byte aligned (one 16-byte access for
  // a whole vector), else element accesses.
  static __device__ __forceinline__ void load(const T *row, int64_t cols, int64_t c, float fill,
                                              float (&v)[EPV], bool vec) {
    const int64_t e0 = c * EPV;
    if (vec && e0 + EPV <= cols) {
      const u32x4 raw = *reinterpret_cast<const u32x4 *>(row + e0);
      const T *t = reinterpret_cast<const T *>(&raw);
#pragma unroll
      for (int i = 0; i < EPV; ++i) v[i] = (float)t[i];
    } else {
#pragma unroll
      for (int i = 0; i < EPV; ++i) v[i] = e0 + i < cols ? (float)row[e0 + i] : fill;
    }
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

// Merge the states of the threads of one row: across the 64 lanes, then (WPR
// = 4) across the four waves through LDS.  Every thread ends with the row's
// state.
template <int WPR, typename S, typename F>
__device__ __forceinline__ S row_merge(S s, F merge, S *lds) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    S o;
    float *po = reinterpret_cast<float *>(&o);
    const float *ps = reinterpret_cast<const float *>(&s);
#pragma unroll
    for (int k = 0; k < (int)(sizeof(S) / 4); ++k) po[k] = __shfl_xor(ps[k], off);
    s = merge(s, o);
  }
  if constexpr (WPR > 1) {
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = s;
    __syncthreads();
    s = lds[0];
#pragma unroll
    for (int w = 1; w < WPR; ++w) s = merge(s, lds[w]);
  }
  return s;
}

template <typename T, int WPR, bool RES>
__global__ void __launch_bounds__(256) softmax_rows_kernel(RedParams p) {
  using IO = RowIO<T>;
  constexpr int EPV = IO::EPV, NT = 64 * WPR, NV = RES ? kResVecs : 1;
  __shared__ SmState lds[WPR];
  const int wave = threadIdx.x >> 6;
  const int64_t row = WPR == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
  if (row >= p.rows) return;  // uniform over the wave (WPR 1) or the workgroup (WPR 4)
  const int tid = WPR == 1 ? (threadIdx.x & 63) : threadIdx.x;
  const T *x = static_cast<const T *>(p.x) + row * p.ldx;
  T *y = static_cast<T *>(p.y) + row * p.ldy;
  const int64_t cols = p.cols, nvec = (cols + EPV - 1) / EPV;

  float keep[NV][EPV];
  SmState s = {-INFINITY, 0.f};
  auto absorb = [&](float (&v)[EPV]) {
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPV; ++i) {
      v[i] *= kLog2e;
      mb = fmaxf(mb, v[i]);
    }
    if (mb == -INFINITY) return;
    float lb = 0.f;
#pragma unroll
    for (int i = 0; i < EPV; ++i) lb += fast_exp2(v[i] - mb);
    s = sm_merge(s, {mb, lb});
  };
  if constexpr (RES) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t c = tid + (int64_t)k * NT;
      if (c < nvec) {
        IO::load(x, cols, c, -INFINITY, keep[k], p.vec);
        absorb(keep[k]);
      }
    }
  } else {
    for (int64_t c = tid; c < nvec; c += NT) {
      float v[EPV];
      IO::load(x, cols, c, -INFINITY, v, p.vec);
      absorb(v);
    }
  }
  s = row_merge<WPR>(s, sm_merge, lds);
  const bool empty = s.m == -INFINITY;  // every entry -inf: y = 0, lse = -inf
  const float inv = empty ? 0.f : 1.f / s.l;
  auto emit = [&](int64_t c, float (&v)[EPV]) {
#pragma unroll
    for (int i = 0; i < EPV; ++i) v[i] = empty ? 0.f : fast_exp2(v[i] - s.m) * inv;
    IO::store(y, cols, c, v, p.vec);
  };
  if constexpr (RES) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t c = tid + (int64_t)k * NT;
      if (c < nvec) emit(c, keep[k]);
    }
  } else {
    for (int64_t c = tid; c < nvec; c += NT) {
      float v[EPV];
      IO::load(x, cols, c, -INFINITY, v, p.vec);
#pragma unroll
      for (int i = 0; i < EPV; ++i) v[i] *= kLog2e;
      emit(c, v);
    }
  }
  if (p.lse && tid == 0) p.lse[row] = empty ? -INFINITY : (s.m + log2f(s.l)) * kLn2;
}

template <typename T, int WPR, bool RES>
__global__ void __launch_bounds__(256) layernorm_rows_kernel(RedParams p) {
  using IO = RowIO<T>;
  constexpr int EPV = IO::EPV, NT = 64 * WPR, NV = RES ? kResVecs : 1;
  __shared__ MoState lds[WPR];
  const int wave = threadIdx.x >> 6;
  const int64_t row = WPR == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
  if (row >= p.rows) return;
  const int tid = WPR == 1 ? (threadIdx.x & 63) : threadIdx.x;
  const T *x = static_cast<const T *>(p.x) + row * p.ldx;
  T *y = static_cast<T *>(p.y) + row * p.ldy;
  const int64_t cols = p.cols, nvec = (cols + EPV - 1) / EPV;

  float keep[NV][EPV];
  MoState s = {0.f, 0.f, 0.f};
  auto absorb = [&](int64_t c, const float (&v)[EPV]) {
    const int64_t left = cols - c * EPV;
    const int cnt = left < EPV ? (int)left : EPV;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < EPV; ++i) sum += i < cnt ? v[i] : 0.f;
    const float mb = sum / (float)cnt;
    float m2 = 0.f;
#pragma unroll
    for (int i = 0; i < EPV; ++i) {
      const float d = v[i] - mb;
      m2 += i < cnt ? d * d : 0.f;
    }
    s = mo_merge(s, {(float)cnt, mb, m2});
  };
  if constexpr (RES) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t c = tid + (int64_t)k * NT;
      if (c < nvec) {
        IO::load(x, cols, c, 0.f, keep[k], p.vec);
        absorb(c, keep[k]);
      }
    }
  } else {
    for (int64_t c = tid; c < nvec; c += NT) {
      float v[EPV];
      IO::load(x, cols, c, 0.f, v, p.vec);
      absorb(c, v);
    }
  }
  s = row_merge<WPR>(s, mo_merge, lds);
  const float mean = s.mean, rstd = 1.f / sqrtf(s.m2 / s.n + p.eps);
  const T *gamma = static_cast<const T *>(p.gamma), *beta = static_cast<const T *>(p.beta);
  const int64_t cbase = (row % p.groups) * p.cpg;  // first channel of this row
  const bool plain = p.groups == 1 && p.inner == 1;  // LayerNorm: channel = element
  auto emit = [&](int64_t c, float (&v)[EPV]) {
    const int64_t e0 = c * EPV;
    if (plain && e0 + EPV <= cols) {
      float g[EPV], b[EPV];
      if (gamma) IO::load(gamma, cols, c, 1.f, g, p.gvec);
      if (beta) IO::load(beta, cols, c, 0.f, b, p.gvec);
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        float t = (v[i] - mean) * rstd;
        if (gamma) t *= g[i];
        if (beta) t += b[i];
        v[i] = t;
      }
      IO::store(y, cols, c, v, p.vec);
      return;
    }
    // channel of element e0 + i: cbase + (e0 + i) / inner
    const int64_t q0 = e0 / p.inner, r0 = e0 - q0 * p.inner;
#pragma unroll
    for (int i = 0; i < EPV; ++i) {
      const int64_t ch = cbase + (p.inner >= EPV ? q0 + (r0 + i >= p.inner ? 1 : 0) : (e0 + i) / p.inner);
      float t = (v[i] - mean) * rstd;
      if (e0 + i < cols) {
        if (gamma) t *= (float)gamma[ch];
        if (beta) t += (float)beta[ch];
      }
      v[i] = t;
    }
    IO::store(y, cols, c, v, p.vec);
  };
  if constexpr (RES) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t c = tid + (int64_t)k * NT;
      if (c < nvec) emit(c, keep[k]);
    }
  } else {
    for (int64_t c = tid; c < nvec; c += NT) {
      float v[EPV];
      IO::load(x, cols, c, 0.f, v, p.vec);
      emit(c, v);
    }
  }
  if (tid == 0) {
    if (p.mean) p.mean[row] = mean;
    if (p.rstd) p.rstd[row] = rstd;
  }
}

// Shape choice: one wavefront per row when there are enough rows to fill the
// GPU with four-row workgroups, else one workgroup per row; registers hold
// the row when it fits in kResVecs vectors per thread.  The four instances
// of each kernel are named here directly, so that each is compiled for the
// device.
struct RowShape {
  int wpr;
  bool res;
  int64_t grid;
};
template <typename T>
static RowShape row_shape(const RedParams &p) {
  constexpr int EPV = RowIO<T>::EPV;
  const int64_t nvec = (p.cols + EPV - 1) / EPV;
  if (p.rows >= 2048) return {1, nvec <= 64 * kResVecs, (p.rows + 3) / 4};
  return {4, nvec <= 256 * kResVecs, p.rows};
}

static hipError_t launch1(const void *fn, const RedParams &p, int64_t grid, hipStream_t s) {
  RedParams a = p;
  void *args[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, s);
}

template <typename T>
static hipError_t softmax_t(const RedParams &p, hipStream_t s) {
  const RowShape r = row_shape<T>(p);
  const void *fn = r.wpr == 1
      ? (r.res ? reinterpret_cast<const void *>(&softmax_rows_kernel<T, 1, true>)
               : reinterpret_cast<const void *>(&softmax_rows_kernel<T, 1, false>))
      : (r.res ? reinterpret_cast<const void *>(&softmax_rows_kernel<T, 4, true>)
               : reinterpret_cast<const void *>(&softmax_rows_kernel<T, 4, false>));
  return launch1(fn, p, r.grid, s);
}

template <typename T>
static hipError_t layernorm_t(const RedParams &p, hipStream_t s) {
  const RowShape r = row_shape<T>(p);
  const void *fn = r.wpr == 1
      ? (r.res ? reinterpret_cast<const void *>(&layernorm_rows_kernel<T, 1, true>)
               : reinterpret_cast<const void *>(&layernorm_rows_kernel<T, 1, false>))
      : (r.res ? reinterpret_cast<const void *>(&layernorm_rows_kernel<T, 4, true>)
               : reinterpret_cast<const void *>(&layernorm_rows_kernel<T, 4, false>));
  return launch1(fn, p, r.grid, s);
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
