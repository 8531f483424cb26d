// Merge of partial attention results over disjoint key sets (fa_merge_partials).
//
// Method: FlashAttention summary page (paper 2205.14135), section
// "Incremental softmax tracking", the merge equation: the statistics of a
// score row split into parts combine by rescaling each part's exponential sum
// with exp(part max - overall max).  A part here is the output of a forward
// pass over one subset of the keys -- its O_s already divided by its own sum,
// and its LSE_s = m_s + ln l_s -- so the same rule reads, in log-sum-exp form,
//     LSE = log sum_s exp(LSE_s),      O = sum_s exp(LSE_s - LSE) O_s.
// This is what combines the per-hop results of context-parallel (ring)
// attention, where each device holds a query shard and the key / value shards
// visit it one by one (same page, "Limitations and open questions": multi-GPU
// attention is left open there).
//
// HBM-bound: per query row it reads S rows of O_s (d elements each) and S
// floats of LSE_s and writes one row of O and one float.  A row is split over
// d * sizeof(T) / 16 adjacent lanes (8, 16 or 32), each moving one 16-byte
// vector per part, so every load instruction of a wave covers whole rows.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <typename T, int D>
struct MergeCfg {
  static constexpr int E = sizeof(T);
  static constexpr int LPR = D * E / 16;  // lanes per row (divides 64)
  static constexpr int RPB = 256 / LPR;   // rows per workgroup
  static constexpr int EPL = 16 / E;      // elements per lane
};

template <typename T, int D>
__global__ void __launch_bounds__(256) merge_parts_kernel(MergeParams p) {
  using C = MergeCfg<T, D>;
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  const int64_t row = (int64_t)blockIdx.x * C::RPB + threadIdx.x / C::LPR;
  const int c = (int)(threadIdx.x % C::LPR);
  // a row's lanes lie in one wave and leave together
  if (row >= rows) return;
  const int n = (int)(row % p.Nq);
  const int64_t bh = row / p.Nq;
  const int b = (int)(bh / p.H), hh = (int)(bh % p.H);
  const int64_t off = ((int64_t)b * p.sb + (int64_t)hh * p.sh + (int64_t)n * p.sn) * C::E + 16 * c;
  // The largest LSE_s first, so every weight exp(LSE_s - m) is at most 1.
  float m = -INFINITY;
  for (int s = 0; s < p.S; ++s) m = fmaxf(m, p.lse_parts[s][row]);
  float acc[C::EPL];
#pragma unroll
  for (int e = 0; e < C::EPL; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    // Parts in groups of kGroup: the group's loads are all in flight before
    // the first is used.  A part that saw no key (LSE_s = -inf) weighs 0
    // whatever its O_s holds (its terms are skipped by a select, not
    // multiplied by 0, so a NaN there cannot leak in).
    constexpr int kGroup = 4;
    for (int s0 = 0; s0 < p.S; s0 += kGroup) {
      u32x4 raw[kGroup];
      float w[kGroup];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        const int s = min(s0 + g, p.S - 1);
        raw[g] = ldg16(static_cast<const char *>(p.o_parts[s]) + off);
        w[g] = s0 + g < p.S ? expf(p.lse_parts[s][row] - m) : 0.f;
      }
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        wsum += w[g];
        const T *x = reinterpret_cast<const T *>(&raw[g]);
#pragma unroll
        for (int e = 0; e < C::EPL; ++e) acc[e] = w[g] == 0.f ? acc[e] : fmaf(w[g], to_f32(x[e]), acc[e]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  u32x4 out;
  T *y = reinterpret_cast<T *>(&out);
#pragma unroll
  for (int e = 0; e < C::EPL; ++e) y[e] = from_f32<T>(acc[e] * inv);
  stg16(static_cast<char *>(p.o) + off, out);
  if (c == 0) p.lse[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

template <typename T, int D>
static hipError_t launch_merge_t(const MergeParams &p, hipStream_t s) {
  using C = MergeCfg<T, D>;
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  MergeParams a = p;
  void *args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void *>(&merge_parts_kernel<T, D>),
                         dim3((unsigned)((rows + C::RPB - 1) / C::RPB)), dim3(256), args, 0, s);
}

template <typename T>
static hipError_t launch_merge_dt(const MergeParams &p, hipStream_t s) {
  return p.d == 64 ? launch_merge_t<T, 64>(p, s) : launch_merge_t<T, 128>(p, s);
}

hipError_t launch_merge(const MergeParams &p, fa_dtype_t dt, hipStream_t s) {
  switch (dt) {
    case FA_DTYPE_F32: return launch_merge_dt<float>(p, s);
    case FA_DTYPE_F16: return launch_merge_dt<_Float16>(p, s);
    case FA_DTYPE_BF16: return launch_merge_dt<__bf16>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
