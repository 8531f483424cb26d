// Forward pass of exact attention on gfx950: one workgroup per (batch, head,
// 128-query tile), one wavefront per 32 queries, K/V streamed through LDS in
// tiles of BC keys with a running row max / row sum.
//
// Method (FlashAttention summary page, paper 2205.14135):
//  * section "Incremental softmax tracking", steps 1-4 for query block i and
//    key/value block j: block scores, block max / exp / sum, running max/sum
//    update, rescaled output accumulation.  Here the division by the running
//    sum is deferred to the epilogue (identical in exact arithmetic) and the
//    exponentials are taken directly against the running max (the block-local
//    exp(S - m_block) times exp(m_block - m_new) of the page, folded).
//  * section "Key ideas", tiling bullet: Q, K, V are cut into blocks that fit
//    on chip; the N x N matrices never reach device memory.
//  * Math-properties page, section 7: the loop keeps one query tile resident
//    (outer loop) and streams key/value tiles (inner loop); the carried state
//    is the running max, the exponential sum and the partial output.
//  * section "Block-Sparse FlashAttention": only key tiles whose mask block is
//    set are visited.
//
// gfx950 mapping.  Scores are formed transposed, S^T = K Q^T, on 32x32 MFMAs
// (A = K rows from LDS, B = this wave's Q rows kept in registers for the whole
// loop), so every lane owns one query (column) of each 32-query block and 16
// of its keys per 32-key block; its partner lane (l ^ 32) owns the other 16.  The row max therefore
// needs one cross-half exchange, and P^T, converted in registers, is directly
// the B operand of O^T += V^T P^T.  V^T fragments come from the row-major V
// tile in LDS through the transposing LDS read (ds_read_b64_tr_b16).
// Exponentials are base 2 with scale*log2(e) folded into one FMA.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

template <typename T, int D, bool SPARSE>
struct FwdCfg {
  static constexpr int E = sizeof(T);
  static constexpr int KPL = Mma<T>::KPL;
  static constexpr int WAVES = 4;
  // 32-query blocks per wavefront.  Two would give each wave two independent
  // softmax chains and halve the LDS reads per MFMA, but the extra registers
  // cost occupancy: measured slower on gfx950 (16K dense: 1.24 -> 1.46 ms,
  // 4K causal: 0.24 -> 0.27 ms), so one.  QB > 1 must stay off for the
  // block-sparse path, whose tiles may not span two rows of the block mask.
  static constexpr int QB = 1;
  static constexpr int QPW = 32 * QB;             // queries per wavefront
  static constexpr int BR = QPW * WAVES;          // queries per workgroup
  static constexpr int BC = (E == 4) ? 32 : 64;   // keys per LDS tile
  static constexpr int NSB = BC / 32;             // 32-key score blocks per tile
  static constexpr int NOB = D / 32;              // 32-wide blocks of the output
  static constexpr int KSTEPS = D / (2 * KPL);    // MFMA steps over d
  static constexpr int PSTEPS = 16 / KPL;         // MFMA steps over 32 keys
  // LDS row pitches, chosen so that the reads of each tile are free of bank
  // conflicts (measured on gfx950): K rows are read 16 bytes per lane down 16
  // consecutive rows (pitch = 16 mod 32 bytes); V rows are read by the
  // transposing read, 4 rows x 64 bytes per half-wave (pitch = 64 mod 256).
  static constexpr int PITCH = D * E + 16;        // K tile row pitch (bytes)
  static constexpr int VPITCH = (E == 4) ? D * E + 16 : D * E + 64;  // V tile row pitch
  static constexpr int KTILE = BC * PITCH;
  static constexpr int VTILE = BC * VPITCH;
  static constexpr int TILE_BYTES = KTILE + VTILE;  // one stage: K then V
  static constexpr int CPR = D * E / 16;          // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / (64 * WAVES);  // chunks per thread
  static_assert(BC * CPR % (64 * WAVES) == 0, "tile must split evenly");
};

constexpr int kMaxMaskBlocks = 1024;


// V^T fragment for step t of 32-key block sb and 32-wide output block nb:
// element e is V[sb*32 + reg_row(KPL*t + e, h)][nb*32 + l32].
template <typename T, int PITCH>
__device__ __forceinline__ typename Mma<T>::frag vt_frag(const char *vl, int sb, int t, int nb) {
  const int lane = threadIdx.x & 63;
  if constexpr (Mma<T>::KPL == 1) {
    const int row = sb * 32 + reg_row(t, lane >> 5);
    return *reinterpret_cast<const float *>(vl + row * PITCH + (nb * 32 + (lane & 31)) * 4);
  } else {
    const int g = lane >> 4, s16 = lane & 15;
    const int row0 = sb * 32 + 16 * t + 4 * (g >> 1) + (s16 >> 2);
    const int col = nb * 32 + 16 * (g & 1) + 4 * (s16 & 3);
    const i16x4 lo = lds_tr4(vl, row0 * PITCH + col * 2);
    const i16x4 hi = lds_tr4(vl, (row0 + 8) * PITCH + col * 2);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(typename Mma<T>::frag, v);
  }
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(256) fwd_kernel(AttnParams p) {
  using C = FwdCfg<T, D, SPARSE>;
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KPL = C::KPL, PITCH = C::PITCH, E = C::E;

  __shared__ __attribute__((aligned(16))) char smem[2 * C::TILE_BYTES];
  __shared__ uint16_t blist[SPARSE ? kMaxMaskBlocks : 1];
  __shared__ int nlist_s;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int N = p.N;
  const int nqt = (N + C::BR - 1) / C::BR;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nqt;
  int qt = logical - bh * nqt;
  if (CAUSAL) qt = nqt - 1 - qt;  // longest rows first
  const int b = bh / p.H, hh = bh - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)hh * p.sh;
  const T *Q = static_cast<const T *>(p.q) + base;
  const T *K = static_cast<const T *>(p.k) + base;
  const T *V = static_cast<const T *>(p.v) + base;
  T *O = static_cast<T *>(p.o) + base;

  int kv_len = N;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), N);
  const int q_tile0 = qt * C::BR;
  const int qw0 = q_tile0 + C::QPW * wave;  // first query of this wave
  // this lane's query in query block qb is qw0 + 32*qb + l32
  int kv_hi = kv_len;                   // keys >= kv_hi are invisible to the whole tile
  if (CAUSAL) kv_hi = min(kv_hi, q_tile0 + C::BR);

  // ---- the list of key tiles this workgroup visits
  int ntiles;
  int tiles_per_blk = 1;
  if constexpr (SPARSE) {
    tiles_per_blk = p.mb / C::BC;
    const uint8_t *mrow = p.mask + (int64_t)hh * p.mask_hstride + (int64_t)(q_tile0 / p.mb) * p.nblk;
    if (wave == 0) {
      int count = 0;
      for (int j0 = 0; j0 < p.nblk; j0 += 64) {
        const int j = j0 + lane;
        const bool set = j < p.nblk && j * p.mb < kv_hi && mrow[j] != 0;
        const uint64_t bal = __ballot(set);
        if (set) blist[count + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)j;
        count += __popcll(bal);
      }
      if (lane == 0) nlist_s = count;
    }
    __syncthreads();
    const int nl = nlist_s;
    if (nl == 0) {
      ntiles = 0;
    } else {
      const int last0 = (int)blist[nl - 1] * p.mb;
      const int in_last = min(tiles_per_blk, (kv_hi - last0 + C::BC - 1) / C::BC);
      ntiles = (nl - 1) * tiles_per_blk + in_last;
    }
  } else {
    ntiles = (kv_hi + C::BC - 1) / C::BC;
  }
  auto tile_start = [&](int t) -> int {
    if constexpr (SPARSE) {
      const int bi = t / tiles_per_blk;
      return (int)blist[bi] * p.mb + (t - bi * tiles_per_blk) * C::BC;
    } else {
      return t * C::BC;
    }
  };

  // ---- this wave's Q rows, held as MFMA B operands for the whole loop.
  // Step s, half h covers d = h*D/2 + s*KPL + e: each lane reads a contiguous
  // half row.
  frag qf[C::QB][C::KSTEPS];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int qi = qw0 + 32 * qb + l32;
    if (qi < N) {
      const T *qrow = Q + (int64_t)qi * p.sn + h * (D / 2);
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qf[qb][s] = *reinterpret_cast<const frag *>(qrow + s * KPL);
    } else {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qf[qb][s] = frag{};
    }
  }

  // ---- K/V staging: buffer loads (next tile) -> registers -> LDS (double
  // buffer).  Lane offsets inside a tile are loop invariant; the tile start
  // goes in the scalar offset, and rows past N read as zeros.
  const uint32_t kv_bytes = (uint32_t)(((int64_t)(N - 1) * p.sn + D) * E);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, kv_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V, kv_bytes);
  const int row_bytes = (int)(p.sn * E);
  int voff[C::CPT];
#pragma unroll
  for (int u = 0; u < C::CPT; ++u) {
    const int c = tid + 256 * u, row = c / C::CPR, col = c - row * C::CPR;
    voff[u] = row * row_bytes + col * 16;
  }
  u32x4 stk[C::CPT], stv[C::CPT];
  auto load_tile = [&](int kv0) {
    const int so = kv0 * row_bytes;
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      stk[u] = buf_load16(krs, voff[u], so);
      stv[u] = buf_load16(vrs, voff[u], so);
    }
  };
  auto store_tile = [&](int buf) {
    char *kl = smem + buf * C::TILE_BYTES;
    char *vl = kl + C::KTILE;
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int c = tid + 256 * u, row = c / C::CPR, col = c - row * C::CPR;
      *reinterpret_cast<u32x4 *>(kl + row * PITCH + col * 16) = stk[u];
      *reinterpret_cast<u32x4 *>(vl + row * C::VPITCH + col * 16) = stv[u];
    }
  };

  float m_run[C::QB], l_run[C::QB];  // per query block: running max of
  f32x16 oacc[C::QB][C::NOB];          // scale*log2(e)*S, this lane's half-sum
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < C::NOB; ++nb) oacc[qb][nb] = f32x16{};
  }
  const float c2 = p.scale_log2;

  // Tiles that no mask touches form a prefix of the list (tiles ascend): a key
  // tile is whole for every query of the workgroup when it ends at or before
  // the padding length and (causal) at or before the tile's first query.
  const int lim = CAUSAL ? min(kv_len, q_tile0 + 1) : kv_len;
  int n_full;
  if constexpr (SPARSE) {
    n_full = 0;
    for (int bi = 0; bi * tiles_per_blk < ntiles; ++bi) {
      const int f = min(tiles_per_blk, max(0, (lim - (int)blist[bi] * p.mb) / C::BC));
      n_full += f;
      if (f < tiles_per_blk) break;
    }
    n_full = min(n_full, ntiles);
  } else {
    n_full = min(ntiles, lim / C::BC);
  }

  // One key tile: scores, (masking), running max / rescale, exp, PV, for every
  // query block of the wave.
  auto tile = [&](const char *kl, const char *vl, int kv0, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    // step 1: S^T = K_j Q_i^T (each K fragment feeds every query block)
    f32x16 sacc[C::QB][C::NSB];
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) sacc[qb][sb] = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        const frag a = lds_frag<T>(kl, (sb * 32 + l32) * PITCH + (h * (D / 2) + s * KPL) * E);
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) sacc[qb][sb] = M::mma32(a, qf[qb][s], sacc[qb][sb]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const int qi = qw0 + 32 * qb + l32;
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (MASK) {
            const int key = kv0 + sb * 32 + reg_row(r, h);
            if (!(key < kv_len && (!CAUSAL || key <= qi))) sacc[qb][sb][r] = -INFINITY;
          }
          mx = fmaxf(mx, sacc[qb][sb][r]);
        }
      // steps 2-3: running max; the carried state is rescaled only when some
      // lane's max grew (exp2(0) = 1 for the others)
      mx = fmaxf(mx, xor32(mx));
      const float mt = (MASK && mx == -INFINITY) ? -INFINITY : mx * c2;
      const float m_new = fmaxf(m_run[qb], mt);
      const float m_use = (MASK && m_new == -INFINITY) ? 0.f : m_new;
      if (__ballot(m_new > m_run[qb]) != 0) {
        const float alpha = fast_exp2(m_run[qb] - m_use);
        l_run[qb] *= alpha;
#pragma unroll
        for (int nb = 0; nb < C::NOB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][nb][r] *= alpha;
      }
      m_run[qb] = m_new;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = fast_exp2(fmaf(sacc[qb][sb][r], c2, -m_use));
          if constexpr (MASK) {
            if (sacc[qb][sb][r] == -INFINITY) x = 0.f;
          }
          sacc[qb][sb][r] = x;
        }
    }
    // step 4: O_i^T += V_j^T P^T; the row sum takes the same rounded P.  Each
    // V^T fragment feeds every query block.
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb)
#pragma unroll
      for (int t = 0; t < C::PSTEPS; ++t) {
        frag pb[C::QB];
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          pb[qb] = pack_frag<T>(sacc[qb][sb], t * KPL);
          l_run[qb] = frag_sum<T>(pb[qb], l_run[qb]);
        }
#pragma unroll
        for (int nb = 0; nb < C::NOB; ++nb) {
          const frag va = vt_frag<T, C::VPITCH>(vl, sb, t, nb);
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) oacc[qb][nb] = M::mma32(va, pb[qb], oacc[qb][nb]);
        }
      }
  };

  if (ntiles > 0) {
    load_tile(tile_start(0));
    store_tile(0);
  }
  // Retire every outstanding load (Q fragments included) on all paths into
  // the loop; otherwise the compiler keeps them "pending" at the loop header
  // and waits on the next tile's prefetch before the first MFMA of each tile.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  int it = 0;
  for (; it < n_full; ++it) {
    const bool has_next = it + 1 < ntiles;
    if (has_next) load_tile(tile_start(it + 1));
    const char *kl = smem + (it & 1) * C::TILE_BYTES;
    tile(kl, kl + C::KTILE, tile_start(it), std::integral_constant<bool, false>{});
    if (has_next) store_tile((it + 1) & 1);
    __syncthreads();
  }
  for (; it < ntiles; ++it) {
    const int kv0 = tile_start(it);
    const bool has_next = it + 1 < ntiles;
    if (has_next) load_tile(tile_start(it + 1));
    const char *kl = smem + (it & 1) * C::TILE_BYTES;
    if (!(CAUSAL && kv0 > qw0 + C::QPW - 1))  // some key of the tile is visible to this wave
      tile(kl, kl + C::KTILE, kv0, std::integral_constant<bool, true>{});
    if (has_next) store_tile((it + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O / l, LSE = (m + log2 l) ln 2
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int qi = qw0 + 32 * qb + l32;
    const float l_tot = l_run[qb] + xor32(l_run[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qi < N) {
      T *orow = O + (int64_t)qi * p.sn;
#pragma unroll
      for (int nb = 0; nb < C::NOB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = nb * 32 + 8 * i + 4 * h;
          if constexpr (E == 4) {
            f32x4 v = {oacc[qb][nb][4 * i] * inv, oacc[qb][nb][4 * i + 1] * inv,
                       oacc[qb][nb][4 * i + 2] * inv, oacc[qb][nb][4 * i + 3] * inv};
            *reinterpret_cast<f32x4 *>(orow + d0) = v;
          } else {
            typedef T t4 __attribute__((ext_vector_type(4)));
            t4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = (T)(oacc[qb][nb][4 * i + j] * inv);
            *reinterpret_cast<t4 *>(orow + d0) = v;
          }
        }
      if (h == 0)
        p.lse[(int64_t)bh * N + qi] = l_tot > 0.f ? (m_run[qb] + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_fwd_t(const AttnParams &p, hipStream_t s) {
  using C = FwdCfg<T, D, SPARSE>;
  const int64_t nqt = (p.N + C::BR - 1) / C::BR;
  const int64_t grid = (int64_t)p.B * p.H * nqt;
  AttnParams a = p;
  void *args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void *>(&fwd_kernel<T, D, CAUSAL, SPARSE>),
                         dim3((unsigned)grid), dim3(256), args, 0, s);
}

template <typename T, int D>
static hipError_t launch_fwd_d(const AttnParams &p, bool sparse, hipStream_t s) {
  if (sparse) return p.causal ? launch_fwd_t<T, D, true, true>(p, s) : launch_fwd_t<T, D, false, true>(p, s);
  return p.causal ? launch_fwd_t<T, D, true, false>(p, s) : launch_fwd_t<T, D, false, false>(p, s);
}

template <typename T>
static hipError_t launch_fwd_dt(const AttnParams &p, bool sparse, hipStream_t s) {
  return p.d == 64 ? launch_fwd_d<T, 64>(p, sparse, s) : launch_fwd_d<T, 128>(p, sparse, s);
}

hipError_t launch_fwd(const AttnParams &p, fa_dtype_t dt, bool sparse, hipStream_t s) {
  switch (dt) {
    case FA_DTYPE_F32: return launch_fwd_dt<float>(p, sparse, s);
    case FA_DTYPE_F16: return launch_fwd_dt<_Float16>(p, sparse, s);
    case FA_DTYPE_BF16: return launch_fwd_dt<__bf16>(p, sparse, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
