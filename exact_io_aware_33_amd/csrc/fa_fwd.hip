// Forward pass of exact attention on gfx950: one workgroup per (batch, head,
// 128-query tile), K/V streamed through LDS in tiles of BC keys with a running
// row max / row sum.
//
// Method (FlashAttention summary page, paper 2205.14135):
//  * section "Incremental softmax tracking", steps 1-4 for query block i and
//    key/value block j: block scores, block max / exp / sum, running max/sum
//    update, rescaled output accumulation.  Here the division by the running
//    sum is deferred to the epilogue (identical in exact arithmetic) and the
//    exponentials are taken directly against a running reference point (the
//    block-local exp(S - m_block) times exp(m_block - m_new) of the page,
//    folded; see kMaxSlack for how the reference point moves).
//  * section "Key ideas", tiling bullet: Q, K, V are cut into blocks that fit
//    on chip; the N x N matrices never reach device memory.
//  * Math-properties page, section 7: the loop keeps one query tile resident
//    (outer loop) and streams key/value tiles (inner loop); the carried state
//    is the running max, the exponential sum and the partial output.
//  * section "Block-Sparse FlashAttention": only key tiles whose mask block is
//    set are visited.
//
// gfx950 mapping.  Scores are formed transposed, S^T = K Q^T, on 32x32 MFMAs
// (A = K rows from LDS, B = the wave's Q rows kept in registers for the whole
// loop), so every lane owns one query (column) of each 32-query block and 16
// of its keys per 32-key block; its partner lane (l ^ 32) owns the other 16.
// The row max therefore needs one cross-half exchange, and P^T, converted in
// registers, is directly the B operand of O^T += V^T P^T.  V^T fragments come
// from the row-major V tile in LDS through the transposing LDS read
// (ds_read_b64_tr_b16).  Exponentials are base 2 with scale*log2(e) folded
// into one FMA.  A wave owns QB 32-query blocks: every K / V fragment read
// from LDS feeds QB MFMAs, which is what keeps LDS bandwidth below the
// matrix-core rate for d = 64.
//
// Schedule.  K and V tiles move from memory into XOR-swizzled LDS slots by
// LDS-DMA.  Iteration j overlaps (A) the PV MFMAs of tile j-1 with the
// packing / row sums of P_{j-1} and the x*c - m of tile j, then (B) the score
// MFMAs of tile j+1 with the exponentials of tile j, then (C) takes the row
// max of tile j+1.  The MFMA / vector groups are fenced so that the source
// order is the issue order.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_dropout.hpp"
#include "fa_internal.hpp"

namespace fa {

// W: wavefronts per workgroup, so B_r = 32 W queries per workgroup (64, 128
// or 256): the K / V tiles a workgroup streams through LDS serve that many
// queries, so the K / V re-reads of the tile model scale as 1 / B_r.
template <typename T, int D, bool SPARSE, int W = 4>
struct FwdCfg {
  static constexpr int E = sizeof(T);
  static constexpr int KPL = Mma<T>::KPL;
  // 32-query blocks per wavefront.  Two (each K / V fragment feeding two
  // MFMAs, half the LDS reads per MFMA, 2-wave workgroups) were measured
  // slower on gfx950 than one block per wave at three waves per SIMD
  // (16K causal 0.69 vs 0.65 ms): LDS bandwidth is not what limits this
  // kernel.  The code keeps QB general.
  static constexpr int QB = 1;
  static constexpr int WAVES = W / QB;
  static constexpr int NTHR = 64 * WAVES;
  static constexpr int QPW = 32 * QB;             // queries per wavefront
  static constexpr int BR = QPW * WAVES;          // queries per workgroup (B_r)
  static constexpr int BC = (E == 4 || QB == 2) ? 32 : 64;  // keys per LDS tile
  static constexpr int NSB = BC / 32;             // 32-key score blocks per tile
  static constexpr int NBLK = QB * NSB;           // 32x32 score blocks per wave
  static constexpr int NEL = NBLK * 16;           // score elements per lane
  static constexpr int NOB = D / 32;              // 32-wide blocks of the output
  static constexpr int KSTEPS = D / (2 * KPL);    // MFMA steps over d
  static constexpr int PSTEPS = 16 / KPL;         // MFMA steps over 32 keys
  // LDS tiles.  16-bit types: unpadded rows whose 16-byte chunks are permuted
  // by an XOR swizzle (Layout), filled straight from memory by LDS-DMA buffer
  // loads; both read patterns (K rows 16 bytes per lane down 16 consecutive
  // rows; V through the transposing read, 4 rows x 64 bytes per half-wave) are
  // then free of bank conflicts.  fp32: padded rows filled from registers.
  static constexpr bool DMA = (E == 2);
  static constexpr int ROWB = D * E;
  static constexpr int PITCH = DMA ? ROWB : ROWB + 16;
  using LT = Layout<PITCH, ROWB, DMA>;
  static constexpr int TILE = BC * PITCH;         // one K or V tile (bytes)
  static constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / NTHR;     // chunks per thread
  static_assert(BC * CPR % NTHR == 0, "tile must split evenly");
  static_assert(!SPARSE || 128 % BR == 0, "a block-sparse workgroup must lie in one mask block row");
};

constexpr int kMaxMaskBlocks = 1024;

// Slack of the running reference point, in log2 units: the stored max is
// raised only when some lane's tile max exceeds it by more than this, so the
// exponentials stay below 2^kMaxSlack.  Any reference point gives the same
// O = (sum p v) / l and LSE = m + log l in exact arithmetic; this one makes
// the rescale of the carried state rare instead of frequent.
constexpr float kMaxSlack = 8.0f;

// Scheduling fence: the compiler keeps the instructions on each side of it
// apart, so the source order of the interleaved MFMA / vector groups below is
// the issue order.
#define FA_FENCE() __builtin_amdgcn_sched_barrier(0)

// DROP: dropout on P (keep decisions regenerated per tile, see fa_dropout.hpp).
// SPLIT: the workgroup covers one of p.nsplit contiguous ranges of the key
// tiles its query tile sees and writes an fp32 partial (O_s = sum p v / l_s,
// LSE_s) for the merge kernel below.
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool SPLIT = false, int W = 4>
// d = 64: registers bounded for three waves per SIMD (the few spills this
// costs sit outside the tile loops); two with dropout, whose generator needs
// the registers.
__global__ void __launch_bounds__((FwdCfg<T, D, SPARSE, W>::NTHR), (D == 64 ? (DROP ? 2 : 3) : 1))
    fwd_kernel(AttnParams p) {
  using C = FwdCfg<T, D, SPARSE, W>;
  using M = Mma<T>;
  using frag = typename M::frag;
  using LT = typename C::LT;
  constexpr int KPL = C::KPL, E = C::E, QB = C::QB, NSB = C::NSB, NBLK = C::NBLK, NEL = C::NEL;
  using ffalse = std::integral_constant<bool, false>;
  using ftrue = std::integral_constant<bool, true>;

  // Two K slots and two V slots.  Iteration j reads V_{j-1} and K_{j+1} and
  // fills the other two slots with V_j and K_{j+2}.
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE];
  __shared__ uint16_t blist[SPARSE ? kMaxMaskBlocks : 1];
  __shared__ int nlist_s;

  const int tid = threadIdx.x, wave = tid >> 6;
  // Not const: recomputed after the steady loop (see there).
  int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nqt = (Nq + C::BR - 1) / C::BR;
  int split = 0, bh, qt;
  if constexpr (SPLIT) {
    const int logical0 = xcd_remap(blockIdx.x, gridDim.x);
    split = logical0 % p.nsplit;
    const int logical = logical0 / p.nsplit;
    bh = logical / nqt;
    qt = logical - bh * nqt;
  } else {
    tile_of(blockIdx.x, gridDim.x, nqt, CAUSAL, p.cu_fill, bh, qt);
  }
  if (CAUSAL) qt = nqt - 1 - qt;  // longest rows first
  const int b = bh / p.H, hh = bh - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)hh * p.sh;     // Q, O
  const int64_t kbase = (int64_t)b * p.ksb + (int64_t)hh * p.ksh;  // K, V
  const T *Q = static_cast<const T *>(p.q) + base;
  const T *K = static_cast<const T *>(p.k) + kbase;
  const T *V = static_cast<const T *>(p.v) + kbase;
  T *O = static_cast<T *>(p.o) + base;

  int kv_len = Nk;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), Nk);
  const int cs = CAUSAL ? p.cshift : 0;  // causal: key j visible to query i iff j <= i + cs
  const int q_tile0 = qt * C::BR;
  const int qw0 = q_tile0 + C::QPW * wave;  // first query of this wave
  // this lane's query in query block qb is qw0 + 32*qb + l32
  int kv_hi = kv_len;                       // keys >= kv_hi are invisible to the whole tile
  if (CAUSAL) kv_hi = min(kv_hi, q_tile0 + C::BR + cs);

  // ---- the list of key tiles this workgroup visits
  int ntiles;
  int tiles_per_blk = 1;
  if constexpr (SPARSE) {
    tiles_per_blk = p.mb / C::BC;
    const uint8_t *mrow = p.mask + (int64_t)hh * p.mask_hstride + (int64_t)(q_tile0 / p.mb) * p.nblk_k;
    if (wave == 0) {
      int count = 0;
      for (int j0 = 0; j0 < p.nblk_k; j0 += 64) {
        const int j = j0 + lane;
        const bool set = j < p.nblk_k && j * p.mb < kv_hi && mrow[j] != 0;
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
    ntiles = kv_hi > 0 ? (kv_hi + C::BC - 1) / C::BC : 0;
  }
  int tbase = 0;  // first tile of this workgroup's range (split-KV)
  auto tile_start = [&](int t) -> int {
    t += tbase;
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
  frag qf[QB][C::KSTEPS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw0 + 32 * qb + l32;
    if (qi < Nq) {
      const T *qrow = Q + (int64_t)qi * p.sn + h * (D / 2);
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qf[qb][s] = *reinterpret_cast<const frag *>(qrow + s * KPL);
    } else {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qf[qb][s] = frag{};
    }
  }

  // ---- K/V tiles into LDS.  Buffer loads with the tile start in the scalar
  // offset; rows past N read as zeros.  16-bit types: LDS-DMA, each wave
  // instruction writing 1 KB of the tile (lane i -> byte 16 i) and fetching
  // the chunk that the swizzle places there.  fp32: through registers.
  const uint32_t kv_bytes = (uint32_t)(((int64_t)(Nk - 1) * p.ksn + D) * E);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K, kv_bytes), vrs = make_rsrc(V, kv_bytes);
  const i32x4 kwords = rsrc_words(K, kv_bytes), vwords = rsrc_words(V, kv_bytes);
  const uint32_t lds0 = lds_addr(smem);
  const int row_bytes = (int)(p.ksn * E);
  int voff[C::CPT];
#pragma unroll
  for (int u = 0; u < C::CPT; ++u) {
    if constexpr (C::DMA) {
      const int c = 64 * (C::WAVES * u + wave) + lane;  // physical chunk
      const int row = c / C::CPR, pc = c - row * C::CPR;
      voff[u] = row * row_bytes + ((pc ^ LT::swz(row)) << 4);
    } else {
      const int c = tid + C::NTHR * u, row = c / C::CPR, col = c - row * C::CPR;
      voff[u] = row * row_bytes + col * 16;
    }
  }
  u32x4 stk[C::DMA ? 1 : C::CPT], stv[C::DMA ? 1 : C::CPT];
  auto kslot = [&](int t) -> char * { return smem + (t & 1) * C::TILE; };
  auto vslot = [&](int t) -> char * { return smem + (2 + (t & 1)) * C::TILE; };
  // fetch1: start moving part u of tile `kv0` towards LDS slot `dst` (staged
  // in `st` for fp32); commit: finish (fp32 register stores).  The caller
  // waits for the memory counter and synchronises before the slot is read.
  auto fetch1 = [&](bool is_v, u32x4 *st, char *dst, int kv0, int u) {
    const int so = __builtin_amdgcn_readfirstlane(kv0 * row_bytes);
    if constexpr (C::DMA) {
      const uint32_t la = lds0 + (uint32_t)(dst - smem) + 1024 * (C::WAVES * u + wave);
      buf_load16_lds(is_v ? vwords : kwords, __builtin_amdgcn_readfirstlane(la), voff[u], so);
    } else {
      st[u] = buf_load16(is_v ? vrs : krs, voff[u], so);
    }
  };
  auto fetch = [&](bool is_v, u32x4 *st, char *dst, int kv0) {
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) fetch1(is_v, st, dst, kv0, u);
  };
  auto commit = [&](const u32x4 *st, char *dst) {
    if constexpr (!C::DMA) {
#pragma unroll
      for (int u = 0; u < C::CPT; ++u) {
        const int c = tid + C::NTHR * u, row = c / C::CPR, col = c - row * C::CPR;
        *reinterpret_cast<u32x4 *>(dst + row * C::PITCH + col * 16) = st[u];
      }
    }
  };

  // Carried state per query block (section "Incremental softmax tracking"):
  // m_run is the reference point of the exponentials (a running max of
  // scale*log2(e)*S, raised lazily), lpart this lane's share of the
  // exponential sum (four independent partial sums), oacc the unnormalised
  // output O^T.
  float m_run[QB];
  float lpart[QB][4];
  f32x16 oacc[QB][C::NOB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) lpart[qb][q] = 0.f;
#pragma unroll
    for (int nb = 0; nb < C::NOB; ++nb) oacc[qb][nb] = f32x16{};
  }
  const float c2 = p.scale_log2;

  // Tiles that no mask touches form a prefix of the list (tiles ascend): a key
  // tile is whole for every query of the workgroup when it ends at or before
  // the padding length and (causal) at or before the tile's first query.
  const int lim = CAUSAL ? min(kv_len, q_tile0 + 1 + cs) : kv_len;
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
    n_full = min(ntiles, max(lim, 0) / C::BC);
  }
  if constexpr (SPLIT) {
    // this workgroup's range [t0, t1) of the tile list; the unmasked tiles
    // stay a prefix of it
    const int t0 = (int)((int64_t)ntiles * split / p.nsplit);
    const int t1 = (int)((int64_t)ntiles * (split + 1) / p.nsplit);
    n_full = min(max(n_full - t0, 0), t1 - t0);
    tbase = t0;
    ntiles = t1 - t0;
  }

  // Operand fragments.  K fragment i (step s = i / NSB over d, key block
  // sb = i % NSB): rows = keys, 16 bytes per lane.  V^T fragment (k, nb)
  // (key block sb = k / PSTEPS, step t = k % PSTEPS, output block nb): rows =
  // keys in register order, through the transposing read.
  auto kfrag = [&](const char *kl, int i) -> frag {
    const int s = i / NSB, sb = i - s * NSB;
    return lds_frag<T>(kl, LT::off(sb * 32 + l32, (h * (D / 2) + s * KPL) * E));
  };
  auto vfrag = [&](const char *vl, int k, int nb) -> frag {
    const int sb = k / C::PSTEPS, t = k - sb * C::PSTEPS;
    return regorder_frag<T, LT>(vl, sb * 32, t, nb * 32, lane);
  };
  constexpr int NS1 = NSB * C::PSTEPS;   // PV steps
  constexpr int NG1 = NS1 * C::NOB;      // PV groups (one V fragment, QB MFMAs each)
  constexpr int NG2 = NSB * C::KSTEPS;   // score groups (one K fragment, QB MFMAs each)
#define EL(a, e) a[(e) / 16][(e) % 16]

  // Row sums: the four bf16/f16 pairs of a P fragment go to four independent
  // partial sums (v_dot2 with ones: the sum of exactly the rounded values the
  // MFMA consumes).
  auto rowsum = [&](int qb, frag pb) {
    if constexpr (KPL == 1) {
      lpart[qb][0] += pb;
    } else {
      typedef T t2 __attribute__((ext_vector_type(2)));
      const t2 one = {(T)1.0f, (T)1.0f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const t2 v = {pb[2 * q], pb[2 * q + 1]};
        if constexpr (__is_same(T, __bf16))
          lpart[qb][q] = __builtin_amdgcn_fdot2_f32_bf16(v, one, lpart[qb][q], false);
        else
          lpart[qb][q] = __builtin_amdgcn_fdot2(v, one, lpart[qb][q], false);
      }
    }
  };

  // step 1: S^T = K_j Q_i^T for the tile whose K rows are at kl (blocks
  // b = qb*NSB + sb).
  auto scores = [&](const char *kl, f32x16 (&S)[NBLK]) {
#pragma unroll
    for (int b = 0; b < NBLK; ++b) S[b] = f32x16{};
#pragma unroll
    for (int i = 0; i < NG2; ++i) {
      const int s = i / NSB, sb = i - s * NSB;
      const frag a = kfrag(kl, i);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[qb * NSB + sb] = M::mma32(a, qf[qb][s], S[qb * NSB + sb]);
      FA_FENCE();  // bounds the operand reads in flight (register pressure)
    }
  };
  // Masking of the tile at kv0 (invisible scores -> -inf): key kv0 + o is
  // visible to the lane's query of block qb iff o < its bound.
  auto apply_mask = [&](f32x16 (&S)[NBLK], int kv0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = qw0 + 32 * qb + l32;
      const int lim_o = (CAUSAL ? min(kv_len, qi + 1 + cs) : kv_len) - kv0;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!(sb * 32 + reg_row(r, 0) + 4 * h < lim_o)) S[qb * NSB + sb][r] = -INFINITY;
    }
  };
  // steps 2-3 for the scores in S: the row max over both half-waves (four
  // independent max chains, IEEE maximum: a NaN score propagates, and no
  // NaN-quieting instruction precedes each max as for maxNum), scaled by
  // scale*log2(e).  The reference point
  // moves only when some lane's max passed it by more than the slack; then
  // the carried state -- O, the partial sums and the exponentials P of the
  // previous tile, not yet added to O -- is rescaled by exp2(old - new).
  auto update_max = [&](f32x16 (&S)[NBLK], f32x16 (&P)[NBLK], auto masked) {
    float mt[QB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int e = 0; e < NSB * 16; ++e) mx[e & 3] = __builtin_elementwise_maximum(mx[e & 3], EL(S, qb * NSB * 16 + e));
      float m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx[0], mx[1]),
                                              __builtin_elementwise_maximum(mx[2], mx[3]));
      m = __builtin_elementwise_maximum(m, xor32(m));
      mt[qb] = (decltype(masked)::value && m == -INFINITY) ? -INFINITY : m * c2;
      grow = grow || mt[qb] > m_run[qb] + kMaxSlack;
    }
    if (__ballot(grow) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = fmaxf(m_run[qb], mt[qb]);
        if (m_new != -INFINITY) {
          const float alpha = fast_exp2(m_run[qb] - m_new);
#pragma unroll
          for (int q = 0; q < 4; ++q) lpart[qb][q] *= alpha;
#pragma unroll
          for (int nb = 0; nb < C::NOB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][nb][r] *= alpha;
#pragma unroll
          for (int e = 0; e < NSB * 16; ++e) EL(P, qb * NSB * 16 + e) *= alpha;
          m_run[qb] = m_new;
        }
      }
    }
  };
  // step 4: O_i^T += V_j^T P^T for P in `P` (the tile at key kv0), plus the
  // row sums.  With dropout the row sums take P and the product P o Z (Z's
  // common factor 1 / (1 - p) is applied in the epilogue).
  const uint32_t drop_add = keep_pair_add(p.drop_thr);
  auto pv = [&](const char *vl, const f32x16 (&P)[NBLK], int kv0) {
    uint32_t keepb[QB][4];
#pragma unroll
    for (int k = 0; k < NS1; ++k) {
      const int sb = k / C::PSTEPS, t = k - sb * C::PSTEPS;
      frag pb[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (DROP) {
          if (t == 0) keep_bytes_query_col(keepb[qb], p, bh, qw0 + 32 * qb + l32, kv0 + 32 * sb, lane);
        }
        pb[qb] = pack_frag<T>(P[qb * NSB + sb], t * KPL);
        rowsum(qb, pb[qb]);
        if constexpr (DROP) pb[qb] = drop_frag<T>(pb[qb], keepb[qb], t * KPL, p.drop_thr, drop_add);
      }
#pragma unroll
      for (int nb = 0; nb < C::NOB; ++nb) {
        const frag va = vfrag(vl, k, nb);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][nb] = M::mma32(va, pb[qb], oacc[qb][nb]);
        FA_FENCE();  // bounds the operand reads in flight (register pressure)
      }
    }
  };

  // Every iteration j starts with X = S_j (scores of tile j, whose max is
  // already folded into m_run) and Y = P_{j-1} (exponentials of tile j-1,
  // already on the m_run scale) and ends with X = P_j, Y = S_{j+1}.
  //
  // Generic iteration: any mask, any visibility.  Straight-line code: a tile
  // that the wave cannot see is fully masked, so its exponentials are 0 and
  // its PV adds nothing; past the last tile everything is masked.
  auto iter_any = [&](int j, auto first, f32x16 (&X)[NBLK], f32x16 (&Y)[NBLK]) {
    fetch(true, stv, vslot(j), tile_start(j));
    fetch(false, stk, kslot(j), tile_start(min(j + 2, ntiles - 1)));
    if constexpr (!decltype(first)::value) pv(vslot(j - 1), Y, tile_start(j - 1));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_use = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
#pragma unroll
      for (int e = qb * NSB * 16; e < (qb + 1) * NSB * 16; ++e) {
        const float x = fast_exp2(fmaf(EL(X, e), c2, -m_use));
        EL(X, e) = EL(X, e) == -INFINITY ? 0.f : x;  // masked keys (also for scale 0)
      }
    }
    scores(kslot(j + 1), Y);
    apply_mask(Y, j + 1 < ntiles ? tile_start(j + 1) : kv_len);  // all masked past the end
    update_max(Y, X, ftrue{});
    commit(stv, vslot(j));
    commit(stk, kslot(j));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // Iteration j for unmasked tiles j and j+1 with j >= 1:
  //  A: PV MFMAs of tile j-1 | packing and row sums of P_{j-1}, x*c - m of
  //     tile j; the LDS-DMA of V_j and K_{j+2} is issued here too
  //  B: score MFMAs of tile j+1 | exponentials of tile j
  //  C: row max of tile j+1 and the (rare) rescale.
  // Operand reads run two groups ahead of their MFMA.  `par` is the parity of
  // j (a compile-time constant in the unrolled loop, so every LDS address is
  // a loop-invariant register plus an immediate).
  //
  // With dropout (QB = 1): KX holds the keep bytes of tile j-1, applied to the
  // PV operands as they are packed (after their row sums: l sums P, not
  // P o Z); the generator rounds for tile j's bytes (into KY, one call per
  // 32-key block) ride on the MFMA groups of both phases.
  constexpr int NGRP = NG1 + NG2;                 // MFMA groups per iteration
  static_assert(!DROP || (QB == 1 && NGRP % NSB == 0), "dropout steady iteration: one query block per wave");
  auto iter_steady = [&](int j, auto par, f32x16 (&X)[NBLK], f32x16 (&Y)[NBLK], uint32_t (&KX)[NSB][4],
                         uint32_t (&KY)[NSB][4]) {
    constexpr int P = decltype(par)::value;
    const char *vl = vslot(P ^ 1), *kl = kslot(P ^ 1);
    const int kv_v = tile_start(j), kv_k = tile_start(min(j + 2, ntiles - 1));
    float m_use[QB];  // finite: every lane sees a key of tile j
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_use[qb] = m_run[qb];
    // generator rounds of MFMA group G: block G / GB, rounds spread evenly
    constexpr int GB = NGRP / NSB;
    auto gen = [&](int G) {
      if constexpr (DROP) {
        const int sb = G / GB, g = G - sb * GB;
#pragma unroll
        for (int r = g * kPhiloxRounds / GB; r < (g + 1) * kPhiloxRounds / GB; ++r)
          philox_round(KY[sb], p.drop_key0, p.drop_key1, r);
        if (g == GB - 1) keep_finish_query_col(KY[sb], lane);
      }
    };
    if constexpr (DROP) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) keep_ctr_query_col(KY[sb], p, bh, qw0 + l32, kv_v + 32 * sb, lane);
    }
    // with DROP: row sum of the packed operand, then the keep mask
    auto drop_op = [&](frag &f, int sb, int t) {
      if constexpr (DROP) {
        rowsum(0, f);
        f = drop_frag<T>(f, KX[sb], t * KPL, p.drop_thr, drop_add);
      }
    };
    // ---- A
    frag vf[3], pbf[2][QB];
    auto vf_of = [&](int g) { return vfrag(vl, g / C::NOB, g % C::NOB); };
    vf[0] = vf_of(0);
    if (NG1 > 1) vf[1] = vf_of(1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) pbf[0][qb] = pack_frag<T>(Y[qb * NSB], 0);
    drop_op(pbf[0][0], 0, 0);
    FA_FENCE();
#pragma unroll
    for (int g = 0; g < NG1; ++g) {
      const int k = g / C::NOB, nb = g % C::NOB, cb = k & 1;
      if (g + 2 < NG1) vf[(g + 2) % 3] = vf_of(g + 2);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[qb][nb] = M::mma32(vf[g % 3], pbf[cb][qb], oacc[qb][nb]);
      // LDS-DMA of the next tiles, spread over the first groups
#pragma unroll
      for (int u = 0; u < C::CPT; ++u) {
        if (g == u % NG1) fetch1(true, stv, vslot(P), kv_v, u);
        if (g == (C::CPT + u) % NG1) fetch1(false, stk, kslot(P), kv_k, u);
      }
      if (nb == 0) {
        if (k + 1 < NS1) {
          const int sb = (k + 1) / C::PSTEPS, t = (k + 1) - sb * C::PSTEPS;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) pbf[cb ^ 1][qb] = pack_frag<T>(Y[qb * NSB + sb], t * KPL);
          drop_op(pbf[cb ^ 1][0], sb, t);
        }
        if constexpr (!DROP) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) rowsum(qb, pbf[cb][qb]);
        }
      }
#pragma unroll
      for (int e = g * NEL / NG1; e < (g + 1) * NEL / NG1; ++e)
        EL(X, e) = fmaf(EL(X, e), c2, -m_use[e / (NSB * 16)]);
      gen(g);
      FA_FENCE();
    }
    // ---- B
    frag kf[3];
    kf[0] = kfrag(kl, 0);
    if (NG2 > 1) kf[1] = kfrag(kl, 1);
    FA_FENCE();
#pragma unroll
    for (int i = 0; i < NG2; ++i) {
      const int s = i / NSB, sb = i - s * NSB;
      if (i + 2 < NG2) kf[(i + 2) % 3] = kfrag(kl, i + 2);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        Y[qb * NSB + sb] = M::mma32(kf[i % 3], qf[qb][s], s == 0 ? f32x16{} : Y[qb * NSB + sb]);
#pragma unroll
      for (int e = i * NEL / NG2; e < (i + 1) * NEL / NG2; ++e) EL(X, e) = fast_exp2(EL(X, e));
      gen(NG1 + i);
      FA_FENCE();
    }
    // ---- C
    update_max(Y, X, ffalse{});
    commit(stv, vslot(P));
    commit(stk, kslot(P));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // ---- prologue: K_0, K_1 into LDS, S_0 and its max.
  // SB holds the current tile's scores and SA the previous tile's
  // exponentials at the top of every iteration (the two arrays trade roles
  // inside an iteration; `rotate` swaps them back where needed).
  f32x16 SA[NBLK], SB[NBLK];
#pragma unroll
  for (int b = 0; b < NBLK; ++b) SA[b] = f32x16{};
  auto rotate = [&]() {
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const f32x16 t = SA[b];
      SA[b] = SB[b];
      SB[b] = t;
    }
  };
  if (ntiles > 0) {
    fetch(false, stk, kslot(0), tile_start(0));
    fetch(false, stv, kslot(1), tile_start(min(1, ntiles - 1)));
    commit(stk, kslot(0));
    commit(stv, kslot(1));
  }
  // Retire every outstanding load (Q fragments included) on all paths into
  // the loop; otherwise the compiler keeps them "pending" at the loop header.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (ntiles > 0) {
    scores(kslot(0), SB);
    apply_mask(SB, tile_start(0));
    update_max(SB, SA, ftrue{});
  }
  __syncthreads();  // K_0's slot is refilled by the first iteration

  int j = 0;
  if (ntiles > 0) {
    iter_any(j++, ftrue{}, SB, SA);
    rotate();
  }
  {
    // tiles j and j+1 unmasked; when no tile is masked, also the last tile,
    // whose successor is the last tile again (the ring fetches it once more:
    // its scores only ever raise the reference point to a max already seen)
    const int j_steady = n_full >= ntiles ? ntiles : n_full - 1;
    // Two iterations per trip restore the roles at the loop back edge, so the
    // steady loop needs no register copies.
    using odd = std::integral_constant<int, 1>;
    using even = std::integral_constant<int, 0>;
    uint32_t KA[NSB][4], KB[NSB][4];  // keep bytes of the previous / current tile (DROP)
    if (DROP && j < j_steady) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
        keep_bytes_query_col(KA[sb], p, bh, qw0 + l32, tile_start(j - 1) + 32 * sb, lane);
    }
    for (; j + 1 < j_steady; j += 2) {
      iter_steady(j, odd{}, SB, SA, KA, KB);
      iter_steady(j + 1, even{}, SA, SB, KB, KA);
    }
    if (j < j_steady) {
      iter_steady(j++, odd{}, SB, SA, KA, KB);
      rotate();
    }
  }
  // The lane indices again, from an opaque copy of the thread id: what the
  // tail iterations and the epilogue derive from them (LDS offsets, query
  // rows) is then computed here instead of being hoisted above the steady
  // loop and kept alive across it, where at this register budget it spilled.
  {
    int t = tid;
    asm volatile("" : "+v"(t));
    lane = t & 63;
    h = lane >> 5;
    l32 = lane & 31;
  }
  for (; j < ntiles; ++j) {
    iter_any(j, ffalse{}, SB, SA);
    rotate();
  }
  if (ntiles > 0) pv(vslot(ntiles - 1), SA, tile_start(ntiles - 1));
#undef EL

  // ---- epilogue: O = O / l (times 1 / (1 - p) with dropout), LSE = (m + log2 l) ln 2
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qw0 + 32 * qb + l32;
    const float l_half = (lpart[qb][0] + lpart[qb][1]) + (lpart[qb][2] + lpart[qb][3]);
    const float l_tot = l_half + xor32(l_half);
    const float inv = l_tot > 0.f ? (DROP ? p.drop_scale : 1.f) / l_tot : 0.f;
    if constexpr (SPLIT) {
      if (qi < Nq) {
        const int64_t prow = ((int64_t)split * p.B * p.H + bh) * Nq + qi;
        float *po = p.part_o + prow * D;
#pragma unroll
        for (int nb = 0; nb < C::NOB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4 *>(po + nb * 32 + 8 * i + 4 * h) =
                f32x4{oacc[qb][nb][4 * i] * inv, oacc[qb][nb][4 * i + 1] * inv,
                      oacc[qb][nb][4 * i + 2] * inv, oacc[qb][nb][4 * i + 3] * inv};
        if (h == 0) p.part_lse[prow] = l_tot > 0.f ? (m_run[qb] + log2f(l_tot)) * kLn2 : -INFINITY;
      }
      continue;
    }
    if (qi < Nq) {
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
            for (int jj = 0; jj < 4; ++jj) v[jj] = (T)(oacc[qb][nb][4 * i + jj] * inv);
            *reinterpret_cast<t4 *>(orow + d0) = v;
          }
        }
      if (h == 0)
        p.lse[(int64_t)bh * Nq + qi] = l_tot > 0.f ? (m_run[qb] + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV merge (summary page, section "Incremental softmax tracking": the
// statistics of a row split into parts combine by rescaling each part's sum
// with exp(part max - total max); here in log-sum-exp form, with each part's
// output already divided by its own sum):
//     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
// One wavefront per query row; lanes run along d.  Parts that saw no key
// carry LSE_s = -inf and weigh 0; a row no part saw gets O = 0, LSE = -inf.
template <typename T, int D>
__global__ void __launch_bounds__(256) splitkv_merge_kernel(AttnParams p) {
  constexpr int PER = D / 64;  // elements per lane
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // whole wavefronts only
  const int S = p.nsplit;
  float m = -INFINITY;
  for (int sp = 0; sp < S; ++sp) m = fmaxf(m, p.part_lse[(int64_t)sp * rows + row]);
  const int qi = (int)(row % p.Nq);
  const int64_t bh = row / p.Nq;
  const int b = (int)(bh / p.H), hh = (int)(bh % p.H);
  T *orow = static_cast<T *>(p.o) + (int64_t)b * p.sb + (int64_t)hh * p.sh + (int64_t)qi * p.sn;
  float acc[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) acc[c] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int sp = 0; sp < S; ++sp) {
      const int64_t prow = (int64_t)sp * rows + row;
      const float w = expf(p.part_lse[prow] - m);  // exp(-inf) = 0 for empty parts
      wsum += w;
      const float *po = p.part_o + prow * D;
#pragma unroll
      for (int c = 0; c < PER; ++c) acc[c] = fmaf(w, po[lane + 64 * c], acc[c]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int c = 0; c < PER; ++c) orow[lane + 64 * c] = (T)(acc[c] * inv);
  if (lane == 0) p.lse[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool SPLIT = false, int W = 4>
static hipError_t launch_fwd_t(const AttnParams &p, hipStream_t s) {
  using C = FwdCfg<T, D, SPARSE, W>;
  const int64_t nqt = (p.Nq + C::BR - 1) / C::BR;
  const int64_t grid = (int64_t)p.B * p.H * nqt * (SPLIT ? p.nsplit : 1);
  const void *fn = reinterpret_cast<const void *>(&fwd_kernel<T, D, CAUSAL, SPARSE, DROP, SPLIT, W>);
  static const int fill = resident_per_cu(fn, C::NTHR);
  AttnParams a = p;
  a.cu_fill = fill;
  void *args[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(C::NTHR), args, 0, s);
}

template <typename T, int D, bool DROP, int W>
static hipError_t launch_fwd_w(const AttnParams &p, bool sparse, hipStream_t s) {
  if (sparse) {
    if constexpr (128 % (32 * W) == 0)
      return p.causal ? launch_fwd_t<T, D, true, true, DROP, false, W>(p, s)
                      : launch_fwd_t<T, D, false, true, DROP, false, W>(p, s);
    return hipErrorInvalidValue;  // refused by the argument checks
  }
  return p.causal ? launch_fwd_t<T, D, true, false, DROP, false, W>(p, s)
                  : launch_fwd_t<T, D, false, false, DROP, false, W>(p, s);
}

// Query tile: 128 unless the caller asked for 64 or 256 (16-bit types without
// dropout only; the argument checks refuse the other combinations).
template <typename T, int D, bool DROP>
static hipError_t launch_fwd_dd(const AttnParams &p, bool sparse, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && !DROP) {
    if (p.qtile == 64) return launch_fwd_w<T, D, DROP, 2>(p, sparse, s);
    if (p.qtile == 256) return launch_fwd_w<T, D, DROP, 8>(p, sparse, s);
  }
  return launch_fwd_w<T, D, DROP, 4>(p, sparse, s);
}

template <typename T, int D>
static hipError_t launch_fwd_d(const AttnParams &p, bool sparse, hipStream_t s) {
  return p.drop_thr ? launch_fwd_dd<T, D, true>(p, sparse, s) : launch_fwd_dd<T, D, false>(p, sparse, s);
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

template <typename T, int D>
static hipError_t launch_splitkv_d(const AttnParams &p, bool sparse, hipStream_t s) {
  hipError_t e;
  if (sparse)
    e = p.causal ? launch_fwd_t<T, D, true, true, false, true>(p, s)
                 : launch_fwd_t<T, D, false, true, false, true>(p, s);
  else
    e = p.causal ? launch_fwd_t<T, D, true, false, false, true>(p, s)
                 : launch_fwd_t<T, D, false, false, false, true>(p, s);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  AttnParams a = p;
  void *args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void *>(&splitkv_merge_kernel<T, D>),
                         dim3((unsigned)((rows + 3) / 4)), dim3(256), args, 0, s);
}

template <typename T>
static hipError_t launch_splitkv_dt(const AttnParams &p, bool sparse, hipStream_t s) {
  return p.d == 64 ? launch_splitkv_d<T, 64>(p, sparse, s) : launch_splitkv_d<T, 128>(p, sparse, s);
}

hipError_t launch_fwd_splitkv(const AttnParams &p, fa_dtype_t dt, bool sparse, hipStream_t s) {
  switch (dt) {
    case FA_DTYPE_F32: return launch_splitkv_dt<float>(p, sparse, s);
    case FA_DTYPE_F16: return launch_splitkv_dt<_Float16>(p, sparse, s);
    case FA_DTYPE_BF16: return launch_splitkv_dt<__bf16>(p, sparse, s);
  }
  return hipErrorInvalidValue;
}

int fwd_key_tile(fa_dtype_t dt) {
  return dt == FA_DTYPE_F32 ? FwdCfg<float, 64, false>::BC : FwdCfg<__bf16, 64, false>::BC;
}

}  // namespace fa
