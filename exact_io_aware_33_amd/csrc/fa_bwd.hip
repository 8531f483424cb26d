// Backward pass of exact attention on gfx950.
//
// Method.  FlashAttention summary page (paper 2205.14135), section "Key
// ideas", recomputation bullet: the backward pass keeps no N x N matrix; it
// rebuilds S and P tile by tile on chip from Q, K, V and the saved softmax
// statistics (kept here as LSE, so P = exp(S*scale - LSE)).  The gradient
// formulas are the analytic derivatives of O = softmax(scale Q K^T) V for the
// loss <dO, O> (the pages do not print them):
//     dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij = sum_c dO_ic O_ic,
//     dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// Block-sparse section of the same page: zero mask blocks are skipped here too.
// With dropout (O = (P o Z) V, Z regenerated from the same Philox counters as
// the forward's, fa_dropout.hpp) the same derivation with Z held fixed gives
//     dV = (P o Z)^T dO,  dS = P * (Z o dP - D),  D_i = sum_c dO_ic O_ic
// (D is unchanged in form: sum_j P_ij Z_ij dP_ij = dO_i . O_i).  In those
// instances (DROP) the steady iterations generate the next block's keep
// bytes while the current block is processed.
//
// Kernels (all on the caller's stream):
//  1. bwd_pre:   D = rowsum(dO * O) per query row (the only workspace: one
//                float per row, O(N) extra memory).
//  2. bwd_main:  dK and dV.  One workgroup per (batch, head, 128-key tile), one
//                wavefront per 32 keys; K and V rows of the wave stay in
//                registers, query blocks of 32 rows (Q, dO, LSE, D) stream
//                through LDS.  Per block: S = Q K^T and dP = dO V^T on 32x32
//                MFMAs (rows = queries in register order), P and dS in fp32,
//                then dV^T += dO^T P and dK^T += Q^T dS with P and dS fed back
//                from registers and dO^T / Q^T read through the transposing
//                LDS read.
//  3. bwd_dq:    dQ.  One workgroup per (batch, head, 128-query tile), laid out
//                like the forward: each lane owns one query; S^T = K Q^T and
//                dP^T = V dO^T per key tile, dS^T in registers, then
//                dQ^T += K^T dS^T with K^T read through the transposing LDS
//                read.  dQ is written once per row: no atomics, and the result
//                does not depend on scheduling.
// bwd_main and bwd_dq both read D and are independent of each other.  The
// full sequence (fa_bwd) is two launches: bwd_dq with dq_pre set does step 1
// for its own queries (bitwise as bwd_pre does it) and fills the workspace,
// then bwd_main; bwd_pre runs when a caller asks for that stage alone.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_dropout.hpp"
#include "fa_internal.hpp"

namespace fa {

constexpr int kMaxMaskBlocksB = 1024;

// Scheduling fence: the compiler keeps the instructions on each side of it
// apart, so the source order of interleaved MFMA / vector groups is the issue
// order.
#define FA_FENCE() __builtin_amdgcn_sched_barrier(0)


// ---------------------------------------------------------------------------
// 1. -D = -rowsum(dO * O) and LSE * log2(e).  A row of O and of dO is
// D * sizeof(T) / 16 (8, 16 or 32) sixteen-byte chunks; that many adjacent
// lanes take one chunk each, so a wave reads whole consecutive rows (every
// load instruction is one contiguous run of memory), and the partial dot
// products meet by xor shuffles inside the lane group.
template <typename T, int D>
struct PreCfg {
  static constexpr int LPR = D * (int)sizeof(T) / 16;  // lanes per row
  static constexpr int RPB = 256 / LPR;                // rows per workgroup
};
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(AttnParams p) {
  using C = PreCfg<T, D>;
  constexpr int EPC = 16 / (int)sizeof(T);
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  const int64_t row = (int64_t)blockIdx.x * C::RPB + threadIdx.x / C::LPR;
  const int c = (int)(threadIdx.x % C::LPR);
  // LPR divides 64: a lane group lies in one wave and leaves together
  if (row >= rows) return;
  const int n = (int)(row % p.Nq);
  const int64_t bh = row / p.Nq;
  const int b = (int)(bh / p.H), hh = (int)(bh % p.H);
  const int64_t off = (int64_t)b * p.sb + (int64_t)hh * p.sh + (int64_t)n * p.sn;
  const char *o = reinterpret_cast<const char *>(static_cast<const T *>(p.o_in) + off);
  const char *g = reinterpret_cast<const char *>(static_cast<const T *>(p.dout) + off);
  const u32x4 a = ldg16(o + 16 * c), bq = ldg16(g + 16 * c);
  const T *ta = reinterpret_cast<const T *>(&a);
  const T *tb = reinterpret_cast<const T *>(&bq);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc = fmaf((float)ta[e], (float)tb[e], acc);
#pragma unroll
  for (int w = C::LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w);
  if (c != 0) return;
  // stored negated: the dP MFMAs accumulate onto it (acc = dP - D)
  p.ws_negd[row] = -acc;
  // the saved statistics in the base-2 domain: P = exp2(S*scale*log2e - lse2);
  // a row that sees no key (LSE = -inf) gets +inf, so its P is 0
  const float l = p.lse[row];
  p.ws_lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
}

// ---------------------------------------------------------------------------
// 2. dK, dV (key-stationary).
template <typename T, int D>
struct BwdCfg {
  static constexpr int E = sizeof(T);
  static constexpr int KPL = Mma<T>::KPL;
  static constexpr int WAVES = 4;
  static constexpr int BKC = 32 * WAVES;        // keys per workgroup
  static constexpr int BQ = 32;                 // queries per block
  static constexpr int KSTEPS = D / (2 * KPL);  // 32x32 MFMA steps over d
  static constexpr int TSTEPS = 16 / KPL;       // 32x32 MFMA steps over 32 queries
  static constexpr int NOB = D / 32;            // 32-wide d blocks of dK, dV
  // Q / dO rows are read two ways: 16 bytes per lane down 16 rows (MFMA A
  // operand) and 4 rows x 64 bytes per half-wave (transposing read).  No
  // padding is conflict-free for both, so 16-bit rows are unpadded with
  // XOR-swizzled 16-byte chunks (Layout) and arrive by LDS-DMA; fp32 rows are
  // padded by 16 bytes and staged through registers.
  static constexpr bool DMA = (E == 2);
  static constexpr int ROWB = D * E;
  static constexpr int PITCH = DMA ? ROWB : ROWB + 16;
  static constexpr int QBYTES = BQ * PITCH;     // one Q (or dO) block
  // One slot: Q block, dO block, then lse*log2(e) and -D of 64 rows (one
  // 4-byte LDS-DMA; the first 32 belong to the block).
  static constexpr int LSE_OFF = 2 * QBYTES, D_OFF = LSE_OFF + 256;
  static constexpr int SLOT = 2 * QBYTES + 512;
  // Ring of query blocks in LDS: iteration i reads blocks i and i+1 while
  // blocks i+2 (landed or landing) and i+3 (requested now) are in flight.
  static constexpr int NSLOT = 4;
  static constexpr int AHEAD = 3;
  // vector-memory operations per wave per fetched block (16-bit: all DMA)
  static constexpr int FETCH_OPS = 2 * (BQ * ROWB / 16 / (64 * WAVES)) + 1;
  static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
  static constexpr int CPTQ = BQ * CPR / (64 * WAVES);  // chunks per thread per tensor
  static_assert(BQ * CPR % (64 * WAVES) == 0, "query block must split evenly");
};

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ void __launch_bounds__(256) bwd_main_kernel(AttnParams p) {
  using C = BwdCfg<T, D>;
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KPL = C::KPL, E = C::E;
  using LQ = Layout<C::PITCH, C::ROWB, C::DMA>;
  using ffalse = std::integral_constant<bool, false>;
  using ftrue = std::integral_constant<bool, true>;

  __shared__ __attribute__((aligned(1024))) char smem[C::NSLOT * C::SLOT];
  __shared__ uint16_t blist[SPARSE ? kMaxMaskBlocksB : 1];
  __shared__ int nlist_s;

  // the wave index is made explicitly uniform (it selects scalar operands)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nkt = (Nk + C::BKC - 1) / C::BKC;
  int bh, kt;  // causal: key tile 0 sees the most queries, so rank = kt is longest first
  tile_of(blockIdx.x, gridDim.x, nkt, CAUSAL, p.cu_fill, bh, kt);
  const int b = bh / p.H, hh = bh - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)hh * p.sh;     // Q, dO
  const int64_t kbase = (int64_t)b * p.ksb + (int64_t)hh * p.ksh;  // K, V, dK, dV
  const T *Q = static_cast<const T *>(p.q) + base;
  const T *K = static_cast<const T *>(p.k) + kbase;
  const T *V = static_cast<const T *>(p.v) + kbase;
  const T *dO = static_cast<const T *>(p.dout) + base;
  T *dK = static_cast<T *>(p.dk) + kbase;
  T *dV = static_cast<T *>(p.dv) + kbase;
  const float *LSE = p.lse + (int64_t)bh * Nq;
  const float *negD = p.ws_negd + (int64_t)bh * Nq;

  int kv_len = Nk;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), Nk);
  const int cs = CAUSAL ? p.cshift : 0;  // causal: key j visible to query i iff i >= j - cs
  const int k0 = kt * C::BKC;
  const int kw0 = k0 + 32 * wave;  // first key of this wave
  const int key = kw0 + l32;       // this lane's key (column of S)

  // dV accumulates (P o Z / (1 - p))^T dO: the common factor goes here.
  const float vscale = DROP ? p.drop_scale : 1.f;
  auto store_dkdv = [&](const f32x16 *dkacc, const f32x16 *dvacc) {
    if (key >= Nk) return;
    T *krow = dK + (int64_t)key * p.ksn;
    T *vrow = dV + (int64_t)key * p.ksn;
#pragma unroll
    for (int nb = 0; nb < C::NOB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = nb * 32 + 8 * i + 4 * h;
        if constexpr (E == 4) {
          *reinterpret_cast<f32x4 *>(krow + d0) =
              f32x4{dkacc[nb][4 * i] * p.scale, dkacc[nb][4 * i + 1] * p.scale,
                    dkacc[nb][4 * i + 2] * p.scale, dkacc[nb][4 * i + 3] * p.scale};
          *reinterpret_cast<f32x4 *>(vrow + d0) =
              f32x4{dvacc[nb][4 * i] * vscale, dvacc[nb][4 * i + 1] * vscale,
                    dvacc[nb][4 * i + 2] * vscale, dvacc[nb][4 * i + 3] * vscale};
        } else {
          typedef T t4 __attribute__((ext_vector_type(4)));
          t4 kv4, vv4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            kv4[j] = (T)(dkacc[nb][4 * i + j] * p.scale);
            vv4[j] = (T)(dvacc[nb][4 * i + j] * vscale);
          }
          *reinterpret_cast<t4 *>(krow + d0) = kv4;
          *reinterpret_cast<t4 *>(vrow + d0) = vv4;
        }
      }
  };

  f32x16 dkacc[C::NOB], dvacc[C::NOB];
#pragma unroll
  for (int nb = 0; nb < C::NOB; ++nb) {
    dkacc[nb] = f32x16{};
    dvacc[nb] = f32x16{};
  }

  // Key tile entirely beyond the padding length: every gradient row is zero.
  if (k0 >= kv_len) {
    store_dkdv(dkacc, dvacc);
    return;
  }

  // ---- the list of query blocks this workgroup visits
  const int nqb_all = (Nq + C::BQ - 1) / C::BQ;
  int nq, first_skip = 0, per = 1;
  if constexpr (SPARSE) {
    per = p.mb / C::BQ;
    const int kb = k0 / p.mb;
    const uint8_t *mcol = p.mask + (int64_t)hh * p.mask_hstride + kb;
    if (wave == 0) {
      int count = 0;
      for (int i0 = 0; i0 < p.nblk_q; i0 += 64) {
        const int i = i0 + lane;
        // causal: query block i reaches this key tile iff its last query
        // sees the tile's first key
        const bool set = i < p.nblk_q && (!CAUSAL || (i + 1) * p.mb - 1 + cs >= k0) &&
                         mcol[(int64_t)i * p.nblk_k] != 0;
        const uint64_t bal = __ballot(set);
        if (set) blist[count + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)i;
        count += __popcll(bal);
      }
      if (lane == 0) nlist_s = count;
    }
    __syncthreads();
    const int nl = nlist_s;
    // causal: queries below k0 - cs see no key of this tile
    if (CAUSAL && nl > 0) first_skip = min(per, max(0, k0 - cs - (int)blist[0] * p.mb) / C::BQ);
    nq = nl * per - first_skip;
  } else {
    first_skip = CAUSAL ? max(0, k0 - cs) / C::BQ : 0;
    nq = max(0, nqb_all - first_skip);
  }
  auto qblock_start = [&](int t) -> int {
    const int u = t + first_skip;
    if constexpr (SPARSE) {
      const int bi = u / per;
      return (int)blist[bi] * p.mb + (u - bi * per) * C::BQ;
    } else {
      return u * C::BQ;
    }
  };

  // ---- K, V rows of this wave as the B operands of S and dP
  frag kf[C::KSTEPS], vf[C::KSTEPS];
  if (key < Nk) {
    const T *kr = K + (int64_t)key * p.ksn + h * (D / 2);
    const T *vr = V + (int64_t)key * p.ksn + h * (D / 2);
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      kf[s] = *reinterpret_cast<const frag *>(kr + s * KPL);
      vf[s] = *reinterpret_cast<const frag *>(vr + s * KPL);
    }
  } else {
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      kf[s] = frag{};
      vf[s] = frag{};
    }
  }

  // ---- query blocks into the LDS ring (block t -> slot t % NSLOT).  Q, dO:
  // buffer loads with the block start in the scalar offset, rows past N read
  // as zeros (16-bit: LDS-DMA, fp32: through registers).  lse*log2(e) and -D
  // from the workspace by 4-byte LDS-DMA (waves 0 and 2 the one, 1 and 3 the
  // other, so every wave issues the same number of operations).  Rows past N
  // read zeros there too: with zero Q and dO rows they add nothing to dK, dV.
  const uint32_t q_bytes = (uint32_t)(((int64_t)(Nq - 1) * p.sn + D) * E);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q, q_bytes), dors = make_rsrc(dO, q_bytes);
  const i32x4 qwords = rsrc_words(Q, q_bytes), dowords = rsrc_words(dO, q_bytes);
  const i32x4 statwords = (wave & 1) ? rsrc_words(negD, (uint32_t)Nq * 4u)
                                     : rsrc_words(p.ws_lse2 + (int64_t)bh * Nq, (uint32_t)Nq * 4u);
  const uint32_t lds0 = lds_addr(smem);
  const int row_bytes = (int)(p.sn * E);
  int voff[C::CPTQ];
#pragma unroll
  for (int u = 0; u < C::CPTQ; ++u) {
    if constexpr (C::DMA) {
      const int c = 64 * (C::WAVES * u + wave) + lane;  // physical chunk
      const int row = c / C::CPR, pc = c - row * C::CPR;
      voff[u] = row * row_bytes + ((pc ^ LQ::swz(row)) << 4);
    } else {
      const int c = tid + 256 * u, row = c / C::CPR, col = c - row * C::CPR;
      voff[u] = row * row_bytes + col * 16;
    }
  }
  u32x4 sq[C::DMA ? 1 : C::CPTQ], sdo[C::DMA ? 1 : C::CPTQ];
  auto slot = [&](int t) -> char * { return smem + (t & (C::NSLOT - 1)) * C::SLOT; };
  // fetch1: part u of query block t (clamped to the list; u = CPTQ is the
  // statistics); commit: finish the fp32 register staging before the barrier.
  // Past the end of the list the last block is fetched again, into the
  // block's own ring slot (free: its previous block was consumed).
  auto fetch1 = [&](int t, int u) {
    const int q0 = qblock_start(min(t, nq - 1));
    const uint32_t la = lds0 + (uint32_t)(slot(t) - smem);
    if (u == C::CPTQ) {
      buf_load4_lds(statwords, __builtin_amdgcn_readfirstlane(la + ((wave & 1) ? C::D_OFF : C::LSE_OFF)),
                    lane * 4, __builtin_amdgcn_readfirstlane(q0 * 4));
      return;
    }
    const int so = __builtin_amdgcn_readfirstlane(q0 * row_bytes);
    if constexpr (C::DMA) {
      const uint32_t lu = la + 1024 * (C::WAVES * u + wave);
      buf_load16_lds(qwords, __builtin_amdgcn_readfirstlane(lu), voff[u], so);
      buf_load16_lds(dowords, __builtin_amdgcn_readfirstlane(lu + C::QBYTES), voff[u], so);
    } else {
      sq[u] = buf_load16(qrs, voff[u], so);
      sdo[u] = buf_load16(dors, voff[u], so);
    }
  };
  auto fetch = [&](int t) {
#pragma unroll
    for (int u = 0; u <= C::CPTQ; ++u) fetch1(t, u);
  };
  auto commit = [&](int t) {
    if constexpr (!C::DMA) {
      char *ql = slot(t);
#pragma unroll
      for (int u = 0; u < C::CPTQ; ++u) {
        const int c = tid + 256 * u, row = c / C::CPR, col = c - row * C::CPR;
        *reinterpret_cast<u32x4 *>(ql + LQ::off(row, col * 16)) = sq[u];
        *reinterpret_cast<u32x4 *>(ql + C::QBYTES + LQ::off(row, col * 16)) = sdo[u];
      }
    }
  };
  // End of an iteration: the block fetched one iteration ago has landed (the
  // one requested in this iteration may still be in flight), and every wave
  // is done with the slot that the next iteration refills.
  auto sync_ring = [&]() {
    if constexpr (C::DMA) __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::FETCH_OPS));
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  const float c2 = p.scale_log2;
  // Operand fragments from a slot.  qfrag(i): step s = i / 2 over d, tensor
  // i % 2 (0 = Q, 1 = dO): rows = queries, 16 bytes per lane.  tfrag(g):
  // step t = g / (2 NOB) over queries, output block nb, tensor (0 = dO for
  // dV, 1 = Q for dK): rows = queries in register order, through the
  // transposing read.
  auto qfrag = [&](const char *ql, int i) -> frag {
    const int s = i >> 1, which = i & 1;
    return lds_frag<T>(ql + which * C::QBYTES, LQ::off(l32, (h * (D / 2) + s * KPL) * E));
  };
  auto tfrag = [&](const char *ql, int g) -> frag {
    const int t = g / (2 * C::NOB), nb = (g >> 1) % C::NOB, which = g & 1;
    return regorder_frag<T, LQ>(ql + (which ? 0 : C::QBYTES), 0, t, nb * 32);
  };
  constexpr int NGA = 2 * C::KSTEPS;            // S / dP MFMAs per block
  constexpr int NGB = 2 * C::TSTEPS * C::NOB;   // dV / dK MFMAs per block
  // Issue order of the S / dP MFMAs: three S steps first (so the -D addend of
  // the first dP step has time to arrive from LDS), then dP and S alternate.
  // Returns the qfrag index 2 s + tensor.
  auto sdp_order = [](int g) constexpr -> int {
    constexpr int K = C::KSTEPS;
    if (g < 3) return 2 * g;
    if (g < 3 + 2 * (K - 3)) {
      const int k = g - 3;
      return (k & 1) ? 2 * (3 + k / 2) : 2 * (k / 2) + 1;
    }
    return 2 * ((K - 3) + (g - 3 - 2 * (K - 3))) + 1;
  };
  // -D of the block's 32 rows in register order (the addend of the first dP
  // MFMA: the accumulator then holds dP - D)
  auto load_negd = [&](const char *qs) -> f32x16 {
    const float *dd = reinterpret_cast<const float *>(qs + C::D_OFF);
    f32x16 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(dd + 8 * q + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) r[4 * q + j] = v[j];
    }
    return r;
  };

  // S = Q K^T, dP = dO V^T for the block in `ql` (rows = queries in register
  // order, column = this lane's key).
  auto sdp = [&](const char *ql, f32x16 &S, f32x16 &DP) {
    S = f32x16{};
    if constexpr (DROP) DP = f32x16{};  // dP alone: -D enters after the keep factor
    else DP = load_negd(ql);
#pragma unroll
    for (int i = 0; i < NGA; ++i) {
      const int s = i >> 1;
      if (i & 1) DP = M::mma32(qfrag(ql, i), vf[s], DP);
      else S = M::mma32(qfrag(ql, i), kf[s], S);
      FA_FENCE();  // bounds the operand reads in flight (register pressure)
    }
  };
  // P = exp2(S*scale*log2e - LSE*log2e), dS = P (dP - D) with DP = dP - D
  // already, in place; with MASK, invisible (query, key) pairs get
  // P = dS = 0.
  // With DROP (DP = dP): P o Z / (1 - p) into S and dS = P (Z dP - D) into DP.
  auto softmax_grad = [&](const char *ql, int q0, f32x16 &S, f32x16 &DP, auto masked) {
    const float *ll = reinterpret_cast<const float *>(ql + C::LSE_OFF);
    const float *dd = reinterpret_cast<const float *>(ql + C::D_OFF);
    const int lim_q = CAUSAL ? key - cs - q0 : -1;  // query row qr visible iff qr >= lim_q
    uint32_t keepb[4];
    if constexpr (DROP) keep_bytes_key_col(keepb, p, bh, q0, key, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(ll + 8 * i + 4 * h);
      f32x4 nd4;
      if constexpr (DROP) nd4 = *reinterpret_cast<const f32x4 *>(dd + 8 * i + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * i + j;
        float pv = fast_exp2(fmaf(S[r], c2, -l4[j]));
        if constexpr (decltype(masked)::value) {
          if (!(key < kv_len && reg_row(r, h) >= lim_q)) pv = 0.f;
        }
        if constexpr (DROP) {
          const bool kp = kept(keepb, r, p.drop_thr);
          S[r] = kp ? pv : 0.f;
          DP[r] = pv * fmaf(kp ? p.drop_scale : 0.f, DP[r], nd4[j]);
        } else {
          S[r] = pv;
          DP[r] = pv * DP[r];
        }
      }
    }
  };
  // dV^T += dO^T P, dK^T += Q^T dS (rows = d, column = this lane's key).
  auto dvdk = [&](const char *ql, const f32x16 &P, const f32x16 &DS) {
#pragma unroll
    for (int t = 0; t < C::TSTEPS; ++t) {
      const frag pb = pack_frag<T>(P, t * KPL);
      const frag sb = pack_frag<T>(DS, t * KPL);
#pragma unroll
      for (int nb = 0; nb < C::NOB; ++nb) {
        const int g = 2 * (t * C::NOB + nb);
        dvacc[nb] = M::mma32(tfrag(ql, g), pb, dvacc[nb]);
        dkacc[nb] = M::mma32(tfrag(ql, g + 1), sb, dkacc[nb]);
        FA_FENCE();  // bounds the operand reads in flight (register pressure)
      }
    }
  };

  // Every iteration i starts with (SX, DX) = (S_i, dP_i) and ends with
  // (SX, DX) = (P_i, dS_i) consumed and (SY, DY) = (S_{i+1}, dP_{i+1}).
  //
  // Generic iteration: any mask.  Straight-line code; past the last block the
  // next-block products are computed on a repeated block and never used.
  // `masked` false: block i is unmasked, the per-element mask is left out.
  auto iter_any = [&](int i, auto masked, f32x16 &SX, f32x16 &DX, f32x16 &SY, f32x16 &DY) {
    fetch(i + C::AHEAD);
    const char *ql = slot(i), *qn = slot(i + 1);
    softmax_grad(ql, qblock_start(i), SX, DX, masked);
    sdp(qn, SY, DY);
    dvdk(ql, SX, DX);
    commit(i + C::AHEAD);
    sync_ring();
  };
  // Iteration i for an unmasked block i, as one sequence of
  // MFMA groups (NGA score / dP MFMAs of block i+1, then NGB dV / dK MFMAs of
  // block i), each paired with a slice of the vector work of block i:
  //  during the score MFMAs: P, dS of the first 8 rows (register order), then
  //    the packing of step 0;
  //  during the first half of the dV / dK MFMAs: P, dS of the last 8 rows,
  //    and the packing of step t+1 at the end of step t.
  // Operand reads run two groups ahead of their MFMA; the next block's
  // LDS-DMA is spread over the first groups.  `par` is i mod NSLOT (a
  // compile-time constant in the unrolled loop, so every LDS address is a
  // loop-invariant register plus an immediate).  For the last block the
  // next-block products are computed on the repeated last block (the ring
  // fetches it again past the end) and never used, as in the generic
  // iteration.
  // With DROP, KX holds the keep bytes of block i (its dP MFMAs started from
  // 0, -D enters per row as in softmax_grad) and the generator rounds for
  // block i+1's bytes (into KY) ride one per MFMA group.
  static_assert(!DROP || NGA + NGB >= kPhiloxRounds, "one generator round per MFMA group");
  auto iter_steady = [&](int i, auto par, f32x16 &SX, f32x16 &DX, f32x16 &SY, f32x16 &DY,
                         uint32_t (&KX)[4], uint32_t (&KY)[4]) {
    constexpr int P = decltype(par)::value;
    char *const ql = smem + P * C::SLOT;
    char *const qn = smem + ((P + 1) % C::NSLOT) * C::SLOT;
    const float *ll = reinterpret_cast<const float *>(ql + C::LSE_OFF);
    const float *dd = reinterpret_cast<const float *>(ql + C::D_OFF);
    f32x4 l4[2], nd4[2];
    // P, dS of row r (quad q = r / 4 prefetched one quad ahead)
    auto row = [&](int r) {
      const int q = r >> 2, j = r & 3;
      if (j == 0 && q + 1 < 4) {
        l4[(q + 1) & 1] = *reinterpret_cast<const f32x4 *>(ll + 8 * (q + 1) + 4 * h);
        if constexpr (DROP) nd4[(q + 1) & 1] = *reinterpret_cast<const f32x4 *>(dd + 8 * (q + 1) + 4 * h);
      }
      const float pv = fast_exp2(fmaf(SX[r], c2, -l4[q & 1][j]));
      if constexpr (DROP) {
        const bool kp = kept(KX, r, p.drop_thr);
        SX[r] = kp ? pv : 0.f;
        DX[r] = pv * fmaf(kp ? p.drop_scale : 0.f, DX[r], nd4[q & 1][j]);
      } else {
        SX[r] = pv;
        DX[r] = pv * DX[r];
      }
    };
    auto gen = [&](int grp) {
      if constexpr (DROP) {
        if (grp < kPhiloxRounds) philox_round(KY, p.drop_key0, p.drop_key1, grp);
        if (grp == kPhiloxRounds - 1) keep_finish_key_col(KY, lane);
      }
    };
    if constexpr (DROP) keep_ctr_key_col(KY, p, bh, qblock_start(min(i + 1, nq - 1)), key, lane);
    // ---- score / dP MFMAs of block i+1
    frag af[3];
    af[0] = qfrag(qn, sdp_order(0));
    af[1] = qfrag(qn, sdp_order(1));
    const f32x16 negd_n = DROP ? f32x16{} : load_negd(qn);
    l4[0] = *reinterpret_cast<const f32x4 *>(ll + 4 * h);
    if constexpr (DROP) nd4[0] = *reinterpret_cast<const f32x4 *>(dd + 4 * h);
    SY = f32x16{};
    FA_FENCE();
#pragma unroll
    for (int g = 0; g < NGA; ++g) {
      const int fi = sdp_order(g), s = fi >> 1;
      if (g + 2 < NGA) af[(g + 2) % 3] = qfrag(qn, sdp_order(g + 2));
      if (fi & 1) DY = M::mma32(af[g % 3], vf[s], s == 0 ? negd_n : DY);
      else SY = M::mma32(af[g % 3], kf[s], SY);
      if (g <= C::CPTQ) fetch1(i + C::AHEAD, g);
#pragma unroll
      for (int r = 8 * g / NGA; r < 8 * (g + 1) / NGA; ++r) row(r);
      gen(g);
      FA_FENCE();
    }
    // ---- dV / dK MFMAs of block i
    frag tf[3], pb[2], sbf[2];
    tf[0] = tfrag(ql, 0);
    tf[1] = tfrag(ql, 1);
    pb[0] = pack_frag<T>(SX, 0);
    sbf[0] = pack_frag<T>(DX, 0);
    FA_FENCE();
#pragma unroll
    for (int g = 0; g < NGB; ++g) {
      const int t = g / (2 * C::NOB), nb = (g >> 1) % C::NOB;
      if (g + 2 < NGB) tf[(g + 2) % 3] = tfrag(ql, g + 2);
      if (g & 1) dkacc[nb] = M::mma32(tf[g % 3], sbf[t & 1], dkacc[nb]);
      else dvacc[nb] = M::mma32(tf[g % 3], pb[t & 1], dvacc[nb]);
      if (g < NGB / 2) {
#pragma unroll
        for (int r = 8 + 8 * g / (NGB / 2); r < 8 + 8 * (g + 1) / (NGB / 2); ++r) row(r);
      }
      if (g % (2 * C::NOB) == 2 * C::NOB - 1 && t + 1 < C::TSTEPS) {
        // the next step's operands, once its rows are done
        pb[(t + 1) & 1] = pack_frag<T>(SX, (t + 1) * KPL);
        sbf[(t + 1) & 1] = pack_frag<T>(DX, (t + 1) * KPL);
      }
      gen(NGA + g);
      FA_FENCE();
    }
    commit(i + C::AHEAD);
    sync_ring();
  };

  // ---- prologue: the first AHEAD blocks into the ring, S_0 and dP_0.
  f32x16 SA, DA, SB, DB;
  if (nq > 0) {
#pragma unroll
    for (int t = 0; t < C::AHEAD; ++t) {
      fetch(t);
      commit(t);
    }
  }
  // Retire every outstanding load (K/V operands included) on all paths into
  // the loop, so the compiler does not wait on a later prefetch inside it.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nq > 0) sdp(slot(0), SA, DA);

  // Blocks some mask touches come first: the causal diagonal (queries before
  // the end of this key tile), or every block when the key tile crosses the
  // padding length.
  int n_masked = 0;
  if (k0 + C::BKC > kv_len) {
    n_masked = nq;
  } else if (CAUSAL) {
    while (n_masked < nq && qblock_start(n_masked) < k0 + C::BKC - cs) ++n_masked;
  }
  // (SA, DA) holds the current block's products at the top of every trip.
  auto swap_ab = [&]() {
    const f32x16 ts = SA, td = DA;
    SA = SB;
    DA = DB;
    SB = ts;
    DB = td;
  };
  int i = 0;
  for (; i < n_masked && i < nq; ++i) {
    iter_any(i, ftrue{}, SA, DA, SB, DB);
    swap_ab();
  }
  // Steady blocks in trips of NSLOT (so the slots are compile-time
  // constants); the trip must start at a block index that is 0 mod NSLOT.
  {
    for (; i < nq - 1 && (i & (C::NSLOT - 1)) != 0; ++i) {
      iter_any(i, ffalse{}, SA, DA, SB, DB);
      swap_ab();
    }
    using s0 = std::integral_constant<int, 0>;
    using s1 = std::integral_constant<int, 1>;
    using s2 = std::integral_constant<int, 2>;
    using s3 = std::integral_constant<int, 3>;
    uint32_t KA[4], KB[4];  // keep bytes of the current / next block (DROP)
    if (DROP && i + C::NSLOT <= nq) keep_bytes_key_col(KA, p, bh, qblock_start(i), key, lane);
    for (; i + C::NSLOT <= nq; i += C::NSLOT) {
      iter_steady(i, s0{}, SA, DA, SB, DB, KA, KB);
      iter_steady(i + 1, s1{}, SB, DB, SA, DA, KB, KA);
      iter_steady(i + 2, s2{}, SA, DA, SB, DB, KA, KB);
      iter_steady(i + 3, s3{}, SB, DB, SA, DA, KB, KA);
    }
  }
  // the rest: fewer than NSLOT unmasked blocks
  for (; i < nq; ++i) {
    iter_any(i, ffalse{}, SA, DA, SB, DB);
    swap_ab();
  }

  store_dkdv(dkacc, dvacc);
}

// ---------------------------------------------------------------------------
// 3. dQ (query-stationary, same tiling as the forward pass).
template <typename T, int D>
struct DqCfg {
  static constexpr int E = sizeof(T);
  static constexpr int KPL = Mma<T>::KPL;
  static constexpr int WAVES = 4;
  static constexpr int BR = 32 * WAVES;           // queries per workgroup
  static constexpr int BC = 32;                   // keys per tile
  static constexpr int NOB = D / 32;              // 32-wide blocks of dQ
  static constexpr int KSTEPS = D / (2 * KPL);    // MFMA steps over d
  static constexpr int PSTEPS = 16 / KPL;         // MFMA steps over 32 keys
  // K rows are read 16 bytes per lane (A operand of S^T) and through the
  // transposing read (A operand of dQ^T): swizzled 16-bit rows as in bwd_main,
  // filled by LDS-DMA; fp32 rows padded and staged through registers.
  static constexpr bool DMA = (E == 2);
  static constexpr int ROWB = D * E;
  static constexpr int PITCH = DMA ? ROWB : ROWB + 16;
  static constexpr int KTILE = BC * PITCH;
  static constexpr int SLOT = 2 * KTILE;          // K tile, then V tile
  static constexpr int NSLOT = 4;                 // ring of key tiles in LDS
  static constexpr int AHEAD = 3;                 // tiles requested ahead
  static constexpr int CPR = ROWB / 16;
  static constexpr int CPT = BC * CPR / (64 * WAVES);
  static constexpr int FETCH_OPS = 2 * CPT;       // vector-memory ops per wave per tile
  static_assert(BC * CPR % (64 * WAVES) == 0, "tile must split evenly");
};

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
// d = 128: at most 256 VGPRs, so that two waves share each SIMD
__global__ void __launch_bounds__(256, (D == 128 ? 2 : 1)) bwd_dq_kernel(AttnParams p) {
  using C = DqCfg<T, D>;
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KPL = C::KPL, E = C::E;
  using LK = Layout<C::PITCH, C::ROWB, C::DMA>;
  using ffalse = std::integral_constant<bool, false>;
  using ftrue = std::integral_constant<bool, true>;

  __shared__ __attribute__((aligned(1024))) char smem[C::NSLOT * C::SLOT];
  __shared__ uint16_t blist[SPARSE ? kMaxMaskBlocksB : 1];
  __shared__ int nlist_s;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nqt = (Nq + C::BR - 1) / C::BR;
  int bh, qt;
  tile_of(blockIdx.x, gridDim.x, nqt, CAUSAL, p.cu_fill, bh, qt);
  if (CAUSAL) qt = nqt - 1 - qt;  // longest rows first
  const int b = bh / p.H, hh = bh - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)hh * p.sh;     // Q, dO, dQ
  const int64_t kbase = (int64_t)b * p.ksb + (int64_t)hh * p.ksh;  // K, V
  const T *Q = static_cast<const T *>(p.q) + base;
  const T *K = static_cast<const T *>(p.k) + kbase;
  const T *V = static_cast<const T *>(p.v) + kbase;
  const T *dO = static_cast<const T *>(p.dout) + base;
  T *dQ = static_cast<T *>(p.dq) + base;

  int kv_len = Nk;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), Nk);
  const int cs = CAUSAL ? p.cshift : 0;  // causal: key j visible to query i iff j <= i + cs
  const int q_tile0 = qt * C::BR;
  const int qw0 = q_tile0 + 32 * wave;
  const int qi = qw0 + l32;
  int kv_hi = kv_len;
  if (CAUSAL) kv_hi = min(kv_hi, q_tile0 + C::BR + cs);

  // ---- key tiles visited (as in the forward pass)
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
  auto tile_start = [&](int t) -> int {
    if constexpr (SPARSE) {
      const int bi = t / tiles_per_blk;
      return (int)blist[bi] * p.mb + (t - bi * tiles_per_blk) * C::BC;
    } else {
      return t * C::BC;
    }
  };
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

  // ---- this wave's Q and dO rows (B operands), lse*log2(e) and D of the
  // lane's query.  dP^T accumulates onto -D (the first MFMA takes it as its
  // addend), so the MFMA result is already dP - D.
  frag qf[C::KSTEPS], gf[C::KSTEPS];
  float lse2 = INFINITY, negdl = 0.f;
  if (qi < Nq) {
    const T *qrow = Q + (int64_t)qi * p.sn + h * (D / 2);
    const T *grow = dO + (int64_t)qi * p.sn + h * (D / 2);
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      qf[s] = *reinterpret_cast<const frag *>(qrow + s * KPL);
      gf[s] = *reinterpret_cast<const frag *>(grow + s * KPL);
    }
    if (!p.dq_pre) {
      lse2 = p.ws_lse2[(int64_t)bh * Nq + qi];  // +inf when no key is visible: P = 0
      negdl = p.ws_negd[(int64_t)bh * Nq + qi];
    }
  } else {
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      qf[s] = frag{};
      gf[s] = frag{};
    }
  }
  if (p.dq_pre) {
    // The preprocessing step for this lane's query, bitwise as bwd_pre_kernel
    // computes it: the row's 16-byte chunks of O and dO (LPR of them) each
    // give an FMA chain, and the chunk sums meet pairwise at strides LPR/2,
    // LPR/4, ..., 1 (the preprocessing kernel's xor shuffles).  This lane
    // holds the chunks of its half row (its dO ones are already in gf); the
    // stride-LPR/2 pairs are this lane's and its partner's (lane ^ 32).
    constexpr int EPC = 16 / E, LPR = D * E / 16, HALF = LPR / 2;
    const T *O = static_cast<const T *>(p.o_in) + base;
    float cs_[HALF];
#pragma unroll
    for (int c = 0; c < HALF; ++c) {
      u32x4 ov = u32x4{};
      if (qi < Nq) ov = ldg16(reinterpret_cast<const char *>(O + (int64_t)qi * p.sn + h * (D / 2)) + 16 * c);
      const T *ot = reinterpret_cast<const T *>(&ov);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int idx = c * EPC + e;  // element of the half row
        T g;
        if constexpr (KPL == 1) g = gf[idx];
        else g = gf[idx / KPL][idx % KPL];
        acc = fmaf((float)ot[e], (float)g, acc);
      }
      cs_[c] = acc;
    }
#pragma unroll
    for (int c = 0; c < HALF; ++c) cs_[c] = cs_[c] + xor32(cs_[c]);
#pragma unroll
    for (int w = HALF / 2; w >= 1; w >>= 1)
#pragma unroll
      for (int c = 0; c < w; ++c) cs_[c] = cs_[c] + cs_[c + w];
    if (qi < Nq) {
      negdl = -cs_[0];
      const float l = p.lse[(int64_t)bh * Nq + qi];
      lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
      if (h == 0) {  // for the dK/dV pass, which runs after this one
        p.ws_negd[(int64_t)bh * Nq + qi] = negdl;
        p.ws_lse2[(int64_t)bh * Nq + qi] = lse2;
      }
    }
  }
  f32x16 negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = negdl;

  // ---- key tiles into the LDS ring (tile t -> slot t % NSLOT): buffer loads
  // with the tile start in the scalar offset, rows past N read as zeros
  // (16-bit: LDS-DMA, fp32: through registers).
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
      voff[u] = row * row_bytes + ((pc ^ LK::swz(row)) << 4);
    } else {
      const int c = tid + 256 * u, row = c / C::CPR, col = c - row * C::CPR;
      voff[u] = row * row_bytes + col * 16;
    }
  }
  u32x4 stk[C::DMA ? 1 : C::CPT], stv[C::DMA ? 1 : C::CPT];
  auto slot = [&](int t) -> char * { return smem + (t & (C::NSLOT - 1)) * C::SLOT; };
  // Past the end of the list the last tile is fetched again, into the tile's
  // own ring slot (free: its previous tile was consumed).
  auto fetch1 = [&](int t, int u) {
    const int so = __builtin_amdgcn_readfirstlane(tile_start(min(t, ntiles - 1)) * row_bytes);
    if constexpr (C::DMA) {
      const uint32_t la = lds0 + (uint32_t)(slot(t) - smem) + 1024 * (C::WAVES * u + wave);
      buf_load16_lds(kwords, __builtin_amdgcn_readfirstlane(la), voff[u], so);
      buf_load16_lds(vwords, __builtin_amdgcn_readfirstlane(la + C::KTILE), voff[u], so);
    } else {
      stk[u] = buf_load16(krs, voff[u], so);
      stv[u] = buf_load16(vrs, voff[u], so);
    }
  };
  auto fetch = [&](int t) {
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) fetch1(t, u);
  };
  auto commit = [&](int t) {
    if constexpr (!C::DMA) {
      char *kl = slot(t);
#pragma unroll
      for (int u = 0; u < C::CPT; ++u) {
        const int c = tid + 256 * u, row = c / C::CPR, col = c - row * C::CPR;
        *reinterpret_cast<u32x4 *>(kl + LK::off(row, col * 16)) = stk[u];
        *reinterpret_cast<u32x4 *>(kl + C::KTILE + LK::off(row, col * 16)) = stv[u];
      }
    }
  };
  auto sync_ring = [&]() {
    if constexpr (C::DMA) __builtin_amdgcn_s_waitcnt(waitcnt_vm(C::FETCH_OPS));
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  f32x16 qacc[C::NOB];
#pragma unroll
  for (int nb = 0; nb < C::NOB; ++nb) qacc[nb] = f32x16{};
  const float c2 = p.scale_log2;

  // Fragments from a slot.  kvfrag(i): step s = i / 2 over d, tensor i % 2
  // (0 = K for S^T, 1 = V for dP^T), rows = keys, 16 bytes per lane.
  // ktfrag(g): K^T for step t = g / NOB over keys, output block nb = g % NOB,
  // rows = keys in register order, through the transposing read.
  auto kvfrag = [&](const char *kl, int i) -> frag {
    return lds_frag<T>(kl + (i & 1) * C::KTILE, LK::off(l32, (h * (D / 2) + (i >> 1) * KPL) * E));
  };
  auto ktfrag = [&](const char *kl, int g) -> frag {
    return regorder_frag<T, LK>(kl, 0, g / C::NOB, (g % C::NOB) * 32);
  };
  constexpr int NGA = 2 * C::KSTEPS;       // S^T / dP^T MFMAs per tile
  constexpr int NGB = C::PSTEPS * C::NOB;  // dQ^T MFMAs per tile

  // S^T = K Q^T and dP^T - D = V dO^T - D for the tile in `kl`.
  auto sdp = [&](const char *kl, f32x16 &S, f32x16 &DP) {
    S = f32x16{};
#pragma unroll
    for (int i = 0; i < NGA; ++i) {
      const int s = i >> 1;
      if (i & 1) DP = M::mma32(kvfrag(kl, i), gf[s], s == 0 ? (DROP ? f32x16{} : negd) : DP);
      else S = M::mma32(kvfrag(kl, i), qf[s], S);
      FA_FENCE();  // bounds the operand reads in flight (register pressure)
    }
  };
  // P = exp2(S*scale*log2e - lse2), dS^T = P (dP - D) in place (row r of the
  // register layout); masked keys get 0.
  auto grad_row = [&](f32x16 &S, f32x16 &DP, int r) {
    const float pv = fast_exp2(fmaf(S[r], c2, -lse2));
    DP[r] = pv * DP[r];
  };
  // With DROP (DP = dP^T): dS^T = P (Z dP - D).
  auto grad_row_drop = [&](f32x16 &S, f32x16 &DP, int r, const uint32_t (&keepb)[4]) {
    const float pv = fast_exp2(fmaf(S[r], c2, -lse2));
    DP[r] = pv * fmaf(kept(keepb, r, p.drop_thr) ? p.drop_scale : 0.f, DP[r], negdl);
  };
  // dQ^T += K^T dS^T  (rows = d, column = this lane's query)
  auto dqacc = [&](const char *kl, const f32x16 &DS) {
#pragma unroll
    for (int t = 0; t < C::PSTEPS; ++t) {
      const frag sf = pack_frag<T>(DS, t * KPL);
#pragma unroll
      for (int nb = 0; nb < C::NOB; ++nb) {
        qacc[nb] = M::mma32(ktfrag(kl, t * C::NOB + nb), sf, qacc[nb]);
        FA_FENCE();
      }
    }
  };

  // Every iteration j starts with (SX, DX) = (S^T_j, dP^T_j - D) and ends
  // with (SY, DY) = (S^T_{j+1}, dP^T_{j+1} - D).
  //
  // Generic iteration: any mask, straight-line; past the last tile the
  // next-tile products are computed on a repeated tile and never used.
  // `masked` false: tile j is unmasked, the per-element mask is left out.
  auto iter_any = [&](int j, auto masked, f32x16 &SX, f32x16 &DX, f32x16 &SY, f32x16 &DY) {
    fetch(j + C::AHEAD);
    const char *kl = slot(j), *kn = slot(j + 1);
    const int lim_o = (CAUSAL ? min(kv_len, qi + 1 + cs) : kv_len) - tile_start(j);
    uint32_t keepb[4];
    if constexpr (DROP) keep_bytes_query_col(keepb, p, bh, qi, tile_start(j), lane);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (DROP) grad_row_drop(SX, DX, r, keepb);
      else grad_row(SX, DX, r);
      if constexpr (decltype(masked)::value) {
        if (!(reg_row(r, 0) + 4 * h < lim_o)) DX[r] = 0.f;  // key kv0 + row invisible
      }
    }
    sdp(kn, SY, DY);
    dqacc(kl, DX);
    commit(j + C::AHEAD);
    sync_ring();
  };
  // Iteration j for an unmasked tile j (its successor may be masked, or past
  // the end the repeated last tile, whose products go unused): the NGA score / dP
  // MFMAs of tile j+1 carry dS of the first 8 rows of tile j (then the
  // packing of step 0), the first half of the NGB dQ MFMAs carry the last 8
  // rows; operand reads two groups ahead; the next tile's LDS-DMA spread over
  // the first groups.  `par` is j mod NSLOT (compile-time slot addresses).
  // With DROP, KX holds the keep bytes of tile j and the generator rounds for
  // tile j+1's (into KY) ride one per MFMA group.
  constexpr int NGRP = NGA + NGB;
  static_assert(!DROP || NGRP >= kPhiloxRounds, "one generator round per MFMA group");
  auto iter_steady = [&](int j, auto par, f32x16 &SX, f32x16 &DX, f32x16 &SY, f32x16 &DY,
                         uint32_t (&KX)[4], uint32_t (&KY)[4]) {
    constexpr int P = decltype(par)::value;
    char *const kl = smem + P * C::SLOT;
    char *const kn = smem + ((P + 1) % C::NSLOT) * C::SLOT;
    auto row = [&](int r) {
      if constexpr (DROP) grad_row_drop(SX, DX, r, KX);
      else grad_row(SX, DX, r);
    };
    auto gen = [&](int grp) {
      if constexpr (DROP) {
        if (grp < kPhiloxRounds) philox_round(KY, p.drop_key0, p.drop_key1, grp);
        if (grp == kPhiloxRounds - 1) keep_finish_query_col(KY, lane);
      }
    };
    if constexpr (DROP) keep_ctr_query_col(KY, p, bh, qi, tile_start(min(j + 1, ntiles - 1)), lane);
    frag af[3];
    af[0] = kvfrag(kn, 0);
    af[1] = kvfrag(kn, 1);
    SY = f32x16{};
    FA_FENCE();
#pragma unroll
    for (int g = 0; g < NGA; ++g) {
      const int s = g >> 1;
      if (g + 2 < NGA) af[(g + 2) % 3] = kvfrag(kn, g + 2);
      if (g & 1) DY = M::mma32(af[g % 3], gf[s], s == 0 ? (DROP ? f32x16{} : negd) : DY);
      else SY = M::mma32(af[g % 3], qf[s], SY);
      if (g < C::CPT) fetch1(j + C::AHEAD, g);
#pragma unroll
      for (int r = 8 * g / NGA; r < 8 * (g + 1) / NGA; ++r) row(r);
      gen(g);
      FA_FENCE();
    }
    frag tf[3], sf[2];
    tf[0] = ktfrag(kl, 0);
    if (NGB > 1) tf[1] = ktfrag(kl, 1);
    sf[0] = pack_frag<T>(DX, 0);
    FA_FENCE();
#pragma unroll
    for (int g = 0; g < NGB; ++g) {
      const int t = g / C::NOB, nb = g % C::NOB;
      if (g + 2 < NGB) tf[(g + 2) % 3] = ktfrag(kl, g + 2);
      qacc[nb] = M::mma32(tf[g % 3], sf[t & 1], qacc[nb]);
      if (g < NGB / 2) {
#pragma unroll
        for (int r = 8 + 8 * g / (NGB / 2); r < 8 + 8 * (g + 1) / (NGB / 2); ++r) row(r);
      }
      if (g % C::NOB == C::NOB - 1 && t + 1 < C::PSTEPS) sf[(t + 1) & 1] = pack_frag<T>(DX, (t + 1) * KPL);
      gen(NGA + g);
      FA_FENCE();
    }
    commit(j + C::AHEAD);
    sync_ring();
  };

  // ---- prologue
  f32x16 SA, DA, SB, DB;
  if (ntiles > 0) {
#pragma unroll
    for (int t = 0; t < C::AHEAD; ++t) {
      fetch(t);
      commit(t);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (ntiles > 0) sdp(slot(0), SA, DA);
  auto swap_ab = [&]() {
    const f32x16 ts = SA, td = DA;
    SA = SB;
    DA = DB;
    SB = ts;
    DB = td;
  };
  // unmasked tiles first (a prefix), in trips of NSLOT; then the rest
  int j = 0;
  using s0 = std::integral_constant<int, 0>;
  using s1 = std::integral_constant<int, 1>;
  using s2 = std::integral_constant<int, 2>;
  using s3 = std::integral_constant<int, 3>;
  {
    // tile j unmasked; its successor is a masked tile or, past the end, the
    // last tile again (the ring fetches it once more), whose products are
    // never used
    const int j_steady = n_full;
    uint32_t KA[4], KB[4];  // keep bytes of the current / next tile (DROP)
    if (DROP && j + C::NSLOT <= j_steady) keep_bytes_query_col(KA, p, bh, qi, tile_start(j), lane);
    for (; j + C::NSLOT <= j_steady; j += C::NSLOT) {
      iter_steady(j, s0{}, SA, DA, SB, DB, KA, KB);
      iter_steady(j + 1, s1{}, SB, DB, SA, DA, KB, KA);
      iter_steady(j + 2, s2{}, SA, DA, SB, DB, KA, KB);
      iter_steady(j + 3, s3{}, SB, DB, SA, DA, KB, KA);
    }
  }
  for (; j < min(n_full, ntiles); ++j) {  // unmasked
    iter_any(j, ffalse{}, SA, DA, SB, DB);
    swap_ab();
  }
  for (; j < ntiles; ++j) {
    iter_any(j, ftrue{}, SA, DA, SB, DB);
    swap_ab();
  }

  // ---- dQ = scale * (dS K)
  if (qi < Nq) {
    T *qrow = dQ + (int64_t)qi * p.sn;
#pragma unroll
    for (int nb = 0; nb < C::NOB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = nb * 32 + 8 * i + 4 * h;
        if constexpr (E == 4) {
          *reinterpret_cast<f32x4 *>(qrow + d0) =
              f32x4{qacc[nb][4 * i] * p.scale, qacc[nb][4 * i + 1] * p.scale,
                    qacc[nb][4 * i + 2] * p.scale, qacc[nb][4 * i + 3] * p.scale};
        } else {
          typedef T t4 __attribute__((ext_vector_type(4)));
          t4 v;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v[jj] = (T)(qacc[nb][4 * i + jj] * p.scale);
          *reinterpret_cast<t4 *>(qrow + d0) = v;
        }
      }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
static hipError_t launch_main_t(const AttnParams &p, hipStream_t s) {
  using C = BwdCfg<T, D>;
  const int64_t nkt = (p.Nk + C::BKC - 1) / C::BKC;
  const int64_t grid = (int64_t)p.B * p.H * nkt;
  const void *fn = reinterpret_cast<const void *>(&bwd_main_kernel<T, D, CAUSAL, SPARSE, DROP>);
  static const int fill = resident_per_cu(fn, 256);
  AttnParams a = p;
  a.cu_fill = fill;
  void *args[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, s);
}

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
static hipError_t launch_dq_t(const AttnParams &p, hipStream_t s) {
  using C = DqCfg<T, D>;
  const int64_t nqt = (p.Nq + C::BR - 1) / C::BR;
  const int64_t grid = (int64_t)p.B * p.H * nqt;
  const void *fn = reinterpret_cast<const void *>(&bwd_dq_kernel<T, D, CAUSAL, SPARSE, DROP>);
  static const int fill = resident_per_cu(fn, 256);
  AttnParams a = p;
  a.cu_fill = fill;
  void *args[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, s);
}

template <typename T, int D, bool DROP>
static hipError_t launch_bwd_dd(const AttnParams &p, bool sparse, unsigned stages, hipStream_t s) {
  AttnParams a = p;
  void *args[] = {&a};
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  hipError_t e = hipSuccess;
  auto main_pass = [&]() {
    if (sparse)
      return p.causal ? launch_main_t<T, D, true, true, DROP>(p, s) : launch_main_t<T, D, false, true, DROP>(p, s);
    return p.causal ? launch_main_t<T, D, true, false, DROP>(p, s) : launch_main_t<T, D, false, false, DROP>(p, s);
  };
  auto dq_pass = [&](const AttnParams &q) {
    if (sparse)
      return q.causal ? launch_dq_t<T, D, true, true, DROP>(q, s) : launch_dq_t<T, D, false, true, DROP>(q, s);
    return q.causal ? launch_dq_t<T, D, true, false, DROP>(q, s) : launch_dq_t<T, D, false, false, DROP>(q, s);
  };
  if ((stages & FA_BWD_PRE) && (stages & FA_BWD_DQ)) {
    // The dQ pass does the preprocessing of its own queries and fills the
    // workspace; the dK/dV pass, if asked for, runs after it.
    AttnParams f = p;
    f.dq_pre = 1;
    if ((e = dq_pass(f)) != hipSuccess) return e;
    if (stages & FA_BWD_MAIN) e = main_pass();
    return e;
  }
  if (stages & FA_BWD_PRE) {
    constexpr int rpb = PreCfg<T, D>::RPB;
    e = hipLaunchKernel(reinterpret_cast<const void *>(&bwd_pre_kernel<T, D>),
                        dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), args, 0, s);
    if (e != hipSuccess) return e;
  }
  if (stages & FA_BWD_MAIN) {
    if ((e = main_pass()) != hipSuccess) return e;
  }
  if (stages & FA_BWD_DQ) e = dq_pass(p);
  return e;
}

template <typename T, int D>
static hipError_t launch_bwd_d(const AttnParams &p, bool sparse, unsigned stages, hipStream_t s) {
  return p.drop_thr ? launch_bwd_dd<T, D, true>(p, sparse, stages, s)
                    : launch_bwd_dd<T, D, false>(p, sparse, stages, s);
}

template <typename T>
static hipError_t launch_bwd_dt(const AttnParams &p, bool sparse, unsigned stages, hipStream_t s) {
  return p.d == 64 ? launch_bwd_d<T, 64>(p, sparse, stages, s) : launch_bwd_d<T, 128>(p, sparse, stages, s);
}

hipError_t launch_bwd(const AttnParams &p, fa_dtype_t dt, bool sparse, unsigned stages,
                      hipStream_t s) {
  switch (dt) {
    case FA_DTYPE_F32: return launch_bwd_dt<float>(p, sparse, stages, s);
    case FA_DTYPE_F16: return launch_bwd_dt<_Float16>(p, sparse, stages, s);
    case FA_DTYPE_BF16: return launch_bwd_dt<__bf16>(p, sparse, stages, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
