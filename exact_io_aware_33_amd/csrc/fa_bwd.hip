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
//
// Kernels (all on the caller's stream):
//  1. bwd_pre:   D = rowsum(dO * O) per query row, and zero the fp32 dQ
//                accumulator (a fill kernel, no memset node).
//  2. bwd_main:  one workgroup per (batch, head, 128-key tile), one wavefront
//                per 32 keys.  K and V rows of the wave stay in registers;
//                query blocks of 32 rows (Q, dO, LSE, D) stream through LDS,
//                double buffered.  Per block: S = Q K^T and dP = dO V^T on
//                32x32 MFMAs (scores in "register order", rows = queries), P
//                and dS in fp32, then dV^T += dO^T P and dK^T += Q^T dS with
//                P, dS fed back from registers, dO^T / Q^T from LDS through
//                the transposing read.  dS^T goes to LDS; after one barrier
//                every wave computes a 32 x d/4 slice of dQ = dS K over the
//                workgroup's 128 keys on 16x16 MFMAs and adds it into the
//                fp32 accumulator with global float atomics.
//  3. bwd_dq:    dQ = scale * accumulator, converted to the storage dtype.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

constexpr int kMaxMaskBlocksB = 1024;

template <typename T, int D>
struct BwdCfg {
  static constexpr int E = sizeof(T);
  static constexpr int KPL = Mma<T>::KPL;
  static constexpr int WAVES = 4;
  static constexpr int BKC = 32 * WAVES;        // keys per workgroup
  static constexpr int BQ = 32;                 // queries per iteration
  static constexpr int KSTEPS = D / (2 * KPL);  // 32x32 MFMA steps over d
  static constexpr int TSTEPS = 16 / KPL;       // 32x32 MFMA steps over 32 queries
  static constexpr int NOB = D / 32;            // 32-wide d blocks of dK, dV
  // LDS layouts.  Q / dO (and, during set-up, K) rows are read two ways: 16
  // bytes per lane down 16 consecutive rows (MFMA A operand) and 4 rows x 64
  // bytes per half-wave (transposing read).  No row padding is free of bank
  // conflicts for both, so 16-bit rows are unpadded and their 16-byte chunks
  // are XOR-swizzled per row (see Layout); fp32 rows are padded by 16 bytes.
  static constexpr int PITCH = (E == 4) ? D * E + 16 : D * E;  // Q / dO / K rows
  static constexpr int QBYTES = BQ * PITCH;     // one staged Q (or dO) block
  static constexpr int DSP = (E == 4) ? BQ * E + 16 : BQ * E;  // dS^T rows (rows = keys)
  static constexpr int DBW = D / 64;            // 16-wide d blocks of dQ per wave
  static constexpr int QSTEPS = BKC / (4 * KPL);  // 16x16 MFMA steps over 128 keys
  static constexpr int CPR = D * E / 16;        // 16-byte chunks per row
  static constexpr int CPTQ = BQ * CPR / (64 * WAVES);   // staged chunks / thread / tensor
  static constexpr int CPTK = BKC * CPR / (64 * WAVES);  // K-tile chunks / thread
  static_assert(BQ * CPR % (64 * WAVES) == 0, "query block must split evenly");
  static_assert(4 * QBYTES == BKC * PITCH, "K tile aliases the staging buffers");
};

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
__device__ __forceinline__ typename Mma<T>::frag regorder_frag(const char *lds, int row0, int t, int col0) {
  const int lane = threadIdx.x & 63;
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

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O); zero the dQ accumulator.  One thread per row.
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(AttnParams p) {
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int n = (int)(row % p.N);
  const int64_t bh = row / p.N;
  const int b = (int)(bh / p.H), hh = (int)(bh % p.H);
  const int64_t off = (int64_t)b * p.sb + (int64_t)hh * p.sh + (int64_t)n * p.sn;
  const char *o = reinterpret_cast<const char *>(static_cast<const T *>(p.o_in) + off);
  const char *g = reinterpret_cast<const char *>(static_cast<const T *>(p.dout) + off);
  constexpr int CH = D * (int)sizeof(T) / 16;
  constexpr int EPC = 16 / (int)sizeof(T);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const u32x4 a = ldg16(o + 16 * c), bq = ldg16(g + 16 * c);
    const T *ta = reinterpret_cast<const T *>(&a);
    const T *tb = reinterpret_cast<const T *>(&bq);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc = fmaf((float)ta[e], (float)tb[e], acc);
  }
  p.ws_delta[row] = acc;
  float *dq = p.ws_dq + row * D;
#pragma unroll
  for (int c = 0; c < D / 4; ++c) reinterpret_cast<f32x4 *>(dq)[c] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------------------
// 3. dQ = scale * accumulator -> storage dtype.  One thread per 16 output bytes.
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_dq_kernel(AttnParams p) {
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int CPR = D / EPC;
  const int64_t total = (int64_t)p.B * p.H * p.N * CPR;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= total) return;
  const int64_t row = id / CPR;
  const int c = (int)(id % CPR);
  const int n = (int)(row % p.N);
  const int64_t bh = row / p.N;
  const int b = (int)(bh / p.H), hh = (int)(bh % p.H);
  const float *src = p.ws_dq + row * D + c * EPC;
  T *dst = static_cast<T *>(p.dq) + (int64_t)b * p.sb + (int64_t)hh * p.sh + (int64_t)n * p.sn + c * EPC;
  u32x4 out;
  T *to = reinterpret_cast<T *>(&out);
#pragma unroll
  for (int e = 0; e < EPC; ++e) to[e] = (T)(src[e] * p.scale);
  stg16(dst, out);
}

// ---------------------------------------------------------------------------
// 2. Main backward kernel.
template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(256) bwd_main_kernel(AttnParams p) {
  using C = BwdCfg<T, D>;
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KPL = C::KPL, E = C::E;
  using LQ = Layout<C::PITCH, D * E, E != 4>;    // Q / dO / K tiles
  using LS = Layout<C::DSP, C::BQ * E, E != 4>;  // dS^T

  // stage[buf][0=Q,1=dO][BQ rows]; the K tile aliases it during set-up.
  __shared__ __attribute__((aligned(16))) char stage[4 * C::QBYTES];
  __shared__ __attribute__((aligned(16))) char dst_lds[2][C::BKC * C::DSP];  // dS^T [key][q]
  __shared__ __attribute__((aligned(16))) float lsed[2][2][C::BQ];           // [buf][lse2, D]
  __shared__ uint16_t blist[SPARSE ? kMaxMaskBlocksB : 1];
  __shared__ int nlist_s;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int N = p.N;
  const int nkt = (N + C::BKC - 1) / C::BKC;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / nkt;
  const int kt = logical - bh * nkt;
  const int b = bh / p.H, hh = bh - b * p.H;
  const int64_t base = (int64_t)b * p.sb + (int64_t)hh * p.sh;
  const T *Q = static_cast<const T *>(p.q) + base;
  const T *K = static_cast<const T *>(p.k) + base;
  const T *V = static_cast<const T *>(p.v) + base;
  const T *dO = static_cast<const T *>(p.dout) + base;
  T *dK = static_cast<T *>(p.dk) + base;
  T *dV = static_cast<T *>(p.dv) + base;
  const float *LSE = p.lse + (int64_t)bh * N;
  const float *Dl = p.ws_delta + (int64_t)bh * N;
  float *dQacc = p.ws_dq + (int64_t)bh * N * D;

  int kv_len = N;
  if (p.key_lens) kv_len = min(max(p.key_lens[b], 0), N);
  const int k0 = kt * C::BKC;
  const int kw0 = k0 + 32 * wave;  // first key of this wave
  const int key = kw0 + l32;       // this lane's key (column of S)

  auto store_dkdv = [&](const f32x16 *dkacc, const f32x16 *dvacc) {
    if (key >= N) return;
    T *krow = dK + (int64_t)key * p.sn;
    T *vrow = dV + (int64_t)key * p.sn;
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
              f32x4{dvacc[nb][4 * i], dvacc[nb][4 * i + 1], dvacc[nb][4 * i + 2], dvacc[nb][4 * i + 3]};
        } else {
          typedef T t4 __attribute__((ext_vector_type(4)));
          t4 kv4, vv4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            kv4[j] = (T)(dkacc[nb][4 * i + j] * p.scale);
            vv4[j] = (T)dvacc[nb][4 * i + j];
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
  const int nqb_all = (N + C::BQ - 1) / C::BQ;
  int nq, first_skip = 0, per = 1;
  if constexpr (SPARSE) {
    per = p.mb / C::BQ;
    const int kb = k0 / p.mb;
    const uint8_t *mcol = p.mask + (int64_t)hh * p.mask_hstride + kb;
    if (wave == 0) {
      int count = 0;
      for (int i0 = 0; i0 < p.nblk; i0 += 64) {
        const int i = i0 + lane;
        const bool set = i < p.nblk && (!CAUSAL || i >= kb) && mcol[(int64_t)i * p.nblk] != 0;
        const uint64_t bal = __ballot(set);
        if (set) blist[count + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)i;
        count += __popcll(bal);
      }
      if (lane == 0) nlist_s = count;
    }
    __syncthreads();
    const int nl = nlist_s;
    if (CAUSAL && nl > 0 && blist[0] == kb) first_skip = (k0 - kb * p.mb) / C::BQ;
    nq = nl * per - first_skip;
  } else {
    first_skip = CAUSAL ? k0 / C::BQ : 0;
    nq = nqb_all - first_skip;
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

  // ---- set-up: K tile through LDS (for the dQ operand); K, V rows of this
  // wave into registers as S / dP operands.
  {
#pragma unroll
    for (int u = 0; u < C::CPTK; ++u) {
      const int c = tid + 256 * u, row = c / C::CPR, col = c - row * C::CPR;
      const int kk = k0 + row;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (kk < N) v = ldg16(reinterpret_cast<const char *>(K + (int64_t)kk * p.sn) + col * 16);
      *reinterpret_cast<u32x4 *>(stage + LQ::off(row, col * 16)) = v;
    }
  }
  frag kf[C::KSTEPS], vf[C::KSTEPS];
  if (key < N) {
    const T *kr = K + (int64_t)key * p.sn + h * (D / 2);
    const T *vr = V + (int64_t)key * p.sn + h * (D / 2);
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
  __syncthreads();
  // dQ operand: K[key][d] for this wave's d blocks (d = (wave*DBW + db)*16 + i)
  frag kq[C::DBW][C::QSTEPS];
#pragma unroll
  for (int db = 0; db < C::DBW; ++db)
#pragma unroll
    for (int st = 0; st < C::QSTEPS; ++st)
      kq[db][st] = colfrag16<T, LQ>(stage, st * 4 * KPL, (wave * C::DBW + db) * 16);
  __syncthreads();  // the staging buffers are reused from here on

  // ---- query-block staging: buffer loads -> registers -> LDS (double
  // buffer).  Lane offsets inside a block are loop invariant, the block start
  // goes in the scalar offset, and rows past N read as zeros.
  const uint32_t q_bytes = (uint32_t)(((int64_t)(N - 1) * p.sn + D) * E);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q, q_bytes);
  const __amdgpu_buffer_rsrc_t dors = make_rsrc(dO, q_bytes);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(LSE, (uint32_t)N * 4u);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(Dl, (uint32_t)N * 4u);
  const int row_bytes = (int)(p.sn * E);
  int voff[C::CPTQ];
#pragma unroll
  for (int u = 0; u < C::CPTQ; ++u) {
    const int c = tid + 256 * u, row = c / C::CPR, col = c - row * C::CPR;
    voff[u] = row * row_bytes + col * 16;
  }
  u32x4 sq[C::CPTQ], sdo[C::CPTQ];
  float slse = 0.f, sdel = 0.f;
  auto load_q = [&](int q0) {
    const int so = q0 * row_bytes;
#pragma unroll
    for (int u = 0; u < C::CPTQ; ++u) {
      sq[u] = buf_load16(qrs, voff[u], so);
      sdo[u] = buf_load16(dors, voff[u], so);
    }
    if (tid < C::BQ) {
      const int so4 = __builtin_amdgcn_readfirstlane(q0 * 4);
      slse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, tid * 4, so4, 0));
      sdel = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(drs, tid * 4, so4, 0));
    }
  };
  auto store_q = [&](int buf, int q0) {
    char *ql = stage + buf * 2 * C::QBYTES;
    char *dl = ql + C::QBYTES;
#pragma unroll
    for (int u = 0; u < C::CPTQ; ++u) {
      const int c = tid + 256 * u, row = c / C::CPR, col = c - row * C::CPR;
      *reinterpret_cast<u32x4 *>(ql + LQ::off(row, col * 16)) = sq[u];
      *reinterpret_cast<u32x4 *>(dl + LQ::off(row, col * 16)) = sdo[u];
    }
    if (tid < C::BQ) {
      // rows past N, and rows that see no key (LSE = -inf), get P = 0
      const bool in = q0 + tid < N;
      lsed[buf][0][tid] = (!in || slse == -INFINITY) ? INFINITY : slse * kLog2e;
      lsed[buf][1][tid] = in ? sdel : 0.f;
    }
  };

  const float c2 = p.scale_log2;
  if (nq > 0) {
    load_q(qblock_start(0));
    store_q(0, qblock_start(0));
  }
  // Retire every outstanding load (K/V operands included) on all paths into
  // the loop, so the compiler does not wait on the next block's prefetch
  // inside the loop.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int it = 0; it < nq; ++it) {
    const int buf = it & 1;
    const int q0 = qblock_start(it);
    const bool has_next = it + 1 < nq;
    if (has_next) load_q(qblock_start(it + 1));
    const char *ql = stage + buf * 2 * C::QBYTES;
    const char *dl = ql + C::QBYTES;
    char *dsl = dst_lds[buf];

    // Does any (query, key) pair of this block survive the masks for this wave?
    const bool skip = (kw0 >= kv_len) || (CAUSAL && kw0 > q0 + C::BQ - 1);
    if (!skip) {
      // S = Q K^T and dP = dO V^T  (rows = queries in register order, col = key)
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int st = 0; st < C::KSTEPS; ++st) {
        const int off = LQ::off(l32, (h * (D / 2) + st * KPL) * E);
        s = M::mma32(lds_frag<T>(ql, off), kf[st], s);
        dp = M::mma32(lds_frag<T>(dl, off), vf[st], dp);
      }
      const bool need_mask = (kw0 + 32 > kv_len) || (CAUSAL && kw0 + 31 > q0);
      // P = exp2(S*scale*log2e - LSE*log2e); dS = P (dP - D)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&lsed[buf][0][8 * i + 4 * h]);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&lsed[buf][1][8 * i + 4 * h]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * i + j;
          float pv = fast_exp2(fmaf(s[r], c2, -l4[j]));
          if (need_mask) {
            const int qq = q0 + reg_row(r, h);
            const bool ok = key < kv_len && (!CAUSAL || key <= qq);
            if (!ok) pv = 0.f;
          }
          s[r] = pv;
          dp[r] = pv * (dp[r] - d4[j]);
        }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS   (rows = d, cols = keys)
#pragma unroll
      for (int t = 0; t < C::TSTEPS; ++t) {
        const frag pb = pack_frag<T>(s, t * KPL);
        const frag sb = pack_frag<T>(dp, t * KPL);
#pragma unroll
        for (int nb = 0; nb < C::NOB; ++nb) {
          dvacc[nb] = M::mma32(regorder_frag<T, LQ>(dl, 0, t, nb * 32), pb, dvacc[nb]);
          dkacc[nb] = M::mma32(regorder_frag<T, LQ>(ql, 0, t, nb * 32), sb, dkacc[nb]);
        }
      }
      // dS^T -> LDS: row = key (this lane), 4 consecutive queries per group
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qc = 8 * i + 4 * h;
        char *dst = dsl + LS::off(32 * wave + l32, qc * E);
        if constexpr (E == 4) {
          *reinterpret_cast<f32x4 *>(dst) = f32x4{dp[4 * i], dp[4 * i + 1], dp[4 * i + 2], dp[4 * i + 3]};
        } else {
          typedef T t4 __attribute__((ext_vector_type(4)));
          t4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (T)dp[4 * i + j];
          *reinterpret_cast<t4 *>(dst) = v;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        char *dst = dsl + LS::off(32 * wave + l32, (8 * i + 4 * h) * E);
        if constexpr (E == 4) {
          *reinterpret_cast<f32x4 *>(dst) = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
          *reinterpret_cast<u32x2 *>(dst) = u32x2{0u, 0u};
        }
      }
    }
    if (has_next) store_q(buf ^ 1, qblock_start(it + 1));
    __syncthreads();

    // dQ[q0 .. q0+31][wave's d slice] += dS K over the workgroup's keys
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      f32x4 acc[C::DBW];
#pragma unroll
      for (int db = 0; db < C::DBW; ++db) acc[db] = f32x4{};
#pragma unroll
      for (int st = 0; st < C::QSTEPS; ++st) {
        const frag a = colfrag16<T, LS>(dsl, st * 4 * KPL, qh * 16);
#pragma unroll
        for (int db = 0; db < C::DBW; ++db) acc[db] = M::mma16(a, kq[db][st], acc[db]);
      }
      const int g = lane >> 4, i = lane & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qq = q0 + qh * 16 + 4 * g + r;
        if (qq < N) {
#pragma unroll
          for (int db = 0; db < C::DBW; ++db)
            unsafeAtomicAdd(dQacc + (int64_t)qq * D + (wave * C::DBW + db) * 16 + i, acc[db][r]);
        }
      }
    }
  }

  store_dkdv(dkacc, dvacc);
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_main_t(const AttnParams &p, hipStream_t s) {
  using C = BwdCfg<T, D>;
  const int64_t nkt = (p.N + C::BKC - 1) / C::BKC;
  const int64_t grid = (int64_t)p.B * p.H * nkt;
  AttnParams a = p;
  void *args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void *>(&bwd_main_kernel<T, D, CAUSAL, SPARSE>),
                         dim3((unsigned)grid), dim3(256), args, 0, s);
}

template <typename T, int D>
static hipError_t launch_bwd_d(const AttnParams &p, bool sparse, unsigned stages, hipStream_t s) {
  AttnParams a = p;
  void *args[] = {&a};
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  hipError_t e = hipSuccess;
  if (stages & FA_BWD_PRE) {
    e = hipLaunchKernel(reinterpret_cast<const void *>(&bwd_pre_kernel<T, D>),
                        dim3((unsigned)((rows + 255) / 256)), dim3(256), args, 0, s);
    if (e != hipSuccess) return e;
  }
  if (stages & FA_BWD_MAIN) {
    if (sparse)
      e = p.causal ? launch_main_t<T, D, true, true>(p, s) : launch_main_t<T, D, false, true>(p, s);
    else
      e = p.causal ? launch_main_t<T, D, true, false>(p, s) : launch_main_t<T, D, false, false>(p, s);
    if (e != hipSuccess) return e;
  }
  if (stages & FA_BWD_DQ) {
    const int64_t chunks = rows * (D / (16 / (int)sizeof(T)));
    e = hipLaunchKernel(reinterpret_cast<const void *>(&bwd_dq_kernel<T, D>),
                        dim3((unsigned)((chunks + 255) / 256)), dim3(256), args, 0, s);
  }
  return e;
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
