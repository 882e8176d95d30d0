// Backward pass that rebuilds the score and probability tiles instead of
// storing them ("What Ordinary Autograd Saves", section "Why this is
// FlashAttention's second idea": keep O and the row statistic L, rebuild the
// rest; "Backward Pass Implementation", section "The Recomputation Strategy").
//
// Three launches on one stream:
//  1. bwd_pre_kernel: D_i = rowsum(dO_i * O_i), L_i in log2 units (+inf for
//     rows without keys, so their probabilities vanish), zero the fp32 dQ
//     accumulator.  D and L2 rows are padded to a multiple of 64 per head
//     (padding: D = 0, L2 = +inf), so query blocks load them without checks.
//  2. bwd_kernel: one workgroup per (128-key block, b, K/V head).  Each of the
//     4 waves owns 32 keys; their K and V rows sit in registers and dK, dV
//     accumulate in registers across every query block of every query head of
//     the group (the group sum of the GQA backward, "The Autograd Memory
//     Trap", section "Tracing the Autograd Graph").  Q / dO / L / D blocks
//     are double-buffered in LDS and filled by direct global->LDS loads issued
//     one block ahead; LDS tiles are unpadded with XOR-swizzled 16-byte chunks.
//     Per query block:
//     S = Q K^T and dP = dO V^T (lane = key), P = exp2(S c - L2),
//     dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS (transposed LDS reads of
//     the natural Q / dO tiles), dS goes through LDS and dQ = dS K is added to
//     the fp32 accumulator with hardware float atomics.
//  3. dq_convert_kernel (bf16 only): accumulator -> bf16 dQ.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int EPL = D / 16;                       // elements per lane (16 lanes per row)
  const long long prows = (long long)a.B * a.Hq * a.Tqp;
  const long long prow = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const long long bh = prow / a.Tqp;
  const int q = (int)(prow - bh * a.Tqp);
  const bool ok = prow < prows && q < a.Tq;        // a real query row (else padding)
  const long long row = bh * a.Tq + q;
  float acc = 0.f;
  if (ok) {
    const T* o = reinterpret_cast<const T*>(a.O) + row * D + j * EPL;
    const T* g = reinterpret_cast<const T*>(a.dO) + row * D + j * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc += (float)o[e] * (float)g[e];
  }
#pragma unroll
  for (int msk = 8; msk >= 1; msk >>= 1) acc += __shfl_xor(acc, msk, 64);
  if (prow >= prows) return;
  if (j == 0) {
    const float l = ok ? a.L[row] : -INFINITY;
    a.Dvec[prow] = acc;
    a.Lg[prow] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
  if (!ok) return;
  float* z = a.dQacc + row * D + j * EPL;
#pragma unroll
  for (int e = 0; e < EPL; e += 4) store4(z + e, 0.f, 0.f, 0.f, 0.f);
}

// Dispatch order: each XCD (workgroup id mod 8) gets one contiguous range of
// the logical order (group, then key block, heaviest first when causal), so
// the key blocks of one (batch, K/V head) group share that XCD's L2 for the
// group's Q / dO rows.
struct BwdWork {
  int b, hk, kb;
};

__device__ inline BwdWork bwd_work(const BwdArgs& a, int nkb) {
  const int N = gridDim.x, p = blockIdx.x;
  const int x = p & 7, slot = p >> 3, per = N >> 3, rem = N & 7;
  const int logical = x * per + min(x, rem) + slot;
  BwdWork w;
  w.kb = logical % nkb;
  const int grp = logical / nkb;
  w.b = grp / a.Hkv;
  w.hk = grp % a.Hkv;
  return w;
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_kernel(BwdArgs a) {
  using M = MM<T>;
  using TL = SwzTile<T, D>;
  typedef typename M::Op Op;
  constexpr int BK = 128;                           // keys per workgroup, 32 per wave
  constexpr int BQ = (sizeof(T) == 4 && D == 128) ? 32 : 64;
  constexpr int KPER = M::KPER;
  constexpr int LDSS = BK + 32 / (int)sizeof(T);    // sdS row stride (32-byte padding)
  constexpr int NSD = (D / 2) / KPER;
  constexpr int NSQ = (BQ / 2) / KPER;
  constexpr int NSK = (BK / 2) / KPER;
  constexpr int NDT = D / 32, NQT = BQ / 32;
  constexpr int NT_W = NQT * NDT / 4;               // dQ tiles per wave
  constexpr int NATOM = NT_W * 16;                  // dQ atomics per wave per query block
  static_assert(NT_W * 4 == NQT * NDT, "dQ tiles must split evenly over the 4 waves");
  static_assert(NATOM < 64, "vmcnt accounting");
  // Q / dO / L / D blocks are double-buffered; the next block is loaded by
  // direct global->LDS loads while the current one is processed.
  __shared__ __attribute__((aligned(16))) T sK[BK * D];
  __shared__ __attribute__((aligned(16))) T sQ[2][BQ * D];
  __shared__ __attribute__((aligned(16))) T sdO[2][BQ * D];
  __shared__ __attribute__((aligned(16))) T sdS[BQ * LDSS];
  __shared__ __attribute__((aligned(16))) float sL[2][64];
  __shared__ __attribute__((aligned(16))) float sD[2][64];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int nkb = (a.Tk + BK - 1) / BK;
  const BwdWork wk = bwd_work(a, nkb);
  const int bhk = wk.b * a.Hkv + wk.hk, G = a.Hq / a.Hkv;
  const int k0 = wk.kb * BK, kw = k0 + 32 * w, mykey = kw + n;
  const int off = a.Tk - a.Tq;
  const float c = a.scale_log2;
  const bool key_ok = mykey < a.Tk;

  const T* Kp = reinterpret_cast<const T*>(a.K) + (size_t)bhk * a.Tk * D;
  const T* Vp = reinterpret_cast<const T*>(a.V) + (size_t)bhk * a.Tk * D;

  // Work list: every (query head of the group, query block that can see a key
  // of this block); the next item's Q / dO / L / D are loaded during the current one.
  const int nqb = (a.Tq + BQ - 1) / BQ;
  const int qb0 = CAUSAL ? min(nqb, max(0, k0 - off) / BQ) : 0;
  const int per_head = nqb - qb0, total = G * per_head;
  auto item = [&](int it, int& bh, int& q0) {
    bh = wk.b * a.Hq + wk.hk * G + it / per_head;
    q0 = (qb0 + it % per_head) * BQ;
  };
  // L2 and D rows are padded to 64 per head, so 64 floats can always be loaded.
  auto issue = [&](int it, int buf) {
    int bh, q0;
    item(it, bh, q0);
    const size_t qbase = (size_t)bh * a.Tq * D;
    dma_rows<T, D, BQ, 256>(sQ[buf], reinterpret_cast<const T*>(a.Q) + qbase, q0, a.Tq);
    dma_rows<T, D, BQ, 256>(sdO[buf], reinterpret_cast<const T*>(a.dO) + qbase, q0, a.Tq);
    const int q64 = q0 & ~63;                       // 64-row aligned window holding this block
    if (w == 0) dma_floats64(sL[buf], a.Lg + (size_t)bh * a.Tqp + q64);
    if (w == 1) dma_floats64(sD[buf], a.Dvec + (size_t)bh * a.Tqp + q64);
  };

  dma_rows<T, D, BK, 256>(sK, Kp, k0, a.Tk);
  if (total > 0) issue(0, 0);

  Op kop[NSD], vop[NSD];
  {
    const size_t ro = (size_t)(key_ok ? mykey : 0) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      kop[s] = M::ld(Kp + ro + s * KPER);
      vop[s] = M::ld(Vp + ro + s * KPER);
      if (!key_ok) { kop[s] = Op{}; vop[s] = Op{}; }
    }
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) { dk[t] = f32x16{}; dv[t] = f32x16{}; }
  NatFetch<T, D> nat;
  nat.init(n, h);
  TrPermFetch<T, D> trp;
  trp.init(lane);
  // dQ tiles of this wave: idx = w + 4 j; with NDT | 4 the d-tile is the same for every j
  static_assert(4 % NDT == 0, "one d-tile per wave");
  TrNatFetch<T, D, BK> trk;
  trk.init(lane, w % NDT);
  wait_vmcnt<0>();
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
    if (it + 1 < total) issue(it + 1, buf ^ 1);
    int bh, q0;
    item(it, bh, q0);
    const T* cQ = sQ[buf];
    const T* cdO = sdO[buf];
    const float* cL = sL[buf] + (q0 & 63);          // this block's rows within the 64-row window
    const float* cD = sD[buf] + (q0 & 63);

    // S = Q K^T and dP = dO V^T for 32-query tiles x this wave's 32 keys.
    f32x16 sacc[NQT], dpacc[NQT];
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      sacc[t] = f32x16{};
      dpacc[t] = f32x16{};
#pragma unroll
      for (int s = 0; s < NSD; ++s) {
        sacc[t] = M::mma(nat.ld(cQ, t, s), kop[s], sacc[t]);
        dpacc[t] = M::mma(nat.ld(cdO, t, s), vop[s], dpacc[t]);
      }
    }
    sched_interleave<2 * NQT * NSD, 4>();

    // P = exp2(S c - L2) and dS = P (dP - D), one 32-query tile at a time.
    // Padding query rows carry L2 = +inf, so only the diagonal and the ragged
    // key end need explicit masks.
    const bool need_mask = !key_ok || (CAUSAL && k0 + BK - 1 > q0 + off);
    Op pop[NSQ], dsop[NSQ];
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qg = 32 * t + 8 * g + 4 * h;      // queries of registers 4g .. 4g+3
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&cL[qg]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&cD[qg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          p[i] = fast_exp2(__builtin_fmaf(sacc[t][i], c, -l4[e]));
          ds[i] = dpacc[t][i] - d4[e];
        }
      }
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = q0 + 32 * t + 8 * (i >> 2) + 4 * h + (i & 3);
          if (!key_ok || (CAUSAL && mykey > q + off)) p[i] = 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] *= p[i];
#pragma unroll
      for (int s = 0; s < 16 / KPER; ++s) {
        pop[t * (16 / KPER) + s] = M::pack(p + s * KPER);
        dsop[t * (16 / KPER) + s] = M::pack(ds + s * KPER);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sdS[perm_index(h, 16 * t + i) * LDSS + 32 * w + n] = (T)ds[i];
    }

#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int s = 0; s < NSQ; ++s) {
        dv[t] = M::mma(trp.ld(cdO, t, s), pop[s], dv[t]);
        dk[t] = M::mma(trp.ld(cQ, t, s), dsop[s], dk[t]);
      }
    }
    sched_interleave<2 * NDT * NSQ, 4, (sizeof(T) == 2 ? 2 : 1)>();
    __syncthreads();

    // dQ tiles of this wave: dQ[q0 + 32 qt .., 32 dt ..] += scale * dS K.
    // Exactly NATOM atomics per wave (rows past Tq add 0 to the last row), so
    // the wait below can count them.
    float* dQp = a.dQacc + (size_t)bh * a.Tq * D;
    f32x16 qacc[NT_W];
#pragma unroll
    for (int j = 0; j < NT_W; ++j) {
      const int idx = w + 4 * j, qt = idx / NDT, dt = idx % NDT;
      qacc[j] = f32x16{};
      const T* arow = sdS + (qt * 32 + n) * LDSS + h * (BK / 2);
#pragma unroll
      for (int s = 0; s < NSK; ++s)
        qacc[j] = M::mma(M::ld(arow + s * KPER), trk.ld(sK, s), qacc[j]);
    }
    sched_interleave<NT_W * NSK, 4, (sizeof(T) == 2 ? 3 : 2)>();
#pragma unroll
    for (int j = 0; j < NT_W; ++j) {
      const int idx = w + 4 * j, qt = idx / NDT, dt = idx % NDT;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0 + qt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        const bool ok = q < a.Tq;
        unsafeAtomicAdd(dQp + (size_t)(ok ? q : a.Tq - 1) * D + dt * 32 + n, ok ? qacc[j][i] * a.scale : 0.f);
      }
    }
    wait_vmcnt<NATOM>();                           // this wave's loads for the next item have landed
    __syncthreads();
  }

  if (key_ok) {
    T* dKr = reinterpret_cast<T*>(a.dK) + ((size_t)bhk * a.Tk + mykey) * D;
    T* dVr = reinterpret_cast<T*>(a.dV) + ((size_t)bhk * a.Tk + mykey) * D;
    const float sc = a.scale;
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = t * 32 + 8 * g + 4 * h;
        store4(dKr + d0, dk[t][4 * g] * sc, dk[t][4 * g + 1] * sc, dk[t][4 * g + 2] * sc,
               dk[t][4 * g + 3] * sc);
        store4(dVr + d0, dv[t][4 * g], dv[t][4 * g + 1], dv[t][4 * g + 2], dv[t][4 * g + 3]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ src, bf16* __restrict__ dst,
                                                        long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 lo = reinterpret_cast<const f32x4*>(src)[2 * i];
  const f32x4 hi = reinterpret_cast<const f32x4*>(src)[2 * i + 1];
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = (bf16)lo[e]; v[4 + e] = (bf16)hi[e]; }
  reinterpret_cast<bf16x8*>(dst)[i] = v;
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, unsigned stages, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq * a.Tq;
  const long long prows = (long long)a.B * a.Hq * a.Tqp;
  if ((stages & kStagePre) && rows > 0) {
    hipError_t e = launch(bwd_pre_kernel<T, D>, (prows + 15) / 16, stream, a);
    if (e != hipSuccess) return e;
  }
  const long long kblocks = (long long)((a.Tk + 127) / 128) * a.B * a.Hkv;
  if ((stages & kStageMain) && kblocks > 0) {
    hipError_t e = launch(bwd_kernel<T, D, CAUSAL>, kblocks, stream, a);
    if (e != hipSuccess) return e;
  }
  if ((stages & kStageFinish) && sizeof(T) == 2 && rows > 0) {
    const long long n8 = rows * D / 8;
    return launch(dq_convert_kernel, (n8 + 255) / 256, stream, (const float*)a.dQacc, (bf16*)a.dQ, n8);
  }
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs& a, int dtype_bf16, int d, int causal, unsigned stages,
                      hipStream_t stream) {
#define FA_BWD_CASE(T, DD)                                                                         \
  if (d == DD)                                                                                     \
    return causal ? launch_bwd_t<T, DD, true>(a, stages, stream) : launch_bwd_t<T, DD, false>(a, stages, stream);
  if (dtype_bf16) {
    FA_BWD_CASE(bf16, 64)
    FA_BWD_CASE(bf16, 128)
  } else {
    FA_BWD_CASE(float, 64)
    FA_BWD_CASE(float, 128)
  }
#undef FA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
