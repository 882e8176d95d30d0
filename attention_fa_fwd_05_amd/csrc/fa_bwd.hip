// Backward pass that rebuilds the score and probability tiles instead of
// storing them ("What Ordinary Autograd Saves", section "Why this is
// FlashAttention's second idea": keep O and the row statistic L, rebuild the
// rest; "Backward Pass Implementation", section "The Recomputation Strategy").
//
// Three launches on one stream:
//  1. bwd_pre_kernel: D_i = rowsum(dO_i * O_i) and L_i in log2 units (+inf for
//     rows without keys, so their probabilities vanish).  Rows are padded to a
//     multiple of 64 per head (padding: D = 0, L2 = +inf).
//  2. dkdv_kernel: one workgroup per (128-key block, b, K/V head); each of the
//     4 waves owns 32 keys, whose K and V rows sit in registers, and dK, dV
//     accumulate in registers across every query block of every query head of
//     the group (the group sum of the GQA backward, "The Autograd Memory
//     Trap", section "Tracing the Autograd Graph").  Per query block:
//     S = Q K^T, dP = dO V^T (lane = key), P = exp2(S c - L2), dS = P (dP - D),
//     dV^T += dO^T P, dK^T += Q^T dS.  Q / dO / L2 / D blocks are
//     double-buffered in LDS and fetched by direct global->LDS loads one block
//     ahead.
//  3. dq_kernel: one workgroup per query block, the forward's structure: lane =
//     query, S^T = K Q^T and dP^T = V dO^T per key tile, dS^T from L2 and D
//     held per lane, dQ^T += K^T dS^T in registers, written once.
// dQ is thus produced without atomics: the recompute of S and dP in the dQ
// pass costs 3 extra matrix products per tile, but no fp32 accumulator has to
// be zeroed, read-modify-written from every key block and converted.
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
  if (prow >= prows || j != 0) return;
  const float l = ok ? a.L[row] : -INFINITY;
  a.Dvec[prow] = acc;
  a.Lg[prow] = (l == -INFINITY) ? INFINITY : l * kLog2e;
}

// Key-block kernels: logical order = group, then key block (heaviest first
// when causal: low key blocks see the most query blocks).
struct KWork {
  int b, hk, kb;
};
__device__ inline KWork kblock_work(const BwdArgs& a, int nkb) {
  const int logical = xcd_logical_block();
  KWork w;
  w.kb = logical % nkb;
  const int grp = logical / nkb;
  w.b = grp / a.Hkv;
  w.hk = grp % a.Hkv;
  return w;
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void dkdv_kernel(BwdArgs a) {
  using M = MM<T>;
  typedef typename M::Op Op;
  constexpr int BK = 128;                           // keys per workgroup, 32 per wave
  constexpr int BQ = (sizeof(T) == 4 && D == 128) ? 32 : 64;
  constexpr int KPER = M::KPER;
  constexpr int NSD = (D / 2) / KPER;
  constexpr int NSQ = (BQ / 2) / KPER;
  constexpr int NDT = D / 32, NQT = BQ / 32;
  // Q / dO / L2 / D blocks are double-buffered; the next block is loaded by
  // direct global->LDS loads while the current one is processed.
  __shared__ __attribute__((aligned(16))) T sQ[2][BQ * D];
  __shared__ __attribute__((aligned(16))) T sdO[2][BQ * D];
  __shared__ __attribute__((aligned(16))) float sL[2][64];
  __shared__ __attribute__((aligned(16))) float sD[2][64];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int nkb = (a.Tk + BK - 1) / BK;
  const KWork wk = kblock_work(a, nkb);
  const int bhk = wk.b * a.Hkv + wk.hk, G = a.Hq / a.Hkv;
  const int k0 = wk.kb * BK, kw = k0 + 32 * w, mykey = kw + n;
  const int off = a.Tk - a.Tq;
  const float c = a.scale_log2;
  const bool key_ok = mykey < a.Tk;

  const T* Kp = reinterpret_cast<const T*>(a.K) + (size_t)bhk * a.Tk * D;
  const T* Vp = reinterpret_cast<const T*>(a.V) + (size_t)bhk * a.Tk * D;

  // Work list: every (query head of the group, query block that can see a key
  // of this block); the next item's Q / dO / L2 / D are loaded during the current one.
  const int nqb = (a.Tq + BQ - 1) / BQ;
  const int qb0 = CAUSAL ? min(nqb, max(0, k0 - off) / BQ) : 0;
  const int per_head = nqb - qb0, total = G * per_head;
  auto item = [&](int it, int& bh, int& q0) {
    bh = wk.b * a.Hq + wk.hk * G + it / per_head;
    q0 = (qb0 + it % per_head) * BQ;
  };
  // L2 and D rows are padded to 64 per head, so a 64-row window always loads.
  auto issue = [&](int it, int buf) {
    int bh, q0;
    item(it, bh, q0);
    const size_t qbase = (size_t)bh * a.Tq * D;
    dma_rows<T, D, BQ, 256>(sQ[buf], reinterpret_cast<const T*>(a.Q) + qbase, q0, a.Tq);
    dma_rows<T, D, BQ, 256>(sdO[buf], reinterpret_cast<const T*>(a.dO) + qbase, q0, a.Tq);
    const int q64 = q0 & ~63;
    if (w == 0) dma_floats64(sL[buf], a.Lg + (size_t)bh * a.Tqp + q64);
    if (w == 1) dma_floats64(sD[buf], a.Dvec + (size_t)bh * a.Tqp + q64);
  };
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
    wait_vmcnt<0>();                               // this wave's loads of the next block have landed
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

// Waves per dQ workgroup: 8 (256 query rows), or 4 where fp32 d = 128
// operands would not fit in 256 registers.
template <typename T, int D>
constexpr int dq_waves() { return (sizeof(T) == 4 && D == 128) ? 4 : 8; }

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__((64 * dq_waves<T, D>())) void dq_kernel(BwdArgs a) {
  using M = MM<T>;
  typedef typename M::Op Op;
  constexpr int NW = dq_waves<T, D>(), NTHR = 64 * NW, BQ = 32 * NW, BK = 64;
  constexpr int KPER = M::KPER;
  constexpr int NSD = (D / 2) / KPER;
  constexpr int NSK = (BK / 2) / KPER;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) T sK[2][BK * D];
  __shared__ __attribute__((aligned(16))) T sV[2][BK * D];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int nqb = (a.Tq + BQ - 1) / BQ;
  const QWork wk = qblock_work(a.B, a.Hq, a.Hkv, nqb, CAUSAL);
  const int bh = wk.b * a.Hq + wk.hq;
  const int q0 = wk.qb * BQ, qw = q0 + 32 * w, myq = qw + n;
  const int off = a.Tk - a.Tq;
  const bool q_ok = myq < a.Tq;

  const T* Qp = reinterpret_cast<const T*>(a.Q) + (size_t)bh * a.Tq * D;
  const T* dOp = reinterpret_cast<const T*>(a.dO) + (size_t)bh * a.Tq * D;
  const T* Kp = reinterpret_cast<const T*>(a.K) + (size_t)(wk.b * a.Hkv + wk.hk) * a.Tk * D;
  const T* Vp = reinterpret_cast<const T*>(a.V) + (size_t)(wk.b * a.Hkv + wk.hk) * a.Tk * D;

  int kend = a.Tk;
  if (CAUSAL) kend = min(a.Tk, max(0, q0 + BQ + off));
  const int ntiles = (kend + BK - 1) / BK;

  // Rows past Tk are loaded as copies of the last key; their scores are masked.
  auto issue = [&](int k0, int buf) {
    dma_rows<T, D, BK, NTHR>(sK[buf], Kp, k0, a.Tk);
    dma_rows<T, D, BK, NTHR>(sV[buf], Vp, k0, a.Tk);
  };
  if (ntiles > 0) issue(0, 0);

  // Q^T and dO^T operands for this lane's query, L2 and D of that row.
  Op qop[NSD], gop[NSD];
  {
    const size_t ro = (size_t)(q_ok ? myq : 0) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      qop[s] = M::ld(Qp + ro + s * KPER);
      gop[s] = M::ld(dOp + ro + s * KPER);
      if (!q_ok) { qop[s] = Op{}; gop[s] = Op{}; }
    }
  }
  const float l2 = q_ok ? a.Lg[(size_t)bh * a.Tqp + myq] : INFINITY;
  const float dd = q_ok ? a.Dvec[(size_t)bh * a.Tqp + myq] : 0.f;
  NatFetch<T, D> nat;
  nat.init(n, h);
  TrPermFetch<T, D> trp;
  trp.init(lane);
  wait_vmcnt<0>();
  __syncthreads();

  const float c = a.scale_log2;
  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};

  for (int jt = 0; jt < ntiles; ++jt) {
    const int k0 = jt * BK, buf = jt & 1;
    if (jt + 1 < ntiles) issue(k0 + BK, buf ^ 1);
    const T* cK = sK[buf];
    const T* cV = sV[buf];

    if (!(CAUSAL && k0 > qw + 31 + off)) {          // some key of the tile visible to this wave
      // S^T = K Q^T and dP^T = V dO^T: 64 keys x 32 queries each.
      f32x16 st0 = f32x16{}, st1 = f32x16{}, dp0 = f32x16{}, dp1 = f32x16{};
#pragma unroll
      for (int s = 0; s < NSD; ++s) {
        st0 = M::mma(nat.ld(cK, 0, s), qop[s], st0);
        st1 = M::mma(nat.ld(cK, 1, s), qop[s], st1);
        dp0 = M::mma(nat.ld(cV, 0, s), gop[s], dp0);
        dp1 = M::mma(nat.ld(cV, 1, s), gop[s], dp1);
      }
      sched_interleave<4 * NSD, 4>();
      float ds[32];
      const bool need_mask = (k0 + BK > a.Tk) || (CAUSAL && k0 + BK - 1 > qw + off);
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const float sv = r < 16 ? st0[r] : st1[r - 16];
        const float dpv = r < 16 ? dp0[r] : dp1[r - 16];
        float p = fast_exp2(__builtin_fmaf(sv, c, -l2));
        if (need_mask) {
          const int key = k0 + perm_index(h, r);
          if (key >= a.Tk || (CAUSAL && key > myq + off)) p = 0.f;
        }
        ds[r] = p * (dpv - dd);
      }
      Op dsop[NSK];
#pragma unroll
      for (int s = 0; s < NSK; ++s) dsop[s] = M::pack(ds + s * KPER);
      // dQ^T += K^T dS^T (K^T through transposed reads of the key tile).
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
#pragma unroll
        for (int s = 0; s < NSK; ++s) acc[t] = M::mma(trp.ld(cK, t, s), dsop[s], acc[t]);
      }
      sched_interleave<NDT * NSK, 4, (sizeof(T) == 2 ? 2 : 1)>();
    }
    wait_vmcnt<0>();                                 // this wave's loads of the next tile have landed
    __syncthreads();
  }

  if (q_ok) {
    T* qrow = reinterpret_cast<T*>(a.dQ) + ((size_t)bh * a.Tq + myq) * D;
    const float sc = a.scale;
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = t * 32 + 8 * g + 4 * h;
        store4(qrow + d0, acc[t][4 * g] * sc, acc[t][4 * g + 1] * sc, acc[t][4 * g + 2] * sc,
               acc[t][4 * g + 3] * sc);
      }
    }
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, unsigned stages, hipStream_t stream) {
  const long long prows = (long long)a.B * a.Hq * a.Tqp;
  if ((stages & kStagePre) && prows > 0) {
    hipError_t e = launch(bwd_pre_kernel<T, D>, (prows + 15) / 16, stream, a);
    if (e != hipSuccess) return e;
  }
  const long long kblocks = (long long)((a.Tk + 127) / 128) * a.B * a.Hkv;
  if ((stages & kStageDkDv) && kblocks > 0) {
    hipError_t e = launch(dkdv_kernel<T, D, CAUSAL>, kblocks, stream, a);
    if (e != hipSuccess) return e;
  }
  constexpr int NW = dq_waves<T, D>();
  const long long qblocks = (long long)((a.Tq + 32 * NW - 1) / (32 * NW)) * a.B * a.Hq;
  if ((stages & kStageDq) && qblocks > 0) {
    hipError_t e = launch<64 * NW>(dq_kernel<T, D, CAUSAL>, qblocks, stream, a);
    if (e != hipSuccess) return e;
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
