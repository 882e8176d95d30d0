// Backward pass that rebuilds the score and probability tiles instead of
// storing them ("What Ordinary Autograd Saves", section "Why this is
// FlashAttention's second idea": keep O and the row statistic L, rebuild the
// rest; "Backward Pass Implementation", section "The Recomputation Strategy").
//
// Three launches on one stream:
//  1. bwd_pre_kernel: D_i = rowsum(dO_i * O_i), L_i in log2 units (+inf for
//     rows without keys, so their probabilities vanish), zero the fp32 dQ
//     accumulator.
//  2. bwd_kernel: one workgroup per (128-key block, b, K/V head).  Each of the
//     4 waves owns 32 keys; their K and V rows sit in registers and dK, dV
//     accumulate in registers across every query block of every query head of
//     the group (the group sum of the GQA backward, "The Autograd Memory
//     Trap", section "Tracing the Autograd Graph").  Per query block:
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
  const long long rows = (long long)a.B * a.Hq * a.Tq;
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool ok = row < rows;
  float acc = 0.f;
  if (ok) {
    const T* o = reinterpret_cast<const T*>(a.O) + row * D + j * EPL;
    const T* g = reinterpret_cast<const T*>(a.dO) + row * D + j * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc += (float)o[e] * (float)g[e];
  }
#pragma unroll
  for (int msk = 8; msk >= 1; msk >>= 1) acc += __shfl_xor(acc, msk, 64);
  if (!ok) return;
  if (j == 0) {
    a.Dvec[row] = acc;
    const float l = a.L[row];
    a.Lg[row] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
  float* z = a.dQacc + row * D + j * EPL;
#pragma unroll
  for (int e = 0; e < EPL; e += 4) store4(z + e, 0.f, 0.f, 0.f, 0.f);
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_kernel(BwdArgs a) {
  using M = MM<T>;
  typedef typename M::Op Op;
  constexpr int BK = 128;                           // keys per workgroup, 32 per wave
  constexpr int BQ = (sizeof(T) == 4 && D == 128) ? 32 : 64;
  constexpr int KPER = M::KPER;
  constexpr int PADE = 16 / (int)sizeof(T);
  constexpr int LD = D + PADE;                      // sK, sQ, sdO row stride
  constexpr int LDSS = BK + PADE;                   // sdS row stride
  constexpr int NSD = (D / 2) / KPER;
  constexpr int NSQ = (BQ / 2) / KPER;
  constexpr int NSK = (BK / 2) / KPER;
  constexpr int NDT = D / 32, NQT = BQ / 32, NQR = NQT * 16;
  __shared__ __attribute__((aligned(16))) T sK[BK * LD];
  __shared__ __attribute__((aligned(16))) T sQ[BQ * LD];
  __shared__ __attribute__((aligned(16))) T sdO[BQ * LD];
  __shared__ __attribute__((aligned(16))) T sdS[BQ * LDSS];
  __shared__ float sL[BQ], sDv[BQ];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int BHK = a.B * a.Hkv;
  const int bhk = blockIdx.x % BHK, kb = blockIdx.x / BHK;
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv, G = a.Hq / a.Hkv;
  const int k0 = kb * BK, kw = k0 + 32 * w, mykey = kw + n;
  const int off = a.Tk - a.Tq;
  const float c = a.scale_log2;

  const T* Kp = reinterpret_cast<const T*>(a.K) + (size_t)bhk * a.Tk * D;
  const T* Vp = reinterpret_cast<const T*>(a.V) + (size_t)bhk * a.Tk * D;
  stage_tile<T, D, LD, BK>(sK, Kp + (size_t)k0 * D, a.Tk - k0);

  Op kop[NSD], vop[NSD];
  {
    const bool ok = mykey < a.Tk;
    const size_t ro = (size_t)(ok ? mykey : 0) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      kop[s] = M::ld(Kp + ro + s * KPER);
      vop[s] = M::ld(Vp + ro + s * KPER);
      if (!ok) { kop[s] = Op{}; vop[s] = Op{}; }
    }
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) { dk[t] = f32x16{}; dv[t] = f32x16{}; }

  const int nqb = (a.Tq + BQ - 1) / BQ;
  const int qb0 = CAUSAL ? max(0, k0 - off) / BQ : 0;

  for (int r = 0; r < G; ++r) {
    const int bh = b * a.Hq + hk * G + r;
    const T* Qp = reinterpret_cast<const T*>(a.Q) + (size_t)bh * a.Tq * D;
    const T* dOp = reinterpret_cast<const T*>(a.dO) + (size_t)bh * a.Tq * D;
    const float* Lgp = a.Lg + (size_t)bh * a.Tq;
    const float* Dvp = a.Dvec + (size_t)bh * a.Tq;
    float* dQp = a.dQacc + (size_t)bh * a.Tq * D;

    for (int qb = qb0; qb < nqb; ++qb) {
      const int q0 = qb * BQ;
      __syncthreads();
      stage_tile<T, D, LD, BQ>(sQ, Qp + (size_t)q0 * D, a.Tq - q0);
      stage_tile<T, D, LD, BQ>(sdO, dOp + (size_t)q0 * D, a.Tq - q0);
      if (threadIdx.x < BQ) {
        const int q = q0 + threadIdx.x;
        sL[threadIdx.x] = q < a.Tq ? Lgp[q] : INFINITY;
        sDv[threadIdx.x] = q < a.Tq ? Dvp[q] : 0.f;
      }
      __syncthreads();

      // S = Q K^T and dP = dO V^T for 32-query tiles x this wave's 32 keys.
      f32x16 sacc[NQT], dpacc[NQT];
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        sacc[t] = f32x16{};
        dpacc[t] = f32x16{};
        const T* qrow = sQ + (t * 32 + n) * LD + h * (D / 2);
        const T* grow = sdO + (t * 32 + n) * LD + h * (D / 2);
#pragma unroll
        for (int s = 0; s < NSD; ++s) {
          sacc[t] = M::mma(M::ld(qrow + s * KPER), kop[s], sacc[t]);
          dpacc[t] = M::mma(M::ld(grow + s * KPER), vop[s], dpacc[t]);
        }
      }

      float p[NQR], ds[NQR];
      const bool key_ok = mykey < a.Tk;
#pragma unroll
      for (int rr = 0; rr < NQR; ++rr) {
        const int ql = perm_index(h, rr);
        float pv = fast_exp2(sacc[rr >> 4][rr & 15] * c - sL[ql]);
        if (!key_ok || (CAUSAL && mykey > q0 + ql + off)) pv = 0.f;
        p[rr] = pv;
        ds[rr] = pv * (dpacc[rr >> 4][rr & 15] - sDv[ql]);
      }

      Op pop[NSQ], dsop[NSQ];
#pragma unroll
      for (int s = 0; s < NSQ; ++s) {
        pop[s] = M::pack(p + s * KPER);
        dsop[s] = M::pack(ds + s * KPER);
      }
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
#pragma unroll
        for (int s = 0; s < NSQ; ++s) {
          dv[t] = M::mma(TrPerm<T>::ld(sdO, LD, h, s, t * 32), pop[s], dv[t]);
          dk[t] = M::mma(TrPerm<T>::ld(sQ, LD, h, s, t * 32), dsop[s], dk[t]);
        }
      }

#pragma unroll
      for (int rr = 0; rr < NQR; ++rr) sdS[perm_index(h, rr) * LDSS + 32 * w + n] = (T)ds[rr];
      __syncthreads();

      // dQ tile(s) of this wave: dQ[q0 + 32 qt .., 32 dt ..] += scale * dS K.
      for (int idx = w; idx < NQT * NDT; idx += 4) {
        const int qt = idx / NDT, dt = idx % NDT;
        f32x16 acc = f32x16{};
        const T* arow = sdS + (qt * 32 + n) * LDSS + h * (BK / 2);
#pragma unroll
        for (int s = 0; s < NSK; ++s)
          acc = M::mma(M::ld(arow + s * KPER), TrNat<T, BK>::ld(sK, LD, h, s, dt * 32), acc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = q0 + qt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (q < a.Tq) unsafeAtomicAdd(dQp + (size_t)q * D + dt * 32 + n, acc[i] * a.scale);
        }
      }
    }
  }

  if (mykey < a.Tk) {
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
  if ((stages & kStagePre) && rows > 0) {
    hipError_t e = launch(bwd_pre_kernel<T, D>, (rows + 15) / 16, stream, a);
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
