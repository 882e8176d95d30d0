// Forward pass: tiled exact attention with online softmax on gfx950 matrix cores.
//
// Method ("What Ordinary Autograd Saves: Tiling the Forward Pass Is Only Half
// the Algorithm", section "The implementation under test"): outer loop over
// query blocks, inner loop over key blocks; per query row a running max m, a
// running exponential sum l and an unnormalised output, rescaled once whenever
// the max moves; the output is normalised once at the end and the row
// statistic L = m + ln l is kept for the backward pass ("Why this is
// FlashAttention's second idea").
//
// Mapping onto CDNA4.  One workgroup = 4 waves = 128 query rows of one (b, h);
// each wave owns 32 rows.  The wave computes the transposed score tile
// S^T = K_j Q_i^T (keys x queries) so that one query row lives in one lane
// column: the row max is an in-register reduction plus one exchange between
// the two lane halves, and the probabilities feed O^T += V_j^T P^T straight
// from registers.  K_j and V_j (64 keys) are staged in LDS in natural layout;
// V^T operands are fetched with transposed LDS reads.  Softmax runs in the
// exp2 domain (scores pre-multiplied by scale * log2 e); L is converted back
// to a natural log at the end.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  using M = MM<T>;
  typedef typename M::Op Op;
  constexpr int BQ = 128, BK = 64;
  constexpr int KPER = M::KPER;
  constexpr int LD = D + 16 / (int)sizeof(T);       // LDS row stride (elements)
  constexpr int NSD = (D / 2) / KPER;               // steps over the head dim
  constexpr int NSK = (BK / 2) / KPER;              // steps over a key tile
  constexpr int NDT = D / 32;                       // 32-wide output tiles
  __shared__ __attribute__((aligned(16))) T sK[BK * LD];
  __shared__ __attribute__((aligned(16))) T sV[BK * LD];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int BH = a.B * a.Hq;
  const int nqb = (a.Tq + BQ - 1) / BQ;
  const int bh = blockIdx.x % BH;
  int qb = blockIdx.x / BH;
  if (CAUSAL) qb = nqb - 1 - qb;                    // longest rows first
  const int b = bh / a.Hq, hq = bh % a.Hq, hk = hq / (a.Hq / a.Hkv);
  const int q0 = qb * BQ, qw = q0 + 32 * w, myq = qw + n;
  const int off = a.Tk - a.Tq;

  const T* Qp = reinterpret_cast<const T*>(a.Q) + (size_t)bh * a.Tq * D;
  const T* Kp = reinterpret_cast<const T*>(a.K) + (size_t)(b * a.Hkv + hk) * a.Tk * D;
  const T* Vp = reinterpret_cast<const T*>(a.V) + (size_t)(b * a.Hkv + hk) * a.Tk * D;

  // Q^T operand for this lane: query myq, head-dim half h.
  Op qop[NSD];
  {
    const bool ok = myq < a.Tq;
    const T* qrow = Qp + (size_t)(ok ? myq : 0) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      qop[s] = M::ld(qrow + s * KPER);
      if (!ok) qop[s] = Op{};
    }
  }

  const float c = a.scale_log2;
  float m = -INFINITY, lsum = 0.f;
  f32x16 o[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) o[t] = f32x16{};

  int kend = a.Tk;
  if (CAUSAL) kend = min(a.Tk, max(0, q0 + BQ + off));
  const int ntiles = (kend + BK - 1) / BK;

  for (int jt = 0; jt < ntiles; ++jt) {
    const int k0 = jt * BK;
    __syncthreads();
    stage_tile<T, D, LD, BK>(sK, Kp + (size_t)k0 * D, a.Tk - k0);
    stage_tile<T, D, LD, BK>(sV, Vp + (size_t)k0 * D, a.Tk - k0);
    __syncthreads();
    if (CAUSAL && k0 > qw + 31 + off) continue;     // every key hidden from this wave

    // S^T tile: 64 keys x 32 queries as two 32x32 accumulators.
    f32x16 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = f32x16{};
      const T* krow = sK + (t * 32 + n) * LD + h * (D / 2);
#pragma unroll
      for (int s = 0; s < NSD; ++s) st[t] = M::mma(M::ld(krow + s * KPER), qop[s], st[t]);
    }

    float x[32];
    const bool need_mask = (k0 + BK > a.Tk) || (CAUSAL && k0 + BK - 1 > qw + off);
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      x[r] = st[r >> 4][r & 15] * c;
      if (need_mask) {
        const int key = k0 + perm_index(h, r);
        if (key >= a.Tk || (CAUSAL && key > myq + off)) x[r] = -INFINITY;
      }
    }
    float mt = x[0];
#pragma unroll
    for (int r = 1; r < 32; ++r) mt = fmaxf(mt, x[r]);
    mt = wave_xor32_max(mt);
    const float m_new = fmaxf(m, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      x[r] = fast_exp2(x[r] - m_use);
      ps += x[r];
    }
    lsum = lsum * alpha + ps;
    m = m_new;
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[t] *= alpha;

    Op pop[NSK];
#pragma unroll
    for (int s = 0; s < NSK; ++s) pop[s] = M::pack(x + s * KPER);
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int s = 0; s < NSK; ++s) o[t] = M::mma(TrPerm<T>::ld(sV, LD, h, s, t * 32), pop[s], o[t]);
    }
  }

  const float ltot = wave_xor32_sum(lsum);
  if (myq < a.Tq) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    T* orow = reinterpret_cast<T*>(a.O) + ((size_t)bh * a.Tq + myq) * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = t * 32 + 8 * g + 4 * h;
        store4(orow + d0, o[t][4 * g] * inv, o[t][4 * g + 1] * inv, o[t][4 * g + 2] * inv,
               o[t][4 * g + 3] * inv);
      }
    }
    if (h == 0) a.L[(size_t)bh * a.Tq + myq] = ltot > 0.f ? m * kLn2 + logf(ltot) : -INFINITY;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.Tq + 127) / 128;
  const long long blocks = (long long)nqb * a.B * a.Hq;
  if (blocks == 0) return hipSuccess;
  return launch(fwd_kernel<T, D, CAUSAL>, blocks, stream, a);
}

hipError_t launch_fwd(const FwdArgs& a, int dtype_bf16, int d, int causal, hipStream_t stream) {
#define FA_FWD_CASE(T, DD)                                                              \
  if (d == DD) return causal ? launch_fwd_t<T, DD, true>(a, stream) : launch_fwd_t<T, DD, false>(a, stream);
  if (dtype_bf16) {
    FA_FWD_CASE(bf16, 64)
    FA_FWD_CASE(bf16, 128)
  } else {
    FA_FWD_CASE(float, 64)
    FA_FWD_CASE(float, 128)
  }
#undef FA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
