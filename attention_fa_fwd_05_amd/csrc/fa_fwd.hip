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
// Mapping onto CDNA4.  One workgroup = 8 waves = 256 query rows of one (b, h);
// each wave owns 32 rows.  The wave computes the transposed score tile
// S^T = K_j Q_i^T (keys x queries) so that one query row lives in one lane
// column: the row max is an in-register reduction plus one exchange between
// the two lane halves, and the probabilities feed O^T += V_j^T P^T straight
// from registers.  K_j and V_j (64 keys) are staged in LDS as swizzled
// row-major tiles, double-buffered and filled by direct global->LDS loads one
// tile ahead; V^T operands are fetched with transposed LDS reads.  Softmax runs in the
// exp2 domain (scores pre-multiplied by scale * log2 e); L is converted back
// to a natural log at the end.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

// Lazy rescale threshold (log2 units): the reference max m_run only moves when
// a row's true max exceeds it by more than 2^TAU, so probabilities stay <= 2^8
// and the O accumulator is rescaled only on the rare tiles where that happens.
constexpr float kTau = 8.0f;

// Waves per workgroup: 8 (256 query rows, two waves per SIMD), or 4 where the
// fp32 d = 128 operands would not fit in 256 registers.
template <typename T, int D>
constexpr int fwd_waves() { return (sizeof(T) == 4 && D == 128) ? 4 : 8; }

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__((64 * fwd_waves<T, D>())) void fwd_kernel(FwdArgs a) {
  using M = MM<T>;
  typedef typename M::Op Op;
  constexpr int NW = fwd_waves<T, D>(), NTHR = 64 * NW, BQ = 32 * NW, BK = 64;
  constexpr int KPER = M::KPER;
  constexpr int NSD = (D / 2) / KPER;               // steps over the head dim
  constexpr int NSK = (BK / 2) / KPER;              // steps over a key tile
  constexpr int NDT = D / 32;                       // 32-wide output tiles
  // K / V tiles, swizzled, double-buffered; the next tile is fetched by direct
  // global->LDS loads while the current one is used.
  __shared__ __attribute__((aligned(16))) T sK[2][BK * D];
  __shared__ __attribute__((aligned(16))) T sV[2][BK * D];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int nqb = (a.Tq + BQ - 1) / BQ;
  const QWork wk = qblock_work(a.B, a.Hq, a.Hkv, nqb, CAUSAL);
  const int bh = wk.b * a.Hq + wk.hq;
  const int q0 = wk.qb * BQ, qw = q0 + 32 * w, myq = qw + n;
  const int off = a.Tk - a.Tq;

  const T* Qp = reinterpret_cast<const T*>(a.Q) + (size_t)bh * a.Tq * D;
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
  NatFetch<T, D> nat;
  nat.init(n, h);
  TrPermFetch<T, D> trp;
  trp.init(lane);
  wait_vmcnt<0>();
  __syncthreads();

  const float c = a.scale_log2;
  float m_run = -INFINITY, lsum = 0.f;
  f32x16 o[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) o[t] = f32x16{};

  for (int jt = 0; jt < ntiles; ++jt) {
    const int k0 = jt * BK, buf = jt & 1;
    if (jt + 1 < ntiles) issue(k0 + BK, buf ^ 1);
    const T* cK = sK[buf];
    const T* cV = sV[buf];

    if (!(CAUSAL && k0 > qw + 31 + off)) {          // some key of the tile visible to this wave
      f32x16 st0 = f32x16{}, st1 = f32x16{};
#pragma unroll
      for (int s = 0; s < NSD; ++s) {
        st0 = M::mma(nat.ld(cK, 0, s), qop[s], st0);
        st1 = M::mma(nat.ld(cK, 1, s), qop[s], st1);
      }
      sched_interleave<2 * NSD, 4>();
      float x[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) { x[i] = st0[i]; x[16 + i] = st1[i]; }
      if ((k0 + BK > a.Tk) || (CAUSAL && k0 + BK - 1 > qw + off)) {
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          const int key = k0 + perm_index(h, r);
          if (key >= a.Tk || (CAUSAL && key > myq + off)) x[r] = -INFINITY;
        }
      }
      float mt = fmaxf(x[0], x[1]);
#pragma unroll
      for (int r = 2; r < 32; r += 2) mt = fmaxf(mt, fmaxf(x[r], x[r + 1]));
      mt = wave_xor32_max(mt) * c;                   // row max, exp2 units
      const bool need = mt > m_run + kTau;
      if (__ballot(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
        lsum *= alpha;
#pragma unroll
        for (int t = 0; t < NDT; ++t) o[t] *= alpha;
        m_run = m_new;
      }
      const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        x[r] = fast_exp2(__builtin_fmaf(x[r], c, nm));
        ps += x[r];
      }
      lsum += ps;

      Op pop[NSK];
#pragma unroll
      for (int s = 0; s < NSK; ++s) pop[s] = M::pack(x + s * KPER);
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
#pragma unroll
        for (int s = 0; s < NSK; ++s) o[t] = M::mma(trp.ld(cV, t, s), pop[s], o[t]);
      }
      sched_interleave<NDT * NSK, 4, (sizeof(T) == 2 ? 2 : 1)>();
    }
    wait_vmcnt<0>();                                 // this wave's loads of the next tile have landed
    __syncthreads();
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
    if (h == 0) {
      const float mref = (m_run == -INFINITY) ? 0.f : m_run;
      a.L[(size_t)bh * a.Tq + myq] = ltot > 0.f ? mref * kLn2 + logf(ltot) : -INFINITY;
    }
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int NW = fwd_waves<T, D>();
  const int nqb = (a.Tq + 32 * NW - 1) / (32 * NW);
  const long long blocks = (long long)nqb * a.B * a.Hq;
  if (blocks == 0) return hipSuccess;
  return launch<64 * NW>(fwd_kernel<T, D, CAUSAL>, blocks, stream, a);
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
