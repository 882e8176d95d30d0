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
// from registers.  K_j and V_j are staged in LDS as swizzled row-major tiles
// (128 keys; 64 for fp32 with d = 128), double-buffered and filled by direct
// global->LDS loads one tile ahead; V^T operands are fetched with transposed
// LDS reads.  Softmax runs in the exp2 domain (scores pre-multiplied by
// scale * log2 e); L is converted back
// to a natural log at the end.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

// Lazy rescale threshold (log2 units): the reference max m_run only moves when
// a row's true max exceeds it by more than 2^TAU, so probabilities stay <= 2^8
// and the O accumulator is rescaled only on the rare tiles where that happens.
constexpr float kTau = 8.0f;

// Workgroup shape.  Each wave owns QT 32-row query tiles; with QT = 2 every
// K / V operand read from LDS feeds two matrix instructions, but a wave then
// needs the whole register file (one wave per SIMD) and its softmax no longer
// overlaps another wave's matrix work, which costs more than the LDS saving:
// QT = 1 with 8 waves (two per SIMD) is faster.
// Keys per tile: 128, so a workgroup meets one barrier per 128 keys.
// fp32: 4 waves (128 query rows) against 64-key tiles.  Its matrix rate is an
// eighth of bf16's, so each tile is long enough that one wave per SIMD keeps
// the unit busy; 128-row blocks give twice the workgroups of 256-row ones
// (the fp32 shapes are small: 32 heads of 1000 rows make 256 workgroups, one
// per compute unit, instead of 128), and 64-key tiles keep a workgroup's LDS
// at 64 KiB (d = dv = 64) so two fit a compute unit, or within the LDS at all
// when d or dv is 128.  bf16 d = 256 takes the same shape: its 256-wide output
// accumulator (128 registers per wave) and Q operands need the register file
// of one wave per SIMD, and 64-key tiles of 512-byte rows fill 128 KiB.
// Decode shape (DEC): a packed workgroup of 4 waves, one per query head of a
// K/V group with up to 32 rows each, against 64-key tiles.  Its 64 KiB of LDS
// and at most 256 registers per wave (two waves per SIMD, asked of the
// compiler through the launch bounds) let two workgroups share a compute
// unit, so twice the
// K/V loads are in flight; few query rows make these loads, not the matrix
// work, the bound.
template <typename T, int D, bool DEC = false> struct FwdShape {
  static constexpr int QT = 1;
  static constexpr int NW = DEC ? 4 : (sizeof(T) == 4 || D == 256) ? 4 : 8;
  static constexpr int BQ = 32 * QT * NW;
  static constexpr int BK = DEC ? 64 : (sizeof(T) == 4 || D == 256) ? 64 : 128;
};

// D: head dim of Q and K; DV: head dim of V and O.  MASK: scores are also
// masked by a caller's boolean mask (FwdArgs::mask).
template <typename T, int D, bool CAUSAL, bool WIN, bool DEC, int DV = D, bool MASK = false>
__global__ __launch_bounds__((64 * FwdShape<T, D, DEC>::NW), (DEC ? 2 : 1)) void fwd_kernel(FwdArgs a) {
  using M = MM<T>;
  typedef typename M::Op Op;
  using SH = FwdShape<T, D, DEC>;
  constexpr int QT = SH::QT, NW = SH::NW, NTHR = 64 * NW, BQ = SH::BQ, BK = SH::BK;
  constexpr int NKT = BK / 32;                      // 32-key sub-tiles per key tile
  constexpr int NE = 16 * NKT;                      // scores per lane per query tile
  constexpr int KPER = M::KPER;
  constexpr int NSD = (D / 2) / KPER;               // steps over the head dim
  constexpr int NSK = (BK / 2) / KPER;              // steps over a key tile
  constexpr int NDT = DV / 32;                      // 32-wide output tiles
  // K / V tiles, swizzled, double-buffered; the next tile is fetched by direct
  // global->LDS loads while the current one is used.
  __shared__ __attribute__((aligned(16))) T sK[2][BK * D];
  __shared__ __attribute__((aligned(16))) T sV[2][BK * DV];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n = lane & 31;
  const int G = a.Hq / a.Hkv;
  // Work of this workgroup and wave.  Usually one (b, query head, block of BQ
  // rows), 32 rows per wave.  Packed (few query rows, as when one block of
  // new tokens attends to a long prefix): one (b, K/V head) with all Tq rows
  // of each of its G query heads, NW / G waves per head, so every K/V tile is
  // loaded once for the whole group.
  int b, hk, hq, q0, qlast, qw;
  bool active;
  if (a.pack) {
    const int grp = xcd_logical_block();
    const int wph = NW / G, r = w / wph;
    b = grp / a.Hkv;
    hk = grp % a.Hkv;
    hq = hk * G + min(r, G - 1);
    q0 = 0;
    qlast = a.Tq - 1;
    qw = 32 * QT * (w % wph);
    active = r < G && qw < a.Tq;
  } else {
    const int nqb = (a.Tq + BQ - 1) / BQ;
    const QWork wk = qblock_work(a.B, a.Hq, a.Hkv, nqb, CAUSAL);
    b = wk.b;
    hk = wk.hk;
    hq = wk.hq;
    q0 = wk.qb * BQ;
    qlast = min(a.Tq - 1, q0 + BQ - 1);
    qw = q0 + 32 * QT * w;                          // this wave's rows: qw .. qw + 32 QT - 1
    active = qw < a.Tq;
  }
  // This workgroup's sequence (a variable-length batch: its own lengths and
  // rows; the grid covers the longest).  Nothing of it here: leave before
  // any barrier (uniform).
  const SeqView sq = seq_view(a, b);
  const int Tq = sq.Tq, Tk = sq.Tk;
  if (q0 >= Tq) return;
  active = active && qw < Tq;
  qlast = min(qlast, Tq - 1);
  const size_t qrow0 = sq.q_row(hq);       // row of query 0 of (b, hq) in Q, O, L
  const int off = Tk - Tq;

  const T* Qp = reinterpret_cast<const T*>(a.Q) + qrow0 * D;
  const T* Kp = reinterpret_cast<const T*>(a.K) + sq.k_row(hk) * D;
  const T* Vp = reinterpret_cast<const T*>(a.V) + sq.k_row(hk) * DV;

  // Key tiles jt0 .. ntiles - 1: those before the sliding window of the
  // block's first query, and those after the causal bound of its last, are
  // never loaded.  Split over keys, slice blockIdx.y takes the next run of
  // `per` tiles.  Fixed layout: the workgroup's own tiles in equal shares.
  // Sequences of their own lengths (offsets or a page table): runs as long as
  // the longest sequence's share, so a short sequence fills the first slices
  // and leaves the others empty (they store only L_s = -inf) instead of
  // spreading a few tiles over every slice.
  const int W = WIN ? a.window : 0;               // compile-time 0 without a window
  int kend = Tk;
  if (CAUSAL) kend = min(Tk, max(0, qlast + 1 + off));
  int ntiles = (kend + BK - 1) / BK;
  int jt0 = W > 0 ? min(ntiles, max(0, q0 + off - W + 1) / BK) : 0;
  if (gridDim.y > 1) {
    const bool own_lengths = a.cu_q != nullptr || a.pages != nullptr;
    const int span = own_lengths ? (a.Tk + BK - 1) / BK : ntiles - jt0;
    const int per = (span + (int)gridDim.y - 1) / (int)gridDim.y;
    jt0 = min(ntiles, jt0 + (int)blockIdx.y * per);
    ntiles = min(ntiles, jt0 + per);
  }

  // A whole tile is addressed from a wave-uniform base plus per-lane offsets
  // tabulated once; in the tile holding the key end, rows past Tk are loaded
  // as copies of the last key (their scores are masked).
  using DR = DmaRows<T, D, BK, NTHR>;
  using DRV = DmaRows<T, DV, BK, NTHR>;
  uint32_t src_off[DR::PER], src_offv[DRV::PER];
#pragma unroll
  for (int i = 0; i < DR::PER; ++i) src_off[i] = DR::src_off(i);
#pragma unroll
  for (int i = 0; i < DRV::PER; ++i) src_offv[i] = D == DV ? src_off[i % DR::PER] : DRV::src_off(i);
  // Paged keys: the tile's page from the sequence's page table (clamped into
  // the pool); the whole page exists, so the tile loads without clamping rows
  // (rows past the sequence's end are masked like any ragged tail).
  auto issue = [&](int k0, int buf) {
    if (a.pages != nullptr) {
      const int pg = min(max(__builtin_amdgcn_readfirstlane(a.pages[(size_t)b * a.pages_per_seq + k0 / a.page_size]),
                             0), a.num_pages - 1);
      const size_t row = ((size_t)pg * a.Hkv + hk) * a.page_size + k0 % a.page_size;
      const T* kb = reinterpret_cast<const T*>(a.K) + row * D;
      const T* vb = reinterpret_cast<const T*>(a.V) + row * DV;
#pragma unroll
      for (int i = 0; i < DR::PER; ++i) dma16s(kb, src_off[i], lds_addr(sK[buf]) + DR::lds_off(i));
#pragma unroll
      for (int i = 0; i < DRV::PER; ++i) dma16s(vb, src_offv[i], lds_addr(sV[buf]) + DRV::lds_off(i));
    } else if (k0 + BK <= Tk) {
      const T* kb = Kp + (size_t)k0 * D;
      const T* vb = Vp + (size_t)k0 * DV;
#pragma unroll
      for (int i = 0; i < DR::PER; ++i) dma16s(kb, src_off[i], lds_addr(sK[buf]) + DR::lds_off(i));
#pragma unroll
      for (int i = 0; i < DRV::PER; ++i) dma16s(vb, src_offv[i], lds_addr(sV[buf]) + DRV::lds_off(i));
    } else {
      dma_rows<T, D, BK, NTHR>(sK[buf], Kp, k0, Tk);
      dma_rows<T, DV, BK, NTHR>(sV[buf], Vp, k0, Tk);
    }
  };
  if (jt0 < ntiles) issue(jt0 * BK, 0);

  // Q^T operands for this lane's queries qw + 32 u + n, head-dim half h.
  Op qop[QT][NSD];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int q = qw + 32 * u + n;
    const bool ok = q < Tq;
    const T* qrow = Qp + (size_t)(ok ? q : 0) * D + h * (D / 2);
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      qop[u][s] = M::ld(qrow + s * KPER);
      if (!ok) qop[u][s] = Op{};
    }
  }
  NatFetch<T, D> nat;
  nat.init(n, h);
  TrPermFetch<T, DV> trp;
  trp.init(lane);
  // Boolean mask: this lane's row of bits (query qw + n; rows past Tq read
  // the last row and are never stored), one word per 32-key sub-tile, loaded
  // a tile ahead into registers.
  static_assert(!MASK || (QT == 1 && !DEC), "the masked forward uses the plain shape");
  typedef uint32_t MaskWords __attribute__((ext_vector_type(NKT)));
  const uint32_t* mrow = nullptr;
  MaskWords mcur{}, mnext{};
  if constexpr (MASK) {
    mrow = a.mask + (size_t)b * a.mask_bstride + (size_t)min(qw + n, Tq - 1) * a.mask_row_words;
    if (jt0 < ntiles) mcur = *reinterpret_cast<const MaskWords*>(mrow + jt0 * NKT);
  }
  wait_vmcnt<0>();
  __syncthreads();

  const float c = a.scale_log2;
  float m_run[QT], lsum[QT];
  f32x16 o[QT][NDT];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    m_run[u] = -INFINITY;
    lsum[u] = 0.f;
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[u][t] = f32x16{};
  }

  for (int jt = jt0; jt < ntiles; ++jt) {
    const int k0 = jt * BK, buf = (jt - jt0) & 1;
    if (jt + 1 < ntiles) issue(k0 + BK, buf ^ 1);
    const T* cK = sK[buf];
    const T* cV = sV[buf];
    bool any = true;
    if constexpr (MASK) {
      if (jt + 1 < ntiles) mnext = *reinterpret_cast<const MaskWords*>(mrow + (jt + 1) * NKT);
      uint32_t orr = 0;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) orr |= mcur[kt];
      any = __ballot(orr != 0) != 0;                 // the mask leaves some key of the tile to the wave
    }

    // Some key of the tile is visible to this wave: not all after the causal
    // bound of its last row, nor all before the window of its first.
    if (active && any && !(CAUSAL && k0 > qw + 32 * QT - 1 + off) && !(W > 0 && k0 + BK - 1 < qw + off - W + 1)) {
      // S^T = K Q^T: NKT key sub-tiles x QT query tiles; each K operand feeds QT products.
      f32x16 st[QT][NKT];
#pragma unroll
      for (int u = 0; u < QT; ++u)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) st[u][kt] = f32x16{};
      wave_prio<1>();
#pragma unroll
      for (int s = 0; s < NSD; ++s) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const Op kop = nat.ld(cK, kt, s);
#pragma unroll
          for (int u = 0; u < QT; ++u) st[u][kt] = M::mma(kop, qop[u][s], st[u][kt]);
        }
      }
      sched_interleave<NKT * NSD * QT, 4 * QT, 1, QT>();
      wave_prio<0>();

      const bool need_mask = (k0 + BK > Tk) || (CAUSAL && k0 + BK - 1 > qw + off) ||
                             (W > 0 && k0 < qw + 32 * QT - 1 + off - W + 1);
      Op pop[QT][NSK];
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        const int myq = qw + 32 * u + n;
        float x[NE];
#pragma unroll
        for (int r = 0; r < NE; ++r) x[r] = st[u][r >> 4][r & 15];
        if (need_mask) {
          // Key k0 + perm_index(h, r) is visible iff lo <= perm_index(0, r) <= lim.
          const int lim = min(Tk - 1, CAUSAL ? myq + off : Tk - 1) - k0 - 4 * h;
          const int lo = W > 0 ? myq + off - W + 1 - k0 - 4 * h : INT_MIN;
#pragma unroll
          for (int r = 0; r < NE; ++r)
            if (perm_index(0, r) > lim || perm_index(0, r) < lo) x[r] = -INFINITY;
        }
        if constexpr (MASK) {
          // Key k0 + perm_index(h, r) is bit perm_index(h, r) % 32 of word r / 16,
          // i.e. bit perm_index(0, r) % 32 after shifting out this half's 4 h.
#pragma unroll
          for (int r = 0; r < NE; ++r) {
            const uint32_t wsh = mcur[r >> 4] >> (4 * h);
            const int keep = (int)(wsh << (31 - perm_index(0, r) % 32)) >> 31;   // 0 or all ones
            x[r] = __int_as_float((__float_as_int(x[r]) & keep) | (int)(0xff800000u & ~(uint32_t)keep));
          }
        }
        float mt = wave_xor32_max(max_tree<NE>(x)) * c;   // row max, exp2 units
        const bool need = mt > m_run[u] + kTau;
        if (__ballot(need)) {
          const float m_new = need ? mt : m_run[u];
          const float alpha = need ? fast_exp2(m_run[u] - m_new) : 1.f;
          lsum[u] *= alpha;
#pragma unroll
          for (int t = 0; t < NDT; ++t) o[u][t] *= alpha;
          m_run[u] = m_new;
        }
        const float nm = (m_run[u] == -INFINITY) ? 0.f : -m_run[u];
#pragma unroll
        for (int r = 0; r < NE; ++r) x[r] = fast_exp2(__builtin_fmaf(x[r], c, nm));
#pragma unroll
        for (int s = 0; s < NSK; ++s) pop[u][s] = M::pack(x + s * KPER);
        // Row sum: of the rounded bf16 probabilities (two per instruction), so
        // the normaliser is the sum of exactly what the PV product weighs.
        float ps4[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int s = 0; s < NSK; ++s) sum_bf16x8(pop[u][s], ps4);
        } else {
#pragma unroll
          for (int r = 0; r < NE; ++r) ps4[r & 3] += x[r];
        }
        lsum[u] += (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
      }

      wave_prio<1>();
      // O^T += V^T P^T; each V^T operand feeds QT products.
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
#pragma unroll
        for (int s = 0; s < NSK; ++s) {
          const Op vop = trp.ld(cV, t, s);
#pragma unroll
          for (int u = 0; u < QT; ++u) o[u][t] = M::mma(vop, pop[u][s], o[u][t]);
        }
      }
      sched_interleave<NDT * NSK * QT, 4 * QT, (sizeof(T) == 2 ? 2 : 1), QT>();
      wave_prio<0>();
    }
    wait_vmcnt<0>();                                 // this wave's loads of the next tile have landed
    __syncthreads();
    if constexpr (MASK) mcur = mnext;
  }

#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int myq = qw + 32 * u + n;
    const float ltot = wave_xor32_sum(lsum[u]);
    if (a.Opart != nullptr) {                         // a key slice: fp32 partials
      if (active && myq < Tq) {
        const size_t rows_all = (a.cu_q != nullptr) ? (size_t)a.Hq * a.total_q : (size_t)a.B * a.Hq * a.Tq;
        const size_t row = (size_t)blockIdx.y * rows_all + qrow0 + myq;
        // A row that saw no key of this slice gets L_s = -inf, which the merge
        // skips without reading O_s: its partial output is not written.
        if (ltot > 0.f) {
          const float inv = 1.f / ltot;
          float* orow = a.Opart + row * DV;
#pragma unroll
          for (int t = 0; t < NDT; ++t) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int d0 = t * 32 + 8 * g + 4 * h;
              store4(orow + d0, o[u][t][4 * g] * inv, o[u][t][4 * g + 1] * inv, o[u][t][4 * g + 2] * inv,
                     o[u][t][4 * g + 3] * inv);
            }
          }
        }
        if (h == 0) {
          const float mref = (m_run[u] == -INFINITY) ? 0.f : m_run[u];
          a.Lpart[row] = ltot > 0.f ? mref * kLn2 + logf(ltot) : -INFINITY;
        }
      }
      continue;
    }
    if (active && myq < Tq) {
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      T* orow = reinterpret_cast<T*>(a.O) + (qrow0 + myq) * DV;
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = t * 32 + 8 * g + 4 * h;
          store4(orow + d0, o[u][t][4 * g] * inv, o[u][t][4 * g + 1] * inv, o[u][t][4 * g + 2] * inv,
                 o[u][t][4 * g + 3] * inv);
        }
      }
      if (h == 0) {
        const float mref = (m_run[u] == -INFINITY) ? 0.f : m_run[u];
        a.L[qrow0 + myq] = ltot > 0.f ? mref * kLn2 + logf(ltot) : -INFINITY;
      }
    }
  }
}

// Merge of the key slices' partials, one row per 16 lanes: with m the largest
// slice logsumexp and w_s = exp(L_s - m), L = m + ln sum_s w_s and
// O = sum_s w_s O_s / sum_s w_s (slices without a visible key have L_s = -inf
// and weigh nothing; a row without any gets O = 0, L = -inf).
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdArgs a, int nsplit) {
  constexpr int EPL = D / 16;
  const long long rows = a.cu_q ? (long long)a.Hq * a.total_q : (long long)a.B * a.Hq * a.Tq;
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, a.Lpart[s * rows + row]);
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float ls = a.Lpart[s * rows + row];
      if (ls == -INFINITY) continue;
      const float wt = __expf(ls - m);
      wsum += wt;
      const float* op = a.Opart + (s * rows + row) * D + j * EPL;
      if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(op + e);
          acc[e] += wt * v[0];
          acc[e + 1] += wt * v[1];
          acc[e + 2] += wt * v[2];
          acc[e + 3] += wt * v[3];
        }
      } else {                                      // d = 32: two elements per lane
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += wt * op[e];
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  T* orow = reinterpret_cast<T*>(a.O) + row * D + j * EPL;
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      store4(orow + e, acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) orow[e] = (T)(acc[e] * inv);
  }
  if (j == 0) a.L[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

template <typename T, int D, bool CAUSAL, int DV = D>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream, int nsplit) {
  using SH = FwdShape<T, D>;
  const int nqb = (a.Tq + SH::BQ - 1) / SH::BQ;
  const long long blocks = a.pack ? (long long)a.B * a.Hkv : (long long)nqb * a.B * a.Hq;
  if (blocks == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  bool launched = false;
  // A boolean mask: the plain shape (its packing only), with or without a
  // window, split or not; no paging.
  if (a.mask != nullptr) {
    e = a.window > 0
            ? launch2<64 * SH::NW>(fwd_kernel<T, D, CAUSAL, true, false, DV, true>, blocks, nsplit, stream, a)
            : launch2<64 * SH::NW>(fwd_kernel<T, D, CAUSAL, false, false, DV, true>, blocks, nsplit, stream, a);
    launched = true;
  }
  if constexpr (sizeof(T) == 2 && D <= 128) {
    if (!launched && a.pack == 2) {
      using SD = FwdShape<T, D, true>;
      e = a.window > 0 ? launch2<64 * SD::NW>(fwd_kernel<T, D, CAUSAL, true, true, DV>, blocks, nsplit, stream, a)
                       : launch2<64 * SD::NW>(fwd_kernel<T, D, CAUSAL, false, true, DV>, blocks, nsplit, stream, a);
      launched = true;
    }
  }
  if (!launched)
    e = a.window > 0 ? launch2<64 * SH::NW>(fwd_kernel<T, D, CAUSAL, true, false, DV>, blocks, nsplit, stream, a)
                     : launch2<64 * SH::NW>(fwd_kernel<T, D, CAUSAL, false, false, DV>, blocks, nsplit, stream, a);
  if (e != hipSuccess || a.Opart == nullptr) return e;
  const long long rows = a.cu_q ? (long long)a.Hq * a.total_q : (long long)a.B * a.Hq * a.Tq;
  if (rows == 0) return hipSuccess;
  return launch(fwd_merge_kernel<T, DV>, (rows + 15) / 16, stream, a, nsplit);
}

// Boolean mask bytes [rows][Tk] (nonzero: visible) to the forward's bit
// layout [rows][row_words]: one thread per 32-bit word, bit e of word w from
// byte 32 w + e; bits past Tk are 0.
__global__ __launch_bounds__(256) void mask_pack_kernel(const uint8_t* in, uint32_t* out, long long rows, int Tk,
                                                         int row_words) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * row_words) return;
  const long long r = i / row_words;
  const int j0 = (int)(i % row_words) * 32;
  const uint8_t* src = in + r * Tk;
  uint32_t v = 0;
  for (int e = 0; e < 32 && j0 + e < Tk; ++e) v |= (src[j0 + e] != 0 ? 1u : 0u) << e;
  out[i] = v;
}

hipError_t launch_mask_pack(const uint8_t* in, uint32_t* out, long long rows, int Tk, int row_words,
                            hipStream_t stream) {
  const long long words = rows * row_words;
  if (words == 0) return hipSuccess;
  return launch(mask_pack_kernel, (words + 255) / 256, stream, in, out, rows, Tk, row_words);
}

int fwd_waves(int dtype_bf16, int d) {
  return dtype_bf16 ? (d == 32    ? FwdShape<bf16, 32>::NW
                       : d == 64  ? FwdShape<bf16, 64>::NW
                       : d == 256 ? FwdShape<bf16, 256>::NW
                                  : FwdShape<bf16, 128>::NW)
                    : (d == 32 ? FwdShape<float, 32>::NW
                               : d == 64 ? FwdShape<float, 64>::NW : FwdShape<float, 128>::NW);
}
int fwd_decode_waves() { return FwdShape<bf16, 128, true>::NW; }
int fwd_decode_block_keys() { return FwdShape<bf16, 128, true>::BK; }
int fwd_block_keys(int dtype_bf16, int d) {
  return dtype_bf16 ? (d == 32    ? FwdShape<bf16, 32>::BK
                       : d == 64  ? FwdShape<bf16, 64>::BK
                       : d == 256 ? FwdShape<bf16, 256>::BK
                                  : FwdShape<bf16, 128>::BK)
                    : (d == 32 ? FwdShape<float, 32>::BK
                               : d == 64 ? FwdShape<float, 64>::BK : FwdShape<float, 128>::BK);
}

hipError_t launch_fwd(const FwdArgs& a, int dtype_bf16, int d, int causal, hipStream_t stream, int nsplit,
                      int dv) {
  if (dv < 0) dv = d;
  if (dv != d) {                                     // d = 128 with dv = 64, and the reverse
#define FA_FWD_DV_CASE(T)                                                                        \
  if (d == 128 && dv == 64)                                                                      \
    return causal ? launch_fwd_t<T, 128, true, 64>(a, stream, nsplit)                            \
                  : launch_fwd_t<T, 128, false, 64>(a, stream, nsplit);                          \
  if (d == 64 && dv == 128)                                                                      \
    return causal ? launch_fwd_t<T, 64, true, 128>(a, stream, nsplit)                            \
                  : launch_fwd_t<T, 64, false, 128>(a, stream, nsplit);
    if (dtype_bf16) {
      FA_FWD_DV_CASE(bf16)
    } else {
      FA_FWD_DV_CASE(float)
    }
#undef FA_FWD_DV_CASE
    return hipErrorInvalidValue;
  }
#define FA_FWD_CASE(T, DD)                                                              \
  if (d == DD)                                                                          \
    return causal ? launch_fwd_t<T, DD, true>(a, stream, nsplit) : launch_fwd_t<T, DD, false>(a, stream, nsplit);
  if (dtype_bf16) {
    FA_FWD_CASE(bf16, 32)
    FA_FWD_CASE(bf16, 64)
    FA_FWD_CASE(bf16, 128)
    FA_FWD_CASE(bf16, 256)
  } else {
    FA_FWD_CASE(float, 32)
    FA_FWD_CASE(float, 64)
    FA_FWD_CASE(float, 128)
  }
#undef FA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
