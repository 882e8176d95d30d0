// dK / dV pass of the backward for bf16, with the work of each key group split
// between two waves that share a SIMD ("What Ordinary Autograd Saves",
// section "Why this is FlashAttention's second idea": rebuild S and P from
// Q, K, V, O and L instead of storing them; "Backward Pass Implementation",
// section "The Recomputation Strategy").
//
// One workgroup per (128-key block, b, K/V head), 8 waves.  Waves w and w + 4
// own the same 32 keys and run on the same SIMD:
//  * the P-wave (w < 4) holds K and accumulates dV: per 64-query block it
//    forms S = Q K^T, P = exp2(S c - L2) (0 where the pair is hidden), writes
//    P (bf16) to LDS and adds dV^T += dO^T P;
//  * the dS-wave (w >= 4) holds V and accumulates dK: per block it forms
//    dP - D = dO V^T seeded with -D, and one block later, once the P-wave's
//    P of that block is in LDS, dS = P (dP - D) and dK^T += Q^T dS.
// Each wave then needs about half the registers of a wave doing all four
// products, so two fit on a SIMD and one's vector work (exponentials, dS)
// runs while the other keeps the matrix unit busy.  The dK and dV sums run
// over every query block of every query head of the group (the GQA group
// sum, "The Autograd Memory Trap", section "Tracing the Autograd Graph").
//
// Query blocks: from the last one down, heads innermost, so the key blocks of
// a group (all on one XCD) step through the same Q / dO blocks together and
// share them in L2.  Blocks are loaded two ahead by direct global->LDS loads:
// Q has four LDS slots (block i - 1 for the dS-wave's Q^T, block i for both
// waves, blocks i + 1 and i + 2 in flight), dO, L2 and -D three (blocks i,
// i + 1, i + 2).  P goes through two LDS buffers.  One barrier per block.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {
namespace {

// Key-block work of the dK / dV pass: logical order = group, then key block
// (heaviest first when causal: low key blocks see the most query blocks).  A
// group with fewer key blocks than the 32 compute units of an XCD is
// interleaved by key block with K - 1 others (K * key blocks = 32), as the
// query-block kernels do (at 16 heads of 2048 keys: -7% for this pass).
struct KWork2 {
  int b, hk, kb;
};
__device__ inline KWork2 kblock_work2(const BwdArgs& a, int nkb) {
  const int logical = xcd_logical_block();
  const int N = gridDim.x, per = N >> 3;
  int K = nkb < 32 ? 32 / nkb : 1;
  if (N % 8 != 0 || per % nkb != 0 || (per / nkb) % K != 0) K = 1;
  KWork2 w;
  int grp;
  if (K > 1) {
    const int u = logical / K;
    w.kb = u % nkb;
    grp = (u / nkb) * K + logical % K;
  } else {
    w.kb = logical % nkb;
    grp = logical / nkb;
  }
  w.b = grp / a.Hkv;
  w.hk = grp % a.Hkv;
  return w;
}

}  // namespace

// D: head dim of Q, K, dK; DV: of V, dO, dV.
template <int D, int DV, bool CAUSAL, bool WIN, bool MASK>
__global__ __launch_bounds__(512) void dkdv_pair_kernel(BwdArgs a) {
  using T = bf16;
  using M = MM<bf16>;
  typedef bf16x8 Op;
  constexpr int BK = 128;                           // keys per workgroup, 32 per wave pair
  constexpr int BQ = 64;                            // queries per block: two 32-query tiles
  constexpr int NTHR = 512;
  constexpr int NSD = D / 16;                       // steps of S = Q K^T (contraction over d)
  constexpr int NSDV = DV / 16;                     // steps of dP = dO V^T
  constexpr int NSQ = BQ / 16;                      // steps over a query block (dV, dK)
  constexpr int NDT = D / 32;                       // 32-wide dK tiles
  constexpr int NDTV = DV / 32;                     // 32-wide dV tiles
  constexpr int NBQ = 4, NB = 3;                    // Q slots; dO, L2, -D (and mask) slots
  static_assert(NSQ == 4, "P in LDS is 4 operands per lane");
  // Tiles 4096-byte aligned (XorFetch): 64 rows of 32, 64 or 128 bf16 are 4, 8 or 16 KiB.
  __shared__ __attribute__((aligned(4096))) T sQ[NBQ][BQ * D];
  __shared__ __attribute__((aligned(4096))) T sdO[NB][BQ * DV];
  __shared__ __attribute__((aligned(16))) bf16x8 sP[2][4][NSQ][64];   // [buffer][key group][step][lane]
  __shared__ __attribute__((aligned(16))) float sL[NB][64];
  __shared__ __attribute__((aligned(16))) float sD[NB][64];          // -D
  __shared__ __attribute__((aligned(16))) uint32_t sM[MASK ? NB * 4 * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = w & 3;                             // key group: keys kw .. kw + 31
  const bool pwave = w < 4;
  const int h = lane >> 5, n = lane & 31;
  const int nkb = (a.Tk + BK - 1) / BK;
  const KWork2 wk = kblock_work2(a, nkb);
  const int G = a.Hq / a.Hkv;
  const int k0 = wk.kb * BK, kw = k0 + 32 * kg, mykey = kw + n;
  const SeqView sq = seq_view(a, wk.b);
  const int Tq = sq.Tq, Tk = sq.Tk;
  if (k0 >= Tk) return;                             // uniform: before any barrier
  const size_t krow0 = sq.k_row(wk.hk);
  const int off = Tk - Tq;
  const float c = a.scale_log2;
  const bool key_ok = mykey < Tk;
  const bool ragged = k0 + BK > Tk;

  // Work list: (query block, head of the group) pairs, query blocks qb1 down
  // to qb0 (those that see some key of this block), heads innermost.
  const int nqb = (Tq + BQ - 1) / BQ;
  const int W = WIN ? a.window : 0;
  const int qb0 = CAUSAL ? min(nqb, max(0, k0 - off) / BQ) : 0;
  const int qlast = W > 0 ? min(Tq - 1, k0 + BK - 1 - off + W - 1) : Tq - 1;
  const int qb1 = qlast < 0 ? -1 : qlast / BQ;
  const int total = G * max(0, qb1 - qb0 + 1);
  // A position in the work list: its query block, head within the group and
  // LDS slot of dO, L2, -D (mod NB).  The loops step cursors forward by one
  // item per block instead of dividing by G.
  struct Cursor {
    int qb, g, buf;
  };
  auto cursor_at = [&](int it) { return Cursor{qb1 - it / G, it % G, it % NB}; };
  auto step = [&](Cursor& c) {
    if (++c.g == G) {
      c.g = 0;
      --c.qb;
    }
    c.buf = c.buf == NB - 1 ? 0 : c.buf + 1;
  };

  // Loads of block it: Q and dO rows (clamped at Tq - 1; the padding rows have
  // L2 = +inf and -D = 0, so they add nothing), L2 and -D (rows padded to 64
  // per head in the workspace), and for a boolean mask each P-wave's bits of
  // its keys (key-major copy, two words per key).  A whole block is addressed
  // from a wave-uniform row pointer plus per-lane byte offsets tabulated once;
  // only the ragged last block clamps its rows.  The loads go out as single
  // instructions ("pieces") spread over a phase of matrix products.  A block
  // of 32-wide rows (4 KiB) is half a slot per thread: the P-waves then load
  // Q and the dS-waves dO, one instruction each.
  constexpr bool SPLIT = BQ * D * 2 / 16 < NTHR;
  static_assert(!SPLIT || D == DV, "split loads for d = dv = 32");
  using DRQ = DmaRows<T, D, BQ, NTHR, 0, SPLIT ? 4 : NTHR / 64>;
  using DRO = DmaRows<T, DV, BQ, NTHR, SPLIT ? 4 : 0, SPLIT ? 4 : NTHR / 64>;
  uint32_t qoff[DRQ::PER], ooff[DRO::PER];
#pragma unroll
  for (int j = 0; j < DRQ::PER; ++j) qoff[j] = DRQ::src_off(j);
#pragma unroll
  for (int j = 0; j < DRO::PER; ++j) ooff[j] = D == DV && !SPLIT ? qoff[j % DRQ::PER] : DRO::src_off(j);
  struct Src {
    const T* q;                                     // Q row q0 of the block's head
    const T* o;                                     // dO row q0
    size_t wrow;                                    // workspace row of query q0
    int q0, qs, buf;                                // Q slot (it mod NBQ), dO / L2 / -D slot
    bool whole;                                     // all BQ rows exist: no clamping
  };
  auto block_src = [&](const Cursor& c, int it) {
    Src r;
    r.q0 = c.qb * BQ;
    r.qs = it & (NBQ - 1);
    r.buf = c.buf;
    const int hq = wk.hk * G + c.g;
    const size_t qr = sq.q_row(hq) + r.q0;
    r.q = reinterpret_cast<const T*>(a.Q) + qr * D;
    r.o = reinterpret_cast<const T*>(a.dO) + qr * DV;
    r.wrow = (size_t)(wk.b * a.Hq + hq) * a.Tqp + r.q0;
    r.whole = r.q0 + BQ <= Tq;
    return r;
  };
  static_assert((NBQ & (NBQ - 1)) == 0, "Q slots by mask");
  // Pieces 0 .. NPC - 1: Q, dO, then the L2 / -D row (waves 0 / 1) and the
  // mask word (P-waves with a mask); a piece a wave has no share of is empty.
  constexpr int NPC = DRQ::PER + DRO::PER + 1 + (MASK ? 1 : 0);
  auto piece = [&](const Src& b, int j) {
    const int buf = b.buf;
    if (j < DRQ::PER) {
      if (!DRQ::mine()) return;
      if (b.whole) dma16s(b.q, qoff[j], lds_addr(sQ[b.qs]) + DRQ::lds_off(j));
      else DRQ::one(sQ[b.qs], b.q - (size_t)b.q0 * D, b.q0, Tq, j);
    } else if (j < DRQ::PER + DRO::PER) {
      const int i = j - DRQ::PER;
      if (!DRO::mine()) return;
      if (b.whole) dma16s(b.o, ooff[i], lds_addr(sdO[buf]) + DRO::lds_off(i));
      else DRO::one(sdO[buf], b.o - (size_t)b.q0 * DV, b.q0, Tq, i);
    } else if (j == DRQ::PER + DRO::PER) {
      if (w == 0) dma_floats64(sL[buf], a.Lg + b.wrow);
      if (w == 1) dma_floats64(sD[buf], a.Dvec + b.wrow);
    } else if constexpr (MASK) {
      if (pwave)
        dma4(a.mask_t + (size_t)wk.b * a.mask_t_bstride +
                 (size_t)min(kw + (lane >> 1), Tk - 1) * a.mask_t_row_words + b.q0 / 32 + (lane & 1),
             lds_addr(sM + (buf * 4 + kg) * 64));
    }
  };
  auto issue = [&](int it) {
    const Src b = block_src(cursor_at(it), it);
#pragma unroll
    for (int j = 0; j < NPC; ++j) piece(b, j);
  };
  // Pieces go out at every other product of a phase when they fit, else at
  // every product (a mask word with d != dv).
  static_assert(NPC <= 2 * NSD && NPC <= 2 * NSDV, "pieces fit in a phase");
  constexpr int SPS = 2 * NPC <= 2 * NSD ? 2 : 1;   // spacing in the S phase (2 NSD products)
  constexpr int SPP = 2 * NPC <= 2 * NSDV ? 2 : 1;  // ... in the dP phase (2 NSDV products)

  // Direct-load instructions this wave issues per block (Q and dO rows: P-
  // and dS-waves differ when the loads are split), so that the wait at the
  // end of block i leaves block i + 2's loads in flight.
  constexpr int NLDP = SPLIT ? DRQ::PER : DRQ::PER + DRO::PER;
  constexpr int NLDS = SPLIT ? DRO::PER : DRQ::PER + DRO::PER;
  auto wait_next = [&](bool two_in_flight) {
    if (!two_in_flight) {
      wait_vmcnt<0>();
    } else if (w < 2) {                             // + the L2 or -D row
      wait_vmcnt<NLDP + 1 + (MASK ? 1 : 0)>();
    } else if (pwave) {
      wait_vmcnt<NLDP + (MASK ? 1 : 0)>();
    } else {
      wait_vmcnt<NLDS>();
    }
  };

  XorFetch<D> xf;
  xf.init(lane);
  XorFetch<DV> xfv;
  xfv.init(lane);

  if (total > 0) issue(0);

  if (pwave) {
    // ------------------------------------------------------------ P-wave
    Op kop[NSD];
    {
      const T* Kp = reinterpret_cast<const T*>(a.K) + (krow0 + (key_ok ? mykey : 0)) * D + h * (D / 2);
#pragma unroll
      for (int s = 0; s < NSD; ++s) {
        kop[s] = M::ld(Kp + s * 8);
        if (!key_ok) kop[s] = Op{};
      }
    }
    f32x16 dv[NDTV];
#pragma unroll
    for (int t = 0; t < NDTV; ++t) dv[t] = f32x16{};
    if (total > 1) issue(1);
    wait_next(total > 1);
    __syncthreads();
    Cursor ccur = cursor_at(0), ncur = cursor_at(2);   // the block worked on, the block loaded
    for (int it = 0; it <= total; ++it, step(ccur), step(ncur)) {
      const int cur = ccur.buf;
      const bool load = it + 2 < total;             // uniform
      const Src nsrc = block_src(ncur, it + 2);     // used only when load
      if (it < total) {
        const int q0 = ccur.qb * BQ;
        const uint32_t qb = lds_addr(sQ[it % NBQ]), ob = lds_addr(sdO[cur]);
        // P = exp2(S c - L2); register i of tile t holds query
        // q0 + 32 t + 8 (i / 4) + 4 h + i % 4.  A boolean mask's hidden pairs
        // get L2 = +inf (bit 4 h + 8 g + e of the tile's word for register
        // 4 g + e).  Element i of tile t, in one of 4 pieces of 4 elements.
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
        float p[2][16];
        f32x4 lt[2][4];
        uint32_t mw[2] = {0, 0};
        auto exp_piece = [&](int t, int g) {
          f32x4 l4 = lt[t][g];
          if constexpr (MASK) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int keep = (int)(mw[t] << (31 - (8 * g + e))) >> 31;
              l4[e] = __int_as_float((__float_as_int(l4[e]) & keep) | (int)(0x7f800000u & ~(uint32_t)keep));
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) p[t][4 * g + e] = fast_exp2(__builtin_fmaf(sacc[t][4 * g + e], c, -l4[e]));
        };
        // Causal diagonal, window edge and ragged key end: only on the blocks
        // that have them (a uniform test), clear hidden pairs; then pack the
        // tile's two P operands and hand them to the dS-wave through LDS.
        Op pop[NSQ];
        auto finish_tile = [&](int t) {
          if (ragged || (CAUSAL && k0 + BK - 1 > q0 + 32 * t + off) ||
              (W > 0 && q0 + 32 * t + 31 > k0 - off + W - 1)) {
            const int thr = !key_ok ? INT_MAX : (CAUSAL ? mykey - off - q0 - 32 * t - 4 * h : INT_MIN);
            const int thr_hi = W > 0 ? mykey - off + W - 1 - q0 - 32 * t - 4 * h : INT_MAX;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (8 * (i >> 2) + (i & 3) < thr || 8 * (i >> 2) + (i & 3) > thr_hi) p[t][i] = 0.f;
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            u32x4 wv;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              wv[e] = __builtin_bit_cast(uint32_t, bf16x2{(bf16)p[t][8 * j + 2 * e], (bf16)p[t][8 * j + 2 * e + 1]});
            pop[2 * t + j] = __builtin_bit_cast(bf16x8, wv);
            sP[it & 1][kg][2 * t + j][lane] = pop[2 * t + j];
          }
        };
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int g = 0; g < 4; ++g) lt[t][g] = *reinterpret_cast<const f32x4*>(&sL[cur][32 * t + 8 * g + 4 * h]);
          if constexpr (MASK) mw[t] = sM[(cur * 4 + kg) * 64 + 2 * n + t] >> (4 * h);
        }
        // S = Q K^T, tile 0 then tile 1 (lane = key); tile 0's exponentials
        // under the last products of tile 1; block it + 2's loads at every
        // other product.
        wave_prio<1>();
        pipelined<2 * NSD, 4, Op>(
            [&](int m) { return XorFetch<D>::nat(qb + xf.nat0, m / NSD, m % NSD); },
            [&](int m, const Op& x) { sacc[m / NSD] = M::mma(x, kop[m % NSD], sacc[m / NSD]); },
            [&](int m) {
              if (m % SPS == SPS - 1 && m / SPS < NPC && load) piece(nsrc, m / SPS);
              if constexpr (2 * NSD >= 5) {
                const int k = m - (2 * NSD - 5);    // 4 pieces over the last 4 products
                if (k >= 0 && k < 4) exp_piece(0, k);
              }
            });
        if constexpr (2 * NSD < 5) {                // d = 32: too few products to hide them
#pragma unroll
          for (int k = 0; k < 4; ++k) exp_piece(0, k);
        }
        finish_tile(0);
        // dV^T += dO^T P (dO^T by transposed reads), query steps of tile 0
        // first; tile 1's exponentials under those products (d = 32: before
        // them, as tile 0's steps are two products only).
        if constexpr (NDTV == 1) {
#pragma unroll
          for (int k = 0; k < 4; ++k) exp_piece(1, k);
          finish_tile(1);
        }
        pipelined<NSQ * NDTV, 4, Op>(
            [&](int m) { return XorFetch<DV>::tr(ob + xfv.tr0, m % NDTV, m / NDTV); },
            [&](int m, const Op& x) { dv[m % NDTV] = M::mma(x, pop[m / NDTV], dv[m % NDTV]); },
            [&](int m) {
              // 4 pieces from product E0 on; tile 1's operands (query steps 2
              // and 3) are complete after product 2 NDTV - 1, before their use.
              if constexpr (NDTV > 1) {
                constexpr int E0 = 2 * NDTV >= 6 ? 1 : 0;
                const int k = m - E0;
                if (k >= 0 && k < 4) exp_piece(1, k);
                if (m == 2 * NDTV - 1) finish_tile(1);
              }
            });
        static_assert(NDTV == 1 || 2 * NDTV - 1 >= (2 * NDTV >= 6 ? 1 : 0) + 3,
                      "tile 1's P is formed before its query steps");
        wave_prio<0>();
      }
      wait_next(load);
      __syncthreads();
    }
    if (key_ok) {
      T* dVr = reinterpret_cast<T*>(a.dV) + (krow0 + mykey) * DV;
#pragma unroll
      for (int t = 0; t < NDTV; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(dVr + t * 32 + 8 * g + 4 * h, dv[t][4 * g], dv[t][4 * g + 1], dv[t][4 * g + 2], dv[t][4 * g + 3]);
    }
  } else {
    // ------------------------------------------------------------ dS-wave
    Op vop[NSDV];
    {
      const T* Vp = reinterpret_cast<const T*>(a.V) + (krow0 + (key_ok ? mykey : 0)) * DV + h * (DV / 2);
#pragma unroll
      for (int s = 0; s < NSDV; ++s) {
        vop[s] = M::ld(Vp + s * 8);
        if (!key_ok) vop[s] = Op{};
      }
    }
    f32x16 dk[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t) dk[t] = f32x16{};
    f32x16 dpacc[2];                                // dP - D of the previous block (lane = key)
    if (total > 1) issue(1);
    wait_next(total > 1);
    __syncthreads();
    Cursor ccur = cursor_at(0), ncur = cursor_at(2);   // the block worked on, the block loaded
    for (int it = 0; it <= total; ++it, step(ccur), step(ncur)) {
      const int cur = ccur.buf;
      const bool load = it + 2 < total;             // uniform
      const Src nsrc = block_src(ncur, it + 2);     // used only when load
      wave_prio<1>();
      if (it > 0) {
        // dS = P (dP - D) of the previous block and dK^T += Q^T dS: the dS
        // operand of query step s + 1 is formed under the products of step s.
        const uint32_t qb = lds_addr(sQ[(it + NBQ - 1) % NBQ]);
        u32x4 pw[NSQ], dsw[NSQ];
#pragma unroll
        for (int s = 0; s < NSQ; ++s) pw[s] = __builtin_bit_cast(u32x4, sP[(it - 1) & 1][kg][s][lane]);
        auto ds_word = [&](int s, int e) {          // word e (elements 2e, 2e+1) of step s
          const f32x16& dp = dpacc[s >> 1];
          const int r = 8 * (s & 1) + 2 * e;
          const float p0 = __uint_as_float(pw[s][e] << 16), p1 = __uint_as_float(pw[s][e] & 0xffff0000u);
          dsw[s][e] = __builtin_bit_cast(uint32_t, bf16x2{(bf16)(p0 * dp[r]), (bf16)(p1 * dp[r + 1])});
        };
        // Step 0's dS words wait on the P read; the first Q^T operand reads
        // (block it - 1's slot, stable since that block) go out before them.
        pipelined_after<NSQ * NDT, 4, Op>(
            [&](int m) { return XorFetch<D>::tr(qb + xf.tr0, m % NDT, m / NDT); },
            [&]() {
#pragma unroll
              for (int e = 0; e < 4; ++e) ds_word(0, e);
            },
            [&](int m, const Op& x) {
              dk[m % NDT] = M::mma(x, __builtin_bit_cast(bf16x8, dsw[m / NDT]), dk[m % NDT]);
            },
            [&](int m) {
              const int s = m / NDT + 1, r = m % NDT;
              if (s < NSQ)
#pragma unroll
                for (int e = r * 4 / NDT; e < (r + 1) * 4 / NDT; ++e) ds_word(s, e);
            });
      }
      if (it < total) {
        // dP - D = dO V^T on a seed of -D (register i of tile t: query
        // 32 t + 8 (i / 4) + 4 h + i % 4); block it + 2's loads at every other
        // product.
        const uint32_t ob = lds_addr(sdO[cur]);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&sD[cur][32 * t + 8 * g + 4 * h]);
#pragma unroll
            for (int e = 0; e < 4; ++e) dpacc[t][4 * g + e] = v[e];
          }
        pipelined<2 * NSDV, 4, Op>(
            [&](int m) { return XorFetch<DV>::nat(ob + xfv.nat0, m & 1, m >> 1); },
            [&](int m, const Op& x) { dpacc[m & 1] = M::mma(x, vop[m >> 1], dpacc[m & 1]); },
            [&](int m) {
              if (m % SPP == SPP - 1 && m / SPP < NPC && load) piece(nsrc, m / SPP);
            });
      }
      wave_prio<0>();
      wait_next(load);
      __syncthreads();
    }
    if (key_ok) {
      T* dKr = reinterpret_cast<T*>(a.dK) + (krow0 + mykey) * D;
      const float sc = a.scale;
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(dKr + t * 32 + 8 * g + 4 * h, dk[t][4 * g] * sc, dk[t][4 * g + 1] * sc, dk[t][4 * g + 2] * sc,
                 dk[t][4 * g + 3] * sc);
    }
  }
}

template <int D, int DV, bool CAUSAL>
hipError_t launch_dkdv_pair_t(const BwdArgs& a, long long blocks, hipStream_t stream) {
  if (a.mask != nullptr)
    return a.window > 0 ? launch<512>(dkdv_pair_kernel<D, DV, CAUSAL, true, true>, blocks, stream, a)
                        : launch<512>(dkdv_pair_kernel<D, DV, CAUSAL, false, true>, blocks, stream, a);
  if (a.window > 0) return launch<512>(dkdv_pair_kernel<D, DV, CAUSAL, true, false>, blocks, stream, a);
  return launch<512>(dkdv_pair_kernel<D, DV, CAUSAL, false, false>, blocks, stream, a);
}

hipError_t launch_dkdv_pair(const BwdArgs& a, int d, int dv, int causal, hipStream_t stream) {
  const long long blocks = (long long)((a.Tk + 127) / 128) * a.B * a.Hkv;
  if (blocks <= 0) return hipSuccess;
#define FA_DKDV_CASE(DD, DDV)                                                                        \
  if (d == DD && dv == DDV)                                                                          \
    return causal ? launch_dkdv_pair_t<DD, DDV, true>(a, blocks, stream)                             \
                  : launch_dkdv_pair_t<DD, DDV, false>(a, blocks, stream);
  FA_DKDV_CASE(128, 128)
  FA_DKDV_CASE(64, 64)
  FA_DKDV_CASE(32, 32)
  FA_DKDV_CASE(128, 64)
  FA_DKDV_CASE(64, 128)
#undef FA_DKDV_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
