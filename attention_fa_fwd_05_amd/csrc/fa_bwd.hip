// Backward pass that rebuilds the score and probability tiles instead of
// storing them ("What Ordinary Autograd Saves", section "Why this is
// FlashAttention's second idea": keep O and the row statistic L, rebuild the
// rest; "Backward Pass Implementation", section "The Recomputation Strategy").
//
// Two launches on one stream (dQ pass first), or three when the caller runs
// the preprocessing on its own:
//  1. bwd_pre_kernel: -D_i = -rowsum(dO_i * O_i) and L_i in log2 units (+inf
//     for rows without keys, so their probabilities vanish).  Rows are padded
//     to a multiple of 64 per head (padding: -D = 0, L2 = +inf).  The negated
//     D seeds the dP accumulators, which then hold dP - D directly.  When the
//     dQ pass runs in the same call it forms these rows itself (each lane has
//     its query's dO in registers and reads O alongside) and writes them for
//     the dK/dV pass, which then follows it; this kernel is skipped.
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
  // 32-bit index arithmetic: B * Hq * Tqp is bounded by the grid limits.  A
  // workgroup's 16 rows lie in one (b, h), since Tqp is a multiple of 64.
  const int prow32 = (int)min(prow, prows - 1);
  const int bh = prow32 / a.Tqp;
  const int q = prow32 - bh * a.Tqp;
  const int b = bh / a.Hq, hq = bh - b * a.Hq;
  const SeqView sq = seq_view(a, b);
  const bool ok = prow < prows && q < sq.Tq;       // a real query row (else padding)
  const long long row = (long long)sq.q_row(hq) + q;
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
  a.Dvec[prow] = -acc;
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

// Position of the m-th instruction of a phase that interleaves NA products of
// kind A with NB of kind B as evenly as possible: true when it is of kind B.
__host__ __device__ constexpr bool interleave_is_b(int m, int na, int nb) {
  return ((m + 1) * nb) / (na + nb) > (m * nb) / (na + nb);
}
__host__ __device__ constexpr int interleave_rank(int m, int na, int nb) {
  // index of instruction m within its own kind
  return interleave_is_b(m, na, nb) ? (m * nb) / (na + nb) : m - ((m + 1) * nb) / (na + nb);
}

__device__ inline void zero_elem(bf16x8& x, int e) { x[e] = (bf16)0.f; }
__device__ inline void zero_elem(f32x4& x, int e) { x[e] = 0.f; }

// LDS words of a boolean mask's bits for the tiles in flight: 64 per wave and
// buffer, written by one 4-byte direct load per wave (lane l: word l % 2 of
// row l / 2 of the wave's 32 rows) and read back as two words per lane.  Only
// the kernels compiled with a mask instantiate it.
template <int N>
__device__ inline uint32_t* mask_lds() {
  __shared__ __attribute__((aligned(16))) uint32_t m[N];
  return m;
}

// Key-major copy of a query-major mask: word (b, w, j) of mask_t holds in bit
// e the bit of (query 32 w + e, key j), 0 past Tq.  One thread per output
// word, key fastest, so neighbouring threads read the same source words.
__global__ __launch_bounds__(256) void mask_transpose_kernel(BwdArgs a, long long entries) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int rwq = a.mask_t_row_words;
  const long long per = (long long)a.Tk * rwq;
  if (i >= entries * per) return;
  const long long b = i / per, r = i % per;
  const int w = (int)(r / a.Tk), j = (int)(r % a.Tk);
  const uint32_t* src = a.mask + b * a.mask_bstride + (j >> 5);
  uint32_t v = 0;
  for (int e = 0; e < 32 && 32 * w + e < a.Tq; ++e)
    v |= ((src[(size_t)(32 * w + e) * a.mask_row_words] >> (j & 31)) & 1u) << e;
  a.mask_t[b * a.mask_t_bstride + (size_t)j * rwq + w] = v;
}

// D: head dim of Q, K, dK; DV: of V, dO, dV.  HSPLIT: each workgroup forms
// one half of the columns of dK and dV (blockIdx.y; S and dP still contract
// over the whole head dim), so that a 256-wide head's accumulators fit.
template <typename T, int D, bool CAUSAL, bool WIN, int DV = D, bool MASK = false, bool HSPLIT = false>
__global__ __launch_bounds__(256) void dkdv_kernel(BwdArgs a) {
  using M = MM<T>;
  typedef typename M::Op Op;
  constexpr int BK = 128;                           // keys per workgroup, 32 per wave
  constexpr int BQ = 64;                            // queries per block: two 32-query tiles
  constexpr int KPER = M::KPER;
  constexpr int NSD = (D / 2) / KPER;               // contraction steps over d (S = Q K^T)
  constexpr int NSDV = (DV / 2) / KPER;             // ... over dv (dP = dO V^T)
  constexpr int NSQ = (BQ / 2) / KPER;              // contraction steps over a query block
  constexpr int NDT = D / (HSPLIT ? 64 : 32);       // 32-wide dK tiles (of this workgroup's half)
  constexpr int NDTV = DV / (HSPLIT ? 64 : 32);     // 32-wide dV tiles
  constexpr int NPS = NDT + NDTV;                   // dV and dK products per query step
  constexpr int NSH = NSQ / 2;                      // steps per 32-query tile
  // Three LDS buffers let block i+2 load while blocks i and i+1 are read;
  // fp32 with d = 128 fits two, and then loads without overlap.
  constexpr int NB = ((sizeof(T) == 4 && D == 128) || D == 256) ? 2 : 3;
  // Software pipeline over the query blocks of the work list, iteration i:
  //   phase 1a: S, dP of block i+1 tile 0  |  dV, dK of block i, first quarter
  //             of its query steps  |  P, dS of block i tile 1;
  //   phase 1b: S, dP of block i+1 tile 1  |  dV, dK of block i, second
  //             quarter  |  P, dS of block i+1 tile 0, first half;
  //   phase 2:  dV, dK of block i, second half  |  P, dS of block i+1 tile 0,
  //             second half.
  // The vector work of an element runs in three stages on successive product
  // steps (x = S c - L2; P = exp2 x; dS = P (dP - D) and packing), so that a
  // step's vector instructions never wait on one another and the in-order
  // issue keeps feeding the matrix unit.  P, dS of a tile overwrite those of
  // the same tile of the previous block once its last product has been
  // issued.  Products and LDS reads go out in a fixed order with a fixed
  // number of operands in flight; the loop is unrolled over the buffers so
  // every LDS address is a lane offset plus a constant.
  constexpr int NS1 = NSD + NSDV;                   // S and dP products per tile
  constexpr int NDQ = (NSH / 2) * NPS;              // dV/dK products per quarter of the steps
  constexpr int NDH = NSH * NPS;                    // ... per half
  constexpr int NPA = NS1 + NDQ;                    // products in phase 1a (and 1b)
  // Operands in flight: a divisor of NPA, so the ring slots line up across phases.
  constexpr int AHEAD = sizeof(T) != 2 ? 4 : NPA % 8 == 0 ? 8 : (D != DV && NPA % 6 == 0) ? 6 : 4;
  static_assert(NSH % 2 == 0, "quarters of the query steps");
  static_assert(NPA % AHEAD == 0, "operand ring slots line up across phases");
  static_assert(NPA >= 12 && NDH >= 8, "room for the vector stages");
  static_assert(NB == 2 || 2 * (DmaRows<T, D, BQ, 256>::PER + DmaRows<T, DV, BQ, 256>::PER + 1) <= NPA,
                "loads fit in phase 1b");
  __shared__ __attribute__((aligned(16))) float sL[NB][64];
  __shared__ __attribute__((aligned(16))) float sD[NB][64];    // -D
  __shared__ __attribute__((aligned(16))) T sQ[NB][BQ * D];
  __shared__ __attribute__((aligned(16))) T sdO[NB][BQ * DV];

  // The wave index is uniform across a wave; readfirstlane tells the compiler,
  // so conditions built from it become scalar branches.
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n = lane & 31;
  const int nkb = (a.Tk + BK - 1) / BK;
  const KWork wk = kblock_work(a, nkb);
  const int G = a.Hq / a.Hkv;
  const int k0 = wk.kb * BK, kw = k0 + 32 * w, mykey = kw + n;
  const int T0 = HSPLIT ? (int)blockIdx.y * NDT : 0;      // first dK tile (and dV tile) of the half
  const int T0V = HSPLIT ? (int)blockIdx.y * NDTV : 0;
  // This workgroup's sequence (a variable-length batch has its own lengths
  // and rows; the grid covers the longest).  No key of it here: leave before
  // any barrier (uniform).
  const SeqView sq = seq_view(a, wk.b);
  const int Tq = sq.Tq, Tk = sq.Tk;
  if (k0 >= Tk) return;
  const size_t krow0 = sq.k_row(wk.hk);  // row of key 0 of (b, hk) in K, V, dK, dV
  const int off = Tk - Tq;
  const float c = a.scale_log2;
  const bool key_ok = mykey < Tk;
  const bool ragged = k0 + BK > Tk;                 // uniform: this block holds the key end

  const T* Kp = reinterpret_cast<const T*>(a.K) + krow0 * D;
  const T* Vp = reinterpret_cast<const T*>(a.V) + krow0 * DV;

  // Work list: every (query block that can see a key of this block, query
  // head of the group), query blocks from the last one down and heads
  // innermost.  All key blocks of a group run at once on one XCD and step
  // through the same query blocks in lockstep (each stops at its diagonal), so
  // every Q / dO block is fetched into that XCD's L2 once, not once per key
  // block.
  // Query blocks qb0 .. qb1 see some key of this block: none before the
  // causal bound of its first key, none past the window of its last.
  const int nqb = (Tq + BQ - 1) / BQ;
  const int W = WIN ? a.window : 0;               // compile-time 0 without a window
  const int qb0 = CAUSAL ? min(nqb, max(0, k0 - off) / BQ) : 0;
  const int qlast = W > 0 ? min(Tq - 1, k0 + BK - 1 - off + W - 1) : Tq - 1;   // last query seeing a key
  const int qb1 = qlast < 0 ? -1 : qlast / BQ;
  const int total = G * max(0, qb1 - qb0 + 1);
  auto item_q0 = [&](int it) { return (qb1 - it / G) * BQ; };
  auto item_bh = [&](int it) { return wk.b * a.Hq + wk.hk * G + it % G; };   // workspace rows (padded)
  auto item_qrow = [&](int it) { return sq.q_row(wk.hk * G + it % G); };   // Q, dO rows
  // L2 and D rows are padded to 64 per head, so a 64-row window always loads.
  // Boolean mask: this wave's keys' bits of a query block (key-major copy),
  // two words per key; lane l loads word l % 2 of key kw + l / 2 (keys past Tk
  // read the last key's row; their results are never stored).
  uint32_t* sM = nullptr;
  if constexpr (MASK) sM = mask_lds<NB * 256>();
  auto mask_src = [&](int it) -> const uint32_t* {
    return a.mask_t + (size_t)wk.b * a.mask_t_bstride +
           (size_t)min(kw + (lane >> 1), Tk - 1) * a.mask_t_row_words + item_q0(it) / 32 + (lane & 1);
  };
  auto issue = [&](int it, int buf) {
    const int bh = item_bh(it);
    const int q0 = item_q0(it);
    const size_t qbase = item_qrow(it) * D, obase = item_qrow(it) * DV;
    dma_rows<T, D, BQ, 256>(sQ[buf], reinterpret_cast<const T*>(a.Q) + qbase, q0, Tq);
    dma_rows<T, DV, BQ, 256>(sdO[buf], reinterpret_cast<const T*>(a.dO) + obase, q0, Tq);
    if (w == 0) dma_floats64(sL[buf], a.Lg + (size_t)bh * a.Tqp + q0);
    if (w == 1) dma_floats64(sD[buf], a.Dvec + (size_t)bh * a.Tqp + q0);
    if constexpr (MASK) dma4(mask_src(it), lds_addr(sM + buf * 256 + w * 64));
  };
  if (total > 0) issue(0, 0);
  if (total > 1) issue(1, 1);
  // The same loads split into single instructions, spread over phase 1b (the
  // phase with the least vector work) so that no step issues a burst and the
  // address unit is never backed up: NDMA pieces, Q rows, dO rows, then L2
  // and -D.
  using DR = DmaRows<T, D, BQ, 256>;
  using DRV = DmaRows<T, DV, BQ, 256>;
  constexpr int NDMA = DR::PER + DRV::PER + 1 + (MASK ? 1 : 0);
  static_assert(NB == 2 || 2 * NDMA <= NPA, "loads fit in phase 1b");
  uint32_t src_off[DR::PER], src_offv[DRV::PER];   // per-lane source byte offsets, one per instruction
#pragma unroll
  for (int j = 0; j < DR::PER; ++j) src_off[j] = DR::src_off(j);
#pragma unroll
  for (int j = 0; j < DRV::PER; ++j) src_offv[j] = D == DV ? src_off[j % DR::PER] : DRV::src_off(j);
  // Uniform description of one block's loads (computed once per iteration).
  struct Src {
    const char* q;                                  // Q row q0 of the head
    const char* o;                                  // dO row q0 of the head
    const float* l;
    const float* d;
    int q0;
    bool whole;                                     // all BQ rows exist: no clamping
    const uint32_t* m;                              // this lane's mask word (MASK)
  };
  auto block_src = [&](int it) {
    Src r;
    if constexpr (MASK) r.m = mask_src(it);
    const int bh = item_bh(it);
    r.q0 = item_q0(it);
    const size_t row = item_qrow(it) + r.q0;
    r.q = reinterpret_cast<const char*>(a.Q) + row * D * sizeof(T);
    r.o = reinterpret_cast<const char*>(a.dO) + row * DV * sizeof(T);
    r.l = a.Lg + (size_t)bh * a.Tqp + r.q0;
    r.d = a.Dvec + (size_t)bh * a.Tqp + r.q0;
    r.whole = r.q0 + BQ <= Tq;
    return r;
  };
  auto dma_piece = [&](const Src& src, int buf, int j) {
    if (j < DR::PER) {
      if (src.whole) {
        dma16s(src.q, src_off[j], lds_addr(sQ[buf]) + DR::lds_off(j));
      } else {                                      // ragged end of the queries: clamped rows
        const T* g = reinterpret_cast<const T*>(src.q) - (size_t)src.q0 * D;
        DR::one(sQ[buf], g, src.q0, Tq, j);
      }
    } else if (j < DR::PER + DRV::PER) {
      const int i = j - DR::PER;
      if (src.whole) {
        dma16s(src.o, src_offv[i], lds_addr(sdO[buf]) + DRV::lds_off(i));
      } else {
        const T* g = reinterpret_cast<const T*>(src.o) - (size_t)src.q0 * DV;
        DRV::one(sdO[buf], g, src.q0, Tq, i);
      }
    } else if (!MASK || j == DR::PER + DRV::PER) {
      if (w == 0) dma_floats64(sL[buf], src.l);
      if (w == 1) dma_floats64(sD[buf], src.d);
    } else {
      dma4(src.m, lds_addr(sM + buf * 256 + w * 64));
    }
  };

  Op kop[NSD], vop[NSDV];
  {
    const size_t ro = (size_t)(key_ok ? mykey : 0) * D + h * (D / 2);
    const size_t rov = (size_t)(key_ok ? mykey : 0) * DV + h * (DV / 2);
    // K and V only feed matrix instructions: keep them in accumulation
    // registers, leaving the vector registers to the softmax work.
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      kop[s] = M::ld(Kp + ro + s * KPER);
      if (!key_ok) kop[s] = Op{};
      if constexpr (sizeof(T) == 2) asm volatile("" : "+a"(kop[s]));
    }
#pragma unroll
    for (int s = 0; s < NSDV; ++s) {
      vop[s] = M::ld(Vp + rov + s * KPER);
      if (!key_ok) vop[s] = Op{};
      if constexpr (sizeof(T) == 2) asm volatile("" : "+a"(vop[s]));
    }
  }
  f32x16 dk[NDT], dv[NDTV];
#pragma unroll
  for (int t = 0; t < NDT; ++t) dk[t] = f32x16{};
#pragma unroll
  for (int t = 0; t < NDTV; ++t) dv[t] = f32x16{};
  // Natural and transposed operand fetchers of the Q tiles (width d) and the
  // dO tiles (width dv).
  NatFetch<T, D> nat;
  nat.init(n, h);
  TrPermFetch<T, D> trp;
  trp.init(lane);
  NatFetch<T, DV> natv;
  TrPermFetch<T, DV> trpv;
  if constexpr (DV != D) {
    natv.init(n, h);
    trpv.init(lane);
  }
  // dO natural / transposed operands through the fetcher of its width.
  auto nat_o = [&](const T* tile, int t, int s) -> Op {
    if constexpr (DV == D) return nat.ld(tile, t, s);
    else return natv.ld(tile, t, s);
  };
  auto tr_o = [&](const T* tile, int t, int s) -> Op {
    if constexpr (DV == D) return trp.ld(tile, t, s);
    else return trpv.ld(tile, t, s);
  };

  f32x16 sacc[2], dpacc[2];                         // S and dP - D of one block (lane = key)
  Op pop[NSQ], dsop[NSQ];                           // P, dS as operands, by query step

  // Seed of tile t's dP accumulator: -D of the tile's queries (register i
  // holds query 32 t + 8 (i / 4) + 4 h + i % 4).
  auto seed_dp = [&](const float* nd, int t) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(nd + 32 * t + 8 * g + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) dpacc[t][4 * g + e] = v[e];
    }
  };
  // S / dP product m of tile t: the NSD products of S = Q K^T first, then
  // those of dP = dO V^T (their seed then has time to arrive).
  auto s_mma = [&](int t, int m, const Op& x) {
    if (m < NSD) sacc[t] = M::mma(x, kop[m], sacc[t]);
    else dpacc[t] = M::mma(x, vop[m - NSD], dpacc[t]);
  };
  // dV / dK product m (0 .. NSQ * NPS): query step m / NPS outermost; within
  // a step the NDTV dV and NDT dK products alternate as evenly as possible
  // (strictly alternating, dV first, when d = dv).
  auto d_mma = [&](int m, const Op& x) {
    const int s = m / NPS, r = m % NPS;
    const int t = interleave_rank(r, NDTV, NDT);
    if (interleave_is_b(r, NDTV, NDT)) dk[t] = M::mma(x, dsop[s], dk[t]);
    else dv[t] = M::mma(x, pop[s], dv[t]);
  };
  // L2 of one tile's queries in accumulator order (block in buffer buf).  A
  // boolean mask enters here: a pair whose bit is 0 gets L2 = +inf, so its
  // P = exp2(S c - L2) and dS are 0 through the ordinary stages (bit
  // 4 h + 8 g + e of the tile's word for register 4 g + e).
  f32x4 lt[4];
  auto load_l = [&](int buf, int t) {
    const float* lg = sL[buf];
#pragma unroll
    for (int g = 0; g < 4; ++g) lt[g] = *reinterpret_cast<const f32x4*>(lg + 32 * t + 8 * g + 4 * h);
    if constexpr (MASK) {
      const uint32_t mw = sM[buf * 256 + w * 64 + 2 * n + t] >> (4 * h);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int keep = (int)(mw << (31 - (8 * g + e))) >> 31;   // 0 or all ones
          lt[g][e] = __int_as_float((__float_as_int(lt[g][e]) & keep) | (int)(0x7f800000u & ~(uint32_t)keep));
        }
    }
  };
  // The three vector stages of register e of tile t.
  float xa[16], pa[16];
  uint32_t ppk[8], dpk[8];                          // packed bf16 pairs (bf16 operands)
  auto st1 = [&](int t, int e) { xa[e] = __builtin_fmaf(sacc[t][e], c, -lt[e >> 2][e & 3]); };
  auto st2 = [&](int e) { pa[e] = fast_exp2(xa[e]); };
  auto st3 = [&](int t, int e) {
    if constexpr (sizeof(T) == 4) {
      if ((e & 3) == 3) {
        const int s = (16 * t + e) / 4;
        pop[s] = f32x4{pa[e - 3], pa[e - 2], pa[e - 1], pa[e]};
        dsop[s] = f32x4{dpacc[t][e - 3] * pa[e - 3], dpacc[t][e - 2] * pa[e - 2],
                        dpacc[t][e - 1] * pa[e - 1], dpacc[t][e] * pa[e]};
      }
    } else if (e & 1) {
      // Whole 32-bit words (one v_cvt_pk_bf16_f32 each) assembled into the
      // operand as words, so no 16-bit lane shuffles are generated.
      ppk[e >> 1] = __builtin_bit_cast(uint32_t, bf16x2{(bf16)pa[e - 1], (bf16)pa[e]});
      dpk[e >> 1] = __builtin_bit_cast(uint32_t, bf16x2{(bf16)(dpacc[t][e - 1] * pa[e - 1]),
                                                         (bf16)(dpacc[t][e] * pa[e])});
      if ((e & 7) == 7) {
        const int s = (16 * t + e) / 8, j = (e >> 1) - 3;
        pop[s] = __builtin_bit_cast(bf16x8, u32x4{ppk[j], ppk[j + 1], ppk[j + 2], ppk[j + 3]});
        dsop[s] = __builtin_bit_cast(bf16x8, u32x4{dpk[j], dpk[j + 1], dpk[j + 2], dpk[j + 3]});
      }
    }
  };
  // Stages due at step m of a schedule whose element e (e0 <= e < e1) starts
  // at step (e - e0) * span / (e1 - e0).
  auto stages = [&](int t, int m, int e0, int e1, int span) {
#pragma unroll
    for (int e = e0; e < e1; ++e) {
      const int f = (e - e0) * span / (e1 - e0);
      if (f + 2 == m) st3(t, e);
      if (f + 1 == m) st2(e);
      if (f == m) st1(t, e);
    }
  };
  constexpr int SPAN1A = NPA - 4;                   // tile 1 of block i over phase 1a
  constexpr int SPAN1B = NPA - 3;                   // tile 0, registers 0..7, over phase 1b
  constexpr int SPAN2 = NDH - 3;                    // tile 0, registers 8..15, over phase 2
  constexpr int LOADL0 = 15 * SPAN1A / 16 + 1;      // after tile 1's last stage 1
  static_assert(15 * SPAN1A / 16 + 2 < NPA - 1, "tile 1 done before its reseed");
  // Causal diagonal and ragged key end, only on the blocks that have them:
  // P and dS of pairs the key may not see are cleared in the packed operands.
  // Register i of tile t holds query q0 + 32 t + 4 h + 8 (i / 4) + i % 4.
  // The sliding window clears pairs whose query is past the key's window.
  // (A boolean mask is applied through L2 in load_l.)
  auto mask_tile = [&](int q0, int t) {
    if (ragged || (CAUSAL && k0 + BK - 1 > q0 + 32 * t + off) || (W > 0 && q0 + 32 * t + 31 > k0 - off + W - 1)) {
      const int thr = !key_ok ? INT_MAX : (CAUSAL ? mykey - off - q0 - 32 * t - 4 * h : INT_MIN);
      const int thr_hi = W > 0 ? mykey - off + W - 1 - q0 - 32 * t - 4 * h : INT_MAX;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (8 * (i >> 2) + (i & 3) < thr || 8 * (i >> 2) + (i & 3) > thr_hi) {
          const int s = (16 * t + i) / KPER;
          zero_elem(pop[s], i % KPER);
          zero_elem(dsop[s], i % KPER);
        }
      }
    }
  };

  wait_vmcnt<0>();
  __syncthreads();
  if (total > 0) {                                  // block 0: S, dP and tile 0's P, dS
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = f32x16{};
      seed_dp(sD[0], t);
#pragma unroll
      for (int m = 0; m < NS1; ++m) s_mma(t, m, m < NSD ? nat.ld(sQ[0], t, m) : nat_o(sdO[0], t, m - NSD));
    }
    load_l(0, 0);
#pragma unroll
    for (int m = 0; m < 18; ++m) stages(0, m, 0, 16, 16);
    mask_tile(item_q0(0), 0);
    load_l(0, 1);
  }

  // One iteration with block i in buffer CUR, block i+1 in the next buffer.
  auto iteration = [&](auto cur_c, int it) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int nxt = (cur + 1) % NB, nn = (cur + 2) % NB;
    // Block i+2 goes to buffer nn (free since the last barrier); past the end
    // of the list the last block is loaded again, harmlessly.
    const Src dsrc = block_src(min(it + 2, total - 1));
    // On the last item buffer nxt holds stale rows: its products are computed
    // and discarded, which keeps the sequence free of branches.
    const int q0 = item_q0(it), nq0 = item_q0(it + 1);
    const T* cQ = sQ[cur];
    const T* cdO = sdO[cur];
    const T* nQ = sQ[nxt];
    const T* ndO = sdO[nxt];

    // S / dP operand of product m of tile t (block i+1), dV / dK operand of
    // product m (block i).
    auto s_fetch = [&](int t, int m) -> Op { return m < NSD ? nat.ld(nQ, t, m) : nat_o(ndO, t, m - NSD); };
    auto d_fetch = [&](int m) -> Op {
      const int s = m / NPS, r = m % NPS;
      const int t = interleave_rank(r, NDTV, NDT);
      return interleave_is_b(r, NDTV, NDT) ? trp.ld(cQ, T0 + t, s) : tr_o(cdO, T0V + t, s);
    };
    // Phases 1a and 1b: tile u of block i+1's S, dP interleaved with quarter u
    // of block i's dV, dK.
    auto p1_fetch = [&](int u, int m) -> Op {
      return interleave_is_b(m, NS1, NDQ) ? d_fetch(u * NDQ + interleave_rank(m, NS1, NDQ))
                                          : s_fetch(u, interleave_rank(m, NS1, NDQ));
    };
    Op ring[AHEAD];
    sacc[0] = f32x16{};
    seed_dp(sD[nxt], 0);
#pragma unroll
    for (int m = 0; m < AHEAD; ++m) ring[m] = p1_fetch(0, m);
    // Half u as a compile-time constant: the phase is one straight sequence.
    auto phase1 = [&](auto u_c) {
      constexpr int u = decltype(u_c)::value;
#pragma unroll
      for (int m = 0; m < NPA; ++m) {
        const Op x = ring[m % AHEAD];
        if (m + AHEAD < NPA) ring[m % AHEAD] = p1_fetch(u, m + AHEAD);
        else if (u == 0) ring[m % AHEAD] = p1_fetch(1, m + AHEAD - NPA);
        else ring[m % AHEAD] = d_fetch(NDH + (m + AHEAD - NPA));
        if (interleave_is_b(m, NS1, NDQ)) d_mma(u * NDQ + interleave_rank(m, NS1, NDQ), x);
        else s_mma(u, interleave_rank(m, NS1, NDQ), x);
        if (NB == 3 && u == 1 && m % 2 == 1 && m / 2 < NDMA) dma_piece(dsrc, nn, m / 2);
        if (u == 0) {
          stages(1, m, 0, 16, SPAN1A);             // tile 1 of block i
          if (m == LOADL0) load_l(nxt, 0);         // L2 of block i+1's tile 0
          if (m == NPA - 1) {                      // tile 1 of block i is done with S, dP
            sacc[1] = f32x16{};
            seed_dp(sD[nxt], 1);
          }
        } else {
          stages(0, m, 0, 8, SPAN1B);              // tile 0 of block i+1, first half
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    phase1(IC<0>{});
    mask_tile(q0, 1);
    phase1(IC<1>{});

    // Phase 2: the second half of block i's dV, dK, with the second half of
    // block i+1's tile-0 probabilities.
#pragma unroll
    for (int m = 0; m < NDH; ++m) {
      const Op x = ring[(2 * NPA + m) % AHEAD];
      if (m + AHEAD < NDH) ring[(2 * NPA + m) % AHEAD] = d_fetch(NDH + m + AHEAD);
      d_mma(NDH + m, x);
      stages(0, m, 8, 16, SPAN2);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask_tile(nq0, 0);
    load_l(nxt, 1);                                // for block i+1's tile-1 probabilities
    if (NB == 3) {
      wait_vmcnt<0>();                             // this wave's loads of block i+2 have landed
      __syncthreads();
    } else {
      __syncthreads();                             // block i's buffer is free
      if (it + 2 < total) issue(it + 2, cur);
      wait_vmcnt<0>();
      __syncthreads();
    }
  };
  for (int it = 0; it < total; it += NB) {
    iteration(IC<0>{}, it);
    if (it + 1 < total) iteration(IC<1>{}, it + 1);
    if (NB == 3 && it + 2 < total) iteration(IC<NB - 1>{}, it + 2);
  }

  if (key_ok) {
    T* dKr = reinterpret_cast<T*>(a.dK) + (krow0 + mykey) * D;
    T* dVr = reinterpret_cast<T*>(a.dV) + (krow0 + mykey) * DV;
    const float sc = a.scale;
#pragma unroll
    for (int t = 0; t < (NDT > NDTV ? NDT : NDTV); ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = t * 32 + 8 * g + 4 * h;
        if (t < NDT)
          store4(dKr + T0 * 32 + d0, dk[t][4 * g] * sc, dk[t][4 * g + 1] * sc, dk[t][4 * g + 2] * sc,
                 dk[t][4 * g + 3] * sc);
        if (t < NDTV)
          store4(dVr + T0V * 32 + d0, dv[t][4 * g], dv[t][4 * g + 1], dv[t][4 * g + 2], dv[t][4 * g + 3]);
      }
    }
  }
}

// Waves per dQ workgroup: 8 (256 query rows), or 4 where fp32 d = 128
// operands would not fit in 256 registers.
template <typename T, int D>
constexpr int dq_waves() { return sizeof(T) == 4 || D == 32 || D == 256 ? 4 : 8; }

// D: head dim of Q, K, dQ; DV: of V and dO.
template <typename T, int D, bool CAUSAL, bool WIN, int DV = D, bool MASK = false>
__global__ __launch_bounds__((64 * dq_waves<T, D>())) void dq_kernel(BwdArgs a) {
  using M = MM<T>;
  typedef typename M::Op Op;
  constexpr int NW = dq_waves<T, D>(), NTHR = 64 * NW, BQ = 32 * NW, BK = 64;
  constexpr int KPER = M::KPER;
  constexpr int NSD = (D / 2) / KPER;
  constexpr int NSDV = (DV / 2) / KPER;              // steps of dP^T = V dO^T
  constexpr int NSK = (BK / 2) / KPER;
  constexpr int NDT = D / 32;
  // K/V buffers.  8 waves (bf16, d <= 128): four, taken two tiles per
  // barrier: tiles j+2 and j+3 load while tiles j and j+1 are read, so the
  // workgroup meets one barrier per 128 keys, and the wave that finishes
  // tile j first goes on to tile j+1 instead of waiting for the others.
  // 4 waves: two (fp32 with d = 128 fits no more; its loads then wait within
  // the tile), one tile per barrier.
  constexpr bool STEP2 = NW == 8;
  constexpr int NBUF = STEP2 ? 4 : 2;
  constexpr int AHEAD = STEP2 ? 2 : 1;             // tiles loaded before the first barrier
  constexpr int TILE = BK * D;                      // elements of one K tile (the V tile follows)
  // Buffer b: K tile, then V tile; 4096-byte alignment for XorFetch (both
  // tile sizes are multiples of 4096 bytes).
  __shared__ __attribute__((aligned(4096))) T sKV[NBUF][BK * (D + DV)];

  // The wave index is uniform across a wave; readfirstlane tells the compiler,
  // so conditions built from it become scalar branches.
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n = lane & 31;
  const int nqb = (a.Tq + BQ - 1) / BQ;
  const QWork wk = qblock_work(a.B, a.Hq, a.Hkv, nqb, CAUSAL);
  const int bh = wk.b * a.Hq + wk.hq;               // workspace rows (padded per head)
  const int q0 = wk.qb * BQ, qw = q0 + 32 * w, myq = qw + n;
  // This workgroup's sequence (its own lengths and rows in a variable-length
  // batch).  No query of it here: leave before any barrier (uniform).
  const SeqView sq = seq_view(a, wk.b);
  const int Tq = sq.Tq, Tk = sq.Tk;
  if (q0 >= Tq) return;
  const size_t qrow0 = sq.q_row(wk.hq);  // row of query 0 of (b, hq) in Q, dO, dQ
  const size_t krow0 = sq.k_row(wk.hk);
  const int off = Tk - Tq;
  const bool q_ok = myq < Tq;

  const T* Qp = reinterpret_cast<const T*>(a.Q) + qrow0 * D;
  const T* dOp = reinterpret_cast<const T*>(a.dO) + qrow0 * DV;
  const T* Kp = reinterpret_cast<const T*>(a.K) + krow0 * D;
  const T* Vp = reinterpret_cast<const T*>(a.V) + krow0 * DV;

  // Key tiles jt0 .. ntiles - 1 (before the window of the block's first
  // query, or after the causal bound of its last, nothing is visible).
  const int W = WIN ? a.window : 0;               // compile-time 0 without a window
  int kend = Tk;
  if (CAUSAL) kend = min(Tk, max(0, q0 + BQ + off));
  const int ntiles = (kend + BK - 1) / BK;
  const int jt0 = W > 0 ? min(ntiles, max(0, q0 + off - W + 1) / BK) : 0;

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
  // Boolean mask: this wave's rows' bits of a key tile (query-major), two
  // words per row; lane l loads word l % 2 of row qw + l / 2 (rows past Tq
  // read the last row; their results are never stored).
  uint32_t* sM = nullptr;
  if constexpr (MASK) sM = mask_lds<NBUF * NW * 64>();
  auto issue = [&](int k0, int buf) {
    T* tk = sKV[buf];
    T* tv = sKV[buf] + TILE;
    if (k0 + BK <= Tk) {
      const T* kb = Kp + (size_t)k0 * D;
      const T* vb = Vp + (size_t)k0 * DV;
#pragma unroll
      for (int i = 0; i < DR::PER; ++i) dma16s(kb, src_off[i], lds_addr(tk) + DR::lds_off(i));
#pragma unroll
      for (int i = 0; i < DRV::PER; ++i) dma16s(vb, src_offv[i], lds_addr(tv) + DRV::lds_off(i));
    } else {
      dma_rows<T, D, BK, NTHR>(tk, Kp, k0, Tk);
      dma_rows<T, DV, BK, NTHR>(tv, Vp, k0, Tk);
    }
    if constexpr (MASK)
      dma4(a.mask + (size_t)wk.b * a.mask_bstride + (size_t)min(qw + (lane >> 1), Tq - 1) * a.mask_row_words +
               k0 / 32 + (lane & 1),
           lds_addr(sM + (buf * NW + w) * 64));
  };
#pragma unroll
  for (int j = 0; j < AHEAD; ++j)
    if (jt0 + j < ntiles) issue((jt0 + j) * BK, j);

  // Q^T and dO^T operands for this lane's query, L2 and D of that row.
  Op qop[NSD], gop[NSDV];
  {
    const size_t ro = (size_t)(q_ok ? myq : 0) * D + h * (D / 2);
    const size_t rov = (size_t)(q_ok ? myq : 0) * DV + h * (DV / 2);
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      qop[s] = M::ld(Qp + ro + s * KPER);
      if (!q_ok) qop[s] = Op{};
    }
#pragma unroll
    for (int s = 0; s < NSDV; ++s) {
      gop[s] = M::ld(dOp + rov + s * KPER);
      if (!q_ok) gop[s] = Op{};
    }
  }
  // L2 and -D of this lane's query: read from the workspace, or formed here
  // (-D = -rowsum(dO * O): this lane's half of the row against its dO
  // operands, then the other half's from lane n + 32 h') and written there
  // for the dK/dV pass, padding rows (+inf, 0) included.
  float l2, ndd;
  if (a.fuse_pre) {
    const T* Orow = reinterpret_cast<const T*>(a.O) + (qrow0 + (q_ok ? myq : 0)) * DV + h * (DV / 2);
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < NSDV; ++s) {
      const Op o = M::ld(Orow + s * KPER);
#pragma unroll
      for (int e = 0; e < KPER; ++e) acc += (float)o[e] * (float)gop[s][e];
    }
    acc = wave_xor32_sum(acc);
    const float l = q_ok ? a.L[qrow0 + myq] : -INFINITY;
    l2 = l == -INFINITY ? INFINITY : l * kLog2e;
    ndd = q_ok ? -acc : 0.f;
    if (h == 0 && myq < a.Tqp) {
      a.Lg[(size_t)bh * a.Tqp + myq] = l2;
      a.Dvec[(size_t)bh * a.Tqp + myq] = ndd;
    }
  } else {
    l2 = q_ok ? a.Lg[(size_t)bh * a.Tqp + myq] : INFINITY;
    ndd = q_ok ? a.Dvec[(size_t)bh * a.Tqp + myq] : 0.f;
  }
  // Operand fetch: bf16 from one base register per tile (XorFetch); fp32
  // (test shapes only) from offset tables.
  XorFetch<D> xf;
  XorFetch<DV> xfv;
  NatFetch<T, D> nat;
  NatFetch<T, DV> natv;
  TrPermFetch<T, D> trp;
  if constexpr (sizeof(T) == 2) {
    xf.init(lane);
    if constexpr (DV != D) xfv.init(lane);
  } else {
    nat.init(n, h);
    natv.init(n, h);
    trp.init(lane);
  }
  // Natural K (kv = 0) or V (kv = 1) operand of key sub-tile t, step s, and
  // transposed K operand of d tile t, step s, from buffer buf.
  auto ld_nat = [&](int buf, int kv, int t, int s) -> Op {
    if constexpr (sizeof(T) == 2) {
      if (kv == 0) return XorFetch<D>::nat(lds_addr(sKV[buf]) + xf.nat0, t, s);
      return XorFetch<DV>::nat(lds_addr(sKV[buf]) + (DV == D ? xf.nat0 : xfv.nat0) + TILE * 2, t, s);
    } else {
      if (kv == 0) return nat.ld(sKV[buf], t, s);
      return natv.ld(sKV[buf] + TILE, t, s);
    }
  };
  auto ld_tr = [&](int buf, int t, int s) -> Op {
    if constexpr (sizeof(T) == 2) {
      return XorFetch<D>::tr(lds_addr(sKV[buf]) + xf.tr0, t, s);
    } else {
      return trp.ld(sKV[buf], t, s);
    }
  };
  wait_vmcnt<0>();
  __syncthreads();

  const float c = a.scale_log2;
  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};
  // S^T = K Q^T and dP^T = V dO^T of one tile: 64 keys x 32 queries each.
  // The dP^T products start from -D (this lane's row), read from a register
  // tile that stays fixed over the loop, so they form dP - D without a
  // per-element add or per-tile copies.
  f32x16 st0, st1, dp0, dp1;
  f32x16 dseed;
#pragma unroll
  for (int r = 0; r < 16; ++r) dseed[r] = ndd;

  // Some key of tile j is visible to this wave's queries.
  auto visible = [&](int j) {
    return !(CAUSAL && j * BK > qw + 31 + off) && !(W > 0 && j * BK + BK - 1 < qw + off - W + 1);
  };
  auto s_phase = [&](int buf) {
    st0 = f32x16{}; st1 = f32x16{}; dp0 = dseed; dp1 = dseed;
    wave_prio<1>();
#pragma unroll
    for (int s = 0; s < (NSD > NSDV ? NSD : NSDV); ++s) {
      if (s < NSD) {
        st0 = M::mma(ld_nat(buf, 0, 0, s), qop[s], st0);
        st1 = M::mma(ld_nat(buf, 0, 1, s), qop[s], st1);
      }
      if (s < NSDV) {
        dp0 = M::mma(ld_nat(buf, 1, 0, s), gop[s], dp0);
        dp1 = M::mma(ld_nat(buf, 1, 1, s), gop[s], dp1);
      }
    }
    sched_interleave<2 * NSD + 2 * NSDV, 4>();
    wave_prio<0>();
  };
  // dS^T from the tile's S^T, dP^T, then dQ^T += K^T dS^T (K^T through
  // transposed reads of the key tile).
  auto dq_phase = [&](int j, int buf) {
    const int k0 = j * BK;
    float ds[32];
    // Boolean mask: key k0 + perm_index(h, r) is bit perm_index(0, r) % 32 of
    // word r / 16 once this half's 4 h are shifted out; a hidden pair's score
    // becomes -inf, so its P and dS are 0.
    uint32_t m0 = 0, m1 = 0;
    if constexpr (MASK) {
      m0 = sM[(buf * NW + w) * 64 + 2 * n] >> (4 * h);
      m1 = sM[(buf * NW + w) * 64 + 2 * n + 1] >> (4 * h);
    }
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      float sv = r < 16 ? st0[r] : st1[r - 16];
      const float dpv = r < 16 ? dp0[r] : dp1[r - 16];
      if constexpr (MASK) {
        const int keep = (int)((r < 16 ? m0 : m1) << (31 - perm_index(0, r) % 32)) >> 31;
        sv = __int_as_float((__float_as_int(sv) & keep) | (int)(0xff800000u & ~(uint32_t)keep));
      }
      ds[r] = fast_exp2(__builtin_fmaf(sv, c, -l2)) * dpv;
    }
    // Only the diagonal tiles and the ragged key end (a uniform test) clear
    // dS of the keys this query may not see; every value above is finite.
    if ((k0 + BK > Tk) || (CAUSAL && k0 + BK - 1 > qw + off) || (W > 0 && k0 < qw + 31 + off - W + 1)) {
      // First and last visible key offsets, less this lane half's 4 h,
      // against the compile-time part of perm_index (no per-lane table).
      const int lim = min(Tk - 1, CAUSAL ? myq + off : Tk - 1) - k0 - 4 * h;
      const int lo = W > 0 ? myq + off - W + 1 - k0 - 4 * h : INT_MIN;
#pragma unroll
      for (int r = 0; r < 32; ++r)
        if (perm_index(0, r) > lim || perm_index(0, r) < lo) ds[r] = 0.f;
    }
    Op dsop[NSK];
#pragma unroll
    for (int s = 0; s < NSK; ++s) dsop[s] = M::pack(ds + s * KPER);
    wave_prio<1>();
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int s = 0; s < NSK; ++s) acc[t] = M::mma(ld_tr(buf, t, s), dsop[s], acc[t]);
    }
    sched_interleave<NDT * NSK, 4, (sizeof(T) == 2 ? 2 : 1)>();
    wave_prio<0>();
  };

  int buf = 0;                                      // buffer of tile jt
  if constexpr (STEP2) {
    // Tiles jt and jt + 1 (buffers buf, buf + 1) between two barriers; the
    // loads of jt + 2 and jt + 3 go to the buffers of jt - 2 and jt - 1,
    // which every wave finished before the last barrier.
    for (int jt = jt0; jt < ntiles; jt += 2) {
      if (jt + 2 < ntiles) issue((jt + 2) * BK, (buf + 2) & 3);
      if (jt + 3 < ntiles) issue((jt + 3) * BK, (buf + 3) & 3);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = jt + u, b = (buf + u) & 3;
        bool any = j < ntiles;
        if constexpr (MASK)                        // the mask leaves the wave some key of the tile
          any = any && __ballot((sM[(b * NW + w) * 64 + 2 * n] | sM[(b * NW + w) * 64 + 2 * n + 1]) != 0) != 0;
        if (any && visible(j)) {
          s_phase(b);
          dq_phase(j, b);
        }
      }
      // This wave's loads of tiles jt + 2 and jt + 3 have landed; the barrier
      // makes every wave's share visible and frees buffers buf, buf + 1.
      wait_vmcnt<0>();
      __syncthreads();
      buf = (buf + 2) & 3;
    }
  } else {
    for (int jt = jt0; jt < ntiles; ++jt) {
      if (jt + 1 < ntiles) issue((jt + 1) * BK, buf ^ 1);
      bool any = true;
      if constexpr (MASK)                          // the mask leaves the wave some key of the tile
        any = __ballot((sM[(buf * NW + w) * 64 + 2 * n] | sM[(buf * NW + w) * 64 + 2 * n + 1]) != 0) != 0;
      if (visible(jt) && any) {
        s_phase(buf);
        dq_phase(jt, buf);
      }
      // This wave's loads of tile jt + 1 have landed; the barrier makes every
      // wave's share visible and frees buffer buf for the loads issued next.
      wait_vmcnt<0>();
      __syncthreads();
      buf ^= 1;
    }
  }

  if (q_ok) {
    T* qrow = reinterpret_cast<T*>(a.dQ) + (qrow0 + myq) * D;
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

template <typename T, int D, bool CAUSAL, int DV = D>
hipError_t launch_bwd_t(const BwdArgs& args, unsigned stages, hipStream_t stream) {
  const long long prows = (long long)args.B * args.Hq * args.Tqp;
  const long long kblocks = (long long)((args.Tk + 127) / 128) * args.B * args.Hkv;
  constexpr int NW = dq_waves<T, D>();
  const long long qblocks = (long long)((args.Tq + 32 * NW - 1) / (32 * NW)) * args.B * args.Hq;
  // bf16: the dK/dV pass on wave pairs (fa_dkdv.hip); d = 256 on the 4-wave
  // kernel, each workgroup forming half the columns of dK and dV (grid y).
  constexpr bool kPair = sizeof(T) == 2 && D <= 128;
  constexpr bool kHalf = D == 256;
  constexpr int kNy = kHalf ? 2 : 1;
  // Order: the dQ pass first, forming every row's -D and L2 itself and
  // writing them for the dK/dV pass (no separate preprocessing pass over O
  // and dO); without the dQ pass, bwd_pre_kernel writes them.
  BwdArgs a = args;
  a.fuse_pre = (stages & kStageDq) && qblocks > 0;
  hipError_t e = hipSuccess;
  if (!a.fuse_pre && (stages & kStagePre) && prows > 0) {
    if ((e = launch(bwd_pre_kernel<T, DV>, (prows + 15) / 16, stream, a)) != hipSuccess) return e;
  }
  if (a.fuse_pre) {
    if (a.mask != nullptr)
      e = a.window > 0 ? launch<64 * NW>(dq_kernel<T, D, CAUSAL, true, DV, true>, qblocks, stream, a)
                       : launch<64 * NW>(dq_kernel<T, D, CAUSAL, false, DV, true>, qblocks, stream, a);
    else
      e = a.window > 0 ? launch<64 * NW>(dq_kernel<T, D, CAUSAL, true, DV>, qblocks, stream, a)
                       : launch<64 * NW>(dq_kernel<T, D, CAUSAL, false, DV>, qblocks, stream, a);
    if (e != hipSuccess) return e;
  }
  if (!(stages & kStageDkDv) || kblocks <= 0) return hipSuccess;
  // A boolean mask: its key-major copy, then the masked pass (with or without
  // a window).
  if (a.mask != nullptr) {
    const long long entries = a.mask_bstride != 0 ? a.B : 1;
    const long long words = entries * a.Tk * a.mask_t_row_words;
    if ((e = launch(mask_transpose_kernel, (words + 255) / 256, stream, a, entries)) != hipSuccess) return e;
    if constexpr (kPair) {
      return launch_dkdv_pair(a, D, DV, CAUSAL, stream);
    } else {
      return a.window > 0 ? launch2(dkdv_kernel<T, D, CAUSAL, true, DV, true, kHalf>, kblocks, kNy, stream, a)
                          : launch2(dkdv_kernel<T, D, CAUSAL, false, DV, true, kHalf>, kblocks, kNy, stream, a);
    }
  }
  if constexpr (kPair) {
    return launch_dkdv_pair(a, D, DV, CAUSAL, stream);
  } else {
    return a.window > 0 ? launch2(dkdv_kernel<T, D, CAUSAL, true, DV, false, kHalf>, kblocks, kNy, stream, a)
                        : launch2(dkdv_kernel<T, D, CAUSAL, false, DV, false, kHalf>, kblocks, kNy, stream, a);
  }
}

hipError_t launch_bwd(const BwdArgs& a, int dtype_bf16, int d, int causal, unsigned stages,
                      hipStream_t stream, int dv) {
  if (dv < 0) dv = d;
  if (dv != d) {                                     // d = 128 with dv = 64, and the reverse
#define FA_BWD_DV_CASE(T)                                                                        \
  if (d == 128 && dv == 64)                                                                      \
    return causal ? launch_bwd_t<T, 128, true, 64>(a, stages, stream)                            \
                  : launch_bwd_t<T, 128, false, 64>(a, stages, stream);                          \
  if (d == 64 && dv == 128)                                                                      \
    return causal ? launch_bwd_t<T, 64, true, 128>(a, stages, stream)                            \
                  : launch_bwd_t<T, 64, false, 128>(a, stages, stream);
    if (dtype_bf16) {
      FA_BWD_DV_CASE(bf16)
    } else {
      FA_BWD_DV_CASE(float)
    }
#undef FA_BWD_DV_CASE
    return hipErrorInvalidValue;
  }
#define FA_BWD_CASE(T, DD)                                                                         \
  if (d == DD)                                                                                     \
    return causal ? launch_bwd_t<T, DD, true>(a, stages, stream) : launch_bwd_t<T, DD, false>(a, stages, stream);
  if (dtype_bf16) {
    FA_BWD_CASE(bf16, 32)
    FA_BWD_CASE(bf16, 64)
    FA_BWD_CASE(bf16, 128)
    FA_BWD_CASE(bf16, 256)
  } else {
    FA_BWD_CASE(float, 32)
    FA_BWD_CASE(float, 64)
    FA_BWD_CASE(float, 128)
  }
#undef FA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
