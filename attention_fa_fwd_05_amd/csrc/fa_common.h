// Shared device helpers for the gfx950 attention kernels: MFMA wrappers, operand
// fetch from LDS in natural (row-major) layout, and the register <-> index maps.
//
// Matrix-core conventions (CDNA4, wave64), checked on the hardware:
//  * v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32 compute D = A B + C with
//    A 32 x K, B K x 32.  Lane l supplies A[l % 32][k] and B[k][l % 32] for the
//    K/2 contraction indices k of lane half h = l / 32.  Accumulator register i
//    of lane l holds D[8 (i / 4) + 4 h + (i % 4)][l % 32].
//  * ds_read_b64_tr_b16: within each 16-lane group, output lane j, element e
//    receives element (j % 4) of the 8 bytes addressed by lane 4 e + j / 4.
//    Letting lane i of the group address row r0 + i / 4, columns c0 + 4 (i % 4)
//    therefore hands lane j the column c0 + j of rows r0 .. r0 + 3: a
//    transposed operand read from a row-major tile.
//
// Contraction order.  A contraction of length KC is split between the two lane
// halves; a "natural" operand lets lane half h walk indices
// h * KC / 2 + s * KPER + e (step s, element e).  An accumulator reused as an
// operand fixes its own order instead: register r of lane half h (tile r / 16,
// register r % 16) holds index perm_index(h, r) below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Index held by accumulator-order register r of lane half h (see header note).
__device__ __host__ inline constexpr int perm_index(int h, int r) {
  return 32 * (r >> 4) + 8 * ((r & 15) >> 2) + 4 * h + (r & 3);
}

template <typename T> struct MM;

template <> struct MM<bf16> {
  static constexpr int KPER = 8;   // contraction elements per lane per step
  typedef bf16x8 Op;
  __device__ static inline f32x16 mma(const Op& a, const Op& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Natural operand: KPER contiguous elements at p.
  __device__ static inline Op ld(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  // Pack fp32 values (register order) into an operand, rounding to nearest even.
  __device__ static inline Op pack(const float* v) {
    Op o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
    return o;
  }
};

// fp32: an operand is 4 consecutive contraction elements per lane, consumed by
// four chained 32x32x2 products (element e feeds the e-th), so that operands
// are 16-byte LDS reads as for bf16.
template <> struct MM<float> {
  static constexpr int KPER = 4;
  typedef f32x4 Op;
  __device__ static inline f32x16 mma(const Op& a, const Op& b, const f32x16& c) {
    f32x16 d = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], d, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], d, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], d, 0, 0, 0);
  }
  __device__ static inline Op ld(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  __device__ static inline Op pack(const float* v) { return f32x4{v[0], v[1], v[2], v[3]}; }
};

// ---------------------------------------------------------------------------
// Unpadded LDS tiles with XOR-swizzled 16-byte chunks.
//
// A [rows x D] tile of T is stored row-major without padding; chunk c of row r
// (16 bytes = 4 of the 64 LDS banks) sits at slot c ^ fsw(r).  For 256-byte
// rows fsw(r) = 4 (r & 3) + ((r >> 2) & 3):
//  * it takes 16 distinct values over any 16 consecutive rows, so 16 lanes
//    reading one chunk of 16 rows (a natural operand) hit 16 different slots;
//  * the 4 rows of an aligned 4-row group differ in bits 2-3, so the 4-chunk
//    run {c .. c+3} (c a multiple of 4) that 32 lanes of a transposed read take
//    from each of the 4 rows lands on 16 distinct slots.
// For 128-byte rows (two rows per bank sweep) the same holds with
// fsw(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3), and for 64-byte rows (four rows
// per sweep, 4 chunks each) with fsw(r) = (r >> 2) & 3: the 16 rows of a
// natural read fall in 4 row classes (r & 3, which picks the sweep quarter)
// times 4 swizzles, and a transposed read takes all 4 chunks of 4 rows of
// distinct r & 3.  fsw depends on r & 15 only, so per-lane offsets can be
// tabulated over a 16-row period.  The layout can be
// filled by direct global->LDS loads, which write 64 consecutive 16-byte slots
// per wave instruction.
template <typename T, int D>
struct SwzTile {
  static constexpr int EPC = 16 / (int)sizeof(T);   // elements per chunk
  static constexpr int NCH = D / EPC;               // chunks per row
  static_assert(NCH == 4 || NCH == 8 || NCH == 16 || NCH == 32, "row must be 4, 8, 16 or 32 chunks");
  __device__ static inline int fsw(int r) {
    return NCH >= 16 ? (4 * (r & 3) + ((r >> 2) & 3))
                     : NCH == 8 ? (4 * ((r >> 1) & 1) + ((r >> 2) & 3)) : ((r >> 2) & 3);
  }
  // element index of (row, col)
  __device__ static inline int elem(int r, int col) {
    return r * D + (((col / EPC) ^ fsw(r)) * EPC) + (col % EPC);
  }
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

// LDS byte address of a pointer into a __shared__ array.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct global->LDS loads, issued as inline assembly so the compiler neither
// tracks them nor inserts waits for them: the caller orders them with
// wait_vmcnt and a workgroup barrier.  M0 holds the wave-uniform LDS base;
// lane l's data lands at base + size * l.
__device__ inline void dma16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// The same with a wave-uniform 64-bit base (scalar registers) and a 32-bit
// per-lane byte offset: no per-lane address arithmetic at the call site.
__device__ inline void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
__device__ inline void dma4(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

// Issue direct loads of global rows [g0, g0 + ROWS) (each clamped to
// nrows - 1, which must be >= 0) into a swizzled tile.  Waves W0 .. W0 + NWS
// - 1 of a workgroup of NTHR threads take part (all of them by default; a
// tile smaller than one 16-byte slot per thread goes to a subset), each
// issuing ROWS * NCH / (64 NWS) instructions; other waves issue none.
template <typename T, int D, int ROWS, int NTHR, int W0 = 0, int NWS = NTHR / 64>
struct DmaRows {
  using TL = SwzTile<T, D>;
  static constexpr int SLOTS = ROWS * TL::NCH, NWV = NWS, PER = SLOTS / (64 * NWS);
  static_assert(PER >= 1 && PER * 64 * NWS == SLOTS, "tile must split evenly over the waves");
  static_assert(W0 >= 0 && W0 + NWS <= NTHR / 64, "waves within the workgroup");
  // This wave takes part (uniform).
  __device__ static inline bool mine() {
    if constexpr (W0 == 0 && NWS == NTHR / 64) return true;
    const int wave = threadIdx.x >> 6;
    return wave >= W0 && wave < W0 + NWS;
  }
  // Instruction i (0 <= i < PER) of this wave.
  __device__ static inline void one(T* tile, const T* g, int g0, int nrows, int i) {
    if (!mine()) return;
    const int wave = (threadIdx.x >> 6) - W0, lane = threadIdx.x & 63;
    const int blk = i * NWV + wave;                 // 64-slot block of this wave instruction
    const int pos = blk * 64 + lane;
    const int r = pos / TL::NCH, x = pos % TL::NCH;
    const int gr = min(g0 + r, nrows - 1);
    dma16(g + (size_t)gr * D + (x ^ TL::fsw(r)) * TL::EPC, lds_addr(tile) + blk * 1024);
  }
  // Byte offset from row 0 of the tile's source rows for instruction i of this
  // lane (rows not clamped), and the LDS byte offset of its 64-slot block.
  __device__ static inline uint32_t src_off(int i) {
    const int wave = (threadIdx.x >> 6) - W0, lane = threadIdx.x & 63;
    const int pos = (i * NWV + wave) * 64 + lane;
    const int r = pos / TL::NCH, x = pos % TL::NCH;
    return (uint32_t)((r * D + (x ^ TL::fsw(r)) * TL::EPC) * (int)sizeof(T));
  }
  __device__ static inline uint32_t lds_off(int i) {
    return (uint32_t)((i * NWV + (threadIdx.x >> 6) - W0) * 1024);
  }
};
template <typename T, int D, int ROWS, int NTHR>
__device__ inline void dma_rows(T* tile, const T* g, int g0, int nrows) {
#pragma unroll
  for (int i = 0; i < DmaRows<T, D, ROWS, NTHR>::PER; ++i) DmaRows<T, D, ROWS, NTHR>::one(tile, g, g0, nrows, i);
}

// 4-byte direct loads of 64 consecutive floats by one wave.
__device__ inline void dma_floats64(float* dst, const float* src) {
  dma4(src + (threadIdx.x & 63), lds_addr(dst));
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt, lgkmcnt left
// at their maxima, i.e. not waited on).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Operand fetchers for swizzled tiles.  The swizzle is periodic in the row
// (16 rows for >= 16-chunk rows, 8 rows otherwise), so every per-lane part of
// an address can be tabulated once per kernel and every per-step part is a
// compile-time byte offset.  Tables hold byte offsets from the tile base.

// A value the optimiser must treat as freshly computed (keeps derived
// addresses from being hoisted out of a loop into long-lived registers).
__device__ inline int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A compile-time constant as a type (for generic lambdas).
template <auto V> struct IC { static constexpr auto value = V; };

// The same for a wave-uniform value, kept in a scalar register.
__device__ inline int opaque_s(int x) {
  x = __builtin_amdgcn_readfirstlane(x);
  asm volatile("" : "+s"(x));
  return x;
}

__device__ inline bf16x8 lds16(const void* base, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(base) + byte_off);
}
__device__ inline bf16x4 lds_tr8(const void* base, int byte_off) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)(reinterpret_cast<const char*>(base) + byte_off));
}
__device__ inline bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Natural operand of lane row n (+ 32 t): element e of step s is
// tile[32 t + n][h * D / 2 + s * KPER + e].
template <typename T, int D> struct NatFetch;
template <int D> struct NatFetch<bf16, D> {
  using TL = SwzTile<bf16, D>;
  static constexpr int NS = D / 16;                 // steps (one chunk each)
  int off[NS];
  __device__ void init(int n, int h) {
#pragma unroll
    for (int s = 0; s < NS; ++s) off[s] = 2 * TL::elem(n, h * (D / 2) + 8 * s);
  }
  __device__ bf16x8 ld(const bf16* tile, int t, int s) const { return lds16(tile + t * 32 * D, off[s]); }
};
template <int D> struct NatFetch<float, D> {
  using TL = SwzTile<float, D>;
  int n_, h_;
  __device__ void init(int n, int h) { n_ = n; h_ = h; }
  __device__ f32x4 ld(const float* tile, int t, int s) const {
    return *reinterpret_cast<const f32x4*>(tile + 32 * t * D + TL::elem(opaque(n_), h_ * (D / 2) + 4 * s));
  }
};

// Transposed operand in accumulator order over rows: element e of step s is
// tile[perm_index(h, s * KPER + e)][32 t + lane % 32].
template <typename T, int D> struct TrPermFetch;
template <int D> struct TrPermFetch<bf16, D> {
  using TL = SwzTile<bf16, D>;
  static constexpr int NT = D / 32;
  int off[2 * NT];                                  // (t, u): rows 8 u + 4 h + i / 4 of a 16-row period
  __device__ void init(int lane) {
    const int h = lane >> 5, i = lane & 15, g16 = (lane >> 4) & 1;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        off[2 * t + u] = 2 * TL::elem(8 * u + 4 * h + (i >> 2), 32 * t + 16 * g16 + 4 * (i & 3));
  }
  __device__ bf16x8 ld(const bf16* tile, int t, int s) const {
    const bf16* base = tile + 16 * s * D;
    return cat(lds_tr8(base, off[2 * t]), lds_tr8(base, off[2 * t + 1]));
  }
};
template <int D> struct TrPermFetch<float, D> {
  int lane_;
  __device__ void init(int lane) { lane_ = lane; }
  __device__ f32x4 ld(const float* tile, int t, int s) const {
    const int l = opaque(lane_), h = l >> 5, col = 32 * t + (l & 31);
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = tile[SwzTile<float, D>::elem(perm_index(h, 4 * s + e), col)];
    return r;
  }
};

// Loads from a 32-bit LDS byte address.
__device__ inline bf16x8 lds16_at(uint32_t addr) {
  typedef __attribute__((address_space(3))) bf16x8 lds_t;
  return *(const lds_t*)addr;
}
__device__ inline bf16x4 lds_tr8_at(uint32_t addr) {
  typedef __attribute__((address_space(3))) bf16x4 lds_t;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_t*)addr);
}

// Register-lean form of the two bf16 fetchers above, for tiles whose buffer is
// chosen at run time.  In a swizzled tile, a lane's natural-operand offset for
// step s is its step-0 offset XOR 16 s, and its transposed-read offset for
// column tile t and row group u is the (0, 0) offset XOR 64 t + (32 + 16 D) u.
// These XOR constants stay below 4096, so with 4096-byte aligned tiles the XOR
// can follow the addition of the tile address.  A wave keeps one base
// register per tile instead of a table of offsets, and spends one v_xor per
// distinct step; the step's row offset is an immediate.
template <int D> struct XorFetch {
  using TL = SwzTile<bf16, D>;
  uint32_t nat0, tr0;                               // byte offsets within a tile
  __device__ void init(int lane) {
    const int h = lane >> 5, n = lane & 31, i = lane & 15, g16 = (lane >> 4) & 1;
    nat0 = 2 * TL::elem(n, h * (D / 2));
    tr0 = 2 * TL::elem(4 * h + (i >> 2), 16 * g16 + 4 * (i & 3));
  }
  // vn = tile address + nat0: tile[32 t + n][h D / 2 + 8 s .. + 7]
  __device__ static bf16x8 nat(uint32_t vn, int t, int s) { return lds16_at((vn ^ (16 * s)) + t * 64 * D); }
  // vt = tile address + tr0: as TrPermFetch::ld
  __device__ static bf16x8 tr(uint32_t vt, int t, int s) {
    return cat(lds_tr8_at((vt ^ (64 * t)) + 32 * s * D), lds_tr8_at((vt ^ (64 * t + 32 + 16 * D)) + 32 * s * D));
  }
};

// Scheduling hint for a straight run of NMMA matrix instructions, each fed by
// RPM LDS reads: issue the reads for the first AHEAD instructions, then
// alternate one matrix instruction with the reads of a later one, so LDS
// latency overlaps matrix work instead of stalling each instruction.
// MPR matrix instructions may share one operand read (MPR consecutive
// instructions per RPM reads).
template <int NMMA, int AHEAD, int RPM = 1, int MPR = 1>
__device__ inline void sched_interleave() {
  constexpr int kMfma = 0x008, kDsRead = 0x100;
  static_assert(NMMA % MPR == 0 && AHEAD % MPR == 0, "groups of MPR matrix instructions");
  __builtin_amdgcn_sched_group_barrier(kDsRead, AHEAD / MPR * RPM, 0);
#pragma unroll
  for (int k = 0; k < (NMMA - AHEAD) / MPR; ++k) {
    __builtin_amdgcn_sched_group_barrier(kMfma, MPR, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, RPM, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, AHEAD, 0);
}

// Issue priority of this wave (s_setprio), fenced so the scheduler keeps it
// at this point of the instruction stream.  Kernels with two waves per SIMD
// raise it around their matrix products: when the other wave is in its vector
// phase, the arbiter then prefers the wave that feeds the matrix unit, and the
// products of one wave overlap the vector work of the other more closely.
template <int P>
__device__ inline void wave_prio() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(P);
  __builtin_amdgcn_sched_barrier(0);
}

// Work items in dispatch order.  Consecutive workgroup ids are spread over
// the 8 XCDs round-robin; giving each XCD one contiguous range of the logical
// order keeps the workgroups of a (batch, K/V head) group on one XCD, so the
// group's tiles stay in that XCD's L2.
__device__ inline int xcd_logical_block() {
  const int N = gridDim.x, p = blockIdx.x;
  const int x = p & 7, slot = p >> 3, per = N >> 3, rem = N & 7;
  return x * per + min(x, rem) + slot;
}

// Query-block kernels (forward, dQ): logical order = group, then query block
// (longest rows first when causal), then query head within the group, so the
// workgroups of a group (which read the same K and V) share an XCD and its L2.
// When a group has fewer workgroups than the 32 compute units of an XCD, K
// groups are interleaved by query block (K * (workgroups per group) = 32):
// each XCD then starts on the longest blocks of K groups at once and ends on
// the shortest, instead of running each group's long block last among a
// group's short ones (at 16 heads of 2048 rows this took the forward and the
// dQ pass 19% and 18% down).  K divides the groups of an XCD's share of the
// grid, else it is 1.
struct QWork {
  int b, hq, hk, qb;
};
__device__ inline QWork qblock_work(int B, int Hq, int Hkv, int nqb, bool causal) {
  const int logical = xcd_logical_block();
  const int G = Hq / Hkv;
  const int N = gridDim.x, per = N >> 3, gsz = nqb * G;
  int K = gsz < 32 ? 32 / gsz : 1;
  if (N % 8 != 0 || per % gsz != 0 || (per / gsz) % K != 0) K = 1;
  const int r = logical % G, t = logical / G;
  const int gk = t % K, u = t / K;
  const int qi = u % nqb, grp = (u / nqb) * K + gk;
  QWork w;
  w.b = grp / Hkv;
  w.hk = grp % Hkv;
  w.hq = w.hk * G + r;
  w.qb = causal ? nqb - 1 - qi : qi;
  return w;
}

// Scheduling hint for matrix work that should hide independent vector-ALU
// work: after AHEAD operand reads, each matrix instruction is followed by up
// to VPM vector-ALU instructions and the read of a later operand.
template <int NMMA, int AHEAD, int VPM>
__device__ inline void sched_interleave_valu() {
  constexpr int kValu = 0x002 | 0x400, kMfma = 0x008, kDsRead = 0x100;  // VALU incl. transcendental
  __builtin_amdgcn_sched_group_barrier(kDsRead, AHEAD, 0);
#pragma unroll
  for (int k = 0; k < NMMA - AHEAD; ++k) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kValu, VPM, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
  }
#pragma unroll
  for (int k = 0; k < AHEAD; ++k) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kValu, VPM, 0);
  }
}

// Issue NP matrix products in a fixed order with AHEAD operands in flight:
// fetch(m) reads product m's LDS operand, mma(m, x) issues product m, and
// between(m) is the other work placed right after product m (vector work of
// a later stage, single direct loads).  A scheduling fence after every step
// keeps exactly this order, so operand reads stay AHEAD products ahead and
// the vector work fills the time the products take.
template <int NP, int AHEAD, typename Op, typename F, typename G, typename H>
__device__ __forceinline__ void pipelined(F&& fetch, G&& mma, H&& between) {
  Op ring[AHEAD];
#pragma unroll
  for (int m = 0; m < AHEAD; ++m) ring[m] = fetch(m);
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    const Op x = ring[m % AHEAD];
    if (m + AHEAD < NP) ring[m % AHEAD] = fetch(m + AHEAD);
    mma(m, x);
    between(m);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// As pipelined, with vector work `pre` that the first product needs placed
// after the first AHEAD operand reads: when `pre` waits on an LDS read of its
// own, the operand reads are already in flight, so the two round trips
// overlap instead of following one another.
template <int NP, int AHEAD, typename Op, typename F, typename P, typename G, typename H>
__device__ __forceinline__ void pipelined_after(F&& fetch, P&& pre, G&& mma, H&& between) {
  Op ring[AHEAD];
#pragma unroll
  for (int m = 0; m < AHEAD; ++m) ring[m] = fetch(m);
  __builtin_amdgcn_sched_barrier(0);
  pre();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    const Op x = ring[m % AHEAD];
    if (m + AHEAD < NP) ring[m % AHEAD] = fetch(m + AHEAD);
    mma(m, x);
    between(m);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane l and lane l ^ 32 combined, on the vector ALU: v_permlane32_swap hands
// every lane the values of lanes l % 32 and l % 32 + 32 (in that order, so
// both halves get bit-identical results) without a round trip through LDS.
__device__ inline void lane_halves(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ inline float wave_xor32_max(float v) {
  float lo, hi;
  lane_halves(v, lo, hi);
  return fmaxf(lo, hi);
}

// Maximum of N values as a tree of three-input maxima (v_max3_f32 once NaNs
// need not be propagated, which the library's build assumes): each level
// takes the values in groups of three, so N values cost about N / 2
// instructions.
template <int N>
__device__ inline float max_tree(const float* v) {
  if constexpr (N == 1) {
    return v[0];
  } else if constexpr (N == 2) {
    return fmaxf(v[0], v[1]);
  } else {
    constexpr int G = N / 3, R = N % 3, M = G + (R ? 1 : 0);
    float t[M];
#pragma unroll
    for (int g = 0; g < G; ++g) t[g] = fmaxf(fmaxf(v[3 * g], v[3 * g + 1]), v[3 * g + 2]);
    if constexpr (R == 1) t[G] = v[3 * G];
    if constexpr (R == 2) t[G] = fmaxf(v[3 * G], v[3 * G + 1]);
    return max_tree<M>(t);
  }
}

// Sum of the 8 bf16 values of an operand, accumulated in fp32 by two-element
// dot products with (1, 1): the sum of exactly the rounded values the matrix
// unit multiplies.
__device__ inline void sum_bf16x8(const bf16x8& p, float* acc4) {
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  acc4[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc4[0], false);
  acc4[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc4[1], false);
  acc4[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc4[2], false);
  acc4[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc4[3], false);
}
__device__ inline float wave_xor32_sum(float v) {
  float lo, hi;
  lane_halves(v, lo, hi);
  return lo + hi;
}

// 16-byte global <-> LDS copy helpers.
__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Store 4 consecutive fp32 values as T.
__device__ inline void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
__device__ inline void store4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}

}  // namespace fa
