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

template <> struct MM<float> {
  static constexpr int KPER = 1;
  typedef float Op;
  __device__ static inline f32x16 mma(Op a, Op b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline Op ld(const float* p) { return *p; }
  __device__ static inline Op pack(const float* v) { return v[0]; }
};

// Transposed bf16 operand for step s from a row-major LDS tile: element
// 4 u + e4 comes from row row_of(u) + e4 and column col0 + (lane % 32).
// rows_u0 / rows_u1: first row of the four rows read by halves u = 0 / 1.
__device__ inline bf16x8 ld_tr_bf16(const bf16* tile, int stride, int rows_u0, int rows_u1, int col0) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15;
  const int c = col0 + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
  const bf16* p0 = tile + (rows_u0 + (i >> 2)) * stride + c;
  const bf16* p1 = tile + (rows_u1 + (i >> 2)) * stride + c;
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Transposed operand whose contraction index follows accumulator order
// (perm_index): step s of lane half h covers registers r = s * KPER + e.
template <typename T> struct TrPerm;
template <> struct TrPerm<bf16> {
  __device__ static inline bf16x8 ld(const bf16* tile, int stride, int h, int s, int col0) {
    // registers s*8 + 4u + e4 hold index 16 s + 8 u + 4 h + e4
    return ld_tr_bf16(tile, stride, 16 * s + 4 * h, 16 * s + 8 + 4 * h, col0);
  }
};
template <> struct TrPerm<float> {
  __device__ static inline float ld(const float* tile, int stride, int h, int s, int col0) {
    return tile[perm_index(h, s) * stride + col0 + (threadIdx.x & 31)];
  }
};

// Transposed operand with natural contraction order over a length-KC range.
template <typename T, int KC> struct TrNat;
template <int KC> struct TrNat<bf16, KC> {
  __device__ static inline bf16x8 ld(const bf16* tile, int stride, int h, int s, int col0) {
    const int r0 = h * (KC / 2) + 8 * s;
    return ld_tr_bf16(tile, stride, r0, r0 + 4, col0);
  }
};
template <int KC> struct TrNat<float, KC> {
  __device__ static inline float ld(const float* tile, int stride, int h, int s, int col0) {
    return tile[(h * (KC / 2) + s) * stride + col0 + (threadIdx.x & 31)];
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float wave_xor32_max(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }
__device__ inline float wave_xor32_sum(float v) { return v + __shfl_xor(v, 32, 64); }

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

// Copy a [rows x D] tile of T from global (row stride D) into LDS (row stride
// LD), rows >= nvalid filled with zeros.  All 256 threads take part.
template <typename T, int D, int LD, int ROWS>
__device__ inline void stage_tile(T* lds, const T* g, int nvalid) {
  constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  constexpr int TOTAL = ROWS * CPR;
  static_assert(TOTAL % 256 == 0, "tile must split evenly over 256 threads");
#pragma unroll
  for (int it = 0; it < TOTAL / 256; ++it) {
    const int idx = it * 256 + threadIdx.x;
    const int row = idx / CPR, ch = idx % CPR;
    uint4 v = {0u, 0u, 0u, 0u};
    if (row < nvalid) v = ld16(g + (size_t)row * D + ch * (16 / sizeof(T)));
    st16(lds + row * LD + ch * (16 / sizeof(T)), v);
  }
}

}  // namespace fa
