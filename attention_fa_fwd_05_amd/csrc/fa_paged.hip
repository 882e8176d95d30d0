// Backward pass through a block table ("The Autograd Memory Trap", sections
// "The Scene" and "The OOM: When Inference Lies": each block of new positions
// gathers its keys and values from a prefix cache of pages, and training
// differentiates through that gather).
//
// The gradient of a gathered page is the sum, over every (sequence, slot) of
// the page tables that points at it, of the gradient of the rows the sequence
// took from it (a page shared by several sequences collects all of them; a
// page no sequence uses gets zero).  Two kernels around the ordinary
// backward:
//  * page_gather_kernel copies each sequence's pages into a contiguous
//    [B][Hkv][pages_per_seq * page_size][d] copy of K and V (the backward's
//    fixed layout, with seqlens_k[b] keys per sequence; the rows past a
//    sequence's key count are zeros, and their table slots are not read);
//  * after the backward has written the per-sequence dK, dV into the same
//    layout, page_reduce_kernel forms each page's gradient: one workgroup per
//    (page, K/V head, 128-row chunk) scans the page table in order and adds,
//    in fp32, the rows of every sequence slot that maps to the page (rows
//    past the sequence's key count are not gradients and are skipped), then
//    writes the page.  The summation order is the table order, so the result
//    does not depend on scheduling.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

// One thread per 16-byte chunk of the gathered copies.
template <typename T, int D>
__global__ __launch_bounds__(256) void page_gather_kernel(PagedBwdArgs p) {
  constexpr int CH = 16 / (int)sizeof(T);            // elements per chunk
  constexpr int NCH = D / CH;                        // chunks per row
  const long long rows = (long long)p.B * p.Hkv * p.tk_max;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * NCH) return;
  const long long row = i / NCH;
  const int c = (int)(i % NCH);
  const int j = (int)(row % p.tk_max);
  const long long bh = row / p.tk_max;
  const int hk = (int)(bh % p.Hkv), b = (int)(bh / p.Hkv);
  const size_t dst = (size_t)row * D + c * CH;
  uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;        // rows past the key count: zeros
  if (j < min(max(p.seqlens[b], 0), p.tk_max)) {
    const int pg = min(max(p.table[(size_t)b * p.pps + j / p.page_size], 0), p.num_pages - 1);
    const size_t src = (((size_t)pg * p.Hkv + hk) * p.page_size + j % p.page_size) * D + c * CH;
    kv = ld16(reinterpret_cast<const T*>(p.K) + src);
    vv = ld16(reinterpret_cast<const T*>(p.V) + src);
  }
  st16(reinterpret_cast<T*>(p.Kg) + dst, kv);
  st16(reinterpret_cast<T*>(p.Vg) + dst, vv);
}

// One workgroup per (page, K/V head, 128-row chunk of the page) and tensor
// (dK for blockIdx.y == 0, dV for 1).  Thread t owns chunk t % NCH of rows
// t / NCH + RPP * k (k < NPASS) of the 128-row chunk.
template <typename T, int D>
__global__ __launch_bounds__(256) void page_reduce_kernel(PagedBwdArgs p) {
  constexpr int CH = 16 / (int)sizeof(T);
  constexpr int NCH = D / CH;
  constexpr int RPP = 256 / NCH;                     // rows per pass
  constexpr int NPASS = 128 / RPP;
  static_assert(RPP * NCH == 256 && NPASS * RPP == 128, "thread layout");
  __shared__ uint64_t smatch[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int chunks = p.page_size / 128;
  const long long blk = blockIdx.x;
  const int chunk = (int)(blk % chunks);
  const long long ph = blk / chunks;
  const int hk = (int)(ph % p.Hkv), pg = (int)(ph / p.Hkv);
  const T* src = reinterpret_cast<const T*>(blockIdx.y == 0 ? p.dKg : p.dVg);
  T* dst = reinterpret_cast<T*>(blockIdx.y == 0 ? p.dK : p.dV);
  const int r0 = tid / NCH, c = tid % NCH;
  float acc[NPASS][CH];
#pragma unroll
  for (int k = 0; k < NPASS; ++k)
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[k][e] = 0.f;
  const long long entries = (long long)p.B * p.pps;
  for (long long base = 0; base < entries; base += 256) {
    const long long e = base + tid;
    const bool m = e < entries && min(max(p.table[e], 0), p.num_pages - 1) == pg;
    const uint64_t ball = __ballot(m);
    __syncthreads();                                 // the previous chunk's masks are consumed
    if (lane == 0) smatch[wv] = ball;
    __syncthreads();
    // The matches of this chunk of the table, in table order.
    for (int w = 0; w < 4; ++w) {
      uint64_t bits = smatch[w];
      while (bits) {
        const int bit = __builtin_ctzll(bits);
        bits &= bits - 1;
        const long long ent = base + 64 * w + bit;
        const int b = (int)(ent / p.pps), slot = (int)(ent % p.pps);
        const int len = min(max(p.seqlens[b], 0), p.tk_max);
        const T* rows = src + ((size_t)b * p.Hkv + hk) * p.tk_max * D;
#pragma unroll
        for (int k = 0; k < NPASS; ++k) {
          const int j = slot * p.page_size + chunk * 128 + r0 + RPP * k;   // key of the sequence
          if (j < len) {
            const uint4 v = ld16(rows + (size_t)j * D + c * CH);
            const T* x = reinterpret_cast<const T*>(&v);
#pragma unroll
            for (int q = 0; q < CH; ++q) acc[k][q] += (float)x[q];
          }
        }
      }
    }
  }
  T* out = dst + (((size_t)pg * p.Hkv + hk) * p.page_size + chunk * 128) * D;
#pragma unroll
  for (int k = 0; k < NPASS; ++k) {
    uint4 v;
    T* x = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int q = 0; q < CH; ++q) x[q] = (T)acc[k][q];
    st16(out + (size_t)(r0 + RPP * k) * D + c * CH, v);
  }
}

template <typename T, int D>
hipError_t launch_paged_t(const PagedBwdArgs& p, int phase, hipStream_t stream) {
  if (phase == 0) {
    const long long n = (long long)p.B * p.Hkv * p.tk_max * (D * (int)sizeof(T) / 16);
    if (n == 0) return hipSuccess;
    return launch(page_gather_kernel<T, D>, (n + 255) / 256, stream, p);
  }
  const long long blocks = (long long)p.num_pages * p.Hkv * (p.page_size / 128);
  if (blocks == 0) return hipSuccess;
  return launch2(page_reduce_kernel<T, D>, blocks, 2, stream, p);
}

hipError_t launch_paged(const PagedBwdArgs& p, int dtype_bf16, int d, int phase, hipStream_t stream) {
  if (dtype_bf16) {
    if (d == 32) return launch_paged_t<bf16, 32>(p, phase, stream);
    if (d == 64) return launch_paged_t<bf16, 64>(p, phase, stream);
    if (d == 128) return launch_paged_t<bf16, 128>(p, phase, stream);
    if (d == 256) return launch_paged_t<bf16, 256>(p, phase, stream);
  } else {
    if (d == 32) return launch_paged_t<float, 32>(p, phase, stream);
    if (d == 64) return launch_paged_t<float, 64>(p, phase, stream);
    if (d == 128) return launch_paged_t<float, 128>(p, phase, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
