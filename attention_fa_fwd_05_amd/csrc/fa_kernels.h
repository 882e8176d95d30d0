// Kernel argument blocks and launchers (host side of the kernels; no validation
// here -- fa_api.hip checks every argument before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  static constexpr bool kPaged = true;   // may describe paged keys and values
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* L;
  int B, Hq, Hkv, Tq, Tk;
  int window;         // > 0: query i sees keys j > i + Tk - Tq - window; else no window
  float scale_log2;   // scale * log2(e): scores are kept in the exp2 domain
  int pack;           // 1: a workgroup holds all Tq rows of every query head of a K/V group;
                      // 2: the same in the 4-wave decode shape (bf16, G * 32-row blocks <= 4)
  // Split over keys (gridDim.y > 1 or Opart set): workgroup slice s = blockIdx.y
  // of the key tiles writes its normalised partial output and row logsumexp,
  // fp32, to Opart[s][row][d] and Lpart[s][row]; fwd_merge combines them.
  float* Opart;
  float* Lpart;
  // Variable-length batch (cu_q != nullptr): sequence b has the rows
  // cu_q[b] .. cu_q[b+1] - 1 of every query head and cu_k[b] .. cu_k[b+1] - 1
  // of every K/V head, tensors packed head-major ([H][total][d], L [Hq][total_q]);
  // Tq and Tk then hold the longest sequence (the grid's extent).
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  // Paged keys and values (pages != nullptr): K and V are pools of num_pages
  // pages, [num_pages][Hkv][page_size][d] (V: [dv]); sequence b's key j is row
  // j % page_size of page pages[b * pages_per_seq + j / page_size], and the
  // sequence has seqlens_k[b] keys (Tk then holds pages_per_seq * page_size).
  // page_size is a multiple of every key tile, so a tile lies in one page.
  const int* pages = nullptr;
  const int* seqlens_k = nullptr;
  int pages_per_seq = 0, page_size = 0, num_pages = 0;
  // Boolean mask (mask != nullptr): bit j % 32 of word mask[b * mask_bstride +
  // i * mask_row_words + j / 32] set means key j is visible to query i (then
  // also subject to the causal rule and j < Tk), for every head of batch
  // entry b; mask_row_words = 4 * ceil(Tk / 128), so a 128-key tile's bits
  // of a row are one aligned 16-byte word group; mask_bstride 0 shares one
  // mask across the batch.
  const uint32_t* mask = nullptr;
  long long mask_bstride = 0;
  int mask_row_words = 0;
};

// One sequence of a batch: its lengths, and where its rows sit.  Row 0 of
// query head hq is q_base + hq * q_hstride (fixed layout: b * Hq * Tq and Tq;
// packed variable-length layout: the sequence's offset and total_q), and
// likewise for keys; all computed once, so each use is one multiply-add.
struct SeqView {
  int Tq, Tk;
  size_t q_base, q_hstride, k_base, k_hstride;
  __device__ size_t q_row(int hq) const { return q_base + (size_t)hq * q_hstride; }
  __device__ size_t k_row(int hk) const { return k_base + (size_t)hk * k_hstride; }
};
template <typename A>
__device__ inline SeqView seq_view(const A& a, int b) {
  SeqView v;
  if (a.cu_q != nullptr) {
    // Clamped so that even inconsistent offsets keep every access inside the
    // packed tensors: 0 <= start, start + length <= total, length <= the
    // longest sequence the grid was sized for.
    const int q0 = __builtin_amdgcn_readfirstlane(a.cu_q[b]), q1 = __builtin_amdgcn_readfirstlane(a.cu_q[b + 1]);
    const int k0 = __builtin_amdgcn_readfirstlane(a.cu_k[b]), k1 = __builtin_amdgcn_readfirstlane(a.cu_k[b + 1]);
    const int qs = min(max(q0, 0), a.total_q), ks = min(max(k0, 0), a.total_k);
    v.Tq = min(min(max(q1 - q0, 0), a.Tq), a.total_q - qs);
    v.Tk = min(min(max(k1 - k0, 0), a.Tk), a.total_k - ks);
    v.q_base = qs;
    v.q_hstride = a.total_q;
    v.k_base = ks;
    v.k_hstride = a.total_k;
  } else {
    v.Tq = a.Tq;
    v.Tk = a.Tk;
    if constexpr (A::kPaged) {
      if (a.seqlens_k != nullptr) v.Tk = min(max(__builtin_amdgcn_readfirstlane(a.seqlens_k[b]), 0), a.Tk);
    }
    v.q_base = (size_t)b * a.Hq * a.Tq;
    v.q_hstride = a.Tq;
    v.k_base = (size_t)b * a.Hkv * a.Tk;
    v.k_hstride = a.Tk;
  }
  return v;
}

struct BwdArgs {
  static constexpr bool kPaged = true;    // may give each sequence its own key count
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const float* L;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  float* Dvec;        // [B*Hq][Tqp] -rowsum(dO * O); 0 in padding rows
  float* Lg;          // [B*Hq][Tqp] L * log2(e); +inf for rows without keys and padding
  // The dQ pass forms its rows' -D and L2 itself (from O, dO and L) and
  // writes them to Dvec and Lg for the dK/dV pass that follows it, instead of
  // reading what bwd_pre_kernel wrote.
  bool fuse_pre = false;
  int B, Hq, Hkv, Tq, Tk;
  int Tqp;            // Tq rounded up to a multiple of 64
  int window;         // as FwdArgs::window
  const int* cu_q;    // as FwdArgs (variable-length batch)
  const int* cu_k;
  int total_q, total_k;
  float scale;
  float scale_log2;
  // Boolean mask (mask != nullptr): the query-major bits of FwdArgs::mask
  // (read by the dQ pass) and a key-major copy in the workspace (written by
  // mask_transpose_kernel, read by the dK/dV pass): bit q % 32 of word
  // mask_t[b * mask_t_bstride + j * mask_t_row_words + q / 32] is the bit of
  // (query q, key j); mask_t_row_words = 4 * ceil(Tq / 128).
  const uint32_t* mask = nullptr;
  long long mask_bstride = 0;
  int mask_row_words = 0;
  uint32_t* mask_t = nullptr;
  long long mask_t_bstride = 0;
  int mask_t_row_words = 0;
  // Per-sequence key counts (seqlens_k != nullptr): sequence b has
  // seqlens_k[b] keys of the fixed layout's Tk rows (the backward through a
  // block table runs on gathered copies of the pages).
  const int* seqlens_k = nullptr;
};

// Backward through a block table: gather of the pages into the fixed layout,
// and the reduction of the per-sequence gradients into gradient pages.
struct PagedBwdArgs {
  const void* K;              // pools [num_pages][Hkv][page_size][d]
  const void* V;
  void* Kg;                   // gathered copies [B][Hkv][tk_max][d]
  void* Vg;
  const void* dKg;            // per-sequence gradients, gathered layout
  const void* dVg;
  void* dK;                   // gradient pools, the layout of K and V
  void* dV;
  const int* table;           // [B][pps] page indices (clamped into the pool)
  const int* seqlens;         // [B] key counts (clamped into [0, tk_max])
  int B, Hkv, pps, page_size, num_pages, tk_max;
};
// phase 0: gather K, V; phase 1: reduce dK, dV into the gradient pools.
hipError_t launch_paged(const PagedBwdArgs& p, int dtype_bf16, int d, int phase, hipStream_t stream);

// Launch a kernel of THREADS threads per workgroup on a 1-D grid and return
// that launch's own status (the thread's sticky last-error state is neither
// read nor cleared).
template <int THREADS = 256, typename... Params, typename... Args>
inline hipError_t launch(void (*kernel)(Params...), long long blocks, hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks), dim3(THREADS), argv,
                         0, stream);
}

// Launch on a 2-D grid (blocks x ny).
template <int THREADS = 256, typename... Params, typename... Args>
inline hipError_t launch2(void (*kernel)(Params...), long long blocks, int ny, hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks, (unsigned)ny),
                         dim3(THREADS), argv, 0, stream);
}

// Forward over nsplit key slices (nsplit >= 1; with Opart/Lpart set, the
// slices' partials are merged into O and L by a second kernel).
// dv: head dim of V and O (d: of Q and K); dv != d only as
// (d, dv) = (128, 64) or (64, 128).
hipError_t launch_fwd(const FwdArgs& a, int dtype_bf16, int d, int causal, hipStream_t stream, int nsplit = 1,
                      int dv = -1);
// Pack a boolean byte mask [rows][Tk] into FwdArgs::mask's bit layout.
hipError_t launch_mask_pack(const uint8_t* in, uint32_t* out, long long rows, int Tk, int row_words,
                            hipStream_t stream);
// Waves per forward workgroup for a dtype and head dim (pack needs G <= waves).
int fwd_waves(int dtype_bf16, int d);
int fwd_block_keys(int dtype_bf16, int d);
// The decode-shape forward (bf16, FwdArgs::pack == 2): waves and keys per tile.
int fwd_decode_waves();
int fwd_decode_block_keys();
// Backward stages (bit mask): preprocess, dK/dV kernel, dQ kernel.
constexpr unsigned kStagePre = 1u, kStageDkDv = 2u, kStageDq = 4u;
hipError_t launch_bwd(const BwdArgs& a, int dtype_bf16, int d, int causal, unsigned stages,
                      hipStream_t stream, int dv = -1);
// The bf16 dK/dV pass on wave pairs (fa_dkdv.hip); a boolean mask needs its
// key-major copy in BwdArgs::mask_t first.
hipError_t launch_dkdv_pair(const BwdArgs& a, int d, int dv, int causal, hipStream_t stream);

}  // namespace fa
