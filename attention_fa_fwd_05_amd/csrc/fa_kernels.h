// Kernel argument blocks and launchers (host side of the kernels; no validation
// here -- fa_api.hip checks every argument before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* L;
  int B, Hq, Hkv, Tq, Tk;
  int window;         // > 0: query i sees keys j > i + Tk - Tq - window; else no window
  float scale_log2;   // scale * log2(e): scores are kept in the exp2 domain
  int pack;           // 1: a workgroup holds all Tq rows of every query head of a K/V group
  // Split over keys (gridDim.y > 1 or Opart set): workgroup slice s = blockIdx.y
  // of the key tiles writes its normalised partial output and row logsumexp,
  // fp32, to Opart[s][row][d] and Lpart[s][row]; fwd_merge combines them.
  float* Opart;
  float* Lpart;
};

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const float* L;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  float* Dvec;        // [B*Hq][Tqp] rowsum(dO * O); 0 in padding rows
  float* Lg;          // [B*Hq][Tqp] L * log2(e); +inf for rows without keys and padding
  int B, Hq, Hkv, Tq, Tk;
  int Tqp;            // Tq rounded up to a multiple of 64
  int window;         // as FwdArgs::window
  float scale;
  float scale_log2;
};

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
hipError_t launch_fwd(const FwdArgs& a, int dtype_bf16, int d, int causal, hipStream_t stream, int nsplit = 1);
// Waves per forward workgroup for a dtype and head dim (pack needs G <= waves).
int fwd_waves(int dtype_bf16, int d);
int fwd_block_keys(int dtype_bf16, int d);
// Backward stages (bit mask): preprocess, dK/dV kernel, dQ kernel.
constexpr unsigned kStagePre = 1u, kStageDkDv = 2u, kStageDq = 4u;
hipError_t launch_bwd(const BwdArgs& a, int dtype_bf16, int d, int causal, unsigned stages,
                      hipStream_t stream);

}  // namespace fa
