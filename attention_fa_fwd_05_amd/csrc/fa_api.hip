// C ABI entry points (include/fa.h): argument validation, workspace layout and
// dispatch to the gfx950 kernels.  Every check runs before any HIP call; the
// library allocates nothing and keeps no state.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include "fa.h"
#include "fa_kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr long long kMaxElems = 1LL << 40;          // element-count ceiling per tensor
constexpr int kMaxSeq = 1 << 24;                     // Tq, Tk ceiling
constexpr int kMaxGrid = 0x7fffffff;

// Text of the HIP error behind the calling thread's most recent FA_ERR_HIP.
thread_local const char* t_hip_error = "no HIP error";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  t_hip_error = hipGetErrorString(e);
  return FA_ERR_HIP;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// The kernels mask invisible scores with -inf before multiplying by the scale
// and take the row maximum of the unscaled scores, both of which hold only for
// a positive scale (the pages' 1/sqrt(d)); zero, negative, NaN and infinite
// scales are rejected.  The test reads the IEEE bits, since the library is
// built without NaN semantics (-fno-honor-nans) and a floating-point compare
// could be folded: positive finite values are exactly the bit patterns
// 0x00000001 .. 0x7f7fffff.
bool bad_scale(float scale) {
  uint32_t bits;
  memcpy(&bits, &scale, sizeof bits);
  return bits - 1u >= 0x7f7fffffu;
}

int elem_bytes(int dtype) { return dtype == FA_DTYPE_BF16 ? 2 : 4; }

// Shared shape checks; returns FA_OK or the first failing status.
int check_common(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 0 || Tk < 0) return FA_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_GQA_RATIO;
  // 32 (the measured configuration of the tiling article), 64 and 128; bf16
  // also 256
  if (d != 32 && d != 64 && d != 128 && !(d == 256 && dtype == FA_DTYPE_BF16)) return FA_ERR_HEAD_DIM;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (Tq > kMaxSeq || Tk > kMaxSeq) return FA_ERR_TOO_LARGE;
  const long long q = (long long)B * Hq * Tq * d, kv = (long long)B * Hkv * Tk * d;
  if (q > kMaxElems || kv > kMaxElems) return FA_ERR_TOO_LARGE;
  // grid sizes: forward (Tq/128) * B * Hq, backward (Tk/128) * B * Hkv, rows/16
  if ((long long)((Tq + 127) / 128) * B * Hq > kMaxGrid) return FA_ERR_TOO_LARGE;
  if ((long long)((Tk + 127) / 128) * B * Hkv > kMaxGrid) return FA_ERR_TOO_LARGE;
  if (((long long)B * Hq * Tq + 15) / 16 > kMaxGrid) return FA_ERR_TOO_LARGE;
  if ((long long)B * Hq * Tq * d / 8 / 256 + 1 > kMaxGrid) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

// A tensor with elements needs a non-NULL, 16-byte aligned pointer.
int check_ptr(const void* p, long long elems) {
  if (elems == 0) return FA_OK;
  if (p == nullptr) return FA_ERR_NULL_PTR;
  if (misaligned(p)) return FA_ERR_ALIGNMENT;
  return FA_OK;
}

struct WsLayout {
  size_t dvec, lg, total;
};

int padded_rows(int Tq) { return (Tq + 63) / 64 * 64; }

WsLayout ws_layout(int B, int Hq, int Tq, int d, int dtype) {
  const size_t rows = (size_t)B * Hq * Tq;
  const size_t prows = (size_t)B * Hq * padded_rows(Tq);
  (void)rows;
  (void)d;
  (void)dtype;
  WsLayout w;
  w.dvec = 0;
  w.lg = align_up(prows * 4);
  w.total = w.lg + align_up(prows * 4);
  return w;
}

// All Tq rows of a K/V group's G query heads fit one forward workgroup: in the
// 4-wave decode shape (bf16; 2), else in the regular one (1); or not (0).
int fwd_pack(int Hq, int Hkv, int Tq, int d, int dtype) {
  const int G = Hq / Hkv;
  const int nd = fa::fwd_decode_waves();
  if (dtype == FA_DTYPE_BF16 && d <= 128 && G <= nd && Tq <= 32 * (nd / G)) return 2;
  const int nw = fa::fwd_waves(dtype == FA_DTYPE_BF16, d);
  return (G <= nw && Tq <= 32 * (nw / G)) ? 1 : 0;
}

// Key slices of a split forward: the requested count, or (nsplit <= 0) enough
// slices for about one workgroup per compute unit (the decode shape fits two,
// and the second slot absorbs uneven slices), each of at least eight key
// tiles, at most 64.  Measured on the 32-query, 8032-key shape: 16 blocks x
// 8 K/V heads run best at 2-4 slices, one block at 12-16.  `target` is the
// number of workgroups aimed at (a variable-length batch raises it).
int fwd_splits(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype, int nsplit, long long target = 256) {
  if (nsplit > 0) return nsplit;
  const int pack = fwd_pack(Hq, Hkv, Tq, d, dtype);
  const int nw = fa::fwd_waves(dtype == FA_DTYPE_BF16, d);
  const int bk = pack == 2 ? fa::fwd_decode_block_keys() : fa::fwd_block_keys(dtype == FA_DTYPE_BF16, d);
  const long long items = pack ? (long long)B * Hkv : (long long)((Tq + 32 * nw - 1) / (32 * nw)) * B * Hq;
  const long long tiles = (Tk + bk - 1) / bk;
  long long ns = items > 0 ? (target + items - 1) / items : 1;
  ns = ns < tiles / 8 ? ns : tiles / 8;
  ns = ns < 64 ? ns : 64;
  return ns < 1 ? 1 : (int)ns;
}

constexpr int kMaxSplits = 1024;
// Key slices of the masked forward, which always runs the regular shape
// (packed when a group's rows fit it): the requested count, or (nsplit <= 0)
// enough for about one workgroup per compute unit, each of at least eight key
// tiles, at most 64 (`target` as for fwd_splits).
int mask_splits(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype, int nsplit, long long target = 256) {
  if (nsplit > 0) return nsplit;
  const int G = Hq / Hkv, nw = fa::fwd_waves(dtype == FA_DTYPE_BF16, d);
  const bool pack = G <= nw && Tq <= 32 * (nw / G);
  const long long items = pack ? (long long)B * Hkv : (long long)((Tq + 32 * nw - 1) / (32 * nw)) * B * Hq;
  const long long tiles = (Tk + fa::fwd_block_keys(dtype == FA_DTYPE_BF16, d) - 1) /
                          fa::fwd_block_keys(dtype == FA_DTYPE_BF16, d);
  long long ns = items > 0 ? (target + items - 1) / items : 1;
  ns = ns < tiles / 8 ? ns : tiles / 8;
  ns = ns < 64 ? ns : 64;
  return ns < 1 ? 1 : (int)ns;
}

// Workgroups aimed at by the automatic slice count of a variable-length
// batch, from the longest key count over the mean, r = max_k * B / total_k
// (the offsets themselves stay in device memory).  Lengths within a factor of
// 4 of the mean: 256, as for the fixed layout.  Beyond that a few long
// sequences set the time while the short ones finish early, and the target
// grows by sqrt(r): between the long sequences' critical path (which wants r)
// and the launch and merge cost of the short ones' extra slices.  Measured on
// 16 batches of 32-query blocks (Hq = 32, Hkv = 8, d = 128, with and without
// a mask): 2% slower than the best slice count on average, 16% at worst
// (256 alone: 17% and 83%; 256 r: 15% and 31%).
long long varlen_split_target(int B, int total_k, int max_k) {
  if (total_k <= 0 || max_k <= 0) return 256;
  const double r = (double)max_k * B / total_k;
  if (r < 4.0) return 256;
  const double t = 256.0 * std::sqrt(r);
  return t > 256.0 * 64 ? 256LL * 64 : (long long)std::ceil(t);
}

// Head dim of V (and O, dO, dV): equal to d, or 64 with d = 128 and 128 with
// d = 64 (both dtypes).
int check_dv(int d, int dv, int dtype) {
  (void)dtype;
  if (dv == d) return FA_OK;
  if ((d == 128 && dv == 64) || (d == 64 && dv == 128)) return FA_OK;
  return FA_ERR_HEAD_DIM;
}

// Variable-length batch arguments: offsets present and 4-byte aligned, sizes
// non-negative, the longest sequence within the totals.  The offsets
// themselves live in device memory and are not read here; the kernels clamp
// each sequence into the packed tensors.
int check_varlen(const int* cu_q, const int* cu_k, int total_q, int total_k, int max_q, int max_k) {
  if (cu_q == nullptr || cu_k == nullptr) return FA_ERR_NULL_PTR;
  if ((reinterpret_cast<uintptr_t>(cu_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_k) & 3u)) return FA_ERR_ALIGNMENT;
  if (total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0) return FA_ERR_BAD_SHAPE;
  if (max_q > total_q || max_k > total_k) return FA_ERR_BAD_SHAPE;
  if (total_q > kMaxSeq * 64 || total_k > kMaxSeq * 64) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

int bwd_core(const void* Q, const void* K, const void* V, const void* O, const float* L,
             const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
             const int* cu_q, const int* cu_k, int B, int Hq, int Hkv, int total_q, int total_k, int Tq,
             int Tk, int d, int dv, int causal, int window, float scale, int dtype, unsigned stages, void* stream,
             const uint32_t* mask = nullptr, long long mask_bstride = 0, bool validate_only = false,
             const int* seqlens_k = nullptr);
// Boolean-mask arguments shared by the forward and the backward: the stride
// is 0 (one mask for the batch) or a multiple of 4 words holding a whole
// entry, and the mask has Tq rows of 4 * ceil(Tk / 128) words.
int check_mask(const uint32_t* mask, long long stride, int B, int Tq, int Tk) {
  const long long rw = 4LL * ((Tk + 127) / 128), mwords = (long long)Tq * rw;
  if (stride < 0 || (stride != 0 && stride < mwords)) return FA_ERR_BAD_SHAPE;
  if (stride % 4 != 0) return FA_ERR_ALIGNMENT;               // every row stays 16-byte aligned
  if (stride > kMaxElems / B) return FA_ERR_TOO_LARGE;
  return check_ptr(mask, mwords);
}
// Bytes of the backward's key-major mask copy (after the rest of its workspace).
size_t mask_t_bytes(int B, int Tq, int Tk, long long stride) {
  const long long entries = stride != 0 ? B : 1;
  return align_up((size_t)entries * Tk * (4 * ((Tq + 127) / 128)) * 4);
}

// Split-forward partials for `rows` output rows: ns * rows fp32 rows of d
// values, then ns * rows logsumexps, each part 256-byte aligned.
size_t splitk_rows_bytes(size_t rows, int d, int ns) {
  return align_up((size_t)ns * rows * d * 4) + align_up((size_t)ns * rows * 4);
}
size_t splitk_ws_bytes(int B, int Hq, int Tq, int d, int ns) {
  return splitk_rows_bytes((size_t)B * Hq * Tq, d, ns);
}

// Workspace of the backward through a block table: the backward's own (-D,
// L2 rows), then the gathered K and V and the per-sequence dK and dV, each
// [B][Hkv][pages_per_seq * page_size][d] in the dtype.
struct PagedWs {
  size_t kg, vg, dkg, dvg, total;
};
PagedWs paged_ws(int B, int Hq, int Hkv, int Tq, long long tk_max, int d, int dtype) {
  PagedWs w;
  const size_t part = align_up((size_t)B * Hkv * tk_max * d * elem_bytes(dtype));
  w.kg = ws_layout(B, Hq, Tq, d, dtype).total;
  w.vg = w.kg + part;
  w.dkg = w.vg + part;
  w.dvg = w.dkg + part;
  w.total = w.dvg + part;
  return w;
}

// Scratch of fa_bwd_noalloc: -D and the log2-domain L of every (padded)
// query row, in the workspace layout of fa_bwd, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy for the life of
// the process.  Host code must never use this name as a device address (on
// the host it is only a stand-in for the symbol): the per-device address
// comes from hipGetSymbolAddress below.
constexpr size_t kScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) {
    t_hip_error = "device ordinal beyond the library's per-device scratch table";
    return FA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) {
      t_hip_error = "hipGetSymbolAddress returned no address for the scratch array";
      return FA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_bwd_paged_workspace_bytes(int B, int Hq, int Hkv, int Tq, int pages_per_seq, int page_size, int d,
                                    int dtype) {
  if (pages_per_seq < 1 || page_size < 1 || page_size % 128 != 0) return 0;
  const long long tk = (long long)pages_per_seq * page_size;
  if (tk > kMaxSeq || check_common(B, Hq, Hkv, Tq, (int)tk, d, dtype) != FA_OK) return 0;
  return paged_ws(B, Hq, Hkv, Tq, tk, d, dtype).total;
}

int fa_bwd_paged(const void* Q, const void* K_pages, const void* V_pages, const void* O, const float* L,
                 const void* dO, void* dQ, void* dK_pages, void* dV_pages, const int* page_table,
                 const int* seqlens_k, int B, int Hq, int Hkv, int Tq, int pages_per_seq, int page_size,
                 int num_pages, int d, int causal, int window, float scale, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (pages_per_seq < 1 || page_size < 1 || num_pages < 1) return FA_ERR_BAD_SHAPE;
  if (page_size % 128 != 0) return FA_ERR_BAD_SHAPE;
  const long long tk = (long long)pages_per_seq * page_size;
  if (tk > kMaxSeq) return FA_ERR_TOO_LARGE;
  int st = check_common(B, Hq, Hkv, Tq, (int)tk, d, dtype);
  if (st != FA_OK) return st;
  if (page_table == nullptr || seqlens_k == nullptr) return FA_ERR_NULL_PTR;
  if ((reinterpret_cast<uintptr_t>(page_table) & 3u) || (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return FA_ERR_ALIGNMENT;
  const long long nq = (long long)B * Hq * Tq * d, npool = (long long)num_pages * Hkv * page_size * d;
  if (npool > kMaxElems) return FA_ERR_TOO_LARGE;
  if ((long long)B * pages_per_seq > kMaxElems) return FA_ERR_TOO_LARGE;
  if ((long long)num_pages * Hkv * (page_size / 128) > kMaxGrid) return FA_ERR_TOO_LARGE;
  if ((st = check_ptr(Q, nq)) || (st = check_ptr(O, nq)) || (st = check_ptr(dO, nq)) || (st = check_ptr(dQ, nq)) ||
      (st = check_ptr(K_pages, npool)) || (st = check_ptr(V_pages, npool)) || (st = check_ptr(dK_pages, npool)) ||
      (st = check_ptr(dV_pages, npool)) || (st = check_ptr(L, (long long)B * Hq * Tq)))
    return st;
  if (bad_scale(scale)) return FA_ERR_SCALE;
  const PagedWs pw = paged_ws(B, Hq, Hkv, Tq, tk, d, dtype);
  if (workspace == nullptr || workspace_bytes < pw.total) return FA_ERR_WORKSPACE;
  if (misaligned(workspace)) return FA_ERR_ALIGNMENT;
  char* wsb = static_cast<char*>(workspace);
  fa::PagedBwdArgs p;
  p.K = K_pages; p.V = V_pages;
  p.Kg = wsb + pw.kg; p.Vg = wsb + pw.vg;
  p.dKg = wsb + pw.dkg; p.dVg = wsb + pw.dvg;
  p.dK = dK_pages; p.dV = dV_pages;
  p.table = page_table; p.seqlens = seqlens_k;
  p.B = B; p.Hkv = Hkv; p.pps = pages_per_seq; p.page_size = page_size; p.num_pages = num_pages;
  p.tk_max = (int)tk;
  const bool bf = dtype == FA_DTYPE_BF16;
  if ((st = hip_status(fa::launch_paged(p, bf, d, 0, (hipStream_t)stream))) != FA_OK) return st;
  st = bwd_core(Q, wsb + pw.kg, wsb + pw.vg, O, L, dO, dQ, wsb + pw.dkg, wsb + pw.dvg, workspace, pw.kg, nullptr,
                nullptr, B, Hq, Hkv, 0, 0, Tq, (int)tk, d, d, causal, window, scale, dtype, FA_BWD_STAGE_ALL, stream,
                nullptr, 0, false, seqlens_k);
  if (st != FA_OK) return st;
  return hip_status(fa::launch_paged(p, bf, d, 1, (hipStream_t)stream));
}

size_t fa_bwd_noalloc_scratch_bytes(void) { return kScratchBytes; }

int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const float* L,
                   const void* dO, void* dQ, void* dK, void* dV,
                   int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
                   int dtype, void* stream) {
  // Every argument is validated (by the same checks as fa_bwd, with the
  // scratch standing in for a workspace of exactly its size) before the
  // scratch address is looked up, so a rejected call makes no HIP call.
  int st = check_common(B, Hq, Hkv, Tq, Tk, d, dtype);
  if (st != FA_OK) return st;
  if (ws_layout(B, Hq, Tq, d, dtype).total > kScratchBytes) return FA_ERR_SCRATCH;
  st = bwd_core(Q, K, V, O, L, dO, dQ, dK, dV, nullptr, kScratchBytes, nullptr, nullptr, B, Hq, Hkv, 0, 0, Tq,
                Tk, d, d, causal, 0, scale, dtype, FA_BWD_STAGE_ALL, stream, nullptr, 0, /*validate_only=*/true);
  if (st != FA_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != FA_OK) return st;
  return bwd_core(Q, K, V, O, L, dO, dQ, dK, dV, ws, kScratchBytes, nullptr, nullptr, B, Hq, Hkv, 0, 0, Tq, Tk,
                  d, d, causal, 0, scale, dtype, FA_BWD_STAGE_ALL, stream);
}

int fa_abi_version(void) { return (2 << 16) | 1; }

const char* fa_hip_error_string(void) { return t_hip_error; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_PTR: return "a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "bad shape: B, Hq, Hkv must be >= 1 and Tq, Tk >= 0";
    case FA_ERR_GQA_RATIO: return "Hq must be a multiple of Hkv";
    case FA_ERR_HEAD_DIM: return "unsupported head dimension (32, 64 or 128, bf16 also 256; dv != d as (128, 64) or (64, 128))";
    case FA_ERR_DTYPE: return "unsupported dtype (FA_DTYPE_F32 or FA_DTYPE_BF16)";
    case FA_ERR_SCALE: return "scale must be finite and positive";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than fa_bwd_workspace_bytes";
    case FA_ERR_ALIGNMENT: return "pointers must be 16-byte aligned";
    case FA_ERR_TOO_LARGE: return "a size exceeds the library's index range";
    case FA_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case FA_ERR_STAGES: return "unknown backward stage bits";
    case FA_ERR_SCRATCH: return "the call needs more than fa_bwd_noalloc's fixed scratch (fa_bwd_noalloc_scratch_bytes)";
    default: return "unknown status";
  }
}

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L,
           int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
           int dtype, void* stream) {
  return fa_fwd_window(Q, K, V, O, L, B, Hq, Hkv, Tq, Tk, d, causal, 0, scale, dtype, stream);
}

int fa_fwd_window(const void* Q, const void* K, const void* V, void* O, float* L,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, int window, float scale,
                  int dtype, void* stream) {
  return fa_fwd_dv(Q, K, V, O, L, B, Hq, Hkv, Tq, Tk, d, d, causal, window, scale, dtype, stream);
}

int fa_fwd_dv(const void* Q, const void* K, const void* V, void* O, float* L, int B, int Hq, int Hkv, int Tq,
              int Tk, int d, int dv, int causal, int window, float scale, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, Tq, Tk, d, dtype);
  if (st != FA_OK) return st;
  if ((st = check_dv(d, dv, dtype)) != FA_OK) return st;
  const long long nq = (long long)B * Hq * Tq * d, nkv = (long long)B * Hkv * Tk * d;
  const long long no = (long long)B * Hq * Tq * dv, nv = (long long)B * Hkv * Tk * dv;
  if ((st = check_ptr(Q, nq)) || (st = check_ptr(O, no)) || (st = check_ptr(K, nkv)) ||
      (st = check_ptr(V, nv)) || (st = check_ptr(L, (long long)B * Hq * Tq)))
    return st;
  if (bad_scale(scale)) return FA_ERR_SCALE;
  if (Tq == 0) return FA_OK;
  fa::FwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.L = L;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq; a.Tk = Tk;
  a.window = window > 0 ? window : 0;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.pack = fwd_pack(Hq, Hkv, Tq, d, dtype);
  a.Opart = nullptr;
  a.Lpart = nullptr;
  a.cu_q = a.cu_k = nullptr;
  a.total_q = a.total_k = 0;
  return hip_status(fa::launch_fwd(a, dtype == FA_DTYPE_BF16, d, causal != 0, (hipStream_t)stream, 1, dv));
}

int fa_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* L, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                  int max_seqlen_k, int d, int causal, int window, float scale, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, dtype);
  if (st != FA_OK) return st;
  if ((st = check_varlen(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k)) != FA_OK)
    return st;
  const long long nq = (long long)Hq * total_q * d, nkv = (long long)Hkv * total_k * d;
  if (nq > kMaxElems || nkv > kMaxElems) return FA_ERR_TOO_LARGE;
  if ((st = check_ptr(Q, nq)) || (st = check_ptr(O, nq)) || (st = check_ptr(K, nkv)) ||
      (st = check_ptr(V, nkv)) || (st = check_ptr(L, (long long)Hq * total_q)))
    return st;
  if (bad_scale(scale)) return FA_ERR_SCALE;
  if (max_seqlen_q == 0 || total_q == 0) return FA_OK;
  fa::FwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.L = L;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = max_seqlen_q; a.Tk = max_seqlen_k;
  a.window = window > 0 ? window : 0;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.pack = fwd_pack(Hq, Hkv, max_seqlen_q, d, dtype);
  a.Opart = nullptr;
  a.Lpart = nullptr;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  return hip_status(fa::launch_fwd(a, dtype == FA_DTYPE_BF16, d, causal != 0, (hipStream_t)stream));
}

int fa_mask_row_words(int Tk) { return Tk < 0 || Tk > kMaxSeq ? -1 : 4 * ((Tk + 127) / 128); }

int fa_mask_pack(const void* mask_bytes, uint32_t* mask_bits, long long rows, int Tk, void* stream) {
  if (rows < 0 || Tk < 0) return FA_ERR_BAD_SHAPE;
  if (Tk > kMaxSeq) return FA_ERR_TOO_LARGE;
  const int rw = fa_mask_row_words(Tk);
  if (rows > kMaxElems / (Tk > 0 ? Tk : 1) || rows * rw / 256 + 1 > kMaxGrid) return FA_ERR_TOO_LARGE;
  if (rows * Tk > 0 && mask_bytes == nullptr) return FA_ERR_NULL_PTR;
  int st;
  if ((st = check_ptr(mask_bits, rows * rw))) return st;
  return hip_status(fa::launch_mask_pack(static_cast<const uint8_t*>(mask_bytes), mask_bits, rows, Tk, rw,
                                         (hipStream_t)stream));
}

int fa_fwd_mask(const void* Q, const void* K, const void* V, void* O, float* L, const uint32_t* mask_bits,
                long long mask_batch_stride, int B, int Hq, int Hkv, int Tq, int Tk, int d, int dv, int causal,
                int window, float scale, int dtype, void* stream) {
  return fa_fwd_mask_splitk(Q, K, V, O, L, mask_bits, mask_batch_stride, nullptr, 0, B, Hq, Hkv, Tq, Tk, d, dv,
                            causal, window, scale, dtype, 1, stream);
}

size_t fa_fwd_mask_splitk_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dv, int dtype,
                                          int nsplit) {
  if (check_common(B, Hq, Hkv, Tq, Tk, d, dtype) != FA_OK || check_dv(d, dv, dtype) != FA_OK) return 0;
  const int ns = mask_splits(B, Hq, Hkv, Tq, Tk, d, dtype, nsplit);
  if (ns > kMaxSplits) return 0;
  return ns == 1 ? 0 : splitk_ws_bytes(B, Hq, Tq, dv, ns);
}

namespace {

// The masked forward for the fixed layout (cu_q == nullptr; Tq, Tk) or a
// variable-length batch (offsets; Tq, Tk the longest sequences), and the
// unmasked variable-length forward (masked == false).  A mask runs the plain
// shape (its packing only); without one the packing of fa_fwd_varlen.  Split
// over ns key slices when ns > 1, the partials indexed by output row.
int fwd_split_core(const void* Q, const void* K, const void* V, void* O, float* L, bool masked,
                   const uint32_t* mask_bits, long long mask_batch_stride, const int* cu_q, const int* cu_k, int B,
                   int Hq, int Hkv, int total_q, int total_k, int Tq, int Tk, int d, int dv, int causal, int window,
                   float scale, int dtype, void* workspace, size_t workspace_bytes, int nsplit, void* stream,
                   long long target = 256) {
  int st = check_common(B, Hq, Hkv, Tq, Tk, d, dtype);
  if (st != FA_OK) return st;
  if ((st = check_dv(d, dv, dtype)) != FA_OK) return st;
  const bool varlen = cu_q != nullptr;
  const long long rows = varlen ? (long long)Hq * total_q : (long long)B * Hq * Tq;
  const long long krows = varlen ? (long long)Hkv * total_k : (long long)B * Hkv * Tk;
  if (rows * d > kMaxElems || rows * dv > kMaxElems || krows * d > kMaxElems || krows * dv > kMaxElems)
    return FA_ERR_TOO_LARGE;
  if ((st = check_ptr(Q, rows * d)) || (st = check_ptr(O, rows * dv)) || (st = check_ptr(K, krows * d)) ||
      (st = check_ptr(V, krows * dv)) || (st = check_ptr(L, rows)))
    return st;
  const long long rw = fa_mask_row_words(Tk);
  if (masked && (st = check_mask(mask_bits, mask_batch_stride, B, Tq, Tk))) return st;
  if (bad_scale(scale)) return FA_ERR_SCALE;
  const int ns = masked ? mask_splits(B, Hq, Hkv, Tq, Tk, d, dtype, nsplit, target)
                        : fwd_splits(B, Hq, Hkv, Tq, Tk, d, dtype, nsplit, target);
  if (ns > kMaxSplits) return FA_ERR_TOO_LARGE;
  const size_t need = ns == 1 ? 0 : splitk_rows_bytes((size_t)rows, dv, ns);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (misaligned(workspace)) return FA_ERR_ALIGNMENT;
  }
  if (Tq == 0 || rows == 0) return FA_OK;
  fa::FwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.L = L;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq; a.Tk = Tk;
  a.window = window > 0 ? window : 0;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  const int G = Hq / Hkv, nw = fa::fwd_waves(dtype == FA_DTYPE_BF16, d);
  a.pack = !masked ? fwd_pack(Hq, Hkv, Tq, d, dtype)
                   : (G <= nw && Tq <= 32 * (nw / G)) ? 1 : 0;   // a mask: the plain shape's packing only
  a.Opart = nullptr;
  a.Lpart = nullptr;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.total_q = varlen ? total_q : 0;
  a.total_k = varlen ? total_k : 0;
  a.mask = masked && Tk > 0 ? mask_bits : nullptr;
  a.mask_bstride = mask_batch_stride;
  a.mask_row_words = (int)rw;
  if (ns > 1) {
    char* wsb = static_cast<char*>(workspace);
    a.Opart = reinterpret_cast<float*>(wsb);
    a.Lpart = reinterpret_cast<float*>(wsb + align_up((size_t)ns * rows * dv * 4));
  }
  return hip_status(fa::launch_fwd(a, dtype == FA_DTYPE_BF16, d, causal != 0, (hipStream_t)stream, ns, dv));
}

}  // namespace

int fa_fwd_mask_splitk(const void* Q, const void* K, const void* V, void* O, float* L, const uint32_t* mask_bits,
                       long long mask_batch_stride, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                       int Tq, int Tk, int d, int dv, int causal, int window, float scale, int dtype, int nsplit,
                       void* stream) {
  return fwd_split_core(Q, K, V, O, L, true, mask_bits, mask_batch_stride, nullptr, nullptr, B, Hq, Hkv, 0, 0, Tq,
                        Tk, d, dv, causal, window, scale, dtype, workspace, workspace_bytes, nsplit, stream);
}

int fa_fwd_varlen_mask(const void* Q, const void* K, const void* V, void* O, float* L, const uint32_t* mask_bits,
                       long long mask_seq_stride, const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq,
                       int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal,
                       int window, float scale, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, dtype);
  if (st != FA_OK) return st;
  if ((st = check_varlen(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k)) != FA_OK)
    return st;
  return fwd_split_core(Q, K, V, O, L, true, mask_bits, mask_seq_stride, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv,
                        total_q, total_k, max_seqlen_q, max_seqlen_k, d, d, causal, window, scale, dtype, nullptr, 0,
                        1, stream);
}

size_t fa_fwd_varlen_splitk_workspace_bytes(int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                                            int max_seqlen_k, int d, int dtype, int nsplit, int masked) {
  if (check_common(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, dtype) != FA_OK) return 0;
  if (total_q < max_seqlen_q || total_q > kMaxSeq * 64) return 0;
  if (total_k < max_seqlen_k || total_k > kMaxSeq * 64) return 0;
  const long long target = varlen_split_target(B, total_k, max_seqlen_k);
  const int ns = masked ? mask_splits(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, dtype, nsplit, target)
                        : fwd_splits(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, dtype, nsplit, target);
  if (ns > kMaxSplits) return 0;
  return ns == 1 ? 0 : splitk_rows_bytes((size_t)Hq * total_q, d, ns);
}

int fa_fwd_varlen_splitk(const void* Q, const void* K, const void* V, void* O, float* L,
                         const uint32_t* mask_bits, long long mask_seq_stride, const int* cu_seqlens_q,
                         const int* cu_seqlens_k, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                         int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal,
                         int window, float scale, int dtype, int nsplit, void* stream) {
  int st = check_common(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, dtype);
  if (st != FA_OK) return st;
  if ((st = check_varlen(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k)) != FA_OK)
    return st;
  return fwd_split_core(Q, K, V, O, L, mask_bits != nullptr, mask_bits, mask_seq_stride, cu_seqlens_q,
                        cu_seqlens_k, B, Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, d, causal, window,
                        scale, dtype, workspace, workspace_bytes, nsplit, stream,
                        varlen_split_target(B, total_k, max_seqlen_k));
}

size_t fa_bwd_mask_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype,
                                   long long mask_batch_stride) {
  if (check_common(B, Hq, Hkv, Tq, Tk, d, dtype) != FA_OK || mask_batch_stride < 0) return 0;
  return ws_layout(B, Hq, Tq, d, dtype).total + mask_t_bytes(B, Tq, Tk, mask_batch_stride);
}

int fa_bwd_mask(const void* Q, const void* K, const void* V, const void* O, const float* L, const void* dO,
                void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, const uint32_t* mask_bits,
                long long mask_batch_stride, int B, int Hq, int Hkv, int Tq, int Tk, int d, int dv, int causal,
                int window, float scale, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, Tq, Tk, d, dtype);
  if (st != FA_OK) return st;
  if ((st = check_dv(d, dv, dtype)) != FA_OK) return st;
  if ((st = check_mask(mask_bits, mask_batch_stride, B, Tq, Tk))) return st;
  return bwd_core(Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, nullptr, nullptr, B, Hq, Hkv, 0, 0,
                  Tq, Tk, d, dv, causal, window, scale, dtype, FA_BWD_STAGE_ALL, stream, mask_bits,
                  mask_batch_stride);
}

int fa_bwd_varlen_mask(const void* Q, const void* K, const void* V, const void* O, const float* L, const void* dO,
                       void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                       const uint32_t* mask_bits, long long mask_seq_stride, const int* cu_seqlens_q,
                       const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                       int max_seqlen_k, int d, int causal, int window, float scale, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, dtype);
  if (st != FA_OK) return st;
  if ((st = check_varlen(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k)) != FA_OK)
    return st;
  if ((st = check_mask(mask_bits, mask_seq_stride, B, max_seqlen_q, max_seqlen_k))) return st;
  return bwd_core(Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, cu_seqlens_q, cu_seqlens_k, B, Hq,
                  Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, d, causal, window, scale, dtype,
                  FA_BWD_STAGE_ALL, stream, mask_bits, mask_seq_stride);
}

size_t fa_fwd_splitk_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype, int nsplit) {
  if (check_common(B, Hq, Hkv, Tq, Tk, d, dtype) != FA_OK) return 0;
  const int ns = fwd_splits(B, Hq, Hkv, Tq, Tk, d, dtype, nsplit);
  if (ns > kMaxSplits) return 0;
  return splitk_ws_bytes(B, Hq, Tq, d, ns);
}

int fa_fwd_splitk(const void* Q, const void* K, const void* V, void* O, float* L, void* workspace,
                  size_t workspace_bytes, int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal,
                  int window, float scale, int dtype, int nsplit, void* stream) {
  int st = check_common(B, Hq, Hkv, Tq, Tk, d, dtype);
  if (st != FA_OK) return st;
  const long long nq = (long long)B * Hq * Tq * d, nkv = (long long)B * Hkv * Tk * d;
  if ((st = check_ptr(Q, nq)) || (st = check_ptr(O, nq)) || (st = check_ptr(K, nkv)) ||
      (st = check_ptr(V, nkv)) || (st = check_ptr(L, (long long)B * Hq * Tq)))
    return st;
  if (bad_scale(scale)) return FA_ERR_SCALE;
  const int ns = fwd_splits(B, Hq, Hkv, Tq, Tk, d, dtype, nsplit);
  if (ns > kMaxSplits) return FA_ERR_TOO_LARGE;
  const size_t need = splitk_ws_bytes(B, Hq, Tq, d, ns);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (misaligned(workspace)) return FA_ERR_ALIGNMENT;
  }
  if (Tq == 0) return FA_OK;
  char* wsb = static_cast<char*>(workspace);
  fa::FwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.L = L;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq; a.Tk = Tk;
  a.window = window > 0 ? window : 0;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.pack = fwd_pack(Hq, Hkv, Tq, d, dtype);
  a.cu_q = a.cu_k = nullptr;
  a.total_q = a.total_k = 0;
  a.Opart = reinterpret_cast<float*>(wsb);
  a.Lpart = reinterpret_cast<float*>(wsb + align_up((size_t)ns * B * Hq * Tq * d * 4));
  return hip_status(fa::launch_fwd(a, dtype == FA_DTYPE_BF16, d, causal != 0, (hipStream_t)stream, ns));
}

size_t fa_fwd_paged_workspace_bytes(int B, int Hq, int Hkv, int Tq, int pages_per_seq, int page_size, int d,
                                    int dtype, int nsplit) {
  if (pages_per_seq < 1 || page_size < 1) return 0;
  const long long tk = (long long)pages_per_seq * page_size;
  if (tk > kMaxSeq) return 0;
  if (nsplit == 1) return 0;
  return fa_fwd_splitk_workspace_bytes(B, Hq, Hkv, Tq, (int)tk, d, dtype, nsplit);
}

int fa_fwd_paged(const void* Q, const void* K_pages, const void* V_pages, void* O, float* L,
                 const int* page_table, const int* seqlens_k, int B, int Hq, int Hkv, int Tq, int pages_per_seq,
                 int page_size, int num_pages, int d, int causal, int window, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, int nsplit, void* stream) {
  if (pages_per_seq < 1 || page_size < 1 || num_pages < 1) return FA_ERR_BAD_SHAPE;
  if (page_size % 128 != 0) return FA_ERR_BAD_SHAPE;
  const long long tk = (long long)pages_per_seq * page_size;
  if (tk > kMaxSeq) return FA_ERR_TOO_LARGE;
  int st = check_common(B, Hq, Hkv, Tq, (int)tk, d, dtype);
  if (st != FA_OK) return st;
  if (page_table == nullptr || seqlens_k == nullptr) return FA_ERR_NULL_PTR;
  if ((reinterpret_cast<uintptr_t>(page_table) & 3u) || (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return FA_ERR_ALIGNMENT;
  const long long nq = (long long)B * Hq * Tq * d, npool = (long long)num_pages * Hkv * page_size * d;
  if (npool > kMaxElems) return FA_ERR_TOO_LARGE;
  if ((st = check_ptr(Q, nq)) || (st = check_ptr(O, nq)) || (st = check_ptr(K_pages, npool)) ||
      (st = check_ptr(V_pages, npool)) || (st = check_ptr(L, (long long)B * Hq * Tq)))
    return st;
  if (bad_scale(scale)) return FA_ERR_SCALE;
  const int ns = nsplit == 1 ? 1 : fwd_splits(B, Hq, Hkv, Tq, (int)tk, d, dtype, nsplit);
  if (ns > kMaxSplits) return FA_ERR_TOO_LARGE;
  const size_t need = ns == 1 ? 0 : splitk_ws_bytes(B, Hq, Tq, d, ns);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (misaligned(workspace)) return FA_ERR_ALIGNMENT;
  }
  if (Tq == 0) return FA_OK;
  fa::FwdArgs a;
  a.Q = Q; a.K = K_pages; a.V = V_pages; a.O = O; a.L = L;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq; a.Tk = (int)tk;
  a.window = window > 0 ? window : 0;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.pack = fwd_pack(Hq, Hkv, Tq, d, dtype);
  a.cu_q = a.cu_k = nullptr;
  a.total_q = a.total_k = 0;
  a.pages = page_table;
  a.seqlens_k = seqlens_k;
  a.pages_per_seq = pages_per_seq;
  a.page_size = page_size;
  a.num_pages = num_pages;
  char* wsb = static_cast<char*>(workspace);
  a.Opart = ns == 1 ? nullptr : reinterpret_cast<float*>(wsb);
  a.Lpart = ns == 1 ? nullptr : reinterpret_cast<float*>(wsb + align_up((size_t)ns * B * Hq * Tq * d * 4));
  return hip_status(fa::launch_fwd(a, dtype == FA_DTYPE_BF16, d, causal != 0, (hipStream_t)stream, ns));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype) {
  if (check_common(B, Hq, Hkv, Tq, Tk, d, dtype) != FA_OK) return 0;
  return ws_layout(B, Hq, Tq, d, dtype).total;
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* L,
           const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
           int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
           int dtype, void* stream) {
  return fa_bwd_stages(Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, B, Hq, Hkv, Tq, Tk, d,
                       causal, scale, dtype, FA_BWD_STAGE_ALL, stream);
}

int fa_bwd_stages(const void* Q, const void* K, const void* V, const void* O, const float* L,
                  const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
                  int dtype, unsigned stages, void* stream) {
  return fa_bwd_window(Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, B, Hq, Hkv, Tq, Tk, d,
                       causal, 0, scale, dtype, stages, stream);
}

int fa_bwd_window(const void* Q, const void* K, const void* V, const void* O, const float* L,
                  const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, int window, float scale,
                  int dtype, unsigned stages, void* stream) {
  return bwd_core(Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, nullptr, nullptr, B, Hq, Hkv,
                  0, 0, Tq, Tk, d, d, causal, window, scale, dtype, stages, stream);
}

int fa_bwd_dv(const void* Q, const void* K, const void* V, const void* O, const float* L, const void* dO,
              void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
              int Tq, int Tk, int d, int dv, int causal, int window, float scale, int dtype, unsigned stages,
              void* stream) {
  return bwd_core(Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, nullptr, nullptr, B, Hq, Hkv,
                  0, 0, Tq, Tk, d, dv, causal, window, scale, dtype, stages, stream);
}

int fa_bwd_varlen(const void* Q, const void* K, const void* V, const void* O, const float* L,
                  const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q,
                  int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal, int window,
                  float scale, int dtype, void* stream) {
  int st = check_varlen(cu_seqlens_q, cu_seqlens_k, total_q, total_k, max_seqlen_q, max_seqlen_k);
  if (st != FA_OK) return st;
  return bwd_core(Q, K, V, O, L, dO, dQ, dK, dV, workspace, workspace_bytes, cu_seqlens_q, cu_seqlens_k, B,
                  Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, d, causal, window, scale, dtype,
                  FA_BWD_STAGE_ALL, stream);
}

}  // extern "C"

namespace {

int bwd_core(const void* Q, const void* K, const void* V, const void* O, const float* L,
             const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
             const int* cu_q, const int* cu_k, int B, int Hq, int Hkv, int total_q, int total_k, int Tq,
             int Tk, int d, int dv, int causal, int window, float scale, int dtype, unsigned stages, void* stream,
             const uint32_t* mask, long long mask_bstride, bool validate_only, const int* seqlens_k) {
  int st = check_common(B, Hq, Hkv, Tq, Tk, d, dtype);
  if (st != FA_OK) return st;
  if ((st = check_dv(d, dv, dtype)) != FA_OK) return st;
  const bool varlen = cu_q != nullptr;
  const long long rows = varlen ? (long long)Hq * total_q : (long long)B * Hq * Tq;
  const long long krows = varlen ? (long long)Hkv * total_k : (long long)B * Hkv * Tk;
  const long long nq = rows * d, no = rows * dv, nk = krows * d, nv = krows * dv;
  if (nq > kMaxElems || no > kMaxElems || nk > kMaxElems || nv > kMaxElems) return FA_ERR_TOO_LARGE;
  if ((st = check_ptr(Q, nq)) || (st = check_ptr(O, no)) || (st = check_ptr(dO, no)) ||
      (st = check_ptr(dQ, nq)) || (st = check_ptr(K, nk)) || (st = check_ptr(V, nv)) ||
      (st = check_ptr(dK, nk)) || (st = check_ptr(dV, nv)) || (st = check_ptr(L, rows)))
    return st;
  if (bad_scale(scale)) return FA_ERR_SCALE;
  if (stages & ~(unsigned)FA_BWD_STAGE_ALL) return FA_ERR_STAGES;
  const WsLayout ws = ws_layout(B, Hq, Tq, d, dtype);
  const bool masked = mask_bstride >= 0 && mask != nullptr && Tq > 0 && Tk > 0;
  if (masked) {                                      // one thread per word of the key-major copy
    const long long words = (mask_bstride != 0 ? (long long)B : 1LL) * Tk * (4LL * ((Tq + 127) / 128));
    if (words / 256 + 1 > kMaxGrid) return FA_ERR_TOO_LARGE;
  }
  const size_t need = ws.total + (masked ? mask_t_bytes(B, Tq, Tk, mask_bstride) : 0);
  if (validate_only) return need <= workspace_bytes ? FA_OK : FA_ERR_WORKSPACE;
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (misaligned(workspace)) return FA_ERR_ALIGNMENT;
  }
  if (Tq == 0 && Tk == 0) return FA_OK;
  if (varlen && total_q == 0 && total_k == 0) return FA_OK;
  char* wsb = static_cast<char*>(workspace);
  fa::BwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.L = L; a.dO = dO;
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.Dvec = ws.total ? reinterpret_cast<float*>(wsb + ws.dvec) : nullptr;
  a.Lg = ws.total ? reinterpret_cast<float*>(wsb + ws.lg) : nullptr;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Tq = Tq; a.Tk = Tk;
  a.Tqp = padded_rows(Tq);
  a.window = window > 0 ? window : 0;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.seqlens_k = seqlens_k;
  if (masked) {
    a.mask = mask;
    a.mask_bstride = mask_bstride;
    a.mask_row_words = 4 * ((Tk + 127) / 128);
    a.mask_t = reinterpret_cast<uint32_t*>(wsb + ws.total);
    a.mask_t_row_words = 4 * ((Tq + 127) / 128);
    a.mask_t_bstride = mask_bstride != 0 ? (long long)Tk * a.mask_t_row_words : 0;
  }
  return hip_status(fa::launch_bwd(a, dtype == FA_DTYPE_BF16, d, causal != 0, stages, (hipStream_t)stream, dv));
}

}  // namespace
