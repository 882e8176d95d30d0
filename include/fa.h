/*
 * fa.h -- C ABI of the gfx950 (MI355X) exact-attention library (libfa05.so).
 *
 * The library computes exact softmax attention with a tiled forward pass that
 * keeps only the output O and the natural-log row logsumexp L, and a backward
 * pass that rebuilds the score and probability tiles from Q, K, V, O and L
 * instead of storing them.
 *
 * Sources (web pages; cited by title and section):
 *  - "What Ordinary Autograd Saves: Tiling the Forward Pass Is Only Half the
 *    Algorithm", section "The implementation under test": the forward returns
 *    O and L = m + ln(l) per row (max m, exponential sum l of the scaled
 *    scores); scale = 1/sqrt(d) there.  Section "Why this is FlashAttention's
 *    second idea": the backward keeps O and L and rebuilds the score and
 *    probability tiles from them.
 *  - "Backward Pass Implementation", sections "Limitations of PyTorch
 *    Autograd" (S = Q K^T / sqrt(d), P = softmax(S), O = P V) and "The
 *    Recomputation Strategy" (O(N) saved statistics; recompute S and P in the
 *    backward); its introduction names arbitrary sequence lengths, causal
 *    masking and GQA as features of the forward.
 *  - "The Autograd Memory Trap: Diagnosing a Backward-Pass OOM in Chunked
 *    Attention", sections "Tracing the Autograd Graph" (the backward of
 *    repeating K/V heads is a sum over the repeats) and "The GQA Expansion
 *    Question" (query heads share K/V heads, 32 over 8).
 *
 * Conventions shared by every entry point
 *  - Layout: contiguous row-major.  Q, O, dO, dQ are [B][Hq][Tq][d]; K, V, dK,
 *    dV are [B][Hkv][Tk][d]; L is [B][Hq][Tq], always float32, natural log.
 *  - dtype: FA_DTYPE_F32 (float) or FA_DTYPE_BF16 (bfloat16 storage, float32
 *    accumulation, outputs rounded to nearest even).  It applies to Q, K, V,
 *    O, dO, dQ, dK, dV.
 *  - d (head dimension, equal for Q/K and V): 32, 64 or 128; bf16 also 256.
 *  - GQA: Hq must be a multiple of Hkv; query head h reads K/V head
 *    h / (Hq / Hkv).  dK and dV are summed over the query heads of a group.
 *  - causal != 0: key j is visible to query i iff j <= i + (Tk - Tq)
 *    (aligned at the end; j <= i when Tq == Tk).  Keys beyond Tk do not exist.
 *  - A query row that sees no key (Tk == 0, or causal with i + Tk - Tq < 0)
 *    gets O = 0, L = -inf and dQ = 0, and adds nothing to dK or dV.
 *  - scale multiplies Q K^T; it must be finite and positive (callers pass
 *    1/sqrt(d), the value of the tiling article's implementation).
 *  - Pointers are device pointers (or host-coherent memory the GPU can reach),
 *    16-byte aligned, and must not alias one another.  A pointer may be NULL
 *    only when the tensor it names has no elements.
 *  - stream is a hipStream_t (NULL = the null stream).  All work is enqueued
 *    on it; nothing synchronises the host, nothing prints, nothing allocates.
 *  - Ownership: the caller owns every buffer.  The library keeps no state
 *    between calls and may be called from several host threads at once
 *    (fa_bwd_noalloc alone keeps a per-device scratch address and shares its
 *    scratch between calls, see there).
 *  - Outputs are overwritten, never accumulated into.
 *  - Errors: arguments are validated before any HIP call and the first failing
 *    check is returned; a failed launch returns FA_ERR_HIP.  No C++ exception
 *    crosses this interface.  Tq == 0 is a successful no-op for fa_fwd.
 */
#ifndef FA05_FA_H
#define FA05_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_PTR = 1,   /* a required pointer is NULL */
  FA_ERR_BAD_SHAPE = 2,  /* B, Hq or Hkv < 1, Tq or Tk < 0 */
  FA_ERR_GQA_RATIO = 3,  /* Hq is not a multiple of Hkv */
  FA_ERR_HEAD_DIM = 4,   /* d is not 32, 64, 128 (bf16: or 256), or an unsupported (d, dv) pair */
  FA_ERR_DTYPE = 5,      /* dtype is not an fa_dtype value */
  FA_ERR_SCALE = 6,      /* scale is NaN, infinite, zero or negative */
  FA_ERR_WORKSPACE = 7,  /* workspace missing or smaller than fa_bwd_workspace_bytes */
  FA_ERR_ALIGNMENT = 8,  /* a pointer is not 16-byte aligned */
  FA_ERR_TOO_LARGE = 9,  /* a size exceeds the library's index range */
  FA_ERR_HIP = 10,       /* a HIP runtime call or kernel launch failed */
  FA_ERR_STAGES = 11,    /* fa_bwd_stages: a bit outside FA_BWD_STAGE_ALL is set */
  FA_ERR_SCRATCH = 12    /* fa_bwd_noalloc: the call needs more than its fixed scratch */
} fa_status;

typedef enum { FA_DTYPE_F32 = 0, FA_DTYPE_BF16 = 1 } fa_dtype;

/*
 * Forward pass.  Computes, per (b, h) and query row i,
 *   S_ij = scale * <Q_i, K_j>, over the visible keys j,
 *   L_i  = ln sum_j exp(S_ij)             (written to L, float32),
 *   O_i  = sum_j exp(S_ij - L_i) V_j      (written to O, dtype),
 * with the online-softmax recurrence over key tiles (running max, running
 * exponential sum, one rescale of the partial output when the max moves,
 * normalisation once at the end).  Reads Q, K, V; writes O and L only.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L,
           int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
           int dtype, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: float32 D and
 * log2-domain L per query row, rows padded to a multiple of 64 per head, each
 * part starting on a 256-byte boundary (8 * B * Hq * ceil(Tq / 64) * 64 bytes
 * plus alignment).  Returns 0 for invalid arguments.  The workspace holds
 * nothing between calls.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype);

/*
 * Backward pass: the gradients of sum(O * dO) with respect to Q, K and V
 * (L receives no cotangent), rebuilt tile by tile from Q, K, V, O, L:
 *   D_i   = sum_c dO_ic O_ic,
 *   P_ij  = exp(scale <Q_i, K_j> - L_i)   (0 for invisible keys),
 *   dP_ij = <dO_i, V_j>,  dS_ij = P_ij (dP_ij - D_i),
 *   dQ_i  = scale sum_j dS_ij K_j,
 *   dK_j  = scale sum_{h in group} sum_i dS_ij Q_i,
 *   dV_j  = sum_{h in group} sum_i P_ij dO_i.
 * O and L must be the outputs of fa_fwd for the same Q, K, V, sizes, causal
 * and scale.  Writes dQ, dK, dV (dtype) and uses `workspace` (at least
 * fa_bwd_workspace_bytes bytes, device memory, 16-byte aligned) as scratch.
 * No T x T tensor is ever formed and no atomics are used: dK, dV come from a
 * pass over key blocks, dQ from a pass over query blocks, each of which
 * rebuilds the score and probability tiles it needs.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* L,
           const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
           int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
           int dtype, void* stream);

/*
 * The backward pass in stages, for callers that time or schedule them
 * separately.  Same arguments and semantics as fa_bwd, plus a bit mask:
 *   FA_BWD_STAGE_PRE   -D = -rowsum(dO * O) and log2-domain L of every query
 *                      row into the workspace, as a pass of its own;
 *   FA_BWD_STAGE_DKDV  rebuild S and P per key block; write dK and dV;
 *   FA_BWD_STAGE_DQ    rebuild S and P per query block; write dQ.  This pass
 *                      forms the rows of PRE itself and writes them to the
 *                      workspace too, so with DQ set PRE does nothing.
 * Within one call the order is PRE (if it runs), DQ, then DKDV.  DKDV reads
 * the rows from the workspace: they must come from PRE or DQ in this call or
 * an earlier call on the same stream with identical arguments.  fa_bwd runs
 * DQ then DKDV.
 */
#define FA_BWD_STAGE_PRE 1u
#define FA_BWD_STAGE_DKDV 2u
#define FA_BWD_STAGE_DQ 4u
#define FA_BWD_STAGE_ALL 7u
int fa_bwd_stages(const void* Q, const void* K, const void* V, const void* O, const float* L,
                  const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
                  int dtype, unsigned stages, void* stream);

/*
 * Sliding-window attention ("The Autograd Memory Trap: Diagnosing a
 * Backward-Pass OOM in Chunked Attention": its sliding-window layers attend
 * over a much smaller key span, 2080 keys, than the full-attention layer's
 * 8032).  With window > 0, query i sees key j only if
 *   j > i + (Tk - Tq) - window,
 * i.e. at most `window` keys ending at its end-aligned diagonal position; this
 * narrows the causal bound when causal != 0 and applies on its own otherwise.
 * window <= 0 means no window, and the calls are then identical to fa_fwd and
 * fa_bwd_stages.  Rows left with no visible key get O = 0, L = -inf, dQ = 0.
 * Key tiles entirely outside a query block's window are neither loaded nor
 * computed, so the work scales with Tq * window instead of Tq * Tk.  All other
 * arguments, layouts, ownership and error behaviour are those of fa_fwd and
 * fa_bwd_stages; O and L passed to fa_bwd_window must come from fa_fwd_window
 * with the same window.
 */
int fa_fwd_window(const void* Q, const void* K, const void* V, void* O, float* L,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, int window, float scale,
                  int dtype, void* stream);
int fa_bwd_window(const void* Q, const void* K, const void* V, const void* O, const float* L,
                  const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                  int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, int window, float scale,
                  int dtype, unsigned stages, void* stream);

/*
 * Forward split over the keys, for few query rows against many keys: one
 * block of new tokens attending to a long prefix ("The Autograd Memory Trap",
 * section "The Scene": 32 new positions against an 8000-key prefix, 8032 keys
 * in all; inference stashes nothing for a backward, "What Ordinary Autograd
 * Saves", section "Why this is FlashAttention's second idea").  The key tiles
 * each workgroup would visit are divided into `nsplit` slices run side by
 * side; slice s writes its normalised partial output O_s and row logsumexp L_s
 * (float32) to the workspace, and a merge writes
 *   L = ln sum_s exp(L_s),  O = sum_s exp(L_s - L) O_s,
 * which is exactly the attention over the union of the slices (a row whose
 * keys all lie outside a slice has L_s = -inf there).  Results equal fa_fwd /
 * fa_fwd_window up to rounding.  nsplit <= 0 picks a count that fills the GPU
 * (about one workgroup per compute unit, at least eight key tiles per slice,
 * at most 64).  The workspace (device memory, 16-byte aligned, at least
 * fa_fwd_splitk_workspace_bytes for the same nsplit) holds nsplit * B * Hq *
 * Tq * (d + 1) floats; it carries nothing between calls.  Errors as fa_fwd,
 * plus FA_ERR_WORKSPACE and FA_ERR_TOO_LARGE (more than 1024 slices);
 * fa_fwd_splitk_workspace_bytes returns 0 for invalid arguments.
 */
size_t fa_fwd_splitk_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype, int nsplit);
int fa_fwd_splitk(const void* Q, const void* K, const void* V, void* O, float* L, void* workspace,
                  size_t workspace_bytes, int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal,
                  int window, float scale, int dtype, int nsplit, void* stream);

/*
 * Variable-length batches: B sequences of different lengths packed together
 * (the chunked-attention article's blocks of new positions each attend to a
 * prefix of their own length, section "The Scene").  Sequence b owns the query
 * rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and the key rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1 of every head; tensors are packed
 * head-major: Q, O, dO, dQ [Hq][total_q][d], K, V, dK, dV [Hkv][total_k][d],
 * L [Hq][total_q].  cu_seqlens_* are device arrays of B + 1 int32 offsets,
 * non-decreasing from 0 to total_*, with no sequence longer than
 * max_seqlen_*; the library does not read them on the host (they are device
 * memory), and the kernels clamp every sequence into the packed tensors, so
 * inconsistent offsets give meaningless rows but no out-of-bounds access.
 * Causal alignment, window, GQA, empty rows and dtypes are per sequence as in
 * fa_fwd_window / fa_bwd_window.  The backward workspace is
 * fa_bwd_workspace_bytes(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, dtype).
 * Errors as fa_fwd / fa_bwd, plus FA_ERR_NULL_PTR for missing offsets,
 * FA_ERR_ALIGNMENT for offsets not 4-byte aligned, FA_ERR_BAD_SHAPE for
 * negative sizes or a max_seqlen above its total.
 */
int fa_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* L, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                  int max_seqlen_k, int d, int causal, int window, float scale, int dtype, void* stream);
int fa_bwd_varlen(const void* Q, const void* K, const void* V, const void* O, const float* L,
                  const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q,
                  int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal, int window,
                  float scale, int dtype, void* stream);

/*
 * A value head dim dv different from the query/key head dim d ("What
 * Ordinary Autograd Saves", section "The implementation under test": V is
 * (Tk, dv)).  Layouts: Q, dQ [B][Hq][Tq][d]; K, dK [B][Hkv][Tk][d]; V, dV
 * [B][Hkv][Tk][dv]; O, dO [B][Hq][Tq][dv]; L as usual.  Supported: dv == d
 * (then identical to fa_fwd_window / fa_bwd_window), and in both dtypes the
 * pairs (d, dv) = (128, 64) and (64, 128); anything else is FA_ERR_HEAD_DIM.  All
 * other arguments, ownership and errors are those of fa_fwd_window and
 * fa_bwd_window (the backward workspace does not depend on d or dv).
 */
int fa_fwd_dv(const void* Q, const void* K, const void* V, void* O, float* L, int B, int Hq, int Hkv, int Tq,
              int Tk, int d, int dv, int causal, int window, float scale, int dtype, void* stream);
int fa_bwd_dv(const void* Q, const void* K, const void* V, const void* O, const float* L, const void* dO,
              void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
              int Tq, int Tk, int d, int dv, int causal, int window, float scale, int dtype, unsigned stages,
              void* stream);

/*
 * Forward over paged keys and values: a pool of fixed-size pages and a page
 * table per sequence, the shape of the chunked-attention article's prefix
 * cache, from which each block of new positions gathers its own prefix
 * (section "The Scene").  K_pages and V_pages are [num_pages][Hkv][page_size][d];
 * sequence b holds seqlens_k[b] keys (at most pages_per_seq * page_size), key
 * j being row j % page_size of page page_table[b * pages_per_seq + j /
 * page_size].  Q, O are [B][Hq][Tq][d] and L [B][Hq][Tq] as in fa_fwd; causal
 * alignment and the window are per sequence (end-aligned on its own key
 * count).  page_table and seqlens_k are device int32 arrays (B * pages_per_seq
 * and B entries) that the host never reads; page indices are clamped into the
 * pool and key counts into [0, pages_per_seq * page_size].  page_size must be a
 * multiple of 128.  nsplit == 1 runs one pass with no workspace; otherwise the
 * keys are split over slices and merged as in fa_fwd_splitk (nsplit <= 0:
 * automatic), with a workspace of fa_fwd_paged_workspace_bytes bytes.  The
 * slices are equal runs of key tiles sized for the longest sequence the table
 * holds (pages_per_seq * page_size keys), so a sequence with few keys leaves
 * the later slices empty.  Errors
 * as fa_fwd_splitk, plus FA_ERR_BAD_SHAPE for a page size that is not a
 * positive multiple of 128 or an empty pool.
 */
size_t fa_fwd_paged_workspace_bytes(int B, int Hq, int Hkv, int Tq, int pages_per_seq, int page_size, int d,
                                    int dtype, int nsplit);
int fa_fwd_paged(const void* Q, const void* K_pages, const void* V_pages, void* O, float* L,
                 const int* page_table, const int* seqlens_k, int B, int Hq, int Hkv, int Tq, int pages_per_seq,
                 int page_size, int num_pages, int d, int causal, int window, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, int nsplit, void* stream);

/*
 * Backward of fa_fwd_paged ("The Autograd Memory Trap: Diagnosing a
 * Backward-Pass OOM in Chunked Attention", sections "The Scene" and "The OOM:
 * When Inference Lies": training differentiates through the gather of each
 * block's prefix from the page pool).  The gradient of a page is the sum, over
 * every table entry (b, slot) that points at it, of the gradients of the rows
 * sequence b took from it: a page shared by several sequences collects all of
 * them, the rows of a page past a sequence's key count contribute nothing, and
 * pages no entry references come back as zeros.  dK_pages and dV_pages are
 * written in full, with the layout of K_pages / V_pages; dQ is [B][Hq][Tq][d].
 * O and L must come from fa_fwd_paged with the same table, key counts, causal
 * flag, window and scale.  Sums run in fp32 in table order (b major, slot
 * minor), so results are reproducible bit for bit.  Sizes, table, key counts
 * and their clamping are those of fa_fwd_paged; d = dv in {64, 128} for bf16,
 * {32, 64, 128} for fp32.
 * Workspace: fa_bwd_paged_workspace_bytes bytes, 16-byte aligned, holding
 * fa_bwd's workspace plus contiguous copies of each sequence's K, V, dK and dV
 * ([B][Hkv][pages_per_seq * page_size][d] each, in the dtype); it returns 0 for
 * invalid sizes.  The call reads K_pages and V_pages, writes dQ, dK_pages and
 * dV_pages, and owns nothing after it returns.  Errors as fa_bwd and
 * fa_fwd_paged (FA_ERR_BAD_SHAPE for a page size that is not a positive
 * multiple of 128 or an empty pool).
 */
size_t fa_bwd_paged_workspace_bytes(int B, int Hq, int Hkv, int Tq, int pages_per_seq, int page_size, int d,
                                    int dtype);
int fa_bwd_paged(const void* Q, const void* K_pages, const void* V_pages, const void* O, const float* L,
                 const void* dO, void* dQ, void* dK_pages, void* dV_pages, const int* page_table,
                 const int* seqlens_k, int B, int Hq, int Hkv, int Tq, int pages_per_seq, int page_size,
                 int num_pages, int d, int causal, int window, float scale, int dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * Boolean attention mask with grouped-query heads ("The Autograd Memory Trap:
 * Diagnosing a Backward-Pass OOM in Chunked Attention", section "The GQA
 * Expansion Question": a caller's boolean mask together with query heads that
 * share K/V heads, here without repeating K and V).  The backward is
 * fa_bwd_mask below.
 *
 * Layout of the mask: 32-bit words, mask_bits[b * mask_batch_stride + i *
 * fa_mask_row_words(Tk) + j / 32], bit j % 32 set meaning key j is visible to
 * query i, for every query head of batch entry b.  Rows hold
 * fa_mask_row_words(Tk) = 4 * ceil(Tk / 128) words (bits past Tk are ignored).
 * mask_batch_stride (in words) is 0 for one mask shared by the whole batch,
 * else at least Tq * fa_mask_row_words(Tk).  fa_mask_row_words returns -1 for
 * Tk < 0 or Tk above the library's sequence limit.
 *
 * fa_mask_pack converts a byte mask, rows x Tk bytes, row-major, nonzero =
 * visible (a torch.bool tensor's storage), to that layout: rows * row words,
 * written in full (padding bits 0).  mask_bits must be 16-byte aligned;
 * neither buffer is read by the host.  Errors: FA_ERR_BAD_SHAPE for negative
 * sizes, FA_ERR_NULL_PTR / FA_ERR_ALIGNMENT for the buffers, FA_ERR_TOO_LARGE,
 * FA_ERR_HIP.
 *
 * fa_fwd_mask computes fa_fwd_dv's O and L where key j is visible to query i
 * iff its mask bit is set, j < Tk, if causal j <= i + Tk - Tq, and with a
 * window (window > 0) j > i + Tk - Tq - window: the mask narrows the causal
 * bound and the sliding window of fa_fwd_window (the drafter of "The Autograd
 * Memory Trap...", sections "The GQA Expansion Question" and "Assumptions and
 * Uncertainties", has full layers under a block mask and sliding-window
 * layers).  Rows without a
 * visible key get O = 0 and L = -inf.  Head dims as fa_fwd_dv: d = dv in
 * {32, 64, 128}, and (d, dv) = (128, 64) or (64, 128);
 * V and O are dv wide.  The mask must be 16-byte aligned (it may be NULL only
 * when Tq * fa_mask_row_words(Tk) == 0).  Errors as fa_fwd_dv, plus
 * FA_ERR_BAD_SHAPE for a mask_batch_stride that is negative or between 0 and
 * Tq * fa_mask_row_words(Tk), FA_ERR_ALIGNMENT for one that is not a multiple
 * of 4.  With a nonzero stride the mask holds B such entries.
 */
int fa_mask_row_words(int Tk);
int fa_mask_pack(const void* mask_bytes, uint32_t* mask_bits, long long rows, int Tk, void* stream);
int fa_fwd_mask(const void* Q, const void* K, const void* V, void* O, float* L, const uint32_t* mask_bits,
                long long mask_batch_stride, int B, int Hq, int Hkv, int Tq, int Tk, int d, int dv, int causal,
                int window, float scale, int dtype, void* stream);

/*
 * fa_fwd_mask with the keys split over slices and merged as in fa_fwd_splitk
 * ("The Autograd Memory Trap...", section "The Scene": blocks of few new
 * positions against a long prefix, here under a mask).  nsplit == 1 is
 * fa_fwd_mask (no workspace); nsplit <= 0 picks the count; otherwise the
 * workspace holds fa_fwd_mask_splitk_workspace_bytes bytes of fp32 partials
 * (dv wide).  Errors as fa_fwd_mask and fa_fwd_splitk; the workspace size
 * function returns 0 for invalid sizes.
 */
size_t fa_fwd_mask_splitk_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dv, int dtype,
                                          int nsplit);
int fa_fwd_mask_splitk(const void* Q, const void* K, const void* V, void* O, float* L, const uint32_t* mask_bits,
                       long long mask_batch_stride, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                       int Tq, int Tk, int d, int dv, int causal, int window, float scale, int dtype, int nsplit,
                       void* stream);

/*
 * The backward under the same mask (bits and stride as for fa_fwd_mask):
 * fa_bwd_dv's dQ, dK, dV where P is 0 on the pairs the mask, the causal bound
 * and the window hide.  O and L must come from fa_fwd_mask with the same
 * mask, causal flag and window.  Head dims as fa_fwd_mask.  The workspace is
 * fa_bwd_mask_workspace_bytes: fa_bwd's plus a key-major copy of the mask
 * (4 * ceil(Tq / 128) words per key and entry) that the call writes before
 * its dK/dV pass.  Errors as fa_bwd_dv, plus the mask errors of fa_fwd_mask.
 * fa_bwd_mask_workspace_bytes returns 0 for invalid sizes.
 */
size_t fa_bwd_mask_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int d, int dtype,
                                   long long mask_batch_stride);
int fa_bwd_mask(const void* Q, const void* K, const void* V, const void* O, const float* L, const void* dO,
                void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, const uint32_t* mask_bits,
                long long mask_batch_stride, int B, int Hq, int Hkv, int Tq, int Tk, int d, int dv, int causal,
                int window, float scale, int dtype, void* stream);

/*
 * A boolean mask over a variable-length batch ("The Autograd Memory Trap...",
 * sections "The Scene" and "The GQA Expansion Question": blocks of new
 * positions with prefixes of their own lengths, under a caller's mask).
 * Layout and offsets as fa_fwd_varlen / fa_bwd_varlen (packed head-major, d =
 * dv, causal alignment and window per sequence).  The mask of sequence b is a
 * [max_seqlen_q][fa_mask_row_words(max_seqlen_k)] array of words at
 * mask_bits + b * mask_seq_stride, indexed by the sequence's own query and key
 * positions (bit j % 32 of word i * row_words + j / 32 for query i, key j of
 * the sequence); rows and bits past the sequence's lengths are ignored.
 * mask_seq_stride is 0 (one mask for every sequence) or at least
 * max_seqlen_q * fa_mask_row_words(max_seqlen_k) and a multiple of 4.  The
 * backward's workspace is fa_bwd_mask_workspace_bytes(B, Hq, Hkv,
 * max_seqlen_q, max_seqlen_k, d, dtype, mask_seq_stride).  The key-split
 * forward is fa_fwd_varlen_splitk.
 * Errors as fa_fwd_varlen / fa_bwd_varlen plus the mask errors of fa_fwd_mask
 * (with max_seqlen_q, max_seqlen_k in place of Tq, Tk).
 */
int fa_fwd_varlen_mask(const void* Q, const void* K, const void* V, void* O, float* L, const uint32_t* mask_bits,
                       long long mask_seq_stride, const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq,
                       int Hkv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal,
                       int window, float scale, int dtype, void* stream);
int fa_bwd_varlen_mask(const void* Q, const void* K, const void* V, const void* O, const float* L, const void* dO,
                       void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                       const uint32_t* mask_bits, long long mask_seq_stride, const int* cu_seqlens_q,
                       const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                       int max_seqlen_k, int d, int causal, int window, float scale, int dtype, void* stream);

/*
 * The variable-length forward with the keys split over slices and merged as
 * in fa_fwd_splitk ("The Autograd Memory Trap", section "The Scene": blocks of
 * few new positions, each against a long prefix of its own length; unsplit,
 * such a batch gives each compute unit a long run of key tiles or nothing).
 * Layout, offsets, causal alignment and window as fa_fwd_varlen (d = dv).
 * mask_bits == NULL: no mask (fa_fwd_varlen's result); otherwise the mask of
 * fa_fwd_varlen_mask, with its mask_seq_stride.  Slice s takes the key tiles
 * s * n .. (s + 1) * n - 1 of the ones a workgroup would visit, with n the
 * longest sequence's tile count over nsplit (rounded up): a short sequence
 * fills the first slices and leaves the others without tiles.  Such a slice
 * gives its rows L_s = -inf, which weighs nothing in the merge.  nsplit == 1 runs the unsplit
 * kernels with no workspace: bit for bit fa_fwd_varlen / fa_fwd_varlen_mask.
 * nsplit <= 0 picks the count as fa_fwd_splitk (fa_fwd_mask_splitk with a
 * mask) would for B sequences of the longest lengths; when the longest key
 * count is 4 or more times the mean (r = max_seqlen_k * B / total_k), its
 * workgroup target grows by sqrt(r), as the few long sequences' slices then
 * set the time.  Otherwise the workspace
 * (device memory, 16-byte aligned, at least
 * fa_fwd_varlen_splitk_workspace_bytes for the same arguments) holds
 * nsplit * Hq * total_q * (d + 1) floats; it carries nothing between calls.
 * The size function's `masked` is 1 for a call with a mask (the automatic
 * count differs).  Errors as fa_fwd_varlen, the mask errors of
 * fa_fwd_varlen_mask when a mask is given, FA_ERR_WORKSPACE and
 * FA_ERR_TOO_LARGE (more than 1024 slices); the size function returns 0 for
 * invalid sizes and when one slice is used.
 */
size_t fa_fwd_varlen_splitk_workspace_bytes(int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                                            int max_seqlen_k, int d, int dtype, int nsplit, int masked);
int fa_fwd_varlen_splitk(const void* Q, const void* K, const void* V, void* O, float* L,
                         const uint32_t* mask_bits, long long mask_seq_stride, const int* cu_seqlens_q,
                         const int* cu_seqlens_k, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                         int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal,
                         int window, float scale, int dtype, int nsplit, void* stream);

/*
 * The backward pass of fa_bwd for callers that cannot allocate memory or pass
 * a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as fa_bwd (bit for bit:
 * the same kernels run), without the workspace: the per-row -D and log2-domain
 * L live in a scratch array of fa_bwd_noalloc_scratch_bytes() bytes (16 MiB)
 * that the library holds in device memory on every GPU it runs on, from load
 * until the process ends.  A call needs 8 bytes per query row with rows padded
 * to a multiple of 64 per head, B * Hq * ceil(Tq / 64) * 64 * 8 bytes, and
 * returns FA_ERR_SCRATCH if that exceeds the scratch (up to 2,097,152 padded
 * rows, e.g. B * Hq = 512 heads of 4096 rows).  Nothing is allocated; the
 * first call on a device looks up that device's scratch address (a HIP symbol
 * lookup, not an allocation) and keeps it.  The work runs on the current
 * device, which must be the stream's.  All calls on one GPU share its scratch
 * and every call rewrites the part it reads before reading it, so nothing has
 * to be cleared between calls; calls that may overlap on one GPU (concurrent
 * streams, host threads) race on it and must be serialised by the caller.
 */
int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const float* L,
                   const void* dO, void* dQ, void* dK, void* dV,
                   int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
                   int dtype, void* stream);
/* Bytes of fa_bwd_noalloc's per-device scratch array. */
size_t fa_bwd_noalloc_scratch_bytes(void);

/* Static English text for a status code (never NULL). */
const char* fa_status_string(int status);

/* Text of the HIP error behind the calling thread's most recent FA_ERR_HIP
 * (static storage, never NULL; "no HIP error" before any).  Diagnostic only. */
const char* fa_hip_error_string(void);

/* Library ABI version: (major << 16) | minor. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA05_FA_H */
