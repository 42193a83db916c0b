/*
 * bi.h -- batch-invariant inference kernels for AMD Instinct MI355X (gfx950).
 *
 * A batch-invariant kernel gives each output row the same bits whatever the
 * batch size M, whatever the other rows hold, and on every run: the
 * floating-point reduction behind each output element runs in one fixed
 * order that depends only on the shape of the row (N, K, head_dim, the
 * sequence's own length), never on M or on the batch composition.
 *
 * The operations are those the pages name:
 *   - mm, addmm, log_softmax, mean: the ops listed as supported by
 *     "thinking-machines-lab/batch_invariant_ops" (catalogue page, section
 *     "When to avoid"), which replaces standard PyTorch kernels ("What it
 *     is"), so each op keeps PyTorch's semantics;
 *   - RMSNorm and attention: named with matmul as the inference kernels whose
 *     output depends on batch size (readhandoff.com, agent-run
 *     reproducibility pinning, section "What does temperature zero actually
 *     guarantee?", and its "Frequently asked questions");
 *   - greedy argmax: the temperature-0 sampler picks the highest-probability
 *     token (same section).
 * The mechanism, fixing the reduction order, is the "TL;DR" of "How to
 * achieve deterministic LLMs with batch invariant inference". The pages give
 * no signatures; the ones below are this library's own.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller. The
 *    library never allocates, frees, copies or synchronises device memory.
 *    Host pointers appear only in bi_decode_plan().
 *  - Row-major storage; ld* is the row stride in ELEMENTS (>= row length).
 *  - bf16 is IEEE-style bfloat16 (the upper half of an fp32); bf16 outputs
 *    are rounded to nearest, ties to even, once, from the fp32 result.
 *  - Every call first validates all of its arguments on the host; on any
 *    error it returns a non-zero bi_status and launches nothing, so an error
 *    never leaves partial work. It never aborts and never throws.
 *  - On success the work is enqueued on `stream` and the call returns before
 *    the GPU finishes (stream-ordered, like any HIP launch). A HIP launch
 *    error is returned as BI_ERR_HIP; the text is in bi_last_error_message().
 *  - m == 0 (or batch == 0) is a valid no-op: BI_OK, nothing launched.
 *  - Alignment: base pointers 16-byte aligned, ld* a multiple of 8 for bf16
 *    and of 4 for fp32 operands (128-bit loads); otherwise BI_ERR_ALIGN.
 *  - Outputs must not overlap inputs (undefined behaviour, not checked).
 *  - Calls are re-entrant and may be issued from several host threads; error
 *    messages are thread-local. The only state the library keeps is the
 *    scratch of bi_decode_attention_noalloc (one per GPU, see there).
 */
#ifndef BI_H_
#define BI_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BI_OK = 0,
  BI_ERR_NULL = 1,        /* a required pointer is NULL                       */
  BI_ERR_SHAPE = 2,       /* a size is negative, or sizes disagree            */
  BI_ERR_STRIDE = 3,      /* a leading dimension is smaller than its row      */
  BI_ERR_ALIGN = 4,       /* pointer or leading dimension misaligned          */
  BI_ERR_DTYPE = 5,       /* dtype code not accepted by this argument         */
  BI_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required          */
  BI_ERR_UNSUPPORTED = 7, /* valid but outside the supported set (see calls)  */
  BI_ERR_HIP = 8          /* the HIP runtime reported an error                */
} bi_status;

typedef enum { BI_BF16 = 0, BI_F32 = 1 } bi_dtype;

/* ------------------------------------------------------------------------
 * bi_mm: C[m,n] = A[m,k] @ B, bf16 inputs, fp32 accumulation.
 *   (mm, "thinking-machines-lab/batch_invariant_ops", "When to avoid")
 *   a       bf16 [m, k], row stride lda.
 *   b       bf16; b_is_nk == 0: B is [k, n] (row stride ldb, torch.mm's mat2);
 *           b_is_nk != 0: B is stored [n, k] (row stride ldb, the nn.Linear
 *           weight layout) and C = A @ B^T.
 *   c       [m, n], row stride ldc, dtype c_dtype (BI_F32 or BI_BF16).
 * Reduction order: for every C element, k runs in increasing order in
 * 16-wide MFMA steps (v_mfma_f32_32x32x16_bf16, k padded with zeros to a
 * multiple of 64), accumulated in fp32 from 0, one chain per element; no
 * split-K, stream-K or atomics. The tile configuration depends on
 * (m, n, k, b_is_nk) (bi_gemm_config reports it), but every configuration
 * runs that same chain with the same operands, so a row of C has the same
 * bits whatever m is and wherever the row sits.
 * Requirements: k % 8 == 0; with b_is_nk == 0 also n % 8 == 0;
 * 256 * lda * 2 and (b_is_nk ? 384 : 64) * ldb * 2 below 2^31 bytes (the
 * largest tile's byte range; BI_ERR_UNSUPPORTED otherwise).
 * k == 0 with m, n > 0: C = beta * bias (addmm) or zeros (mm).
 * ------------------------------------------------------------------------ */
bi_status bi_mm(const void* a, int64_t lda, const void* b, int64_t ldb, int b_is_nk,
                void* c, int64_t ldc, bi_dtype c_dtype,
                int64_t m, int64_t n, int64_t k, hipStream_t stream);

/* ------------------------------------------------------------------------
 * bi_addmm: C = beta * bias + alpha * (A @ B), bias [n] broadcast over rows
 * (torch.addmm with a 1-D input; addmm, same page and section as bi_mm).
 *   bias    [n], dtype bias_dtype (BI_BF16 or BI_F32), contiguous.
 * The bias is applied once, after the whole K reduction, in fp32:
 * t = alpha * acc; t = t + beta * bias[j]; then the single rounding to
 * c_dtype. All other arguments and requirements as bi_mm.
 * ------------------------------------------------------------------------ */
bi_status bi_addmm(const void* bias, bi_dtype bias_dtype, float beta, float alpha,
                   const void* a, int64_t lda, const void* b, int64_t ldb, int b_is_nk,
                   void* c, int64_t ldc, bi_dtype c_dtype,
                   int64_t m, int64_t n, int64_t k, hipStream_t stream);

/* Tile configuration the GEMM uses for (m, n, k, b_is_nk): writes
 * {tile_m, tile_n, tile_k, waves_per_workgroup} to out4. One of
 * {32, 32, 64, 3} and {64, 32, 64, 4} (m <= 64: 32-column strips, a deep
 * load ring), {32, 96, 64, 5} and {64, 96, 64, 8} (m <= 64, 96-column strips
 * where those fill the CUs in one round), {64, 128, 64, 6} and {128, 128, 64, 10} (the same ring with a
 * 64x128 or 128x128 tile), {128, 128, 64, 4}, {256, 256, 64, 8},
 * {256, 384, 64, 8} (only where k % 64 == 0, n % 384 == 0 and its tiles
 * make whole rounds over the 256 CUs). This is the tile table's entry;
 * bi_gemm_plan reports the launches: with {256, 256, 64, 8}, when the last
 * round of tiles over the 256 CUs would be part-empty, either the columns
 * past the last full round run as 256x128 tiles in a second launch, or
 * (wide N, e.g. the LM head) the first columns run as 256x384 tiles in
 * whole rounds and the rest as 256x256 tiles, whichever takes fewer rounds. The
 * choice changes which workgroup computes an element, never how (see
 * bi_mm). Returns BI_ERR_NULL
 * if out4 is NULL, BI_ERR_SHAPE for negative sizes. */
bi_status bi_gemm_config(int64_t m, int64_t n, int64_t k, int b_is_nk, int32_t* out4);

/* ------------------------------------------------------------------------
 * bi_gemm: bi_mm and bi_addmm with flags. bias == NULL gives
 * C = alpha * (A @ B) (bias_dtype and beta unused); otherwise as bi_addmm.
 * flags: 0 (the tile table of bi_gemm_config, chosen by m, n, k and the
 * layout), or BI_GEMM_FIXED_TILE: one tile configuration per (n, k, layout)
 * for every m, and no column split, i.e. no shape-aware tiling at all, which
 * the pages list among the optimisations batch invariance gives up (wiki
 * page "Thinking Machines", section on why it is not the main answer, point
 * 3). Both modes run the same per-element chain, so they give the same
 * bits; the fixed mode is there to measure what the table gains.
 * Other flag bits: BI_ERR_UNSUPPORTED. Requirements as bi_mm.
 * ------------------------------------------------------------------------ */
#define BI_GEMM_FIXED_TILE 1
bi_status bi_gemm(const void* bias, bi_dtype bias_dtype, float beta, float alpha,
                  const void* a, int64_t lda, const void* b, int64_t ldb, int b_is_nk,
                  void* c, int64_t ldc, bi_dtype c_dtype,
                  int64_t m, int64_t n, int64_t k, int flags, hipStream_t stream);

/* The launches a GEMM of these sizes makes with these flags (no device
 * work): *count (1 or 2) entries of five int32 each in out10,
 * {tile_m, tile_n, tile_k, waves_per_workgroup, first output column}; two
 * entries when a 256x256 GEMM is split over its columns (256x256 then
 * 256x128, or 256x384 then 256x256; see bi_gemm_config). Unused entries
 * are zero. BI_ERR_NULL for NULL out10 or count,
 * BI_ERR_SHAPE for negative sizes, BI_ERR_UNSUPPORTED for unknown flags. */
bi_status bi_gemm_plan(int64_t m, int64_t n, int64_t k, int b_is_nk, int flags, int32_t* out10, int32_t* count);

/* ------------------------------------------------------------------------
 * bi_rmsnorm: y[i,j] = (x[i,j] * r_i) * w[j], r_i = 1 / sqrt(ss_i / n + eps),
 * ss_i = sum_j x[i,j]^2 (RMSNorm; readhandoff.com "What does temperature
 * zero actually guarantee?").
 *   x  bf16 [m, n], row stride ldx.     w  bf16 [n], contiguous.
 *   y  [m, n], row stride ldy, dtype y_dtype (BI_BF16 or BI_F32).
 * One workgroup per row; ss_i is an fp32 sum in an order fixed by n alone.
 * ------------------------------------------------------------------------ */
bi_status bi_rmsnorm(const void* x, int64_t ldx, const void* w, float eps,
                     void* y, int64_t ldy, bi_dtype y_dtype,
                     int64_t m, int64_t n, hipStream_t stream);

/* ------------------------------------------------------------------------
 * bi_mean: y[i] = (sum_j x[i,j]) / n, fp32 sum in an order fixed by n
 * (mean, "thinking-machines-lab/batch_invariant_ops", "When to avoid").
 *   x  [m, n], dtype x_dtype (BI_BF16 or BI_F32), row stride ldx.
 *   y  fp32 [m].
 * n == 0 with m > 0 is BI_ERR_SHAPE (the mean of nothing is undefined).
 * ------------------------------------------------------------------------ */
bi_status bi_mean(const void* x, bi_dtype x_dtype, int64_t ldx, float* y,
                  int64_t m, int64_t n, hipStream_t stream);

/* ------------------------------------------------------------------------
 * bi_log_softmax: y[i,j] = (x[i,j] - mx_i) - log(s_i), mx_i = max_j x[i,j],
 * s_i = sum_j exp(x[i,j] - mx_i) (log_softmax, same page and section as
 * bi_mean), plus the greedy choice argmax[i] = the lowest j with
 * x[i,j] == mx_i (the temperature-0 sampler, readhandoff.com "What does
 * temperature zero actually guarantee?").
 *   x  fp32 [m, n], row stride ldx.   y  fp32 [m, n], row stride ldy.
 *   argmax  int64 [m], or NULL to skip it.
 * n must be > 0 (BI_ERR_SHAPE). The argmax is taken over the fp32 input
 * logits, not over the rounded log-probabilities.
 * ------------------------------------------------------------------------ */
bi_status bi_log_softmax(const float* x, int64_t ldx, float* y, int64_t ldy,
                         int64_t* argmax, int64_t m, int64_t n, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode attention over a paged KV cache, split-KV with a fixed split SIZE.
 * (Attention is named as batch-dependent in readhandoff.com "What does
 * temperature zero actually guarantee?"; batch-invariant attention kernels
 * and the cost of the attention kernel are in "Batch-invariant inference
 * kernels (Thinking Machines) -- Evidence & limits", sections "Evidence" and
 * "Limitations".)
 *
 * For sequence b with L_b cached tokens and query head h (kv head
 * g = h / (num_q_heads / num_kv_heads)):
 *   out[b,h,:] = sum_t softmax_t(scale * q[b,h,:] . K[b,g,t,:]) V[b,g,t,:].
 * The tokens of each sequence are cut at multiples of split_tokens of the
 * sequence's own token index, so the split count ceil(L_b / split_tokens)
 * depends on L_b only, never on the batch. Each split reduces its tokens in
 * a fixed order to (m, l, o) partials; a second kernel merges the partials
 * of each (b, h) in increasing split order. A sequence's output therefore has
 * the same bits in any batch.
 * ------------------------------------------------------------------------ */

/* Host-side plan: split_offsets[b] = sum_{b'<b} ceil(L_b' / split_tokens),
 * split_offsets[batch] = total. host_context_lens and host_split_offsets
 * ([batch + 1]) are HOST pointers. Returns the total split count, or -1 on
 * invalid input (NULL pointer, batch < 0, split_tokens <= 0, a length < 1);
 * the message is in bi_last_error_message(). */
int64_t bi_decode_plan(const int32_t* host_context_lens, int64_t batch, int split_tokens,
                       int32_t* host_split_offsets);

/* Bytes of device workspace bi_decode_attention needs for total_splits
 * splits: total_splits * num_q_heads * (head_dim + 2) * 4 (fp32 partials
 * o[head_dim], m, l per split and query head). Returns 0 for invalid sizes. */
size_t bi_decode_workspace_bytes(int64_t total_splits, int num_q_heads, int head_dim);

/* bi_decode_attention
 *   q             bf16 [batch, num_q_heads, head_dim], contiguous.
 *   k_pages       bf16 [num_pages, num_kv_heads, page_size, head_dim],
 *                 contiguous (a key is a contiguous row).
 *   v_pages       bf16 [num_pages, num_kv_heads, head_dim, page_size],
 *                 contiguous (d-major: one head-dim element of a page's
 *                 tokens is a contiguous row, so a value tile of 8 tokens
 *                 is one 16-byte load). Token t of sequence b is in
 *                 physical page block_table[b * max_pages + t / page_size],
 *                 slot t % page_size, of both. Slots past a sequence's
 *                 length may hold any bits (never used).
 *   block_table   int32 [batch, max_pages], contiguous.
 *   context_lens  int32 [batch], each >= 1 and <= max_pages * page_size.
 *   split_offsets int32 [batch + 1] on the DEVICE, as written by
 *                 bi_decode_plan for the same lengths and split_tokens.
 *   total_splits  split_offsets[batch], or any upper bound of it: the
 *                 kernels read the exact count from split_offsets[batch] on
 *                 the device, and workgroups past it exit at once. One
 *                 captured launch can so serve steps whose lengths grow.
 *                 The workspace must hold total_splits splits.
 *   scale         multiplier of q . k (normally 1 / sqrt(head_dim)).
 *   workspace     device buffer of at least bi_decode_workspace_bytes().
 *   out           [batch, num_q_heads, head_dim], contiguous, out_dtype.
 * Supported set (BI_ERR_UNSUPPORTED otherwise): head_dim == 128,
 * page_size == 16, split_tokens == 256, num_q_heads == 4 * num_kv_heads,
 * num_kv_heads >= 1. Device-side contents (lengths, table entries, offsets)
 * are the caller's responsibility: the host cannot read them without a
 * synchronisation, which this call never performs.
 *   flags         0, or BI_DECODE_STREAM_KV: load K and V non-temporal, a
 *                 cache hint only (the results are the same bits). Measured
 *                 on MI355X it makes this call alone 1-5 % slower but a
 *                 decode step whose other kernels keep their cache lines
 *                 ~3 % faster. Any other bit: BI_ERR_UNSUPPORTED.
 */
#define BI_DECODE_STREAM_KV 1
bi_status bi_decode_attention(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, int64_t max_pages,
                              const int32_t* context_lens, const int32_t* split_offsets,
                              int64_t total_splits, int64_t batch,
                              int num_q_heads, int num_kv_heads, int head_dim,
                              int page_size, int split_tokens, float scale,
                              void* workspace, size_t workspace_bytes,
                              void* out, bi_dtype out_dtype, int flags, hipStream_t stream);

/* bi_decode_attention_noalloc: bi_decode_attention without the workspace
 * argument, for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation. The split partials go to a scratch array the library holds in
 * device memory (BI_DECODE_NOALLOC_MAX_BYTES per GPU it runs on, reserved
 * when the library's code is loaded on that GPU and kept until the process
 * ends). The call allocates nothing; the caller passes inputs and outputs
 * as for bi_decode_attention, with the same requirements, and gets the same
 * bits (same kernels).
 * Limit: bi_decode_workspace_bytes(total_splits, num_q_heads, head_dim)
 * must not exceed BI_DECODE_NOALLOC_MAX_BYTES (64 MiB: 4032 splits of 256
 * tokens at 32 query heads, ~1M cached tokens per call); larger calls return
 * BI_ERR_WORKSPACE and launch nothing.
 * All calls on one GPU share the scratch: calls that overlap in time on one
 * GPU (different streams, or host threads) race and give undefined results;
 * calls in one stream are ordered and safe. The stream must belong to the
 * current device (BI_ERR_UNSUPPORTED otherwise). The first call on a device
 * looks the scratch's address up (hipGetSymbolAddress); a failure there is
 * BI_ERR_HIP. */
#define BI_DECODE_NOALLOC_MAX_BYTES ((size_t)64 << 20)
bi_status bi_decode_attention_noalloc(const void* q, const void* k_pages, const void* v_pages,
                                      const int32_t* block_table, int64_t max_pages,
                                      const int32_t* context_lens, const int32_t* split_offsets,
                                      int64_t total_splits, int64_t batch,
                                      int num_q_heads, int num_kv_heads, int head_dim,
                                      int page_size, int split_tokens, float scale,
                                      void* out, bi_dtype out_dtype, int flags, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Prefill / extend attention with the decode split structure.
 *
 * A chunk of new tokens per sequence (already appended to the cache)
 * attends causally: the token at position p sees tokens 0..p of its
 * sequence. Its reduction is cut at the same multiples of split_tokens as a
 * decode step with p + 1 cached tokens, each split is reduced with the very
 * arithmetic of bi_decode_attention's split kernel, and the partials are
 * merged with its combine's arithmetic, term for term. So a token's output
 * has the same bits whether it is
 * prefilled in any chunking, in any batch, or decoded -- the chunked-prefill
 * side of the batch dependence the pages trace to attention (readhandoff.com,
 * agent-run reproducibility pinning, "What does temperature zero actually
 * guarantee?"; "Batch-invariant inference kernels (Thinking Machines) --
 * Evidence & limits", "Evidence" and "Limitations").
 * ------------------------------------------------------------------------ */

/* Host-side plan. Query rows are the chunk tokens of sequence 0, then of
 * sequence 1, ...: sequence b contributes host_chunk_lens[b] rows at
 * positions host_ctx_before[b], host_ctx_before[b] + 1, ... (HOST arrays
 * [batch]). Call once with host_q_pos, host_q_offsets and host_work all NULL
 * to get out_sizes[3] = {rows, total_splits, n_work}; then again with
 *   host_q_pos      int32 [rows]       each row's position,
 *   host_q_offsets  int32 [rows + 1]   split offsets: sum over earlier rows
 *                                      of ceil((pos + 1) / split_tokens),
 *   host_work       int32 [4 n_work]   work items (first row, row count <= 128,
 *                                      sequence, split), split-major per
 *                                      sequence.
 * Returns BI_OK or an error status (the message in bi_last_error_message). */
bi_status bi_prefill_plan(const int32_t* host_chunk_lens, const int32_t* host_ctx_before, int64_t batch,
                          int split_tokens, int32_t* host_q_pos, int32_t* host_q_offsets, int32_t* host_work,
                          int64_t* out_sizes);

/* bi_prefill_attention
 *   q            bf16 [rows, num_q_heads, head_dim], contiguous (row order as
 *                in the plan).
 *   k_pages, v_pages, block_table [batch, max_pages]: as bi_decode_attention;
 *                the cache must already hold every chunk token.
 *   q_pos, q_offsets, work: the plan's arrays, on the DEVICE.
 *   n_work, n_rows, total_splits: the plan's sizes.
 *   workspace    >= bi_decode_workspace_bytes(total_splits, num_q_heads,
 *                head_dim) bytes.
 *   out          [rows, num_q_heads, head_dim], out_dtype.
 * Supported set as bi_decode_attention (BI_ERR_UNSUPPORTED otherwise). The
 * cache must hold finite values in the slots the chunk sees. The plan's
 * arrays are read on the device only: a work item whose rows, sequence,
 * split or pages do not fit the buffers, or a split offset past
 * total_splits, is skipped (those rows' values are then unspecified); the
 * kernels never access memory outside the buffers. */
bi_status bi_prefill_attention(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, int64_t max_pages, const int32_t* q_pos,
                               const int32_t* q_offsets, const int32_t* work, int64_t n_work, int64_t n_rows,
                               int64_t total_splits, int64_t batch, int num_q_heads, int num_kv_heads,
                               int head_dim, int page_size, int split_tokens, float scale,
                               void* workspace, size_t workspace_bytes, void* out, bi_dtype out_dtype,
                               hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-token steps of a decode step (Qwen3-style layer). They carry one
 * sequence's greedy token stream from logits back to the next layer input.
 * The pages trace non-reproducible completions to the batch a request lands
 * in, with a long identical prefix and a fork at one token (readhandoff.com,
 * agent-run reproducibility pinning, sections "What does temperature zero
 * actually guarantee?" and "Where the divergence showed up"), and measure the
 * cost on Qwen3-8B decoding (same page, "Key takeaways"). Each output element
 * depends on its own token's inputs only, through a fixed sequence of fp32
 * operations, so none of these can depend on the batch.
 * ------------------------------------------------------------------------ */

/* bi_add_rmsnorm: residual add fused with the RMSNorm that follows it.
 *   x <- RNE_bf16(x + d)      (in place; fp32 add of the two bf16 values)
 *   y  = bi_rmsnorm(x, w, eps) of the updated x, same rules as bi_rmsnorm.
 *   x  bf16 [m, n], row stride ldx (read, then overwritten).
 *   d  bf16 [m, n], row stride ldd.   w  bf16 [n].   y [m, n] y_dtype.
 * x must not overlap d, w or y. */
bi_status bi_add_rmsnorm(void* x, int64_t ldx, const void* d, int64_t ldd, const void* w, float eps,
                         void* y, int64_t ldy, bi_dtype y_dtype,
                         int64_t m, int64_t n, hipStream_t stream);

/* bi_embed: out[i, :] = table[tokens[i], :] (token embedding lookup).
 *   table  bf16 [vocab, n], row stride ld.   tokens int64 [m] (DEVICE).
 *   out    bf16 [m, n], row stride ldo.
 * n, ld, ldo multiples of 8. A token outside [0, vocab) yields a zero row
 * (the kernel never reads outside the table; the host cannot check device
 * contents). */
bi_status bi_embed(const void* table, int64_t ld, int64_t vocab, const int64_t* tokens,
                   void* out, int64_t ldo, int64_t m, int64_t n, hipStream_t stream);

/* bi_silu_mul: out[i, j] = RNE_bf16(silu(g) * u), g = gu[i, j],
 * u = gu[i, n + j], silu(g) = g / (1 + e^-g), all in fp32 (the gated MLP
 * activation; gate and up come from one GEMM with N = 2n).
 *   gu  bf16 [m, 2n], row stride ldg.   out  bf16 [m, n], row stride ldo.
 * n, ldg, ldo multiples of 8; m <= 65535. */
bi_status bi_silu_mul(const void* gu, int64_t ldg, void* out, int64_t ldo,
                      int64_t m, int64_t n, hipStream_t stream);

/* bi_qknorm_rope_append: the attention prologue of one decode token per
 * sequence.
 *   qkv  bf16 [batch, (num_q_heads + 2 num_kv_heads) * head_dim], row stride
 *        ldqkv: the q heads, then the k heads, then the v heads.
 *   For each q and k head: r = 1 / sqrt(mean(x^2) + eps) over the head,
 *   t = (x * r) * w (w = q_norm_w or k_norm_w, bf16 [head_dim]), then the
 *   rotary embedding at position p = positions[b] on the pairs (i, i + 64):
 *     out[i]      = t[i] * cos[p][i] - t[i+64] * sin[p][i]
 *     out[i + 64] = t[i+64] * cos[p][i] + t[i] * sin[p][i],
 *   rounded once to bf16. q heads go to q_out [batch, num_q_heads, head_dim];
 *   k heads, and v heads unchanged, go to slot p % page_size of page
 *   block_table[b * max_pages + p / page_size] of k_pages
 *   ([num_pages, num_kv_heads, page_size, head_dim]) / v_pages
 *   ([num_pages, num_kv_heads, head_dim, page_size]), the bi_decode_attention
 *   layouts. positions[b] is the new token's index, i.e. the sequence's
 *   length before this token.
 *   cos_tab, sin_tab  fp32 [max_pos, head_dim / 2]: the caller's table.
 * Supported: head_dim == 128. A position outside [0, max_pos) or outside the
 * block table, or a table entry outside [0, num_pages), writes no cache slot
 * and zeros to that token's q_out rows. Pointers need only their element
 * alignment. */
bi_status bi_qknorm_rope_append(const void* qkv, int64_t ldqkv, const void* q_norm_w, const void* k_norm_w,
                                float eps, const float* cos_tab, const float* sin_tab, int64_t max_pos,
                                const int32_t* positions, const int32_t* block_table, int64_t max_pages,
                                int64_t num_pages, void* k_pages, void* v_pages, void* q_out,
                                int64_t batch, int num_q_heads, int num_kv_heads, int head_dim,
                                int page_size, hipStream_t stream);

/* Static text for a status code (never NULL). */
const char* bi_status_string(bi_status s);

/* Thread-local detail of the last error raised on the calling thread
 * (empty string if none); includes the hipError_t text for BI_ERR_HIP. */
const char* bi_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* BI_H_ */
