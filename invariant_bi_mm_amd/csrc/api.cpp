// C-ABI entry points (include/bi.h): argument validation, then dispatch to
// the HIP launchers. Every check runs on the host before any HIP call, so a
// rejected call has launched nothing. No exceptions cross this boundary.
#include "bi.h"

#include <climits>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <string>

#include <algorithm>

#include "bi_internal.h"

namespace {

thread_local std::string g_last_error;

bi_status fail(bi_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bi_status ok() {
  g_last_error.clear();
  return BI_OK;
}

bi_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BI_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool valid_dtype(bi_dtype d) { return d == BI_BF16 || d == BI_F32; }
size_t dsize(bi_dtype d) { return d == BI_BF16 ? 2 : 4; }

bi_status check_gemm(const void* a, int64_t lda, const void* b, int64_t ldb, int b_is_nk, void* c,
                     int64_t ldc, bi_dtype c_dtype, int64_t m, int64_t n, int64_t k, int flags = 0) {
  if (flags & ~BI_GEMM_FIXED_TILE) return fail(BI_ERR_UNSUPPORTED, "unknown GEMM flags 0x%x", flags);
  if (m < 0 || n < 0 || k < 0) return fail(BI_ERR_SHAPE, "negative size (m=%lld n=%lld k=%lld)", (long long)m, (long long)n, (long long)k);
  if (!valid_dtype(c_dtype)) return fail(BI_ERR_DTYPE, "c_dtype %d is not BI_BF16 or BI_F32", (int)c_dtype);
  if (m == 0 || n == 0) return BI_OK;
  if (c == nullptr) return fail(BI_ERR_NULL, "c is NULL");
  if (k > 0 && (a == nullptr || b == nullptr)) return fail(BI_ERR_NULL, "a or b is NULL");
  if (m > INT_MAX || n > INT_MAX || k > INT_MAX) return fail(BI_ERR_UNSUPPORTED, "a size exceeds 2^31-1");
  if (lda < k || ldc < n || ldb < (b_is_nk ? k : n))
    return fail(BI_ERR_STRIDE, "leading dimension smaller than its row (lda=%lld ldb=%lld ldc=%lld)",
                (long long)lda, (long long)ldb, (long long)ldc);
  if (k % 8 != 0) return fail(BI_ERR_UNSUPPORTED, "k=%lld is not a multiple of 8", (long long)k);
  if (!b_is_nk && n % 8 != 0)
    return fail(BI_ERR_UNSUPPORTED, "n=%lld is not a multiple of 8 (B stored [k, n])", (long long)n);
  if (k > 0 && (!aligned(a, 16) || !aligned(b, 16) || lda % 8 != 0 || ldb % 8 != 0))
    return fail(BI_ERR_ALIGN, "a/b must be 16-byte aligned with lda, ldb multiples of 8");
  if (!aligned(c, dsize(c_dtype))) return fail(BI_ERR_ALIGN, "c is not aligned to its element size");
  const bi::GemmPlan plan = bi::gemm_plan(m, n, k, b_is_nk != 0, (flags & BI_GEMM_FIXED_TILE) != 0);
  for (int i = 0; i < plan.count; ++i) {
    const bi::GemmLaunch& L = plan.launch[i];
    const int64_t tiles = ((m + L.cfg.tile_m - 1) / L.cfg.tile_m) * ((L.n_end - L.n_begin + L.cfg.tile_n - 1) / L.cfg.tile_n);
    if (tiles > INT_MAX) return fail(BI_ERR_UNSUPPORTED, "too many output tiles");
  }
  // the kernels address one tile's rows of A and B through 32-bit buffer
  // descriptors: a tile's byte extent must stay below 2^31. Checked for the
  // largest tile of any configuration (256 rows of A; 384 rows of B stored
  // [n, k], 64 k-rows stored [k, n]), so whether a call is accepted does not
  // depend on m.
  const int64_t lim = int64_t(1) << 31;
  if (2 * 256 * lda >= lim || 2 * (b_is_nk ? 384 : 64) * ldb >= lim)
    return fail(BI_ERR_UNSUPPORTED, "leading dimension too large for one tile's 32-bit byte range");
  return BI_OK;
}

bi_status run_gemm(const void* bias, bi_dtype bias_dtype, float beta, float alpha, const void* a, int64_t lda,
                   const void* b, int64_t ldb, int b_is_nk, void* c, int64_t ldc, bi_dtype c_dtype, int64_t m,
                   int64_t n, int64_t k, hipStream_t stream, int flags = 0) {
  bi::GemmParams p;
  p.a = a;
  p.b = b;
  p.c = c;
  p.bias = bias;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.m = m;
  p.n = n;
  p.k = k;
  p.alpha = alpha;
  p.beta = beta;
  p.b_is_nk = b_is_nk != 0;
  p.c_bf16 = c_dtype == BI_BF16;
  p.bias_bf16 = bias_dtype == BI_BF16;
  p.fixed_tile = (flags & BI_GEMM_FIXED_TILE) != 0;
  return hip_status(bi::launch_gemm(p, stream), "gemm launch");
}

}  // namespace

extern "C" {

bi_status bi_mm(const void* a, int64_t lda, const void* b, int64_t ldb, int b_is_nk, void* c, int64_t ldc,
                bi_dtype c_dtype, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  bi_status st = check_gemm(a, lda, b, ldb, b_is_nk, c, ldc, c_dtype, m, n, k);
  if (st != BI_OK) return st;
  if (m == 0 || n == 0) return ok();
  return run_gemm(nullptr, BI_F32, 0.0f, 1.0f, a, lda, b, ldb, b_is_nk, c, ldc, c_dtype, m, n, k, stream);
}

bi_status bi_addmm(const void* bias, bi_dtype bias_dtype, float beta, float alpha, const void* a, int64_t lda,
                   const void* b, int64_t ldb, int b_is_nk, void* c, int64_t ldc, bi_dtype c_dtype, int64_t m,
                   int64_t n, int64_t k, hipStream_t stream) {
  if (!valid_dtype(bias_dtype)) return fail(BI_ERR_DTYPE, "bias_dtype %d is not BI_BF16 or BI_F32", (int)bias_dtype);
  bi_status st = check_gemm(a, lda, b, ldb, b_is_nk, c, ldc, c_dtype, m, n, k);
  if (st != BI_OK) return st;
  if (m == 0 || n == 0) return ok();
  if (bias == nullptr) return fail(BI_ERR_NULL, "bias is NULL");
  if (!aligned(bias, dsize(bias_dtype))) return fail(BI_ERR_ALIGN, "bias is not aligned to its element size");
  return run_gemm(bias, bias_dtype, beta, alpha, a, lda, b, ldb, b_is_nk, c, ldc, c_dtype, m, n, k, stream);
}

bi_status bi_gemm(const void* bias, bi_dtype bias_dtype, float beta, float alpha, const void* a, int64_t lda,
                  const void* b, int64_t ldb, int b_is_nk, void* c, int64_t ldc, bi_dtype c_dtype, int64_t m,
                  int64_t n, int64_t k, int flags, hipStream_t stream) {
  if (bias != nullptr && !valid_dtype(bias_dtype))
    return fail(BI_ERR_DTYPE, "bias_dtype %d is not BI_BF16 or BI_F32", (int)bias_dtype);
  bi_status st = check_gemm(a, lda, b, ldb, b_is_nk, c, ldc, c_dtype, m, n, k, flags);
  if (st != BI_OK) return st;
  if (m == 0 || n == 0) return ok();
  if (bias != nullptr && !aligned(bias, dsize(bias_dtype)))
    return fail(BI_ERR_ALIGN, "bias is not aligned to its element size");
  if (bias == nullptr) {  // mm: C = alpha * (A @ B)
    bias_dtype = BI_F32;
    beta = 0.0f;
  }
  return run_gemm(bias, bias_dtype, beta, alpha, a, lda, b, ldb, b_is_nk, c, ldc, c_dtype, m, n, k, stream, flags);
}

bi_status bi_gemm_plan(int64_t m, int64_t n, int64_t k, int b_is_nk, int flags, int32_t* out10, int32_t* count) {
  if (out10 == nullptr || count == nullptr) return fail(BI_ERR_NULL, "out10 or count is NULL");
  if (m < 0 || n < 0 || k < 0) return fail(BI_ERR_SHAPE, "negative size");
  if (flags & ~BI_GEMM_FIXED_TILE) return fail(BI_ERR_UNSUPPORTED, "unknown GEMM flags 0x%x", flags);
  const bi::GemmPlan plan = bi::gemm_plan(m, n, k, b_is_nk != 0, (flags & BI_GEMM_FIXED_TILE) != 0);
  *count = plan.count;
  for (int i = 0; i < 2; ++i) {
    const bi::GemmLaunch& L = plan.launch[i];
    const bool used = i < plan.count;
    out10[5 * i + 0] = used ? L.cfg.tile_m : 0;
    out10[5 * i + 1] = used ? L.cfg.tile_n : 0;
    out10[5 * i + 2] = used ? L.cfg.tile_k : 0;
    out10[5 * i + 3] = used ? L.cfg.waves : 0;
    out10[5 * i + 4] = used ? (int32_t)L.n_begin : 0;
  }
  return ok();
}

bi_status bi_gemm_config(int64_t m, int64_t n, int64_t k, int b_is_nk, int32_t* out4) {
  if (out4 == nullptr) return fail(BI_ERR_NULL, "out4 is NULL");
  if (m < 0 || n < 0 || k < 0) return fail(BI_ERR_SHAPE, "negative size");
  const bi::GemmConfig c = bi::gemm_config(m, n, k, b_is_nk != 0);
  out4[0] = c.tile_m;
  out4[1] = c.tile_n;
  out4[2] = c.tile_k;
  out4[3] = c.waves;
  return ok();
}

bi_status bi_rmsnorm(const void* x, int64_t ldx, const void* w, float eps, void* y, int64_t ldy, bi_dtype y_dtype,
                     int64_t m, int64_t n, hipStream_t stream) {
  if (m < 0 || n < 0) return fail(BI_ERR_SHAPE, "negative size");
  if (!valid_dtype(y_dtype)) return fail(BI_ERR_DTYPE, "y_dtype %d is not BI_BF16 or BI_F32", (int)y_dtype);
  if (m == 0) return ok();
  if (n == 0) return fail(BI_ERR_SHAPE, "n == 0: RMSNorm of an empty row is undefined");
  if (x == nullptr || w == nullptr || y == nullptr) return fail(BI_ERR_NULL, "x, w or y is NULL");
  if (m > INT_MAX || n > INT_MAX) return fail(BI_ERR_UNSUPPORTED, "a size exceeds 2^31-1");
  if (ldx < n || ldy < n) return fail(BI_ERR_STRIDE, "ldx/ldy smaller than n");
  const int64_t yq = y_dtype == BI_BF16 ? 8 : 4;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || ldx % 8 != 0 || ldy % yq != 0)
    return fail(BI_ERR_ALIGN, "x, w, y must be 16-byte aligned; ldx a multiple of 8, ldy of %lld", (long long)yq);
  return hip_status(bi::launch_rmsnorm(x, ldx, w, eps, y, ldy, y_dtype == BI_BF16, m, n, stream), "rmsnorm launch");
}

bi_status bi_mean(const void* x, bi_dtype x_dtype, int64_t ldx, float* y, int64_t m, int64_t n,
                  hipStream_t stream) {
  if (m < 0 || n < 0) return fail(BI_ERR_SHAPE, "negative size");
  if (!valid_dtype(x_dtype)) return fail(BI_ERR_DTYPE, "x_dtype %d is not BI_BF16 or BI_F32", (int)x_dtype);
  if (m == 0) return ok();
  if (n == 0) return fail(BI_ERR_SHAPE, "n == 0: the mean of an empty row is undefined");
  if (x == nullptr || y == nullptr) return fail(BI_ERR_NULL, "x or y is NULL");
  if (m > INT_MAX || n > INT_MAX) return fail(BI_ERR_UNSUPPORTED, "a size exceeds 2^31-1");
  if (ldx < n) return fail(BI_ERR_STRIDE, "ldx smaller than n");
  const int64_t xq = x_dtype == BI_BF16 ? 8 : 4;
  if (!aligned(x, 16) || ldx % xq != 0 || !aligned(y, 4))
    return fail(BI_ERR_ALIGN, "x must be 16-byte aligned with ldx a multiple of %lld; y 4-byte aligned",
                (long long)xq);
  return hip_status(bi::launch_mean(x, x_dtype == BI_BF16, ldx, y, m, n, stream), "mean launch");
}

bi_status bi_log_softmax(const float* x, int64_t ldx, float* y, int64_t ldy, int64_t* argmax, int64_t m, int64_t n,
                         hipStream_t stream) {
  if (m < 0 || n < 0) return fail(BI_ERR_SHAPE, "negative size");
  if (m == 0) return ok();
  if (n == 0) return fail(BI_ERR_SHAPE, "n == 0: log_softmax of an empty row is undefined");
  if (x == nullptr || y == nullptr) return fail(BI_ERR_NULL, "x or y is NULL");
  if (m > INT_MAX || n > INT_MAX / 4) return fail(BI_ERR_UNSUPPORTED, "a size exceeds the supported range");
  if (ldx < n || ldy < n) return fail(BI_ERR_STRIDE, "ldx/ldy smaller than n");
  if (!aligned(x, 16) || !aligned(y, 16) || ldx % 4 != 0 || ldy % 4 != 0 || !aligned(argmax, 8))
    return fail(BI_ERR_ALIGN, "x, y must be 16-byte aligned with ldx, ldy multiples of 4; argmax 8-byte aligned");
  return hip_status(bi::launch_log_softmax(x, ldx, y, ldy, argmax, m, n, stream), "log_softmax launch");
}

int64_t bi_decode_plan(const int32_t* host_context_lens, int64_t batch, int split_tokens,
                       int32_t* host_split_offsets) {
  if (batch < 0 || split_tokens <= 0) {
    fail(BI_ERR_SHAPE, "batch < 0 or split_tokens <= 0");
    return -1;
  }
  if (host_split_offsets == nullptr || (batch > 0 && host_context_lens == nullptr)) {
    fail(BI_ERR_NULL, "NULL host pointer");
    return -1;
  }
  int64_t total = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t L = host_context_lens[b];
    if (L < 1) {
      fail(BI_ERR_SHAPE, "context_lens[%lld] = %lld < 1", (long long)b, (long long)L);
      return -1;
    }
    host_split_offsets[b] = (int32_t)total;
    total += (L + split_tokens - 1) / split_tokens;
    if (total > INT_MAX) {
      fail(BI_ERR_UNSUPPORTED, "total split count exceeds 2^31-1");
      return -1;
    }
  }
  host_split_offsets[batch] = (int32_t)total;
  ok();
  return total;
}

size_t bi_decode_workspace_bytes(int64_t total_splits, int num_q_heads, int head_dim) {
  if (total_splits < 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return (size_t)total_splits * (size_t)num_q_heads * (size_t)(head_dim + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// Validation and launch shared by bi_decode_attention (caller's workspace)
// and bi_decode_attention_noalloc (the library's scratch, scratch == true:
// workspace and workspace_bytes unused).
bi_status decode_attention_impl(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                                int64_t max_pages, const int32_t* context_lens, const int32_t* split_offsets,
                                int64_t total_splits, int64_t batch, int num_q_heads, int num_kv_heads, int head_dim,
                                int page_size, int split_tokens, float scale, void* workspace, size_t workspace_bytes,
                                void* out, bi_dtype out_dtype, int flags, hipStream_t stream, bool scratch) {
  if (batch < 0 || total_splits < 0 || max_pages < 0) return fail(BI_ERR_SHAPE, "negative size");
  if ((flags & ~BI_DECODE_STREAM_KV) != 0) return fail(BI_ERR_UNSUPPORTED, "unknown flags 0x%x", (unsigned)flags);
  if (!valid_dtype(out_dtype)) return fail(BI_ERR_DTYPE, "out_dtype %d is not BI_BF16 or BI_F32", (int)out_dtype);
  if (head_dim != 128 || page_size != 16 || split_tokens != 256 || num_kv_heads < 1 ||
      num_q_heads != 4 * num_kv_heads)
    return fail(BI_ERR_UNSUPPORTED,
                "supported: head_dim 128, page_size 16, split_tokens 256, num_q_heads = 4 * num_kv_heads "
                "(got %d, %d, %d, %d/%d)",
                head_dim, page_size, split_tokens, num_q_heads, num_kv_heads);
  if (batch == 0) return ok();
  if (q == nullptr || k_pages == nullptr || v_pages == nullptr || block_table == nullptr ||
      context_lens == nullptr || split_offsets == nullptr || out == nullptr)
    return fail(BI_ERR_NULL, "a required pointer is NULL");
  if (max_pages < 1) return fail(BI_ERR_SHAPE, "max_pages must be >= 1");
  const int64_t max_splits_per_seq = (max_pages * page_size + split_tokens - 1) / split_tokens;
  if (total_splits < batch || total_splits > batch * max_splits_per_seq)
    return fail(BI_ERR_SHAPE, "total_splits=%lld inconsistent with batch=%lld and max_pages=%lld",
                (long long)total_splits, (long long)batch, (long long)max_pages);
  // each launch's work items (workgroups x threads) must fit in 32 bits
  if (batch > INT_MAX || num_kv_heads > 65535 || num_q_heads > 65535 ||
      total_splits * num_kv_heads * 256 > (int64_t)UINT32_MAX || batch * num_q_heads * 128 > (int64_t)UINT32_MAX)
    return fail(BI_ERR_UNSUPPORTED, "grid size out of range");
  const size_t need = bi_decode_workspace_bytes(total_splits, num_q_heads, head_dim);
  if (scratch && need > bi::decode_scratch_bytes())
    return fail(BI_ERR_WORKSPACE,
                "the no-allocation entry point's scratch holds %zu bytes; %lld splits of %d heads need %zu "
                "(use bi_decode_attention with a workspace)",
                bi::decode_scratch_bytes(), (long long)total_splits, num_q_heads, need);
  if (!scratch && (workspace == nullptr || workspace_bytes < need))
    return fail(BI_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || (!scratch && !aligned(workspace, 16)) ||
      !aligned(out, dsize(out_dtype)) || !aligned(block_table, 4) || !aligned(context_lens, 4) ||
      !aligned(split_offsets, 4))
    return fail(BI_ERR_ALIGN, "q, k_pages, v_pages, workspace must be 16-byte aligned");
  if (scratch) {
    // every argument is valid: now the scratch of the device the stream runs on
    const hipError_t e = bi::decode_scratch(stream, &workspace);
    if (e == hipErrorInvalidDevice)
      return fail(BI_ERR_UNSUPPORTED, "the stream is not on the current device (the scratch is looked up there)");
    if (e != hipSuccess) return hip_status(e, "scratch lookup");
  }
  bi::DecodeParams p;
  p.q = q;
  p.k_pages = k_pages;
  p.v_pages = v_pages;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.split_offsets = split_offsets;
  p.max_pages = max_pages;
  p.total_splits = total_splits;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.scale = scale;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.ws_o + total_splits * num_q_heads * head_dim;
  p.out = out;
  p.out_bf16 = out_dtype == BI_BF16;
  p.stream_kv = (flags & BI_DECODE_STREAM_KV) != 0;
  return hip_status(bi::launch_decode_attention(p, stream), "decode attention launch");
}

}  // namespace

extern "C" {

bi_status bi_decode_attention(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                              int64_t max_pages, const int32_t* context_lens, const int32_t* split_offsets,
                              int64_t total_splits, int64_t batch, int num_q_heads, int num_kv_heads, int head_dim,
                              int page_size, int split_tokens, float scale, void* workspace, size_t workspace_bytes,
                              void* out, bi_dtype out_dtype, int flags, hipStream_t stream) {
  return decode_attention_impl(q, k_pages, v_pages, block_table, max_pages, context_lens, split_offsets, total_splits,
                               batch, num_q_heads, num_kv_heads, head_dim, page_size, split_tokens, scale, workspace,
                               workspace_bytes, out, out_dtype, flags, stream, false);
}

bi_status bi_decode_attention_noalloc(const void* q, const void* k_pages, const void* v_pages,
                                      const int32_t* block_table, int64_t max_pages, const int32_t* context_lens,
                                      const int32_t* split_offsets, int64_t total_splits, int64_t batch,
                                      int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                                      int split_tokens, float scale, void* out, bi_dtype out_dtype, int flags,
                                      hipStream_t stream) {
  return decode_attention_impl(q, k_pages, v_pages, block_table, max_pages, context_lens, split_offsets, total_splits,
                               batch, num_q_heads, num_kv_heads, head_dim, page_size, split_tokens, scale, nullptr, 0,
                               out, out_dtype, flags, stream, true);
}

bi_status bi_prefill_plan(const int32_t* host_chunk_lens, const int32_t* host_ctx_before, int64_t batch,
                          int split_tokens, int32_t* host_q_pos, int32_t* host_q_offsets, int32_t* host_work,
                          int64_t* out_sizes) {
  if (batch < 0 || split_tokens <= 0) return fail(BI_ERR_SHAPE, "batch < 0 or split_tokens <= 0");
  if (out_sizes == nullptr) return fail(BI_ERR_NULL, "out_sizes is NULL");
  if (batch > 0 && (host_chunk_lens == nullptr || host_ctx_before == nullptr))
    return fail(BI_ERR_NULL, "chunk_lens or ctx_before is NULL");
  const bool fill = host_q_pos != nullptr || host_q_offsets != nullptr || host_work != nullptr;
  if (fill && (host_q_pos == nullptr || host_q_offsets == nullptr || host_work == nullptr))
    return fail(BI_ERR_NULL, "q_pos, q_offsets and work must all be given (or all NULL for the sizes)");
  const int64_t qb = bi::prefill_rows_per_item();
  int64_t rows = 0, splits = 0, items = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t n = host_chunk_lens[b], c0 = host_ctx_before[b];
    if (n < 0 || c0 < 0) return fail(BI_ERR_SHAPE, "chunk_lens[%lld] or ctx_before[%lld] < 0", (long long)b, (long long)b);
    if (c0 + n > INT_MAX) return fail(BI_ERR_UNSUPPORTED, "a position exceeds 2^31-1");
    if (n == 0) continue;
    // rows of this sequence, their positions and split offsets
    for (int64_t i = 0; i < n; ++i) {
      if (fill) {
        host_q_pos[rows + i] = (int32_t)(c0 + i);
        host_q_offsets[rows + i] = (int32_t)splits;
      }
      splits += (c0 + i + split_tokens) / split_tokens;  // ceil((pos + 1) / split_tokens)
      if (splits > INT_MAX) return fail(BI_ERR_UNSUPPORTED, "total split count exceeds 2^31-1");
    }
    // work items: split-major, so the blocks sharing a split's K/V run together
    const int64_t blocks = (n + qb - 1) / qb;
    const int64_t max_split = (c0 + n - 1) / split_tokens;
    for (int64_t sp = 0; sp <= max_split; ++sp) {
      for (int64_t k = 0; k < blocks; ++k) {
        const int64_t r0 = k * qb, nr = std::min(qb, n - r0);
        const int64_t last = c0 + r0 + nr - 1;  // position of the block's last row
        if (last < sp * split_tokens) continue;   // no row of the block sees this split
        if (fill) {
          host_work[4 * items + 0] = (int32_t)(rows + r0);
          host_work[4 * items + 1] = (int32_t)nr;
          host_work[4 * items + 2] = (int32_t)b;
          host_work[4 * items + 3] = (int32_t)sp;
        }
        ++items;
      }
    }
    rows += n;
    if (rows > INT_MAX || items > INT_MAX) return fail(BI_ERR_UNSUPPORTED, "too many rows or work items");
  }
  if (fill) host_q_offsets[rows] = (int32_t)splits;
  out_sizes[0] = rows;
  out_sizes[1] = splits;
  out_sizes[2] = items;
  return ok();
}

bi_status bi_prefill_attention(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                               int64_t max_pages, const int32_t* q_pos, const int32_t* q_offsets, const int32_t* work,
                               int64_t n_work, int64_t n_rows, int64_t total_splits, int64_t batch, int num_q_heads,
                               int num_kv_heads, int head_dim, int page_size, int split_tokens, float scale,
                               void* workspace, size_t workspace_bytes, void* out, bi_dtype out_dtype,
                               hipStream_t stream) {
  if (n_rows < 0 || n_work < 0 || total_splits < 0 || batch < 0 || max_pages < 0)
    return fail(BI_ERR_SHAPE, "negative size");
  if (!valid_dtype(out_dtype)) return fail(BI_ERR_DTYPE, "out_dtype %d is not BI_BF16 or BI_F32", (int)out_dtype);
  if (head_dim != 128 || page_size != 16 || split_tokens != 256 || num_kv_heads < 1 ||
      num_q_heads != 4 * num_kv_heads)
    return fail(BI_ERR_UNSUPPORTED,
                "supported: head_dim 128, page_size 16, split_tokens 256, num_q_heads = 4 * num_kv_heads "
                "(got %d, %d, %d, %d/%d)",
                head_dim, page_size, split_tokens, num_q_heads, num_kv_heads);
  if (n_rows == 0) return ok();
  if (q == nullptr || k_pages == nullptr || v_pages == nullptr || block_table == nullptr || q_pos == nullptr ||
      q_offsets == nullptr || work == nullptr || out == nullptr)
    return fail(BI_ERR_NULL, "a required pointer is NULL");
  if (max_pages < 1 || batch < 1 || n_work < 1) return fail(BI_ERR_SHAPE, "max_pages, batch and n_work must be >= 1");
  if (total_splits < n_rows) return fail(BI_ERR_SHAPE, "total_splits < n_rows (every row has at least one split)");
  // each launch's work items (workgroups x threads) must fit in 32 bits
  if (n_rows > INT_MAX || batch > INT_MAX || total_splits > INT_MAX || num_q_heads > 65535 ||
      n_work * num_kv_heads * 256 > (int64_t)UINT32_MAX || n_rows * (num_q_heads / 4) * 256 > (int64_t)UINT32_MAX)
    return fail(BI_ERR_UNSUPPORTED, "grid size out of range");
  const size_t need = bi_decode_workspace_bytes(total_splits, num_q_heads, head_dim);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(BI_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(workspace, 16) ||
      !aligned(out, dsize(out_dtype)) || !aligned(block_table, 4) || !aligned(q_pos, 4) || !aligned(q_offsets, 4) ||
      !aligned(work, 4))
    return fail(BI_ERR_ALIGN, "q, k_pages, v_pages, workspace must be 16-byte aligned");
  bi::PrefillParams p;
  p.q = q;
  p.k_pages = k_pages;
  p.v_pages = v_pages;
  p.block_table = block_table;
  p.q_pos = q_pos;
  p.q_offsets = q_offsets;
  p.work = work;
  p.max_pages = max_pages;
  p.n_work = n_work;
  p.n_rows = n_rows;
  p.batch = batch;
  p.total_splits = total_splits;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.scale = scale;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_ml = p.ws_o + total_splits * num_q_heads * head_dim;
  p.out = out;
  p.out_bf16 = out_dtype == BI_BF16;
  return hip_status(bi::launch_prefill_attention(p, stream), "prefill attention launch");
}

bi_status bi_add_rmsnorm(void* x, int64_t ldx, const void* d, int64_t ldd, const void* w, float eps, void* y,
                         int64_t ldy, bi_dtype y_dtype, int64_t m, int64_t n, hipStream_t stream) {
  if (m < 0 || n < 0) return fail(BI_ERR_SHAPE, "negative size");
  if (!valid_dtype(y_dtype)) return fail(BI_ERR_DTYPE, "y_dtype %d is not BI_BF16 or BI_F32", (int)y_dtype);
  if (m == 0) return ok();
  if (n == 0) return fail(BI_ERR_SHAPE, "n == 0: RMSNorm of an empty row is undefined");
  if (x == nullptr || d == nullptr || w == nullptr || y == nullptr) return fail(BI_ERR_NULL, "x, d, w or y is NULL");
  if (m > INT_MAX || n > INT_MAX) return fail(BI_ERR_UNSUPPORTED, "a size exceeds 2^31-1");
  if (ldx < n || ldd < n || ldy < n) return fail(BI_ERR_STRIDE, "ldx/ldd/ldy smaller than n");
  const int64_t yq = y_dtype == BI_BF16 ? 8 : 4;
  if (!aligned(x, 16) || !aligned(d, 16) || !aligned(w, 16) || !aligned(y, 16) || ldx % 8 != 0 || ldd % 8 != 0 ||
      ldy % yq != 0)
    return fail(BI_ERR_ALIGN, "x, d, w, y must be 16-byte aligned; ldx, ldd multiples of 8, ldy of %lld",
                (long long)yq);
  return hip_status(bi::launch_add_rmsnorm(x, ldx, d, ldd, w, eps, y, ldy, y_dtype == BI_BF16, m, n, stream),
                    "add_rmsnorm launch");
}

bi_status bi_embed(const void* table, int64_t ld, int64_t vocab, const int64_t* tokens, void* out, int64_t ldo,
                   int64_t m, int64_t n, hipStream_t stream) {
  if (m < 0 || n < 0 || vocab < 0) return fail(BI_ERR_SHAPE, "negative size");
  if (m == 0 || n == 0) return ok();
  if (table == nullptr || tokens == nullptr || out == nullptr) return fail(BI_ERR_NULL, "table, tokens or out is NULL");
  if (vocab == 0) return fail(BI_ERR_SHAPE, "empty table");
  if (m > INT_MAX || n > INT_MAX) return fail(BI_ERR_UNSUPPORTED, "a size exceeds 2^31-1");
  if (ld < n || ldo < n) return fail(BI_ERR_STRIDE, "ld/ldo smaller than n");
  if (n % 8 != 0 || ld % 8 != 0 || ldo % 8 != 0 || !aligned(table, 16) || !aligned(out, 16) || !aligned(tokens, 8))
    return fail(BI_ERR_ALIGN, "table, out 16-byte aligned with n, ld, ldo multiples of 8; tokens 8-byte aligned");
  return hip_status(bi::launch_embed(table, ld, vocab, tokens, out, ldo, m, n, stream), "embed launch");
}

bi_status bi_silu_mul(const void* gu, int64_t ldg, void* out, int64_t ldo, int64_t m, int64_t n, hipStream_t stream) {
  if (m < 0 || n < 0) return fail(BI_ERR_SHAPE, "negative size");
  if (m == 0 || n == 0) return ok();
  if (gu == nullptr || out == nullptr) return fail(BI_ERR_NULL, "gu or out is NULL");
  if (m > 65535 || n > INT_MAX / 2) return fail(BI_ERR_UNSUPPORTED, "m > 65535 or n too large");
  if (ldg < 2 * n || ldo < n) return fail(BI_ERR_STRIDE, "ldg < 2n or ldo < n");
  if (n % 8 != 0 || ldg % 8 != 0 || ldo % 8 != 0 || !aligned(gu, 16) || !aligned(out, 16))
    return fail(BI_ERR_ALIGN, "gu, out 16-byte aligned with n, ldg, ldo multiples of 8");
  return hip_status(bi::launch_silu_mul(gu, ldg, out, ldo, m, n, stream), "silu_mul launch");
}

bi_status bi_qknorm_rope_append(const void* qkv, int64_t ldqkv, const void* q_norm_w, const void* k_norm_w, float eps,
                                const float* cos_tab, const float* sin_tab, int64_t max_pos, const int32_t* positions,
                                const int32_t* block_table, int64_t max_pages, int64_t num_pages, void* k_pages,
                                void* v_pages, void* q_out, int64_t batch, int num_q_heads, int num_kv_heads,
                                int head_dim, int page_size, hipStream_t stream) {
  if (batch < 0 || max_pos < 0 || max_pages < 0 || num_pages < 0) return fail(BI_ERR_SHAPE, "negative size");
  if (head_dim != 128 || page_size < 1 || num_q_heads < 1 || num_kv_heads < 1)
    return fail(BI_ERR_UNSUPPORTED, "supported: head_dim 128, page_size >= 1, at least one q and kv head (got %d, %d, %d/%d)",
                head_dim, page_size, num_q_heads, num_kv_heads);
  if (batch == 0) return ok();
  if (qkv == nullptr || q_norm_w == nullptr || k_norm_w == nullptr || cos_tab == nullptr || sin_tab == nullptr ||
      positions == nullptr || block_table == nullptr || k_pages == nullptr || v_pages == nullptr || q_out == nullptr)
    return fail(BI_ERR_NULL, "a required pointer is NULL");
  if (max_pos < 1 || max_pages < 1 || num_pages < 1) return fail(BI_ERR_SHAPE, "max_pos, max_pages, num_pages must be >= 1");
  const int64_t width = (int64_t)(num_q_heads + 2 * num_kv_heads) * head_dim;
  if (ldqkv < width) return fail(BI_ERR_STRIDE, "ldqkv < (num_q_heads + 2 num_kv_heads) * head_dim");
  if (batch > INT_MAX || num_q_heads + 2 * num_kv_heads > 65535) return fail(BI_ERR_UNSUPPORTED, "grid size out of range");
  if (!aligned(qkv, 2) || !aligned(q_norm_w, 2) || !aligned(k_norm_w, 2) || !aligned(cos_tab, 4) ||
      !aligned(sin_tab, 4) || !aligned(positions, 4) || !aligned(block_table, 4) || !aligned(k_pages, 2) ||
      !aligned(v_pages, 2) || !aligned(q_out, 2))
    return fail(BI_ERR_ALIGN, "a pointer is not aligned to its element size");
  bi::RopeParams p;
  p.qkv = qkv;
  p.ldqkv = ldqkv;
  p.q_norm_w = q_norm_w;
  p.k_norm_w = k_norm_w;
  p.eps = eps;
  p.cos_tab = cos_tab;
  p.sin_tab = sin_tab;
  p.max_pos = max_pos;
  p.positions = positions;
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  p.k_pages = k_pages;
  p.v_pages = v_pages;
  p.q_out = q_out;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.page_size = page_size;
  return hip_status(bi::launch_qknorm_rope_append(p, stream), "qknorm_rope_append launch");
}

const char* bi_status_string(bi_status s) {
  switch (s) {
    case BI_OK: return "BI_OK";
    case BI_ERR_NULL: return "BI_ERR_NULL: a required pointer is NULL";
    case BI_ERR_SHAPE: return "BI_ERR_SHAPE: invalid or inconsistent sizes";
    case BI_ERR_STRIDE: return "BI_ERR_STRIDE: leading dimension smaller than the row";
    case BI_ERR_ALIGN: return "BI_ERR_ALIGN: pointer or leading dimension misaligned";
    case BI_ERR_DTYPE: return "BI_ERR_DTYPE: dtype not accepted";
    case BI_ERR_WORKSPACE: return "BI_ERR_WORKSPACE: workspace missing or too small";
    case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED: outside the supported set";
    case BI_ERR_HIP: return "BI_ERR_HIP: HIP runtime error";
  }
  return "unknown bi_status";
}

const char* bi_last_error_message(void) { return g_last_error.c_str(); }

}  // extern "C"
