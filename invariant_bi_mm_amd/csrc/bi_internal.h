// Internal launcher interface between the host API (api.cpp) and the HIP
// translation units. Arguments arrive here already validated.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace bi {

struct GemmConfig {
  int tile_m, tile_n, tile_k, waves;
};

// Tile configuration for (m, n, k, layout): a pure function of those four.
// Every configuration computes each element with the same chain, so the
// choice never changes a bit (see gemm.hip).
GemmConfig gemm_config(int64_t m, int64_t n, int64_t k, bool b_is_nk);
// The configuration of the fixed-tile mode (BI_GEMM_FIXED_TILE): a function
// of (n, k, layout) only, the same for every m.
GemmConfig gemm_config_fixed(int64_t n, int64_t k, bool b_is_nk);

// The launches one GEMM call makes: up to two, each a configuration applied
// to the output columns [n_begin, n_end).
struct GemmLaunch {
  GemmConfig cfg;
  int64_t n_begin, n_end;
};
struct GemmPlan {
  int count;
  GemmLaunch launch[2];
};
GemmPlan gemm_plan(int64_t m, int64_t n, int64_t k, bool b_is_nk, bool fixed_tile);

struct GemmParams {
  const void* a;
  const void* b;
  void* c;
  const void* bias;  // nullptr for mm
  int64_t lda, ldb, ldc;
  int64_t m, n, k;
  float alpha, beta;
  bool b_is_nk;
  bool c_bf16;
  bool bias_bf16;
  bool fixed_tile;  // BI_GEMM_FIXED_TILE
};
hipError_t launch_gemm(const GemmParams& p, hipStream_t stream);

hipError_t launch_rmsnorm(const void* x, int64_t ldx, const void* w, float eps, void* y,
                          int64_t ldy, bool y_bf16, int64_t m, int64_t n, hipStream_t stream);
hipError_t launch_add_rmsnorm(void* x, int64_t ldx, const void* d, int64_t ldd, const void* w, float eps, void* y,
                              int64_t ldy, bool y_bf16, int64_t m, int64_t n, hipStream_t stream);
hipError_t launch_mean(const void* x, bool x_bf16, int64_t ldx, float* y, int64_t m, int64_t n,
                       hipStream_t stream);
hipError_t launch_log_softmax(const float* x, int64_t ldx, float* y, int64_t ldy, int64_t* argmax,
                              int64_t m, int64_t n, hipStream_t stream);

struct DecodeParams {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const int32_t* context_lens;
  const int32_t* split_offsets;
  int64_t max_pages;
  int64_t total_splits;
  int64_t batch;
  int num_q_heads, num_kv_heads;
  float scale;
  float* ws_o;   // [total_splits, num_q_heads, 128]
  float* ws_ml;  // [total_splits, num_q_heads, 2]
  void* out;
  bool out_bf16;
  bool stream_kv;  // K/V loaded non-temporal
};
hipError_t launch_decode_attention(const DecodeParams& p, hipStream_t stream);
// The no-allocation entry point's scratch (decode_attention.hip): its size,
// and its device address on the device `stream` runs on, which must be the
// current device (hipErrorInvalidDevice otherwise). Looked up once per
// device, on first use.
size_t decode_scratch_bytes();
hipError_t decode_scratch(hipStream_t stream, void** ptr);

struct PrefillParams {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const int32_t* q_pos;
  const int32_t* q_offsets;
  const int32_t* work;
  int64_t max_pages;
  int64_t n_work, n_rows, total_splits, batch;
  int num_q_heads, num_kv_heads;
  float scale;
  float* ws_o;
  float* ws_ml;
  void* out;
  bool out_bf16;
};
hipError_t launch_prefill_attention(const PrefillParams& p, hipStream_t stream);
// Query rows per prefill work item (the kernel's block of rows sharing one split's K/V).
int prefill_rows_per_item();

hipError_t launch_embed(const void* table, int64_t ld, int64_t vocab, const int64_t* tokens, void* out, int64_t ldo,
                        int64_t m, int64_t n, hipStream_t stream);
hipError_t launch_silu_mul(const void* gu, int64_t ldg, void* out, int64_t ldo, int64_t m, int64_t n,
                           hipStream_t stream);

struct RopeParams {
  const void* qkv;
  int64_t ldqkv;
  const void* q_norm_w;
  const void* k_norm_w;
  float eps;
  const float* cos_tab;
  const float* sin_tab;
  int64_t max_pos;
  const int32_t* positions;
  const int32_t* block_table;
  int64_t max_pages, num_pages;
  void* k_pages;
  void* v_pages;
  void* q_out;
  int64_t batch;
  int num_q_heads, num_kv_heads, page_size;
};
hipError_t launch_qknorm_rope_append(const RopeParams& p, hipStream_t stream);

}  // namespace bi
