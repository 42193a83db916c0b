// Host-side check of the C ABI under AddressSanitizer and UndefinedBehavior-
// Sanitizer (test infrastructure, built and run by tests/test_abi_sanitized.py).
//
// Links the library's host code -- argument validation and dispatch
// (api.cpp), the GEMM tile table (gemm_plan.cpp) -- with stub launchers in
// place of the HIP kernels, and drives every entry point through refused
// arguments, empty calls, calls that would launch (the stub records the
// launch and reports "no device") and the host plans with exact-size host
// buffers, so an out-of-bounds write or undefined arithmetic in the host code
// stops the run. No GPU is used.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "bi.h"
#include "bi_internal.h"

namespace bi {
static int g_launches = 0;
static GemmParams g_gemm{};
hipError_t launch_gemm(const GemmParams& p, hipStream_t) {
  ++g_launches;
  g_gemm = p;
  return hipErrorNoDevice;
}
hipError_t launch_rmsnorm(const void*, int64_t, const void*, float, void*, int64_t, bool, int64_t, int64_t,
                          hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_add_rmsnorm(void*, int64_t, const void*, int64_t, const void*, float, void*, int64_t, bool, int64_t,
                              int64_t, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_mean(const void*, bool, int64_t, float*, int64_t, int64_t, hipStream_t) {
  ++g_launches;
  return hipErrorNoDevice;
}
hipError_t launch_log_softmax(const float*, int64_t, float*, int64_t, int64_t*, int64_t, int64_t, hipStream_t) {
  ++g_launches;
  return hipErrorNoDevice;
}
hipError_t launch_decode_attention(const DecodeParams&, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
size_t decode_scratch_bytes() { return BI_DECODE_NOALLOC_MAX_BYTES; }
hipError_t decode_scratch(hipStream_t, void**) { return hipErrorNoDevice; }
hipError_t launch_prefill_attention(const PrefillParams&, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
int prefill_rows_per_item() { return 128; }
hipError_t launch_embed(const void*, int64_t, int64_t, const int64_t*, void*, int64_t, int64_t, int64_t,
                        hipStream_t) { ++g_launches; return hipErrorNoDevice; }
hipError_t launch_silu_mul(const void*, int64_t, void*, int64_t, int64_t, int64_t, hipStream_t) {
  ++g_launches;
  return hipErrorNoDevice;
}
hipError_t launch_qknorm_rope_append(const RopeParams&, hipStream_t) { ++g_launches; return hipErrorNoDevice; }
}  // namespace bi

static int g_fail = 0;
#define CHECK(cond)                                                                     \
  do {                                                                                  \
    if (!(cond)) {                                                                      \
      std::fprintf(stderr, "FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond,        \
                   bi_last_error_message());                                            \
      ++g_fail;                                                                         \
    }                                                                                   \
  } while (0)

static void* A(uintptr_t v) { return reinterpret_cast<void*>(v); }  // fake device address, never dereferenced

int main() {
  const uintptr_t D = 0x10000;  // 16-byte aligned
  // ---- GEMM: refused, empty, and launching calls
  CHECK(bi_mm(A(D), 512, A(D), 512, 0, A(D), 512, BI_F32, -1, 512, 512, nullptr) == BI_ERR_SHAPE);
  CHECK(bi_mm(A(D), 512, A(D), 512, 0, nullptr, 512, BI_F32, 4, 512, 512, nullptr) == BI_ERR_NULL);
  CHECK(bi_mm(A(D + 2), 512, A(D), 512, 0, A(D), 512, BI_F32, 4, 512, 512, nullptr) == BI_ERR_ALIGN);
  CHECK(bi_mm(A(D), 100, A(D), 512, 0, A(D), 512, BI_F32, 4, 512, 512, nullptr) == BI_ERR_STRIDE);
  CHECK(bi_mm(A(D), 512, A(D), 512, 0, A(D), 512, (bi_dtype)7, 4, 512, 512, nullptr) == BI_ERR_DTYPE);
  CHECK(bi_mm(A(D), 512, A(D), 512, 0, A(D), 512, BI_F32, 0, 512, 512, nullptr) == BI_OK);
  CHECK(bi_gemm(nullptr, BI_F32, 0.f, 1.f, A(D), 512, A(D), 512, 0, A(D), 512, BI_F32, 4, 512, 512, 8, nullptr) ==
        BI_ERR_UNSUPPORTED);
  CHECK(bi::g_launches == 0);
  CHECK(bi_mm(A(D), 4096, A(D), 6144, 0, A(D), 6144, BI_F32, 4096, 6144, 4096, nullptr) == BI_ERR_HIP);
  CHECK(bi::g_launches == 1 && bi::g_gemm.m == 4096 && !bi::g_gemm.fixed_tile);
  CHECK(bi_gemm(A(D), BI_BF16, 1.f, 1.f, A(D), 4096, A(D), 4096, 1, A(D), 151936, BI_F32, 256, 151936, 4096,
                BI_GEMM_FIXED_TILE, nullptr) == BI_ERR_HIP);
  CHECK(bi::g_launches == 2 && bi::g_gemm.fixed_tile && bi::g_gemm.bias != nullptr);
  // the tile table over a grid of shapes: plans cover [0, n) in order
  for (int64_t n : {8, 512, 4096, 6136, 6144, 24576, 151936})
    for (int64_t k : {8, 512, 4096, 12288})
      for (int64_t m = 1; m <= 4096; m += (m < 300 ? 1 : 37))
        for (int nk = 0; nk < 2; ++nk)
          for (int flags = 0; flags < 2; ++flags) {
            int32_t out10[10];
            int32_t cnt = -1;
            CHECK(bi_gemm_plan(m, n, k, nk, flags, out10, &cnt) == BI_OK);
            CHECK(cnt == 1 || cnt == 2);
            CHECK(out10[4] == 0);
            if (cnt == 2) CHECK(out10[9] > 0 && out10[9] < n && out10[9] % 256 == 0);
            int32_t c4[4];
            CHECK(bi_gemm_config(m, n, k, nk, c4) == BI_OK);
          }
  // ---- row reductions
  CHECK(bi_rmsnorm(A(D), 4096, A(D), 1e-6f, A(D), 4096, BI_BF16, 5, 0, nullptr) == BI_ERR_SHAPE);
  CHECK(bi_mean(A(D), BI_BF16, 4096, static_cast<float*>(A(D)), 5, 0, nullptr) == BI_ERR_SHAPE);
  CHECK(bi_log_softmax(static_cast<const float*>(A(D)), 1003, static_cast<float*>(A(D)), 1004, nullptr, 2, 1003,
                       nullptr) == BI_ERR_ALIGN);
  CHECK(bi_log_softmax(static_cast<const float*>(A(D)), 1004, static_cast<float*>(A(D)), 1004,
                       static_cast<int64_t*>(A(D + 4)), 2, 1003, nullptr) == BI_ERR_ALIGN);
  CHECK(bi_log_softmax(static_cast<const float*>(A(D)), 151936, static_cast<float*>(A(D)), 151936, nullptr, 7,
                       151936, nullptr) == BI_ERR_HIP);
  // ---- decode plan with exact-size host buffers (ASan bounds)
  std::mt19937 rng(1);
  for (int trial = 0; trial < 200; ++trial) {
    const int64_t batch = rng() % 300;
    std::vector<int32_t> lens(batch);
    for (auto& L : lens) L = 1 + (int32_t)(std::exp(std::uniform_real_distribution<double>(0, std::log(32769.0))(rng))) % 32768;
    int32_t* offs = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (batch + 1)));
    const int64_t total = bi_decode_plan(lens.data(), batch, 256, offs);
    CHECK(total >= batch);
    CHECK(offs[batch] == total);
    std::free(offs);
  }
  {
    int32_t bad[2] = {5, 0};
    int32_t offs[3];
    CHECK(bi_decode_plan(bad, 2, 256, offs) == -1);
    CHECK(bi_decode_plan(bad, 2, 256, nullptr) == -1);
  }
  CHECK(bi_decode_workspace_bytes(-1, 32, 128) == 0);
  // decode attention: refused before the scratch lookup or any launch
  const int before = bi::g_launches;
  CHECK(bi_decode_attention_noalloc(A(D), A(D), A(D), (const int32_t*)A(D), 2048, (const int32_t*)A(D),
                                    (const int32_t*)A(D), 4096, 32, 32, 8, 128, 16, 256, 0.088f, A(D), BI_F32, 0,
                                    nullptr) == BI_ERR_WORKSPACE);
  CHECK(bi_decode_attention(A(D), A(D), A(D), (const int32_t*)A(D), 4, (const int32_t*)A(D), (const int32_t*)A(D), 2,
                            2, 32, 8, 64, 16, 256, 0.1f, A(D), 1 << 20, A(D), BI_F32, 0, nullptr) ==
        BI_ERR_UNSUPPORTED);
  CHECK(bi_decode_attention(A(D), A(D), A(D), (const int32_t*)A(D), 4, (const int32_t*)A(D), (const int32_t*)A(D), 2,
                            2, 32, 8, 128, 16, 256, 0.1f, A(D), 16, A(D), BI_F32, 0, nullptr) == BI_ERR_WORKSPACE);
  CHECK(bi::g_launches == before);
  CHECK(bi_decode_attention_noalloc(A(D), A(D), A(D), (const int32_t*)A(D), 4, (const int32_t*)A(D),
                                    (const int32_t*)A(D), 2, 2, 32, 8, 128, 16, 256, 0.1f, A(D), BI_F32, 0,
                                    nullptr) == BI_ERR_HIP);  // the stub scratch lookup fails
  CHECK(bi::g_launches == before);
  // ---- prefill plan: sizes, then exact-size buffers
  for (int trial = 0; trial < 100; ++trial) {
    const int64_t batch = 1 + rng() % 6;
    std::vector<int32_t> cl(batch), cb(batch);
    for (int64_t b = 0; b < batch; ++b) {
      cl[b] = rng() % 1500;
      cb[b] = rng() % 3000;
    }
    int64_t sizes[3];
    CHECK(bi_prefill_plan(cl.data(), cb.data(), batch, 256, nullptr, nullptr, nullptr, sizes) == BI_OK);
    int32_t* pos = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (sizes[0] ? sizes[0] : 1)));
    int32_t* qo = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (sizes[0] + 1)));
    int32_t* wk = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * 4 * (sizes[2] ? sizes[2] : 1)));
    int64_t sizes2[3];
    CHECK(bi_prefill_plan(cl.data(), cb.data(), batch, 256, pos, qo, wk, sizes2) == BI_OK);
    CHECK(std::memcmp(sizes, sizes2, sizeof sizes) == 0);
    CHECK(qo[sizes[0]] == sizes[1]);
    std::free(pos);
    std::free(qo);
    std::free(wk);
  }
  // ---- per-token kernels
  CHECK(bi_embed(A(D), 4096, 1000, (const int64_t*)A(D), A(D), 4096, 3, 4100, nullptr) != BI_OK);
  CHECK(bi_silu_mul(A(D), 24576, A(D), 12288, 3, 12288, nullptr) == BI_ERR_HIP);
  // ---- status strings
  for (int s = -3; s < 20; ++s) CHECK(bi_status_string((bi_status)s) != nullptr);
  CHECK(bi_last_error_message() != nullptr);
  std::printf("abi host check: %d launches recorded, %d failures\n", bi::g_launches, g_fail);
  return g_fail ? 1 : 0;
}
