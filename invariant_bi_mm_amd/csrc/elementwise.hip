// Per-token kernels of a decode step that do no cross-token reduction, for
// gfx950: embedding row gather, SiLU(gate) * up, and the Qwen3 attention
// prologue (per-head q/k RMSNorm, rotary embedding, paged KV-cache append).
//
// They complete the token path the pages trace through an engine -- one
// sequence's greedy token stream must not change with the batch around it
// (readhandoff.com, agent-run reproducibility pinning, "Where the divergence
// showed up": completions identical for a long prefix, then forking at one
// token; "Batch-invariant inference kernels (Thinking Machines) -- Evidence &
// limits", section "Evidence"). Each output element
// depends only on its own token's inputs through a fixed sequence of fp32
// operations; the only reduction, the per-head sum of squares in the q/k
// RMSNorm, is a fixed wave butterfly over one head. So none of them can
// depend on the batch.
#include "bi_internal.h"
#include "device_common.h"

namespace bi {
namespace {

// out[i, :] = table[tokens[i], :], n bf16 per row, one wave per row. A token
// outside [0, vocab) gives a zero row (the kernel never reads outside the
// table).
__global__ __launch_bounds__(64) void embed_kernel(const uint16_t* __restrict__ table, int64_t ld, int64_t vocab,
                                                    const int64_t* __restrict__ tokens, uint16_t* __restrict__ out,
                                                    int64_t ldo, int n) {
  const int row = blockIdx.x;
  const int64_t t = tokens[row];
  const bool ok = t >= 0 && t < vocab;
  const u32x4* src = reinterpret_cast<const u32x4*>(table + (ok ? t : 0) * ld);
  u32x4* dst = reinterpret_cast<u32x4*>(out + (int64_t)row * ldo);
  for (int c = threadIdx.x; c < n / 8; c += 64) dst[c] = ok ? src[c] : u32x4{0u, 0u, 0u, 0u};
}

// out[i, j] = RNE_bf16(silu(g) * u), g = gu[i, j], u = gu[i, n + j], all in
// fp32: silu(g) = g / (1 + e^-g). 8 elements per lane.
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ gu, int64_t ldg,
                                                        uint16_t* __restrict__ out, int64_t ldo, int n) {
  const int row = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;  // chunk of 8
  if (c >= n / 8) return;
  const uint16_t* r = gu + (int64_t)row * ldg;
  float g[8], u[8], o[8];
  unpack8(reinterpret_cast<const u32x4*>(r)[c], g);
  unpack8(reinterpret_cast<const u32x4*>(r + n)[c], u);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (g[e] / (1.0f + expf(-g[e]))) * u[e];
  reinterpret_cast<u32x4*>(out + (int64_t)row * ldo)[c] =
      u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
}

constexpr int HD = 128;  // head dim
constexpr int HALF = HD / 2;

struct RopeArgs {
  const uint16_t* qkv;
  int64_t ldqkv;
  const uint16_t* qw;  // q-norm weight [HD]
  const uint16_t* kw;  // k-norm weight [HD]
  float eps;
  const float* cos_t;  // [max_pos, HD/2]
  const float* sin_t;
  int64_t max_pos;
  const int32_t* pos;
  const int32_t* bt;
  int64_t max_pages, num_pages;
  uint16_t* kp;
  uint16_t* vp;
  uint16_t* q_out;
  int hq, hkv, page;
};

// One wave per (token, head); lane l owns the rotary pair (l, l + 64).
//   q and k heads: r = 1/sqrt(mean(x^2) + eps) over the head (fixed wave
//   butterfly); t = (x * r) * w; rotated:
//     out[l]      = t[l] cos - t[l+64] sin
//     out[l + 64] = t[l+64] cos + t[l] sin,   cos/sin = table[pos][l];
//   q goes to q_out[b, h, :], k to the cache slot of token pos;
//   v heads are copied unchanged to their slot of the d-major V page
//   ([page][kv head][d][slot]).
// A position outside the table or the block table, or a page outside the
// pool, writes nothing to the cache and zeros to q_out.
__global__ __launch_bounds__(64) void qknorm_rope_append_kernel(RopeArgs a) {
  const int b = blockIdx.x, h = blockIdx.y, l = threadIdx.x;
  const int nq = a.hq, nk = a.hkv;
  const uint16_t* src = a.qkv + (int64_t)b * a.ldqkv + (int64_t)h * HD;
  const int64_t pos = a.pos[b];
  // Out-of-range positions are clamped to 0 for the loads below, which are
  // then all issued together (no load waits behind a branch); the results
  // are masked with ok.
  const bool pos_ok = pos >= 0 && pos < a.max_pos && pos < a.max_pages * a.page;
  const int64_t pc = pos_ok ? pos : 0;
  int64_t page = a.bt[(int64_t)b * a.max_pages + pc / a.page];
  if (!pos_ok || page < 0 || page >= a.num_pages) page = -1;
  const bool ok = page >= 0;
  const uint16_t s0 = src[l], s1 = src[l + HALF];
  const bool is_q = h < nq;
  const uint16_t* w = is_q ? a.qw : a.kw;
  const uint16_t w0 = w[l], w1 = w[l + HALF];
  const float cl = a.cos_t[pc * HALF + l], sl = a.sin_t[pc * HALF + l];
  // keeps the loads above together, ahead of the head-kind branch (the
  // compiler would otherwise sink the weight and table loads past it and
  // wait for the row first)
  asm volatile("" ::"v"(s0), "v"(s1), "v"(w0), "v"(w1), "v"(cl), "v"(sl));
  if (h >= nq + nk) {  // v head: copy
    if (ok) {
      const int g = h - nq - nk;
      // V pages are d-major: [page][kv head][d][slot]
      uint16_t* dst = a.vp + (page * nk + g) * HD * a.page + pos % a.page;
      dst[(int64_t)l * a.page] = s0;
      dst[(int64_t)(l + HALF) * a.page] = s1;
    }
    return;
  }
  const float x0 = __uint_as_float(uint32_t(s0) << 16);
  const float x1 = __uint_as_float(uint32_t(s1) << 16);
  float ss = __builtin_fmaf(x0, x0, x1 * x1);
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
  const float t0 = (x0 * r) * __uint_as_float(uint32_t(w0) << 16);
  const float t1 = (x1 * r) * __uint_as_float(uint32_t(w1) << 16);
  const float c = ok ? cl : 0.0f, s = ok ? sl : 0.0f;
  const float o0 = t0 * c - t1 * s;
  const float o1 = t1 * c + t0 * s;
  const uint16_t b0 = (uint16_t)f32_to_bf16_rne(o0), b1 = (uint16_t)f32_to_bf16_rne(o1);
  if (is_q) {
    uint16_t* dst = a.q_out + ((int64_t)b * nq + h) * HD;
    dst[l] = ok ? b0 : 0;
    dst[l + HALF] = ok ? b1 : 0;
  } else if (ok) {
    const int g = h - nq;
    uint16_t* dst = a.kp + ((page * nk + g) * a.page + pos % a.page) * HD;
    dst[l] = b0;
    dst[l + HALF] = b1;
  }
}

}  // namespace

hipError_t launch_embed(const void* table, int64_t ld, int64_t vocab, const int64_t* tokens, void* out, int64_t ldo,
                        int64_t m, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)m), dim3(64), 0, s, static_cast<const uint16_t*>(table), ld, vocab,
                     tokens, static_cast<uint16_t*>(out), ldo, (int)n);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const void* gu, int64_t ldg, void* out, int64_t ldo, int64_t m, int64_t n,
                           hipStream_t s) {
  const unsigned chunks = (unsigned)(n / 8);
  hipLaunchKernelGGL(silu_mul_kernel, dim3((chunks + 255) / 256, (unsigned)m), dim3(256), 0, s,
                     static_cast<const uint16_t*>(gu), ldg, static_cast<uint16_t*>(out), ldo, (int)n);
  return hipGetLastError();
}

hipError_t launch_qknorm_rope_append(const RopeParams& p, hipStream_t s) {
  RopeArgs a;
  a.qkv = static_cast<const uint16_t*>(p.qkv);
  a.ldqkv = p.ldqkv;
  a.qw = static_cast<const uint16_t*>(p.q_norm_w);
  a.kw = static_cast<const uint16_t*>(p.k_norm_w);
  a.eps = p.eps;
  a.cos_t = p.cos_tab;
  a.sin_t = p.sin_tab;
  a.max_pos = p.max_pos;
  a.pos = p.positions;
  a.bt = p.block_table;
  a.max_pages = p.max_pages;
  a.num_pages = p.num_pages;
  a.kp = static_cast<uint16_t*>(p.k_pages);
  a.vp = static_cast<uint16_t*>(p.v_pages);
  a.q_out = static_cast<uint16_t*>(p.q_out);
  a.hq = p.num_q_heads;
  a.hkv = p.num_kv_heads;
  a.page = p.page_size;
  hipLaunchKernelGGL(qknorm_rope_append_kernel, dim3((unsigned)p.batch, (unsigned)(p.num_q_heads + 2 * p.num_kv_heads)),
                     dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace bi
