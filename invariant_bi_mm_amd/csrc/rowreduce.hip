// Batch-invariant row reductions for gfx950: RMSNorm, mean, log_softmax with
// the greedy argmax.
//
// mean and log_softmax are supported ops of
// "thinking-machines-lab/batch_invariant_ops" (section "When to avoid");
// SGLang took over its mean and log-softmax kernels ("Batch-invariant
// inference kernels (Thinking Machines) -- Evidence & limits", section
// "Evidence"). RMSNorm is named as batch-dependent in readhandoff.com's
// agent-run reproducibility pinning, section "What does temperature zero
// actually guarantee?"; the greedy sampler "picks the highest-probability
// token" (same section).
//
// Invariance: the lane that reads an element, the order each lane folds its
// elements, the butterfly and the fixed-order merge of the waves' partials
// are all functions of n (and the compiled kernel) only, so row i gets the
// same bits for any m and any content of the other rows. A workgroup works
// on one row only; for log_softmax at small m the same wave partials of a row
// are computed by several workgroups and merged by later launches, with the
// same arithmetic (see there). No atomics.
#include "bi_internal.h"
#include "device_common.h"

namespace bi {
namespace {

// ---------------------------------------------------------------------------
// RMSNorm and mean over bf16 rows: one 64-lane wave per row. Lane l owns the
// 16-byte chunks l, l + 64, l + 128, ... of its row (coalesced 128-bit loads),
// keeps up to CPT of them in registers, folds them in increasing order, then
// a wave butterfly gives every lane the row total. Elements past the last
// full chunk (n % 8) are folded last, by lanes 0..n%8-1.
// CPT == 0 selects the streaming variant (no register cache; chunks are read
// again for the output pass) used for rows longer than 64 * 16 chunks.
//
// ADD: residual form. The row first becomes x + d, rounded once to bf16
// (fp32 add of the two bf16 values, then RNE), that sum is written back over
// x and normalised. Every element of x is read before the lane that owns it
// writes it, so the in-place update needs no barrier; the streaming variant
// recomputes the sum in its second pass instead of reading its own writes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 add_bf16x8(const u32x4& a, const u32x4& b) {
  float fa[8], fb[8];
  unpack8(a, fa);
  unpack8(b, fb);
  return u32x4{pack_bf16x2(fa[0] + fb[0], fa[1] + fb[1]), pack_bf16x2(fa[2] + fb[2], fa[3] + fb[3]),
               pack_bf16x2(fa[4] + fb[4], fa[5] + fb[5]), pack_bf16x2(fa[6] + fb[6], fa[7] + fb[7])};
}

template <int CPT, bool ADD>
__global__ __launch_bounds__(64) void rmsnorm_kernel(uint16_t* __restrict__ x, int64_t ldx,
                                                      const uint16_t* __restrict__ d, int64_t ldd,
                                                      const uint16_t* __restrict__ w, float eps,
                                                      void* __restrict__ y, int64_t ldy, int y_bf16,
                                                      int n) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  uint16_t* xr = x + (int64_t)row * ldx;
  const uint16_t* dr = ADD ? d + (int64_t)row * ldd : nullptr;
  const int nch = n >> 3;
  const int tail = n & 7;
  // chunk c of the (updated) row
  auto chunk = [&](int c) {
    const u32x4 v = reinterpret_cast<const u32x4*>(xr)[c];
    if constexpr (ADD) return add_bf16x8(v, reinterpret_cast<const u32x4*>(dr)[c]);
    else return v;
  };
  auto elem = [&](int j) {  // element j (tail) of the updated row, as bf16 bits
    if constexpr (ADD) {
      const float t = __uint_as_float(uint32_t(xr[j]) << 16) + __uint_as_float(uint32_t(dr[j]) << 16);
      return (uint16_t)f32_to_bf16_rne(t);
    } else {
      return xr[j];
    }
  };

  u32x4 cache[CPT > 0 ? CPT : 1];
  u32x4 wcache[CPT > 0 ? CPT : 1];  // the weight chunks, fetched with x (no second round trip)
  float ss = 0.0f;
  if constexpr (CPT > 0) {
    // Every load is unconditional (chunk index clamped to the row's last
    // chunk, the result masked afterwards): a load whose value feeds the add
    // under a per-chunk branch is waited for at the branch's join, which
    // made each chunk a round trip of its own.
    u32x4 xv[CPT], dv[CPT];
    if (nch > 0) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int cc = min(lane + 64 * i, nch - 1);
        xv[i] = reinterpret_cast<const u32x4*>(xr)[cc];
        if constexpr (ADD) dv[i] = reinterpret_cast<const u32x4*>(dr)[cc];
        wcache[i] = reinterpret_cast<const u32x4*>(w)[cc];
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const bool ok = lane + 64 * i < nch;
      u32x4 v = xv[i];
      if constexpr (ADD) v = add_bf16x8(v, dv[i]);
      cache[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      if (!ok) wcache[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      float f[8];
      unpack8(cache[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
    }
  } else {
    for (int c = lane; c < nch; c += 64) {
      float f[8];
      unpack8(chunk(c), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
    }
  }
  uint16_t tail_v = 0;
  if (lane < tail) {
    tail_v = elem(nch * 8 + lane);
    const float t = __uint_as_float(uint32_t(tail_v) << 16);
    ss = __builtin_fmaf(t, t, ss);
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)n + eps);

  auto emit = [&](int c, const u32x4& xv, const u32x4& wv) {
    if constexpr (ADD) reinterpret_cast<u32x4*>(xr)[c] = xv;
    float f[8], wf[8];
    unpack8(xv, f);
    unpack8(wv, wf);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (f[e] * r) * wf[e];
    if (y_bf16) {
      u32x4 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                  pack_bf16x2(o[6], o[7])};
      reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + (int64_t)row * ldy)[c] = pk;
    } else {
      f32x4* yr = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + (int64_t)row * ldy);
      yr[2 * c] = f32x4{o[0], o[1], o[2], o[3]};
      yr[2 * c + 1] = f32x4{o[4], o[5], o[6], o[7]};
    }
  };
  if constexpr (CPT > 0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) emit(c, cache[i], wcache[i]);
    }
  } else {
    for (int c = lane; c < nch; c += 64) emit(c, chunk(c), reinterpret_cast<const u32x4*>(w)[c]);
  }
  if (lane < tail) {
    const int j = nch * 8 + lane;
    if constexpr (ADD) xr[j] = tail_v;
    const float t = __uint_as_float(uint32_t(tail_v) << 16);
    const float wj = __uint_as_float(uint32_t(w[j]) << 16);
    const float o = (t * r) * wj;
    if (y_bf16)
      (reinterpret_cast<uint16_t*>(y) + (int64_t)row * ldy)[j] = (uint16_t)f32_to_bf16_rne(o);
    else
      (reinterpret_cast<float*>(y) + (int64_t)row * ldy)[j] = o;
  }
}

// mean over bf16 (8 per chunk) or fp32 (4 per chunk) rows; same shape as above.
template <bool BF16, int CPT>
__global__ __launch_bounds__(64) void mean_kernel(const void* __restrict__ x, int64_t ldx,
                                                   float* __restrict__ y, int n) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  constexpr int PER = BF16 ? 8 : 4;
  const int nch = n / PER;
  const int tail = n - nch * PER;
  float s = 0.0f;
  if constexpr (BF16) {
    const uint16_t* xr = reinterpret_cast<const uint16_t*>(x) + (int64_t)row * ldx;
    if constexpr (CPT > 0) {
      u32x4 cache[CPT];
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = lane + 64 * i;
        cache[i] = c < nch ? reinterpret_cast<const u32x4*>(xr)[c] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        float f[8];
        unpack8(cache[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = s + f[e];
      }
    } else {
      for (int c = lane; c < nch; c += 64) {
        float f[8];
        unpack8(reinterpret_cast<const u32x4*>(xr)[c], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = s + f[e];
      }
    }
    if (lane < tail) s = s + __uint_as_float(uint32_t(xr[nch * 8 + lane]) << 16);
  } else {
    const float* xr = reinterpret_cast<const float*>(x) + (int64_t)row * ldx;
    if constexpr (CPT > 0) {
      f32x4 cache[CPT];
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = lane + 64 * i;
        cache[i] = c < nch ? reinterpret_cast<const f32x4*>(xr)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) s = s + cache[i].x + cache[i].y + cache[i].z + cache[i].w;
    } else {
      for (int c = lane; c < nch; c += 64) {
        const f32x4 v = reinterpret_cast<const f32x4*>(xr)[c];
        s = s + v.x + v.y + v.z + v.w;
      }
    }
    if (lane < tail) s = s + xr[nch * 4 + lane];
  }
  s = wave_sum(s);
  if (lane == 0) y[row] = s / (float)n;
}

// ---------------------------------------------------------------------------
// log_softmax + argmax over fp32 rows: one workgroup of LS_NT threads per row.
// Pass 1: thread t reads the 16-byte chunks t, t + LS_NT, ... in increasing
// order and keeps a running (max, sum of exp(x - max)) pair, rescaled when
// the max grows, plus the (value, lowest index) of its largest element.
// The pairs are merged by a wave butterfly and then across waves in wave
// order. Pass 2 writes (x - max) - log(sum). Between the passes a thread
// keeps its first LS_REG chunks in registers and the next LS_KEEP in LDS
// (25 of the 38 chunks per thread of a 151936-wide row), so pass 2 re-reads
// only the rest of the row from memory.
// ---------------------------------------------------------------------------
constexpr int LS_NT = 1024;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float exp_dev(float v) { return __builtin_amdgcn_exp2f(v * LOG2E); }

struct MS {
  float m, s;
};
__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return MS{M, 0.0f};
  return MS{M, a.s * exp_dev(a.m - M) + b.s * exp_dev(b.m - M)};
}
struct AM {
  float v;
  int i;
};
__device__ __forceinline__ AM am_merge(AM a, AM b) {
  const bool take_b = (b.v > a.v) || (b.v == a.v && b.i < a.i);
  return take_b ? b : a;
}

// One workgroup per CU (its LDS holds LS_KEEP chunks per thread), so 256
// rows (~155 MB at n = 151936) are in flight at a time and stay inside the
// 256 MB Infinity Cache, which serves pass 2's re-read of the part of a row
// not kept on chip.
constexpr int LS_REG = 16;   // chunks per thread kept in registers between the passes
constexpr int LS_KEEP = 9;   // ... and in LDS

__global__ __launch_bounds__(LS_NT) void log_softmax_kernel(const float* __restrict__ x, int64_t ldx,
                                                             float* __restrict__ y, int64_t ldy,
                                                             int64_t* __restrict__ amax, int n) {
  __shared__ f32x4 keep[LS_KEEP][LS_NT];
  __shared__ float red[4 * (LS_NT / 64)];
  float* sm_m = red;
  float* sm_s = red + LS_NT / 64;
  float* sm_v = red + 2 * (LS_NT / 64);
  int* sm_i = reinterpret_cast<int*>(red + 3 * (LS_NT / 64));
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* xr = x + (int64_t)row * ldx;
  float* yr = y + (int64_t)row * ldy;
  const int nch = n >> 2;
  const int tail = n & 3;

  float m = -INFINITY, s = 0.0f;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  auto fold = [&](float v, int j) {
    // argmax: strictly greater keeps the lowest index within this thread.
    if (v > bv) {
      bv = v;
      bi = j;
    }
  };
  // While every element seen so far is -inf (a masked prefix), m is -inf
  // and v - m would be NaN; the elements are then -inf too, so they are
  // measured against 0 instead, which gives exp(-inf) = 0. A finite m is
  // used as it is, so rows without -inf keep their bits.
  auto fold4 = [&](const f32x4 v, int j0) {
    const float cm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    if (cm > m) {
      s = s * exp_dev(m - cm);
      m = cm;
    }
    const float mr = m == -INFINITY ? 0.0f : m;
    s = s + exp_dev(v.x - mr);
    s = s + exp_dev(v.y - mr);
    s = s + exp_dev(v.z - mr);
    s = s + exp_dev(v.w - mr);
    fold(v.x, j0);
    fold(v.y, j0 + 1);
    fold(v.z, j0 + 2);
    fold(v.w, j0 + 3);
  };

  // The first LS_REG chunks of this thread, all loads in flight together,
  // folded in increasing chunk order and kept in registers for pass 2. The
  // chunks kept on chip (registers, LDS) are loaded non-temporal: they are
  // not read from memory again, and the caches keep more of the part that
  // pass 2 re-reads.
  const f32x4* xv = reinterpret_cast<const f32x4*>(xr);
  f32x4 r[LS_REG];
#pragma unroll
  for (int u = 0; u < LS_REG; ++u) {
    const int cc = tid + u * LS_NT;
    r[u] = cc < nch ? __builtin_nontemporal_load(xv + cc) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int u = 0; u < LS_REG; ++u)
    if (tid + u * LS_NT < nch) fold4(r[u], 4 * (tid + u * LS_NT));
  // the next LS_KEEP chunks, kept in LDS (each thread its own column),
  // three loads in flight at a time
  static_assert(LS_KEEP % 3 == 0, "LDS chunks go in groups of three");
#pragma unroll
  for (int u0 = 0; u0 < LS_KEEP; u0 += 3) {
    f32x4 v[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int cc = tid + (LS_REG + u0 + u) * LS_NT;
      v[u] = cc < nch ? __builtin_nontemporal_load(xv + cc) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int cc = tid + (LS_REG + u0 + u) * LS_NT;
      if (cc < nch) {
        keep[u0 + u][tid] = v[u];
        fold4(v[u], 4 * cc);
      }
    }
  }
  // the rest of the row, six 16-byte loads in flight per thread (eight spill)
  constexpr int U = 6;
  int c = tid + (LS_REG + LS_KEEP) * LS_NT;
  for (; c + (U - 1) * LS_NT < nch; c += U * LS_NT) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = xv[c + u * LS_NT];
#pragma unroll
    for (int u = 0; u < U; ++u) fold4(v[u], 4 * (c + u * LS_NT));
  }
  for (; c < nch; c += LS_NT) fold4(xv[c], 4 * c);
  if (tid < tail) {
    const float v = xr[nch * 4 + tid];
    if (v > m) {
      s = s * exp_dev(m - v);
      m = v;
    }
    s = s + exp_dev(v - (m == -INFINITY ? 0.0f : m));
    fold(v, nch * 4 + tid);
  }

  MS ms{m, s};
  AM am{bv, bi};
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    ms = ms_merge(ms, MS{xor_shfl(ms.m, d), xor_shfl(ms.s, d)});
    am = am_merge(am, AM{xor_shfl(am.v, d), __shfl_xor(am.i, d, 64)});
  }
  if (lane == 0) {
    sm_m[wave] = ms.m;
    sm_s[wave] = ms.s;
    sm_v[wave] = am.v;
    sm_i[wave] = am.i;
  }
  __syncthreads();
  MS tot = MS{sm_m[0], sm_s[0]};
  AM best = AM{sm_v[0], sm_i[0]};
#pragma unroll
  for (int w = 1; w < LS_NT / 64; ++w) {
    tot = ms_merge(tot, MS{sm_m[w], sm_s[w]});
    best = am_merge(best, AM{sm_v[w], sm_i[w]});
  }
  if (tid == 0 && amax != nullptr) amax[row] = (int64_t)(best.i == 0x7fffffff ? 0 : best.i);

  const float mx = tot.m;
  const float lg = __builtin_amdgcn_logf(tot.s) * LN2;  // log2 -> ln
  // the output streams past the caches (non-temporal stores): it is not read
  // again here, and the row's chunks left for the second pass stay cached
  auto out4 = [&](int cc, const f32x4 v) {
    __builtin_nontemporal_store(f32x4{(v.x - mx) - lg, (v.y - mx) - lg, (v.z - mx) - lg, (v.w - mx) - lg},
                                reinterpret_cast<f32x4*>(yr) + cc);
  };
  // the re-read part first, while the end of pass 1 may still hold it in
  // the caches; then the chunks kept in registers and LDS
  constexpr int U2 = 6;
  for (c = tid + (LS_REG + LS_KEEP) * LS_NT; c + (U2 - 1) * LS_NT < nch; c += U2 * LS_NT) {
    f32x4 v[U2];
#pragma unroll
    for (int u = 0; u < U2; ++u) v[u] = xv[c + u * LS_NT];
#pragma unroll
    for (int u = 0; u < U2; ++u) out4(c + u * LS_NT, v[u]);
  }
  for (; c < nch; c += LS_NT) out4(c, xv[c]);
#pragma unroll
  for (int u = 0; u < LS_REG; ++u)
    if (tid + u * LS_NT < nch) out4(tid + u * LS_NT, r[u]);
#pragma unroll
  for (int u = 0; u < LS_KEEP; ++u)
    if (tid + (LS_REG + u) * LS_NT < nch) out4(tid + (LS_REG + u) * LS_NT, keep[u][tid]);
  if (tid < tail) __builtin_nontemporal_store((xr[nch * 4 + tid] - mx) - lg, yr + nch * 4 + tid);
}

// The same row reduction for a few rows, spread over many CUs. In the kernel
// above a row's reduction is 16 wave partials -- wave w, lane l folds the
// units 64 w + l + 1024 u (increasing u; the n % 4 tail elements by threads
// 0..tail-1, last) and then runs the butterfly -- merged in wave order. Those
// 16 partials do not depend on each other, so for a small batch each gets a
// workgroup (one wave) of its own, with all its loads in flight at once,
// instead of sharing one CU with the other 15 (at m = 1 the one-workgroup form
// leaves 255 CUs idle and walks ~38 memory round trips). Three launches in
// stream order; no scratch, no atomics, no waiting between workgroups:
//   ls_partial_kernel  the 16 wave partials of every row, each written as
//                      {max, sum, argmax value, argmax index bits} to floats
//                      [4 w, 4 w + 4) of the row's own output;
//   ls_out_kernel      merges them in wave order (the arithmetic of the kernel
//                      above) and writes every output element from float 64 on;
//   ls_head_kernel     merges them again (same order, same bits), writes
//                      floats 0..63 over the partials, the tail and the argmax.
// Every row therefore gets exactly the bits of log_softmax_kernel.
constexpr int LS_G = 40;  // units a lane of ls_partial_kernel loads at once

__global__ __launch_bounds__(64) void ls_partial_kernel(const float* __restrict__ x, int64_t ldx,
                                                         float* __restrict__ y, int64_t ldy, int n) {
  const int row = blockIdx.x / (LS_NT / 64), w = blockIdx.x % (LS_NT / 64);
  const int lane = threadIdx.x, tid = 64 * w + lane;  // the thread of log_softmax_kernel this lane stands for
  const float* xr = x + (int64_t)row * ldx;
  const f32x4* xv = reinterpret_cast<const f32x4*>(xr);
  const int nch = n >> 2, tail = n & 3;
  float m = -INFINITY, s = 0.0f, bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int u0 = 0; tid + u0 * LS_NT < nch; u0 += LS_G) {
    f32x4 r[LS_G];
#pragma unroll
    for (int u = 0; u < LS_G; ++u) {
      const int cc = tid + (u0 + u) * LS_NT;
      r[u] = cc < nch ? xv[cc] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int u = 0; u < LS_G; ++u) {
      const int cc = tid + (u0 + u) * LS_NT;
      if (cc < nch) {
        const f32x4 v = r[u];
        const float cm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
        if (cm > m) {
          s = s * exp_dev(m - cm);
          m = cm;
        }
        const float mr = m == -INFINITY ? 0.0f : m;
        s = s + exp_dev(v.x - mr);
        s = s + exp_dev(v.y - mr);
        s = s + exp_dev(v.z - mr);
        s = s + exp_dev(v.w - mr);
        const int j0 = 4 * cc;
        if (v.x > bv) { bv = v.x; bi = j0; }
        if (v.y > bv) { bv = v.y; bi = j0 + 1; }
        if (v.z > bv) { bv = v.z; bi = j0 + 2; }
        if (v.w > bv) { bv = v.w; bi = j0 + 3; }
      }
    }
  }
  if (tid < tail) {
    const float v = xr[nch * 4 + tid];
    if (v > m) {
      s = s * exp_dev(m - v);
      m = v;
    }
    s = s + exp_dev(v - (m == -INFINITY ? 0.0f : m));
    if (v > bv) {
      bv = v;
      bi = nch * 4 + tid;
    }
  }
  MS ms{m, s};
  AM am{bv, bi};
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    ms = ms_merge(ms, MS{xor_shfl(ms.m, d), xor_shfl(ms.s, d)});
    am = am_merge(am, AM{xor_shfl(am.v, d), __shfl_xor(am.i, d, 64)});
  }
  if (lane == 0) {
    float* slot = y + (int64_t)row * ldy + 4 * w;
    slot[0] = ms.m;
    slot[1] = ms.s;
    slot[2] = am.v;
    reinterpret_cast<int*>(slot)[3] = am.i;
  }
}

// (max, log sum, argmax) of a row from its 16 wave partials, merged in wave
// order as log_softmax_kernel merges them (all lanes read the same slots).
__device__ __forceinline__ void ls_totals(const float* yr, float& mx, float& lg, AM& best) {
  MS tot{yr[0], yr[1]};
  best = AM{yr[2], reinterpret_cast<const int*>(yr)[3]};
#pragma unroll
  for (int w = 1; w < LS_NT / 64; ++w) {
    tot = ms_merge(tot, MS{yr[4 * w], yr[4 * w + 1]});
    best = am_merge(best, AM{yr[4 * w + 2], reinterpret_cast<const int*>(yr)[4 * w + 3]});
  }
  mx = tot.m;
  lg = __builtin_amdgcn_logf(tot.s) * LN2;  // log2 -> ln
}

// Units 16 .. nch - 1 of every row (the first 16 units hold the partials
// until ls_head_kernel): workgroup (row, slice) writes units 1024 slice ..
// 1024 slice + 1023, four per thread, their loads in flight during the merge.
__global__ __launch_bounds__(256) void ls_out_kernel(const float* __restrict__ x, int64_t ldx,
                                                      float* __restrict__ y, int64_t ldy, int n) {
  const int nch = n >> 2;
  const int slices = (nch + 1023) / 1024;
  const int row = blockIdx.x / slices, slice = blockIdx.x % slices;
  const float* xr = x + (int64_t)row * ldx;
  float* yr = y + (int64_t)row * ldy;
  const f32x4* xv = reinterpret_cast<const f32x4*>(xr);
  f32x4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cc = 1024 * slice + threadIdx.x + 256 * j;
    v[j] = (cc >= 16 && cc < nch) ? xv[cc] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  float mx, lg;
  AM best;
  ls_totals(yr, mx, lg, best);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cc = 1024 * slice + threadIdx.x + 256 * j;
    if (cc >= 16 && cc < nch)
      __builtin_nontemporal_store(f32x4{(v[j].x - mx) - lg, (v[j].y - mx) - lg, (v[j].z - mx) - lg,
                                        (v[j].w - mx) - lg},
                                  reinterpret_cast<f32x4*>(yr) + cc);
  }
}

// Units 0..15 of every row (over its partials), the n % 4 tail and the argmax.
__global__ __launch_bounds__(64) void ls_head_kernel(const float* __restrict__ x, int64_t ldx,
                                                      float* __restrict__ y, int64_t ldy,
                                                      int64_t* __restrict__ amax, int n) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const int nch = n >> 2, tail = n & 3;
  const float* xr = x + (int64_t)row * ldx;
  float* yr = y + (int64_t)row * ldy;
  const f32x4 v = lane < 16 ? reinterpret_cast<const f32x4*>(xr)[lane] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const float t = lane < tail ? xr[nch * 4 + lane] : 0.0f;
  float mx, lg;
  AM best;
  ls_totals(yr, mx, lg, best);
  // every lane's partial reads feed mx and lg, so they precede the stores below
  if (lane < 16)
    __builtin_nontemporal_store(f32x4{(v.x - mx) - lg, (v.y - mx) - lg, (v.z - mx) - lg, (v.w - mx) - lg},
                                reinterpret_cast<f32x4*>(yr) + lane);
  if (lane < tail) __builtin_nontemporal_store((t - mx) - lg, yr + nch * 4 + lane);
  if (lane == 0 && amax != nullptr) amax[row] = (int64_t)(best.i == 0x7fffffff ? 0 : best.i);
}

// Chunks-per-lane template choice for one-wave-per-row kernels: a function
// of n only.
int pick_cpt(int64_t nch) {
  const int64_t per = (nch + 63) / 64;
  if (per <= 1) return 1;
  if (per <= 2) return 2;
  if (per <= 4) return 4;
  if (per <= 8) return 8;
  if (per <= 16) return 16;
  return 0;
}

template <bool ADD>
hipError_t launch_rmsnorm_impl(uint16_t* xp, int64_t ldx, const uint16_t* dp, int64_t ldd, const uint16_t* wp,
                               float eps, void* y, int64_t ldy, bool y_bf16, int64_t m, int64_t n, hipStream_t s) {
  const int yb = y_bf16 ? 1 : 0;
  const dim3 grid((unsigned)m), block(64);
#define BI_RMS(C) hipLaunchKernelGGL((rmsnorm_kernel<C, ADD>), grid, block, 0, s, xp, ldx, dp, ldd, wp, eps, y, ldy, yb, (int)n)
  switch (pick_cpt(n / 8)) {
    case 1: BI_RMS(1); break;
    case 2: BI_RMS(2); break;
    case 4: BI_RMS(4); break;
    case 8: BI_RMS(8); break;
    case 16: BI_RMS(16); break;
    default: BI_RMS(0); break;
  }
#undef BI_RMS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, int64_t ldx, const void* w, float eps, void* y, int64_t ldy,
                          bool y_bf16, int64_t m, int64_t n, hipStream_t s) {
  // the kernel's x is writable only in the residual form; here it is only read
  return launch_rmsnorm_impl<false>(const_cast<uint16_t*>(static_cast<const uint16_t*>(x)), ldx, nullptr, 0,
                                    static_cast<const uint16_t*>(w), eps, y, ldy, y_bf16, m, n, s);
}

hipError_t launch_add_rmsnorm(void* x, int64_t ldx, const void* d, int64_t ldd, const void* w, float eps, void* y,
                              int64_t ldy, bool y_bf16, int64_t m, int64_t n, hipStream_t s) {
  return launch_rmsnorm_impl<true>(static_cast<uint16_t*>(x), ldx, static_cast<const uint16_t*>(d), ldd,
                                   static_cast<const uint16_t*>(w), eps, y, ldy, y_bf16, m, n, s);
}

hipError_t launch_mean(const void* x, bool x_bf16, int64_t ldx, float* y, int64_t m, int64_t n,
                       hipStream_t s) {
  const dim3 grid((unsigned)m), block(64);
  const int cpt = pick_cpt(x_bf16 ? n / 8 : n / 4);
  const int ni = (int)n;
#define BI_MEAN_CASE(B, C) hipLaunchKernelGGL((mean_kernel<B, C>), grid, block, 0, s, x, ldx, y, ni)
  if (x_bf16) {
    switch (cpt) {
      case 1: BI_MEAN_CASE(true, 1); break;
      case 2: BI_MEAN_CASE(true, 2); break;
      case 4: BI_MEAN_CASE(true, 4); break;
      case 8: BI_MEAN_CASE(true, 8); break;
      case 16: BI_MEAN_CASE(true, 16); break;
      default: BI_MEAN_CASE(true, 0); break;
    }
  } else {
    switch (cpt) {
      case 1: BI_MEAN_CASE(false, 1); break;
      case 2: BI_MEAN_CASE(false, 2); break;
      case 4: BI_MEAN_CASE(false, 4); break;
      case 8: BI_MEAN_CASE(false, 8); break;
      case 16: BI_MEAN_CASE(false, 16); break;
      default: BI_MEAN_CASE(false, 0); break;
    }
  }
#undef BI_MEAN_CASE
  return hipGetLastError();
}

// Rows up to which each row's 16 wave partials get workgroups of their own
// (the three-launch form above); the same bits either way. Measured at
// n = 151936: M = 33 27.3 -> 20.3 us, M = 48 27.7 -> 24.2 us, even at
// M = 64 (28.3 / 28.8 us), slower beyond (M = 96 31.3 / 42.6 us).
constexpr int64_t LS_SMALL_M = 48;

hipError_t launch_log_softmax(const float* x, int64_t ldx, float* y, int64_t ldy, int64_t* argmax,
                              int64_t m, int64_t n, hipStream_t s) {
  const int ni = (int)n;
  if (m <= LS_SMALL_M && n >= 4096) {
    const int slices = (ni / 4 + 1023) / 1024;
    hipLaunchKernelGGL(ls_partial_kernel, dim3((unsigned)(m * (LS_NT / 64))), dim3(64), 0, s, x, ldx, y, ldy, ni);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ls_out_kernel, dim3((unsigned)(m * slices)), dim3(256), 0, s, x, ldx, y, ldy, ni);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ls_head_kernel, dim3((unsigned)m), dim3(64), 0, s, x, ldx, y, ldy, argmax, ni);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(log_softmax_kernel, dim3((unsigned)m), dim3(LS_NT), 0, s, x, ldx, y, ldy, argmax, ni);
  return hipGetLastError();
}

}  // namespace bi
