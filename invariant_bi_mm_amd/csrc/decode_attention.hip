// Batch-invariant split-KV decode attention over a paged bf16 KV cache, gfx950.
//
// Attention is one of the inference kernels named as batch-dependent in
// readhandoff.com's agent-run reproducibility pinning ("What does temperature
// zero actually guarantee?"); SGLang wrote its own batch-invariant attention
// and an improved attention kernel recovered much of the cost ("Batch-
// invariant inference kernels (Thinking Machines) -- Evidence & limits",
// sections "Evidence" and "Limitations").
//
// Invariance: a sequence's keys are cut at fixed multiples of SPLIT of its own
// token index, so which tokens form split s, and how many splits there are,
// depends on the sequence's length alone -- never on the batch, on the other
// sequences or on the occupancy of the GPU. Each split is reduced by one
// workgroup in a fixed order; the combine kernel merges the splits of one
// (sequence, head) in increasing split order. The position of the sequence in
// the batch only changes WHICH workgroup does the work.
//
// Kernel 1, one workgroup per (split, kv head), 256 threads = 16 groups of 16
// lanes; lane dl of a group owns head-dim slice [8*dl, 8*dl + 8).
//   phase 1: group i handles slot i of each of the split's (<= 16) pages: the
//            16 groups read one 4 KB head-page together. Scores for the GQA
//            query heads sharing this kv head are 8-term fixed-order dots
//            plus a 16-lane butterfly, kept in LDS (log2 domain: q is
//            pre-multiplied by scale * log2(e)).
//   phase 2: wave h (one per query head) takes the exact max over the split,
//            writes p = 2^(s - max) back and sums it (per-lane fixed order,
//            then butterfly).
//   phase 3: o = sum_t p_t v_t with the same token->group assignment, groups
//            merged by butterfly inside a wave, waves merged in wave order.
//   output : (max, sum p, o[128]) per (split, query head), fp32.
// Kernel 2, one workgroup per (sequence, query head):
//   M = max_s m_s; l = sum_s 2^(m_s - M) l_s; o = sum_s 2^(m_s - M) o_s[d],
//   each sum taken as 8 chains (splits s = r mod 8, increasing s) added in a
//   fixed tree; out = o / l.
#include "bi_internal.h"
#include "device_common.h"

namespace bi {
namespace {

constexpr int HD = 128;     // head dim
constexpr int PAGE = 16;    // tokens per page
constexpr int SPLIT = 256;  // tokens per split
constexpr int GQA = 4;      // query heads per kv head
constexpr int PPS = SPLIT / PAGE;
constexpr float LOG2E = 1.4426950408889634f;

struct SplitArgs {
  const uint16_t* q;
  const uint16_t* kp;
  const uint16_t* vp;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* offs;
  int64_t max_pages;
  int batch;
  int hq, hkv;
  float qscale;
  float* ws_o;
  float* ws_ml;
};

// ---------------------------------------------------------------------------
// The per-(query, split) arithmetic, shared by the decode and the prefill
// kernels so that a token's partials have the same bits whichever computes
// them. Thread layout: 256 threads = 16 groups of 16 lanes; lane dl of group
// grp owns head-dim slice [8 dl, 8 dl + 8) of slot grp of each of the split's
// pages, i.e. of tokens j * PAGE + grp, j = 0..PPS-1.
// ---------------------------------------------------------------------------

// Phase 1: scores S[t][h][key] of the split's SPLIT keys for query rows
// r = GQA t + h, t < ntok tokens, on the matrix cores:
//   S = (sum_d q[r][d] k[key][d]) * qscale   (qscale = scale * log2(e)),
// the sum taken by v_mfma_f32_16x16x32_bf16 over d in four steps of 32
// (exact bf16 products, fp32 accumulation, increasing d), then one fp32
// multiply; keys at or past nt_of(t) get -inf. Wave w covers keys
// [64 w, 64 w + 64) as four 16-key tiles, tile kt being slots 0..15 of page
// 4 w + kt; its MFMA B operand (lane l: key l % 16, d 8 (l / 16) .. +7 of a
// 32-wide step) is read straight from the page with 16-byte loads. Query
// rows go 16 to an MFMA; rows past GQA ntok read zeros and are not stored.
// The element (r, key) gets the same chain whichever row of the MFMA holds
// r, so a token's scores do not depend on the other tokens of the block.
template <int NTOK, typename NtOf>
__device__ __forceinline__ void split_scores(const uint16_t* q0, int64_t q_tok_stride, int ntok, NtOf nt_of,
                                             const uint16_t* kp, const int32_t* bt, int64_t page_stride,
                                             int64_t head_off, int wave, int lane, float qscale,
                                             float (*S)[GQA][SPLIT]) {
  constexpr int RB = (NTOK * GQA + 15) / 16;
  const int nt_max = nt_of(ntok - 1);  // the block's last token sees the most keys
  const int sl = lane & 15, dq = 8 * (lane >> 4);
  u32x4 kf[4][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int pg = 4 * wave + kt;
    if (16 * pg < nt_max) {
      const uint16_t* base = kp + (int64_t)bt[pg] * page_stride + head_off + sl * HD + dq;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kf[kt][ds] = *reinterpret_cast<const u32x4*>(base + 32 * ds);
    } else {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kf[kt][ds] = u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = 16 * rb + sl;  // the query row this lane feeds to the MFMA
    bf16x8 qa[4];
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (r / GQA < ntok)
        v = *reinterpret_cast<const u32x4*>(q0 + (r / GQA) * q_tok_stride + (r % GQA) * HD + 32 * ds + dq);
      qa[ds] = __builtin_bit_cast(bf16x8, v);
    }
    const int t_out = 4 * rb + (lane >> 4);  // token of the 4 rows this lane receives (GQA == 4)
    const int nt_t = t_out < ntok ? nt_of(t_out) : 0;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ds], __builtin_bit_cast(bf16x8, kf[kt][ds]), acc, 0, 0, 0);
      const int key = 64 * wave + 16 * kt + sl;
      if (t_out < ntok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t_out][i][key] = key < nt_t ? acc[i] * qscale : -INFINITY;
      }
    }
  }
}

// Phase 2, one row (query, head) by one wave: exact max, p = 2^(s - max)
// written back, l = sum p (per-lane order, then the wave butterfly).
__device__ __forceinline__ void split_softmax_row(float* row, int lane, float& mx_out, float& l_out) {
  float v[SPLIT / 64];
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < SPLIT / 64; ++r) {
    v[r] = row[lane + 64 * r];
    mx = fmaxf(mx, v[r]);
  }
  mx = wave_max(mx);
  float l = 0.0f;
#pragma unroll
  for (int r = 0; r < SPLIT / 64; ++r) {
    const float pr = __builtin_amdgcn_exp2f(v[r] - mx);  // 2^-inf = 0 for masked slots
    row[lane + 64 * r] = pr;
    l = l + pr;
  }
  mx_out = mx;
  l_out = wave_sum(l);
}

// Phase 3 for one query: o[h][e] = sum_j p(token j * PAGE + grp) v[e] (fma
// chain in j), then the 4 groups of a wave merged (xor 16, then xor 32).
__device__ __forceinline__ void split_pv(const u32x4 (&kv)[PPS], const float (*S)[SPLIT], int grp, float (&o)[GQA][8]) {
#pragma unroll
  for (int h = 0; h < GQA; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;
#pragma unroll
  for (int j = 0; j < PPS; ++j) {
    const int i = j * PAGE + grp;
    float vf[8];
    unpack8(kv[j], vf);
#pragma unroll
    for (int h = 0; h < GQA; ++h) {
      const float pr = S[h][i];  // 0 for masked slots
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = __builtin_fmaf(pr, vf[e], o[h][e]);
    }
  }
#pragma unroll
  for (int h = 0; h < GQA; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = o[h][e];
      t = t + xor_shfl(t, 16);
      t = t + xor_shfl(t, 32);
      o[h][e] = t;
    }
}

// The 4 waves' o merged in wave order, written as the split's partial:
// thread handles (h, d) pairs tid and tid + 256.
__device__ __forceinline__ void write_partial(const float (*O)[GQA][HD], int tid, float* ws_o_base) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int idx = tid + 256 * r;
    const int h = idx >> 7, d = idx & (HD - 1);
    ws_o_base[h * HD + d] = ((O[0][h][d] + O[1][h][d]) + O[2][h][d]) + O[3][h][d];
  }
}

// K (or V) of the split's tokens this thread owns; slots at or past nt read 0.
__device__ __forceinline__ void load_kv(const uint16_t* pages, const int32_t* bt, int64_t page_stride, int64_t slot_off,
                                        int grp, int nt, u32x4 (&kv)[PPS]) {
#pragma unroll
  for (int j = 0; j < PPS; ++j) {
    kv[j] = u32x4{0u, 0u, 0u, 0u};
    if (j * PAGE + grp < nt) {
      const int64_t page = bt[j];
      kv[j] = *reinterpret_cast<const u32x4*>(pages + page * page_stride + slot_off);
    }
  }
}

__global__ __launch_bounds__(256) void decode_split_kernel(SplitArgs a) {
  __shared__ float S[1][GQA][SPLIT];
  __shared__ float O[4][GQA][HD];
  __shared__ float ML[GQA][2];

  // The kv heads of one split are adjacent in dispatch order, so the 4 KB
  // head slices of a physical page (all heads, 32 KB at 8 heads) are read at
  // about the same time.
  const int w = blockIdx.x / a.hkv;  // global split index
  const int g = blockIdx.x % a.hkv;  // kv head
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = tid >> 4;  // 0..15
  const int dl = tid & 15;   // head-dim slice
  // The grid may cover more splits than exist (the host passes an upper
  // bound so one captured launch serves growing lengths): the exact count is
  // split_offsets[batch], and workgroups past it have nothing to do.
  if (w >= a.offs[a.batch]) return;

  // sequence owning split w: the b with offs[b] <= w < offs[b+1]. The
  // offsets are read with coalesced loads and compared in parallel (one
  // memory round trip per 256 sequences instead of a dependent binary search).
  __shared__ int sb;
  if (tid == 0) sb = 0;
  __syncthreads();
  for (int base = 0; base < a.batch; base += 256) {
    const int t = base + tid;
    if (t < a.batch && a.offs[t] <= w && w < a.offs[t + 1]) sb = t;
  }
  __syncthreads();
  const int b = sb;
  const int s = w - a.offs[b];
  const int L = a.lens[b];
  const int t0 = s * SPLIT;
  const int nt = min(SPLIT, L - t0);
  const int32_t* bt = a.bt + (int64_t)b * a.max_pages + t0 / PAGE;

  const int64_t head_stride = (int64_t)PAGE * HD;           // one head-page
  const int64_t page_stride = (int64_t)a.hkv * head_stride;  // one physical page
  const int64_t slot_off = (int64_t)g * head_stride + (int64_t)grp * HD + dl * 8;

  split_scores<1>(a.q + ((int64_t)b * a.hq + g * GQA) * HD, 0, 1, [&](int) { return nt; }, a.kp, bt, page_stride,
                  (int64_t)g * head_stride, wave, lane, a.qscale, S);
  __syncthreads();
  {
    float mx, l;
    split_softmax_row(S[0][wave], lane, mx, l);  // wave h: query head h
    if (lane == 0) {
      ML[wave][0] = mx;
      ML[wave][1] = l;
    }
  }
  __syncthreads();
  u32x4 kv[PPS];
  load_kv(a.vp, bt, page_stride, slot_off, grp, nt, kv);
  float o[GQA][8];
  split_pv(kv, S[0], grp, o);
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < GQA; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) O[wave][h][dl * 8 + e] = o[h][e];
  }
  __syncthreads();
  const int64_t base = (int64_t)w * a.hq + g * GQA;
  write_partial(O, tid, a.ws_o + base * HD);
  if (tid < GQA) {
    a.ws_ml[(base + tid) * 2 + 0] = ML[tid][0];
    a.ws_ml[(base + tid) * 2 + 1] = ML[tid][1];
  }
}

// ---------------------------------------------------------------------------
// Prefill / extend: the tokens of a chunk attend causally to their sequence's
// cache (which already holds them). Query row r at position p uses exactly
// the split structure of a decode step with p + 1 cached tokens: splits
// s = 0 .. ceil((p + 1) / SPLIT) - 1, each reduced by the functions above
// with nt = min(SPLIT, p + 1 - s * SPLIT), merged by the decode combine
// kernel. So a prefilled token's output has the bits a decode step would
// give it, whatever the chunking and the batch.
//
// One workgroup per (work item, kv head); a work item is up to QB
// consecutive query rows of one sequence and one split they see. The split's
// K and V are loaded once for all of them (slots past the last row's nt read
// 0); for an earlier row, the slots it must not see carry p = 0, and
// fma(0, v, o) = o for finite v, so they add nothing.
// ---------------------------------------------------------------------------
constexpr int QB = 8;

struct PrefillArgs {
  const uint16_t* q;  // [rows, hq, HD]
  const uint16_t* kp;
  const uint16_t* vp;
  const int32_t* bt;    // [batch, max_pages]
  const int32_t* pos;   // [rows]
  const int32_t* qoffs; // [rows + 1]
  const int32_t* work;  // [n_work, 4]: row0, n_rows, sequence, split
  int64_t max_pages;
  int hq, hkv;
  float qscale;
  float* ws_o;
  float* ws_ml;
};

__global__ __launch_bounds__(256) void prefill_split_kernel(PrefillArgs a) {
  __shared__ float S[QB][GQA][SPLIT];
  __shared__ float O[4][GQA][HD];
  __shared__ float ML[QB][GQA][2];

  const int wi = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = tid >> 4, dl = tid & 15;
  const int row0 = a.work[4 * wi], nq = a.work[4 * wi + 1], b = a.work[4 * wi + 2], s = a.work[4 * wi + 3];
  const int t0 = s * SPLIT;
  const int nt_max = min(SPLIT, a.pos[row0 + nq - 1] + 1 - t0);
  const int32_t* bt = a.bt + (int64_t)b * a.max_pages + t0 / PAGE;
  const int64_t head_stride = (int64_t)PAGE * HD;
  const int64_t page_stride = (int64_t)a.hkv * head_stride;
  const int64_t slot_off = (int64_t)g * head_stride + (int64_t)grp * HD + dl * 8;

  split_scores<QB>(a.q + ((int64_t)row0 * a.hq + g * GQA) * HD, (int64_t)a.hq * HD, nq,
                   [&](int t) { return min(SPLIT, a.pos[row0 + t] + 1 - t0); }, a.kp, bt, page_stride,
                   (int64_t)g * head_stride, wave, lane, a.qscale, S);
  __syncthreads();
  for (int r = wave; r < nq * GQA; r += 4) {
    float mx, l;
    split_softmax_row(S[r / GQA][r % GQA], lane, mx, l);
    if (lane == 0) {
      ML[r / GQA][r % GQA][0] = mx;
      ML[r / GQA][r % GQA][1] = l;
    }
  }
  __syncthreads();
  u32x4 kv[PPS];
  load_kv(a.vp, bt, page_stride, slot_off, grp, nt_max, kv);
  for (int t = 0; t < nq; ++t) {
    const int row = row0 + t;
    const bool sees = a.pos[row] + 1 - t0 > 0;
    float o[GQA][8];
    split_pv(kv, S[t], grp, o);
    if (lane < 16) {
#pragma unroll
      for (int h = 0; h < GQA; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) O[wave][h][dl * 8 + e] = o[h][e];
    }
    __syncthreads();
    if (sees) {
      const int64_t base = (int64_t)(a.qoffs[row] + s) * a.hq + g * GQA;
      write_partial(O, tid, a.ws_o + base * HD);
      if (tid < GQA) {
        a.ws_ml[(base + tid) * 2 + 0] = ML[t][tid][0];
        a.ws_ml[(base + tid) * 2 + 1] = ML[t][tid][1];
      }
    }
    __syncthreads();
  }
}

// Combine: one workgroup of 256 threads per (sequence, query head), as 8
// groups of 32 lanes; lane c of a group owns o[4c .. 4c+3]. Group r folds the
// splits s = r, r + 8, r + 16, ... in increasing order (m, l, o weighted by
// 2^(m_s - M)); the 8 group sums are then added as
// ((g0 + g1) + (g2 + g3)) + ((g4 + g5) + (g6 + g7)). The order depends only on
// the sequence's split count, and the 8 chains cut the dependent-load chain of
// a 128-split sequence to 16 steps.
__global__ __launch_bounds__(256) void decode_combine_kernel(const int32_t* __restrict__ offs,
                                                              const float* __restrict__ ws_o,
                                                              const float* __restrict__ ws_ml, int hq,
                                                              void* __restrict__ out, int out_bf16) {
  __shared__ float red[4];
  __shared__ float4 po[8][HD / 4];
  __shared__ float pl[8];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid >> 5, c = tid & 31;
  const int w0 = offs[b], ns = offs[b + 1] - w0;
  // exact max of the split maxima (max is order-free)
  float M = -INFINITY;
  for (int s = tid; s < ns; s += 256) M = fmaxf(M, ws_ml[((int64_t)(w0 + s) * hq + h) * 2]);
  M = wave_max(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  float l = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  auto fold = [&](const float2 ml, const float4 ov) {
    const float w = __builtin_amdgcn_exp2f(ml.x - M);
    l = l + w * ml.y;
    o.x = o.x + w * ov.x;
    o.y = o.y + w * ov.y;
    o.z = o.z + w * ov.z;
    o.w = o.w + w * ov.w;
  };
  auto part = [&](int s, float2& ml, float4& ov) {
    const int64_t ph = (int64_t)(w0 + s) * hq + h;
    ml = *reinterpret_cast<const float2*>(ws_ml + ph * 2);
    ov = *reinterpret_cast<const float4*>(ws_o + ph * HD + 4 * c);
  };
  int s = r;
  for (; s + 8 < ns; s += 16) {  // two splits of this group per trip, folded in order
    float2 ml0, ml1;
    float4 o0, o1;
    part(s, ml0, o0);
    part(s + 8, ml1, o1);
    fold(ml0, o0);
    fold(ml1, o1);
  }
  if (s < ns) {
    float2 ml0;
    float4 o0;
    part(s, ml0, o0);
    fold(ml0, o0);
  }
  po[r][c] = o;
  if (c == 0) pl[r] = l;
  __syncthreads();
  if (tid < HD / 4) {
    float4 t[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) t[q] = po[q][tid];
    auto add = [](float4 x, float4 y) { return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w); };
    const float4 os = add(add(add(t[0], t[1]), add(t[2], t[3])), add(add(t[4], t[5]), add(t[6], t[7])));
    const float ls = ((pl[0] + pl[1]) + (pl[2] + pl[3])) + ((pl[4] + pl[5]) + (pl[6] + pl[7]));
    const float res[4] = {os.x / ls, os.y / ls, os.z / ls, os.w / ls};
    const int64_t at = ((int64_t)b * hq + h) * HD + 4 * tid;
    // element stores: out need only be aligned to its element size
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (out_bf16)
        reinterpret_cast<uint16_t*>(out)[at + e] = (uint16_t)f32_to_bf16_rne(res[e]);
      else
        reinterpret_cast<float*>(out)[at + e] = res[e];
    }
  }
}

}  // namespace

hipError_t launch_decode_attention(const DecodeParams& p, hipStream_t s) {
  SplitArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kp = static_cast<const uint16_t*>(p.k_pages);
  a.vp = static_cast<const uint16_t*>(p.v_pages);
  a.bt = p.block_table;
  a.lens = p.context_lens;
  a.offs = p.split_offsets;
  a.max_pages = p.max_pages;
  a.batch = (int)p.batch;
  a.hq = p.num_q_heads;
  a.hkv = p.num_kv_heads;
  a.qscale = p.scale * LOG2E;
  a.ws_o = p.ws_o;
  a.ws_ml = p.ws_ml;
  hipLaunchKernelGGL(decode_split_kernel, dim3((unsigned)(p.total_splits * p.num_kv_heads)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)p.batch, (unsigned)p.num_q_heads), dim3(256), 0, s,
                     p.split_offsets, p.ws_o, p.ws_ml, p.num_q_heads, p.out, p.out_bf16 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_prefill_attention(const PrefillParams& p, hipStream_t s) {
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(p.q);
  a.kp = static_cast<const uint16_t*>(p.k_pages);
  a.vp = static_cast<const uint16_t*>(p.v_pages);
  a.bt = p.block_table;
  a.pos = p.q_pos;
  a.qoffs = p.q_offsets;
  a.work = p.work;
  a.max_pages = p.max_pages;
  a.hq = p.num_q_heads;
  a.hkv = p.num_kv_heads;
  a.qscale = p.scale * LOG2E;
  a.ws_o = p.ws_o;
  a.ws_ml = p.ws_ml;
  hipLaunchKernelGGL(prefill_split_kernel, dim3((unsigned)(p.n_work * p.num_kv_heads)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)p.n_rows, (unsigned)p.num_q_heads), dim3(256), 0, s,
                     p.q_offsets, p.ws_o, p.ws_ml, p.num_q_heads, p.out, p.out_bf16 ? 1 : 0);
  return hipGetLastError();
}

int prefill_rows_per_item() { return QB; }

}  // namespace bi
