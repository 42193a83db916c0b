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
// Kernel 1, one workgroup per (split, kv head), 4 waves of 64 lanes; both
// matrix phases use v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//   phase 1: scores of the GQA query heads sharing this kv head against the
//            split's keys (wave w: keys [64 w, 64 w + 64)), K fragments read
//            straight from the page; kept in LDS in the log2 domain (raw dot
//            times scale * log2(e)).
//   phase 2: wave h (one per query head) takes the exact max over the split,
//            forms p = 2^(s - max), sums it, and writes p back as bf16 hi + lo.
//   phase 3: o = sum_t p_t v_t (wave w: head-dim columns [32 w, 32 w + 32)
//            over all the split's keys), V fragments read straight from the
//            d-major page.
//   output : (max, sum p, o[128]) per (split, query head), fp32.
// Kernel 2, one workgroup per (sequence, query head):
//   M = max_s m_s; l = sum_s 2^(m_s - M) l_s; o = sum_s 2^(m_s - M) o_s[d],
//   each sum taken as 8 chains (splits s = r mod 8, increasing s) added in a
//   fixed tree; out = o / l.
#include "bi_internal.h"
#include "device_common.h"

#include <type_traits>

namespace bi {
namespace {

constexpr int HD = 128;     // head dim
constexpr int PAGE = 16;    // tokens per page
constexpr int SPLIT = 256;  // tokens per split
constexpr int GQA = 4;      // query heads per kv head
constexpr int SROW = SPLIT + 4;  // LDS row stride (floats) of a score row, padded against bank conflicts
// Phase 2 rewrites a row of SROW floats as bf16 parts of p: hi at u16
// [0, SPLIT), lo at u16 [PLO, PLO + SPLIT) (16-byte aligned, inside the row).
constexpr int PLO = SPLIT;
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
// them. Cache layout per physical page: K [kv head][slot][d] (a key is a
// contiguous row), V [kv head][d][slot] (a head-dim row of the page's tokens
// is contiguous), both bf16; PAGE slots per page.
// ---------------------------------------------------------------------------

// Loads. A split's page numbers are read as wave-uniform (scalar) values;
// every fragment is loaded, unconditionally, before the first is used, in
// the order q, K, V, so that the wait for q and K leaves V in flight through
// phases 1 and 2 (a load under a branch would make the compiler wait for it
// at the join). npg >= 1 is the number of pages holding the keys the block
// can see; a tile past it reads the last of them instead (in bounds; its keys
// are masked where they are used).

// K fragments: wave w covers keys [64 w, 64 w + 64) as four 16-key tiles,
// tile kt being slots 0..15 of page 4 w + kt. The MFMA B operand of a 32-wide
// d step (lane l: key l % 16, d 8 (l / 16) .. +7) is one 16-byte load of the
// key row.
// NT: non-temporal loads (the BI_DECODE_STREAM_KV hint of bi_decode_attention).
template <bool NT>
__device__ __forceinline__ void load_k_frags(const uint16_t* kp, const int32_t* bt, int npg, int64_t page_stride,
                                             int64_t head_off, int wave, int lane, u32x4 (&kf)[4][4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const uint16_t* base = kp + (int64_t)bt[min(4 * wave + kt, npg - 1)] * page_stride + head_off +
                           (lane & 15) * HD + 8 * (lane >> 4);
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const u32x4* p = reinterpret_cast<const u32x4*>(base + 32 * ds);
      if constexpr (NT) kf[kt][ds] = __builtin_nontemporal_load(p);
      else kf[kt][ds] = *p;
    }
  }
}

// q fragments (the MFMA A operand) of one block of 16 query rows -- 4
// tokens from q0 on, the GQA heads of each: lane l feeds row r = l % 16
// (token r / GQA, head r % GQA), d 8 (l / 16) .. +7 of each 32-wide step.
// Rows of tokens >= ntok repeat the block's first token (in bounds; those
// rows of the products are never stored).
__device__ __forceinline__ void load_q_block(const uint16_t* q0, int64_t q_tok_stride, int ntok, int lane,
                                             u32x4 (&qa)[4]) {
  const int r = lane & 15;
  const int t = r / GQA < ntok ? r / GQA : 0;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
    qa[ds] = *reinterpret_cast<const u32x4*>(q0 + t * q_tok_stride + (r % GQA) * HD + 32 * ds + 8 * (lane >> 4));
}

// V fragments, the B operand of phase 3: V pages are stored d-major
// ([page][kv head][d][slot]), so for key step ks (keys [32 ks, 32 ks + 32),
// pages 2 ks and 2 ks + 1) lane l's operand -- column d, keys 8 (l / 16) .. +7
// -- is one 16-byte load of a d-row of one page. Wave w owns the columns
// d in [32 w, 32 w + 32), two 16-wide tiles, over all the split's keys.
template <bool NT>
__device__ __forceinline__ void load_v_frags(const uint16_t* vp, const int32_t* bt, int npg, int64_t page_stride,
                                             int64_t head_off, int wave, int lane, u32x4 (&vf)[8][2]) {
  const int q4 = lane >> 4;
  const int d = 32 * wave + (lane & 15);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int32_t p0 = bt[min(2 * ks, npg - 1)], p1 = bt[min(2 * ks + 1, npg - 1)];
    const uint16_t* base = vp + (int64_t)((q4 >> 1) ? p1 : p0) * page_stride + head_off + d * PAGE + 8 * (q4 & 1);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const u32x4* p = reinterpret_cast<const u32x4*>(base + 16 * dt * PAGE);
      if constexpr (NT) vf[ks][dt] = __builtin_nontemporal_load(p);
      else vf[ks][dt] = *p;
    }
  }
}

// Phase 1 for one block of 16 query rows (4 tokens x the GQA heads): the
// scores S[t][h][key] of the split's SPLIT keys, t < ntok tokens of the
// block, on the matrix cores:
//   S = (sum_d q[r][d] k[key][d]) * qscale   (qscale = scale * log2(e)),
// the sum taken by v_mfma_f32_16x16x32_bf16 over d in four steps of 32
// (exact bf16 products, fp32 accumulation, increasing d), then one fp32
// multiply; keys at or past nt_of(t) get -inf. Rows past GQA ntok are not
// stored. The element (r, key) gets the same chain whichever row of the MFMA
// holds r, so a token's scores do not depend on the other tokens of the block.
template <typename NtOf>
__device__ __forceinline__ void scores_block(const u32x4 (&qa)[4], const u32x4 (&kf)[4][4], int ntok, NtOf nt_of,
                                             int wave, int lane, float qscale, float (*S)[GQA][SROW]) {
  const int t_out = lane >> 4;  // token of the 4 rows this lane receives (GQA == 4)
  const int nt_t = t_out < ntok ? nt_of(t_out) : 0;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[ds]),
                                                    __builtin_bit_cast(bf16x8, kf[kt][ds]), acc, 0, 0, 0);
    const int key = 64 * wave + 16 * kt + (lane & 15);
    if (t_out < ntok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[t_out][i][key] = key < nt_t ? acc[i] * qscale : -INFINITY;
    }
  }
}

// Reduction over a full wave without LDS traffic: DPP moves pair lanes
// inside each 16-lane row (xor 1, xor 2, then i <-> 7 - i within 8, then
// i <-> 15 - i within 16), readlane takes the four row totals, combined as
// (r0 op r1) op (r2 op r3). op is commutative, so every lane ends with the
// same bits, and the order is fixed.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_move<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));  // row_half_mirror
  v = op(v, dpp_move<0x140>(v));  // row_mirror
  auto lane_v = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
  return op(op(lane_v(0), lane_v(16)), op(lane_v(32), lane_v(48)));
}

// Phase 2, R rows (query, head) by one wave: for each row, the exact max,
// p = 2^(s - max), l = sum p in fp32 (per-lane order, then wave_reduce).
// p is written back over the row as two bf16 parts, hi = RNE(p)
// and lo = RNE(p - hi) (the difference is exact in fp32), the A operand of
// phase 3. A row's whole contents are in registers (mx depends on every
// element) before its first write. The cross-lane steps are wave_reduce's;
// each row's arithmetic is the same whatever R is.
template <int R>
__device__ __forceinline__ void split_softmax_rows(float* const (&row)[R], int lane, float (&mx_out)[R],
                                                   float (&l_out)[R]) {
  float v[R][SPLIT / 64], mx[R], l[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    mx[i] = -INFINITY;
#pragma unroll
    for (int r = 0; r < SPLIT / 64; ++r) {
      v[i][r] = row[i][lane + 64 * r];
      mx[i] = fmaxf(mx[i], v[i][r]);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) mx[i] = wave_reduce(mx[i], [](float x, float y) { return fmaxf(x, y); });
#pragma unroll
  for (int i = 0; i < R; ++i) {
    l[i] = 0.0f;
    uint16_t* pb = reinterpret_cast<uint16_t*>(row[i]);
#pragma unroll
    for (int r = 0; r < SPLIT / 64; ++r) {
      const float pr = __builtin_amdgcn_exp2f(v[i][r] - mx[i]);  // 2^-inf = 0 for masked slots
      const uint32_t hb = f32_to_bf16_rne(pr);
      pb[lane + 64 * r] = (uint16_t)hb;
      pb[PLO + lane + 64 * r] = (uint16_t)f32_to_bf16_rne(pr - __uint_as_float(hb << 16));
      l[i] = l[i] + pr;
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) l[i] = wave_reduce(l[i], [](float x, float y) { return x + y; });
#pragma unroll
  for (int i = 0; i < R; ++i) {
    mx_out[i] = mx[i];
    l_out[i] = l[i];
  }
}

// Phase 3 on the matrix cores: the split's partial output
//   O[r][d] = sum over its SPLIT keys of p[r][key] v[key][d]
// for one block of 16 query rows (4 tokens x the GQA heads), by
// v_mfma_f32_16x16x32_bf16 with A = p and B = v (fragments from
// load_v_frags). No partial crosses waves: wave w owns columns [32 w, 32 w + 32).
// p enters as its two bf16 parts hi + lo (written by phase 2), so the
// products carry ~16 bits of p; the chain per element is: key steps of 32 in
// increasing order, hi then lo in each, fp32 accumulation. V of keys at or
// past nt is zeroed here (the cache past a sequence's last token may hold
// any bits, and 0 * NaN would poison the sum). acc[dt] = the wave's tile dt:
// lane l holds rows 16 rb + 4 (l / 16) + i (i = 0..3), i.e. token
// 4 rb + l / 16 and GQA head i, column d = 32 w + 16 dt + l % 16. Rows of
// tokens >= ntok repeat token 0's p (never stored).
__device__ __forceinline__ void split_pv(const u32x4 (&vf)[8][2], const float (*S)[GQA][SROW], int rb, int ntok,
                                         int nt, int lane, f32x4 (&acc)[2]) {
  const int r = 16 * rb + (lane & 15);  // the query row this lane feeds
  const int t = r / GQA;
  const int q4 = lane >> 4;
  const uint16_t* prow = reinterpret_cast<const uint16_t*>(S[t < ntok ? t : 0][r % GQA]) + 8 * q4;
  acc[0] = acc[1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const u32x4 hi = *reinterpret_cast<const u32x4*>(prow + 32 * ks);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(prow + PLO + 32 * ks);
    const int valid = nt - (32 * ks + 8 * q4);  // keys of this lane's 8 that exist
    u32x4 keep;
#pragma unroll
    for (int e = 0; e < 4; ++e) keep[e] = (2 * e < valid ? 0xFFFFu : 0u) | (2 * e + 1 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, vf[ks][dt] & keep);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), v, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo), v, acc[dt], 0, 0, 0);
    }
  }
}

// The wave's share of a row block's partials, for the token of this lane's
// rows: out points at that token's [GQA][HD] fp32 partial (or is null).
__device__ __forceinline__ void store_pv(const f32x4 (&acc)[2], int wave, int lane, float* out) {
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i * HD + 32 * wave + 16 * dt + (lane & 15)] = acc[dt][i];
}

template <bool NT>
__global__ __launch_bounds__(256) void decode_split_kernel(SplitArgs a) {
  __shared__ float S[1][GQA][SROW];

  // The kv heads of one split are adjacent in dispatch order, so the 4 KB
  // head slices of a physical page (all heads, 32 KB at 8 heads) are read at
  // about the same time.
  const int w = blockIdx.x / a.hkv;  // global split index
  const int g = blockIdx.x % a.hkv;  // kv head
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The grid may cover more splits than exist (the host passes an upper
  // bound so one captured launch serves growing lengths): the exact count is
  // split_offsets[batch], and workgroups past it have nothing to do.
  const int total = a.offs[a.batch];

  // The sequence owning split w: the one b with offs[b] <= w < offs[b+1]
  // (lengths are >= 1, so the offsets increase strictly). Every thread reads
  // its sequences' offsets and length with coalesced loads issued together
  // with the count above (one memory round trip per 256 sequences), and the
  // owner passes (b, s, L) through LDS.
  __shared__ int sinfo[3];
  for (int base = 0; base < a.batch; base += 256) {
    const int t = base + tid;
    if (t < a.batch) {
      const int o0 = a.offs[t], o1 = a.offs[t + 1], len = a.lens[t];
      // all three loads in flight together (not sunk into the branches below)
      asm volatile("" ::"v"(o0), "v"(o1), "v"(len));
      if (o0 <= w && w < o1) {
        sinfo[0] = t;
        sinfo[1] = w - o0;
        sinfo[2] = len;
      }
    }
  }
  if (w >= total) return;  // uniform over the workgroup
  __syncthreads();
  const int b = __builtin_amdgcn_readfirstlane(sinfo[0]);
  const int s = __builtin_amdgcn_readfirstlane(sinfo[1]);
  const int L = __builtin_amdgcn_readfirstlane(sinfo[2]);
  const int t0 = s * SPLIT;
  const int nt = min(SPLIT, L - t0);
  const int npg = (nt + PAGE - 1) / PAGE;
  const int32_t* bt = a.bt + (int64_t)b * a.max_pages + t0 / PAGE;

  const int64_t head_stride = (int64_t)PAGE * HD;           // one head-page
  const int64_t page_stride = (int64_t)a.hkv * head_stride;  // one physical page
  const int64_t head_off = (int64_t)g * head_stride;

  u32x4 qa[4], kf[4][4], vf[8][2];
  load_q_block(a.q + ((int64_t)b * a.hq + g * GQA) * HD, 0, 1, lane, qa);
  load_k_frags<NT>(a.kp, bt, npg, page_stride, head_off, wave, lane, kf);
  load_v_frags<NT>(a.vp, bt, npg, page_stride, head_off, wave, lane, vf);
  __builtin_amdgcn_sched_barrier(0);  // every load issued before the first MFMA waits
  scores_block(qa, kf, 1, [&](int) { return nt; }, wave, lane, a.qscale, S);
  __syncthreads();
  const int64_t base = (int64_t)w * a.hq + g * GQA;  // partial row of (split w, query head g GQA)
  {
    float mx[1], l[1];
    float* const rows[1] = {S[0][wave]};
    split_softmax_rows<1>(rows, lane, mx, l);  // wave h: query head h
    if (lane == 0) {
      a.ws_ml[(base + wave) * 2 + 0] = mx[0];
      a.ws_ml[(base + wave) * 2 + 1] = l[0];
    }
  }
  __syncthreads();
  f32x4 acc[2];
  split_pv(vf, S, 0, 1, nt, lane, acc);
  if (lane < 16) store_pv(acc, wave, lane, a.ws_o + base * HD);  // rows 0..3: the one token
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
// K and V are loaded once into registers for all of them (keys past the last
// row's nt read 0); the rows then go through the three phases 4 tokens (16
// query rows) at a time, through one block-sized score array in LDS. For an
// earlier row, the keys it must not see carry p = 0, and their products (0
// times a finite cached value) add exact zeros.
// ---------------------------------------------------------------------------
constexpr int QB = 32;

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
  __shared__ float S[4][GQA][SROW];  // one block of 4 tokens

  const int wi = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = a.work[4 * wi], nq = a.work[4 * wi + 1], b = a.work[4 * wi + 2], s = a.work[4 * wi + 3];
  const int t0 = s * SPLIT;
  const int nt_max = min(SPLIT, a.pos[row0 + nq - 1] + 1 - t0);
  const int npg = (nt_max + PAGE - 1) / PAGE;
  const int32_t* bt = a.bt + (int64_t)b * a.max_pages + t0 / PAGE;
  const int64_t head_stride = (int64_t)PAGE * HD;
  const int64_t page_stride = (int64_t)a.hkv * head_stride;
  const int64_t head_off = (int64_t)g * head_stride;
  const int64_t q_tok = (int64_t)a.hq * HD;
  const uint16_t* q0 = a.q + ((int64_t)row0 * a.hq + g * GQA) * HD;
  // the item's row positions and split offsets, read once into LDS (each
  // row block needs them three times)
  __shared__ int spos[QB], soff[QB];
  if (tid < nq) {
    spos[tid] = a.pos[row0 + tid];
    soff[tid] = a.qoffs[row0 + tid];
  }
  // partial row of (chunk row row0 + t, split s, query head g GQA), or -1
  // when that row's position is before the split (it does not see it)
  auto part_row = [&](int t) -> int64_t {
    return spos[t] + 1 - t0 > 0 ? (int64_t)(soff[t] + s) * a.hq + g * GQA : -1;
  };

  u32x4 qa[4], qn[4], kf[4][4], vf[8][2];
  load_q_block(q0, q_tok, min(4, nq), lane, qa);
  load_k_frags<false>(a.kp, bt, npg, page_stride, head_off, wave, lane, kf);
  load_v_frags<false>(a.vp, bt, npg, page_stride, head_off, wave, lane, vf);
  __builtin_amdgcn_sched_barrier(0);  // every load issued before the first MFMA waits
  __syncthreads();                    // spos, soff
  for (int tb = 0; tb < nq; tb += 4) {  // tokens tb .. tb + 3 of the item
    const int nb = min(4, nq - tb);
    if (tb + 4 < nq) load_q_block(q0 + (tb + 4) * q_tok, q_tok, min(4, nq - tb - 4), lane, qn);  // next block
    scores_block(qa, kf, nb, [&](int t) { return min(SPLIT, spos[tb + t] + 1 - t0); }, wave, lane, a.qscale, S);
    __syncthreads();
    {
      // wave h: head h of the block's 4 tokens (rows of tokens >= nb hold
      // nothing of use; they are processed and never read)
      float mx[4], l[4];
      float* const rows[4] = {S[0][wave], S[1][wave], S[2][wave], S[3][wave]};
      split_softmax_rows<4>(rows, lane, mx, l);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < nb) {
          const int64_t base = part_row(tb + t);
          if (lane == 0 && base >= 0) {
            a.ws_ml[(base + wave) * 2 + 0] = mx[t];
            a.ws_ml[(base + wave) * 2 + 1] = l[t];
          }
        }
      }
    }
    __syncthreads();
    f32x4 acc[2];
    split_pv(vf, S, 0, nb, nt_max, lane, acc);
    const int t = lane >> 4;
    if (t < nb) {
      const int64_t base = part_row(tb + t);
      if (base >= 0) store_pv(acc, wave, lane, a.ws_o + base * HD);
    }
    __syncthreads();  // the next block's scores overwrite S
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qa[ds] = qn[ds];
  }
}

// Combine: one workgroup of two waves per (sequence, query head). The split
// partials are folded in 8 groups: group g takes the splits s = g, g + 8,
// g + 16, ... in increasing order (m, l, o weighted by 2^(m_s - M), M the
// exact max of the split maxima), and the 8 group sums are added as
// ((g0 + g1) + (g2 + g3)) + ((g4 + g5) + (g6 + g7)). The order depends only on
// the sequence's split count. The 32-lane quarter q of the workgroup holds
// groups q and q + 4, lane c owning o[4c .. 4c+3]; the tree's first level
// pairs quarters inside a wave, the second goes through LDS. A row of up to
// 8 splits (a context of up to 2048 tokens; almost every prefill row) loads
// its partials at once and takes the max from the loaded values: one memory
// round trip. Longer rows first take the max, then fold 32 splits per trip.
// Two waves per row keep 12 rows per CU in flight (76 VGPRs).
__global__ __launch_bounds__(128) void decode_combine_kernel(const int32_t* __restrict__ offs,
                                                              const float* __restrict__ ws_o,
                                                              const float* __restrict__ ws_ml, int hq,
                                                              void* __restrict__ out, int out_bf16) {
  __shared__ float red[2];
  __shared__ float4 po[2][HD / 4];
  __shared__ float pl[2];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int pg = tid >> 5, c = tid & 31, wv = tid >> 6;
  const int w0 = offs[b], ns = offs[b + 1] - w0;
  float l[2] = {0.0f, 0.0f};
  float4 o[2] = {make_float4(0.0f, 0.0f, 0.0f, 0.0f), make_float4(0.0f, 0.0f, 0.0f, 0.0f)};
  float M = -INFINITY;
  auto wg_max = [&](float v) {
    v = wave_max(v);
    if ((tid & 63) == 0) red[wv] = v;
    __syncthreads();
    return fmaxf(red[0], red[1]);
  };
  auto part = [&](int s, float2& ml, float4& ov) {
    const int64_t ph = (int64_t)(w0 + s) * hq + h;
    ml = *reinterpret_cast<const float2*>(ws_ml + ph * 2);
    ov = *reinterpret_cast<const float4*>(ws_o + ph * HD + 4 * c);
  };
  auto fold = [&](int j, const float2 ml, const float4 ov) {
    const float w = __builtin_amdgcn_exp2f(ml.x - M);
    l[j] = l[j] + w * ml.y;
    o[j].x = o[j].x + w * ov.x;
    o[j].y = o[j].y + w * ov.y;
    o[j].z = o[j].z + w * ov.z;
    o[j].w = o[j].w + w * ov.w;
  };
  if (ns >= 1 && ns <= 8) {
    float2 mls[2];
    float4 ovs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) part(min(pg + 4 * j, ns - 1), mls[j], ovs[j]);
    M = wg_max(fmaxf(mls[0].x, mls[1].x));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (pg + 4 * j < ns) fold(j, mls[j], ovs[j]);
  } else {
    float m = -INFINITY;
    for (int s = tid; s < ns; s += 128) m = fmaxf(m, ws_ml[((int64_t)(w0 + s) * hq + h) * 2]);
    M = wg_max(m);
    for (int t0 = 0; t0 < ns; t0 += 32) {  // splits t0 .. t0 + 31: four per group, in order
      float2 mls[4][2];
      float4 ovs[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 2; ++j) part(min(t0 + 8 * u + pg + 4 * j, ns - 1), mls[u][j], ovs[u][j]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (t0 + 8 * u + pg + 4 * j < ns) fold(j, mls[u][j], ovs[u][j]);
    }
  }
  // wave 0 holds groups 0, 1, 4, 5, wave 1 groups 2, 3, 6, 7
  float lt[2];
  float4 ot[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // g(4j + 2wv) + g(4j + 2wv + 1)
    lt[j] = l[j] + xor_shfl(l[j], 32);
    ot[j].x = o[j].x + xor_shfl(o[j].x, 32);
    ot[j].y = o[j].y + xor_shfl(o[j].y, 32);
    ot[j].z = o[j].z + xor_shfl(o[j].z, 32);
    ot[j].w = o[j].w + xor_shfl(o[j].w, 32);
  }
  if (wv == 1 && (tid & 63) < 32) {
    po[0][c] = ot[0];
    po[1][c] = ot[1];
    if (c == 0) {
      pl[0] = lt[0];
      pl[1] = lt[1];
    }
  }
  __syncthreads();
  if (tid < 32) {
    auto add = [](float4 x, float4 y) { return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w); };
    const float4 os = add(add(ot[0], po[0][c]), add(ot[1], po[1][c]));
    const float ls = (lt[0] + pl[0]) + (lt[1] + pl[1]);
    const float res[4] = {os.x / ls, os.y / ls, os.z / ls, os.w / ls};
    const int64_t at = ((int64_t)b * hq + h) * HD + 4 * c;
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
  if (p.stream_kv)
    hipLaunchKernelGGL(decode_split_kernel<true>, dim3((unsigned)(p.total_splits * p.num_kv_heads)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(decode_split_kernel<false>, dim3((unsigned)(p.total_splits * p.num_kv_heads)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)p.batch, (unsigned)p.num_q_heads), dim3(128), 0, s,
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
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)p.n_rows, (unsigned)p.num_q_heads), dim3(128), 0, s,
                     p.q_offsets, p.ws_o, p.ws_ml, p.num_q_heads, p.out, p.out_bf16 ? 1 : 0);
  return hipGetLastError();
}

int prefill_rows_per_item() { return QB; }

}  // namespace bi
