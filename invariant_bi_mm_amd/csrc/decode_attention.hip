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
#include "bi.h"
#include "bi_internal.h"
#include "device_common.h"

#include <climits>
#include <cstdint>
#include <mutex>
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
// scores S[t][h][key] of the split's SPLIT keys on the matrix cores:
//   S = (sum_d q[r][d] k[key][d]) * qscale   (qscale = scale * log2(e)),
// the sum taken by v_mfma_f32_16x16x32_bf16 over d in four steps of 32
// (exact bf16 products, fp32 accumulation, increasing d), then one fp32
// multiply; keys at or past a token's visible count get -inf. The element
// (r, key) gets the same chain whichever row of the MFMA holds r, so a
// token's scores do not depend on the other tokens of the block. Wave w
// computes keys [64 w, 64 w + 64) as four 16-key tiles; lane l receives the
// rows of token l / 16 (its 4 GQA heads) at key l % 16 of each tile.
//
// scores_step: one d step of the wave's four independent tile chains (FIRST:
// the chains start here, from zeros); scores_store: tile kt's scores of the
// lane's token into S; scores_block: the whole block, for the decode kernel
// (rows of tokens >= ntok are not stored).
template <bool FIRST>
__device__ __forceinline__ void scores_step(const u32x4 (&qa)[4], const u32x4 (&kf)[4][4], int ds, f32x4 (&acc)[4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
    acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[ds]),
                                                      __builtin_bit_cast(bf16x8, kf[kt][ds]),
                                                      FIRST ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[kt], 0, 0, 0);
}
__device__ __forceinline__ void scores_store(const f32x4& acc, int kt, int t_out, int nt_t, int wave, int lane,
                                             float qscale, float (*S)[GQA][SROW]) {
  const int key = 64 * wave + 16 * kt + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) S[t_out][i][key] = key < nt_t ? acc[i] * qscale : -INFINITY;
}
template <typename NtOf>
__device__ __forceinline__ void scores_block(const u32x4 (&qa)[4], const u32x4 (&kf)[4][4], int ntok, NtOf nt_of,
                                             int wave, int lane, float qscale, float (*S)[GQA][SROW]) {
  const int t_out = lane >> 4;  // token of the 4 rows this lane receives (GQA == 4)
  f32x4 acc[4];
  scores_step<true>(qa, kf, 0, acc);
#pragma unroll
  for (int ds = 1; ds < 4; ++ds) scores_step<false>(qa, kf, ds, acc);
  if (t_out < ntok) {
    const int nt_t = nt_of(t_out);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) scores_store(acc[kt], kt, t_out, nt_t, wave, lane, qscale, S);
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
    for (int r = 0; r < SPLIT / 64; r += 2) {  // two keys per conversion
      const float p0 = __builtin_amdgcn_exp2f(v[i][r] - mx[i]);  // 2^-inf = 0 for masked slots
      const float p1 = __builtin_amdgcn_exp2f(v[i][r + 1] - mx[i]);
      const uint32_t hb = cvt_pk_bf16(p0, p1);
      const uint32_t lb = cvt_pk_bf16(p0 - bf16lo(hb), p1 - bf16hi(hb));
      pb[lane + 64 * r] = (uint16_t)hb;
      pb[lane + 64 * (r + 1)] = (uint16_t)(hb >> 16);
      pb[PLO + lane + 64 * r] = (uint16_t)lb;
      pb[PLO + lane + 64 * (r + 1)] = (uint16_t)(lb >> 16);
      l[i] = l[i] + p0;
      l[i] = l[i] + p1;
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

// Phase 2 for four rows at once, 16 lanes per row (the prefill form), in
// stages that the prefill kernel interleaves with matrix instructions: lane
// 16 t + j holds, of row t, the keys 4 j + i + 64 k (i, k = 0..3). The values
// are those of split_softmax_rows, and so is every rounding: the max is exact
// in any order; p, hi and lo are per element; and the sum is the same tree of
// additions. In split_softmax_rows lane L (0..63) first chains keys L,
// L + 64, L + 128, L + 192 from 0, then the lanes are paired by the bits of L
// from the lowest up (xor 1, xor 2, xor 4, xor 8 inside each 16, then
// (R0 + R1) + (R2 + R3) over the four 16-lane rows). Here L = 4 j + i: the
// chains and the first two levels are in the lane, the next four are DPP
// moves inside the 16-lane row (after the first two of them the four lanes
// of a quad hold equal sums, so the half-mirror and mirror moves pair L's
// bits 4 and 5). Every addition adds the same two values, and addition is
// commutative, so the bits are equal.
struct QuadSoftmax {
  f32x4 v[SPLIT / 64];  // this lane's scores; group k becomes p in exp_group(k)
  float mx;
  float leaf[4];
  __device__ __forceinline__ void load(const float* row, int j) {
#pragma unroll
    for (int k = 0; k < SPLIT / 64; ++k) v[k] = *reinterpret_cast<const f32x4*>(row + 4 * j + 64 * k);
  }
  __device__ __forceinline__ void max_lane() {
    mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < SPLIT / 64; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, v[k][i]);
  }
  __device__ __forceinline__ void max_row() {
    auto fmx = [](float x, float y) { return fmaxf(x, y); };
    mx = fmx(mx, dpp_move<0xB1>(mx));   // quad_perm [1,0,3,2]
    mx = fmx(mx, dpp_move<0x4E>(mx));   // quad_perm [2,3,0,1]
    mx = fmx(mx, dpp_move<0x141>(mx));  // row_half_mirror
    mx = fmx(mx, dpp_move<0x140>(mx));  // row_mirror
  }
  // group k: p = 2^(s - max) in place (2^-inf = 0 for masked slots)
  __device__ __forceinline__ void exp_group(int k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[k][i] = __builtin_amdgcn_exp2f(v[k][i] - mx);
  }
  // group k (groups in increasing order): p's bf16 parts written over the
  // row (hi at u16 4 j + 64 k, lo PLO further), p added to the lane's chains
  __device__ __forceinline__ void write_group(float* row, int j, int k) {
    uint16_t* pb = reinterpret_cast<uint16_t*>(row);
    const uint32_t h01 = cvt_pk_bf16(v[k][0], v[k][1]), h23 = cvt_pk_bf16(v[k][2], v[k][3]);
    const uint32_t l01 = cvt_pk_bf16(v[k][0] - bf16lo(h01), v[k][1] - bf16hi(h01));
    const uint32_t l23 = cvt_pk_bf16(v[k][2] - bf16lo(h23), v[k][3] - bf16hi(h23));
    *reinterpret_cast<uint2*>(pb + 4 * j + 64 * k) = make_uint2(h01, h23);
    *reinterpret_cast<uint2*>(pb + PLO + 4 * j + 64 * k) = make_uint2(l01, l23);
#pragma unroll
    for (int i = 0; i < 4; ++i) leaf[i] = (k == 0 ? 0.0f : leaf[i]) + v[k][i];
  }
  __device__ __forceinline__ float sum_row() const {
    float l = (leaf[0] + leaf[1]) + (leaf[2] + leaf[3]);
    l = l + dpp_move<0xB1>(l);
    l = l + dpp_move<0x4E>(l);
    l = l + dpp_move<0x141>(l);
    l = l + dpp_move<0x140>(l);
    return l;
  }
};

// V of keys at or past nt is zeroed in the fragments themselves, once per
// split: the cache past a sequence's last token may hold any bits, and
// 0 * NaN would poison the sum. A full split (nt == SPLIT) has nothing to
// zero.
__device__ __forceinline__ void mask_v(u32x4 (&vf)[8][2], int nt, int lane) {
  if (nt >= SPLIT) return;  // uniform
  const int q4 = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int valid = nt - (32 * ks + 8 * q4);  // keys of this lane's 8 that exist
    u32x4 keep;
#pragma unroll
    for (int e = 0; e < 4; ++e) keep[e] = (2 * e < valid ? 0xFFFFu : 0u) | (2 * e + 1 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) vf[ks][dt] &= keep;
  }
}

// Phase 3 on the matrix cores: the split's partial output
//   O[r][d] = sum over its SPLIT keys of p[r][key] v[key][d]
// for one block of 16 query rows (4 tokens x the GQA heads), by
// v_mfma_f32_16x16x32_bf16 with A = p and B = v (fragments from
// load_v_frags, masked by mask_v). No partial crosses waves: wave w owns
// columns [32 w, 32 w + 32). p enters as its two bf16 parts hi + lo (written
// by phase 2), so the products carry ~16 bits of p; the chain per element
// is: key steps of 32 in increasing order, hi then lo in each, fp32
// accumulation. acc[dt] = the wave's tile dt: lane l holds rows
// 4 (l / 16) + i (i = 0..3), i.e. token l / 16 and GQA head i, column
// d = 32 w + 16 dt + l % 16. Rows of tokens >= ntok repeat token 0's p
// (never stored).
//
// pv_row: the lane's p row (the A operand's row l % 16); pv_operands: one
// key step's hi and lo operands from it; pv_step: that key step for both
// column tiles, hi then lo into each chain.
__device__ __forceinline__ const uint16_t* pv_row(const float (*S)[GQA][SROW], int ntok, int lane) {
  const int r = lane & 15;  // the query row this lane feeds
  const int t = r / GQA;
  return reinterpret_cast<const uint16_t*>(S[t < ntok ? t : 0][r % GQA]) + 8 * (lane >> 4);
}
__device__ __forceinline__ void pv_operands(const uint16_t* prow, int ks, u32x4& hi, u32x4& lo) {
  hi = *reinterpret_cast<const u32x4*>(prow + 32 * ks);
  lo = *reinterpret_cast<const u32x4*>(prow + PLO + 32 * ks);
}
template <bool FIRST>
__device__ __forceinline__ void pv_step(const u32x4 (&vf)[8][2], int ks, const u32x4& hi, const u32x4& lo,
                                        f32x4 (&acc)[2]) {
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi),
                                                      __builtin_bit_cast(bf16x8, vf[ks][dt]),
                                                      FIRST ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[dt], 0, 0, 0);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo),
                                                      __builtin_bit_cast(bf16x8, vf[ks][dt]), acc[dt], 0, 0, 0);
}
__device__ __forceinline__ void split_pv(const u32x4 (&vf)[8][2], const float (*S)[GQA][SROW], int ntok, int lane,
                                         f32x4 (&acc)[2]) {
  const uint16_t* prow = pv_row(S, ntok, lane);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 hi, lo;
    pv_operands(prow, ks, hi, lo);
    if (ks == 0) pv_step<true>(vf, ks, hi, lo, acc);
    else pv_step<false>(vf, ks, hi, lo, acc);
  }
}

// The wave's share of a row block's partials, for the token of this lane's
// rows: out points at that token's [GQA][HD] fp32 partial. NT: non-temporal
// stores (prefill's partials, written once and read back by the combine
// kernel after all of them).
template <bool NT>
__device__ __forceinline__ void store_pv(const f32x4 (&acc)[2], int wave, int lane, float* out) {
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* const at = out + i * HD + 32 * wave + 16 * dt + (lane & 15);
      if constexpr (NT) __builtin_nontemporal_store(acc[dt][i], at);
      else *at = acc[dt][i];
    }
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
  // with the count above (one memory round trip per 256 sequences). Each
  // wave passes the (b, s, L) its lanes found, or b = -1, through its own
  // LDS slot; after the barrier the first slot that holds an owner is used.
  // Offsets that name no owner for w, or a length that does not reach split
  // w or overruns the block table's row, leave the workgroup with nothing to
  // do (contents on the device are the caller's; this keeps every access in
  // bounds whatever they are).
  __shared__ int sinfo[4][3];
  int ob = -1, os = 0, ol = 0;
  for (int base = 0; base < a.batch; base += 256) {
    const int t = base + tid;
    if (t < a.batch) {
      const int o0 = a.offs[t], o1 = a.offs[t + 1], len = a.lens[t];
      // all three loads in flight together (not sunk into the branches below)
      asm volatile("" ::"v"(o0), "v"(o1), "v"(len));
      if (o0 <= w && w < o1) {
        ob = t;
        os = w - o0;
        ol = len;
      }
    }
  }
  if (w >= total) return;  // uniform over the workgroup
  {
    const uint64_t found = __ballot(ob >= 0);
    const int src = found ? (int)__builtin_ctzll(found) : 0;  // wave-uniform
    const int vb = found ? __builtin_amdgcn_readlane(ob, src) : -1;
    const int vs = __builtin_amdgcn_readlane(os, src), vl = __builtin_amdgcn_readlane(ol, src);
    if (lane == 0) {
      sinfo[wave][0] = vb;
      sinfo[wave][1] = vs;
      sinfo[wave][2] = vl;
    }
  }
  __syncthreads();
  int slot = 0;
  while (slot < 3 && sinfo[slot][0] < 0) ++slot;
  const int b = __builtin_amdgcn_readfirstlane(sinfo[slot][0]);
  const int s = __builtin_amdgcn_readfirstlane(sinfo[slot][1]);
  const int L = __builtin_amdgcn_readfirstlane(sinfo[slot][2]);
  const int64_t t0l = (int64_t)s * SPLIT;  // no overflow whatever the offsets
  if (b < 0 || t0l >= L || (t0l + min((int64_t)SPLIT, L - t0l) + PAGE - 1) / PAGE > a.max_pages) return;  // uniform
  const int t0 = (int)t0l;
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
  mask_v(vf, nt, lane);
  split_pv(vf, S, 1, lane, acc);
  if (lane < 16) store_pv<false>(acc, wave, lane, a.ws_o + base * HD);  // rows 0..3: the one token
}

// ---------------------------------------------------------------------------
// Prefill / extend: the tokens of a chunk attend causally to their sequence's
// cache (which already holds them). Query row r at position p uses exactly
// the split structure of a decode step with p + 1 cached tokens: splits
// s = 0 .. ceil((p + 1) / SPLIT) - 1, each reduced by the functions above
// with nt = min(SPLIT, p + 1 - s * SPLIT), merged with the decode combine's
// arithmetic (prefill_combine_kernel). So a prefilled token's output has the
// bits a decode step would give it, whatever the chunking and the batch.
//
// One workgroup per (work item, kv head); a work item is up to QB
// consecutive query rows of one sequence and one split they see. The split's
// K and V are loaded once into registers for all of them (V of keys past the
// last row's nt zeroed once); the rows then go through the three phases 4
// tokens (16 query rows) at a time, pipelined over three block-sized score
// arrays in LDS (see the kernel). For an earlier row, the keys it must not
// see carry p = 0, and their products (0 times a finite cached value) add
// exact zeros. Phase 2 uses the 16-lanes-per-row form (QuadSoftmax), with
// split_softmax_rows's bits.
// ---------------------------------------------------------------------------
constexpr int QB = 128;

struct PrefillArgs {
  const uint16_t* q;  // [rows, hq, HD]
  const uint16_t* kp;
  const uint16_t* vp;
  const int32_t* bt;    // [batch, max_pages]
  const int32_t* pos;   // [rows]
  const int32_t* qoffs; // [rows + 1]
  const int32_t* work;  // [n_work, 4]: row0, n_rows, sequence, split
  int64_t max_pages;
  int n_rows, batch, total_splits;
  int hq, hkv;
  float qscale;
  float* ws_o;
  float* ws_ml;
  int64_t ml_off;     // ws_ml - ws_o, in floats
  uint32_t ws_bytes;  // bytes of ws_o and ws_ml together (below 2^31 when BUFST)
};

// Two workgroups per CU (at most 256 registers per lane, half of a SIMD's),
// so that a second wave on each SIMD fills the first one's gaps.
template <bool BUFST>
__global__ __launch_bounds__(256, 2) void prefill_split_kernel(PrefillArgs a) {
  // Three score buffers of one block (4 tokens) each, in rotation: block i
  // uses buffer i % 3 (separate arrays, so the compiler sees that the
  // buffers of one step never overlap).
  __shared__ __align__(16) float S0[4][GQA][SROW], S1[4][GQA][SROW], S2[4][GQA][SROW];

  const int wi = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = a.work[4 * wi], nq = a.work[4 * wi + 1], b = a.work[4 * wi + 2], s = a.work[4 * wi + 3];
  // The plan's arrays are device data the host does not read: an item that
  // does not fit the buffers (rows, sequence, split, the split's pages in
  // the block table's row) is skipped -- uniformly, before any barrier -- so
  // every access stays in bounds whatever they hold.
  if (row0 < 0 || nq < 1 || nq > QB || row0 > a.n_rows - nq || b < 0 || b >= a.batch || s < 0 ||
      s > INT32_MAX / SPLIT)
    return;
  const int t0 = s * SPLIT;
  const int64_t nt_l = min((int64_t)SPLIT, (int64_t)a.pos[row0 + nq - 1] + 1 - t0);
  if (nt_l < 1 || (t0 + nt_l + PAGE - 1) / PAGE > a.max_pages) return;
  const int nt_max = (int)nt_l;
  const int npg = (nt_max + PAGE - 1) / PAGE;
  const int32_t* bt = a.bt + (int64_t)b * a.max_pages + t0 / PAGE;
  const int64_t head_stride = (int64_t)PAGE * HD;
  const int64_t page_stride = (int64_t)a.hkv * head_stride;
  const int64_t head_off = (int64_t)g * head_stride;
  const int64_t q_tok = (int64_t)a.hq * HD;
  const uint16_t* q0 = a.q + ((int64_t)row0 * a.hq + g * GQA) * HD;
  // Per item row t, worked out once into LDS (each row block needs them
  // three times, and a table read has no branch): the keys of the split it
  // sees (0 for t >= nq), and where its partials go -- the partial row of
  // (chunk row row0 + t, split s, query head g GQA), or -1 when the row's
  // position is before the split (it does not see it), its split slot is
  // outside the workspace's total_splits, or t >= nq. BUFST keeps that row
  // as the byte offsets of its o row and its (m, l) pair in the workspace
  // resource, past the resource's end (dropped stores) for -1. Whether any
  // row sees less than the whole split (the item is masked) is gathered by
  // a ballot of the two waves that fill the tables.
  static_assert(QB % 64 == 0, "the tables are filled by whole waves");
  constexpr uint32_t DROP = 0x80000000u;  // past any resource of BUFST
  __shared__ int s_nt[QB], s_short[QB / 64];
  __shared__ uint32_t s_ooff[BUFST ? QB : 1], s_moff[BUFST ? QB : 1];
  __shared__ int64_t s_row[BUFST ? 1 : QB];
  if (tid < QB) {  // whole waves
    int64_t row = -1;
    int nt = 0;
    if (tid < nq) {
      const int64_t seen = (int64_t)a.pos[row0 + tid] + 1 - t0;
      const int64_t slot = (int64_t)a.qoffs[row0 + tid] + s;
      nt = (int)max((int64_t)0, min((int64_t)SPLIT, seen));
      if (seen > 0 && slot >= 0 && slot < a.total_splits) row = slot * a.hq + g * GQA;
    }
    s_nt[tid] = nt;
    const uint64_t short_rows = __ballot(tid < nq && nt < SPLIT);
    if (lane == 0) s_short[wave] = short_rows != 0;
    if constexpr (BUFST) {
      // in range: the workspace, partials included, is below 2^31 bytes
      s_ooff[tid] = row >= 0 ? (uint32_t)(row * HD) * 4u : DROP;
      s_moff[tid] = row >= 0 ? (uint32_t)(a.ml_off + row * 2) * 4u : DROP;
    } else {
      s_row[tid] = row;
    }
  }

  u32x4 qc[4], kf[4][4], vf[8][2];
  load_q_block(q0, q_tok, min(4, nq), lane, qc);
  load_k_frags<false>(a.kp, bt, npg, page_stride, head_off, wave, lane, kf);
  load_v_frags<false>(a.vp, bt, npg, page_stride, head_off, wave, lane, vf);
  __builtin_amdgcn_sched_barrier(0);  // every load issued before the first MFMA waits
  __syncthreads();                    // the per-row tables
  const int t_lane = lane >> 4;       // the token of this lane's softmax row, scores and p.v outputs
  const int j = lane & 15;            // the lane's place in its softmax row
  const int nblk = (nq + 3) / 4;      // blocks of 4 tokens
  auto nb_of = [&](int i) { return min(4, nq - 4 * i); };
  auto qload = [&](int i) { load_q_block(q0 + 4 * i * q_tok, q_tok, nb_of(i), lane, qc); };
  // BUFST (the workspace is below 2 GiB): the partials go out as raw buffer
  // stores through one resource over ws_o and ws_ml; a lane with nothing to
  // write gets an offset past the resource's end, and the hardware drops its
  // store. So no branch surrounds the stores, and the compiler counts a
  // pipeline step's memory operations exactly: a wait for a load also waits
  // for the stores issued before it, and a branch around the stores made it
  // assume none had been issued, waiting for the previous step's stores.
  // Otherwise, plain stores under a branch.
  const __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.ws_o, 0, (int)a.ws_bytes, 0x00020000);
  constexpr int NT = 2;  // cache policy: non-temporal (written once, read back by the combine)
  // block i's row of this lane (4 i + t_lane < 4 nblk <= QB; rows >= nq
  // have nothing to write)
  auto store_ml = [&](int i, float mx, float l) {
    if constexpr (BUFST) {
      const uint32_t off = j == 0 ? s_moff[4 * i + t_lane] + 8u * wave : DROP;  // DROP + 24 is still past the end
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(mx), __float_as_uint(l)}, ws_rsrc, (int)off, 0, 0);
    } else {
      const int64_t base = s_row[4 * i + t_lane];
      if (j == 0 && base >= 0) {
        a.ws_ml[(base + wave) * 2 + 0] = mx;
        a.ws_ml[(base + wave) * 2 + 1] = l;
      }
    }
  };
  // store_o(-1, zeros) issues the same stores, all dropped (BUFST): the
  // first step does it, so that every step of the pipeline has the same
  // memory operations and the compiler's count at the loop's head is exact.
  auto store_o = [&](int i, const f32x4 (&acc)[2]) {
    if constexpr (BUFST) {
      // + (h HD + 16 dt) 4 below; DROP plus at most 2044 is still past the end
      const uint32_t off = (i >= 0 ? s_ooff[4 * i + t_lane] : DROP) + (uint32_t)(32 * wave + (lane & 15)) * 4u;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int h = 0; h < 4; ++h)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[dt][h]), ws_rsrc,
                                                (int)(off + (uint32_t)(h * HD + 16 * dt) * 4u), 0, NT);
    } else {
      const int64_t base = i >= 0 ? s_row[4 * i + t_lane] : -1;
      if (base >= 0) store_pv<true>(acc, wave, lane, a.ws_o + base * HD);
    }
  };
  using Buf = float (*)[GQA][SROW];
  bool masked = false;  // uniform: some row sees less than the whole split
#pragma unroll
  for (int w = 0; w < QB / 64; ++w) masked = masked || s_short[w] != 0;

  // The item's blocks of 4 tokens run as a pipeline with one barrier per
  // block. Step i takes block i's softmax, block i - 1's p.v and block i + 1's
  // scores, three different buffers (block b uses buffer b % 3). Before the
  // barrier that ends step i, every wave has written block i + 1's scores and
  // block i's p and has read block i - 1's p; so after it, block i + 2's
  // scores may overwrite block i - 1's buffer. Inside a step the work is cut
  // into chunks, each holding one group of matrix instructions (a d step of
  // the scores or a key step of p.v) and one stage of the softmax, so that a
  // wave's vector work sits between its matrix work (and the second wave on
  // the SIMD can fill the gaps); scheduling barriers keep the chunks in order.
  // Where a row of the item does not see the whole split (masked), its keys
  // past its position get -inf scores (p = 0 exactly) and V past the last
  // row's keys is zeroed once, so every product with an unseen key is an
  // exact zero.
  {
    // keys this lane's token of block i sees
    auto nt_tok = [&](int i) { return s_nt[4 * i + t_lane]; };  // 0 past the item's rows
    f32x4 sacc[4], pacc[2];
    u32x4 phi[2], plo[2];
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // has_pv (i >= 1) and has_sc (i + 1 < nblk) are compile-time, so that a
    // step in the middle of the item is straight-line code
    auto step = [&](auto pv_tag, auto sc_tag, int i, Buf Ssm, Buf Spv, Buf Ssc) {
      constexpr bool has_pv = decltype(pv_tag)::value, has_sc = decltype(sc_tag)::value;
      float* const row = Ssm[t_lane][wave];
      const uint16_t* prow = pv_row(Spv, has_pv ? nb_of(i - 1) : 1, lane);
      const int nt_sc = has_sc ? nt_tok(i + 1) : SPLIT;
      QuadSoftmax sm;
      sm.load(row, j);
      if (has_pv) {
        pv_operands(prow, 0, phi[0], plo[0]);
        pv_operands(prow, 1, phi[1], plo[1]);
      }
      fence();
      if (has_sc) scores_step<true>(qc, kf, 0, sacc);
      sm.max_lane();
      fence();
      if (has_sc) scores_step<false>(qc, kf, 1, sacc);
      sm.max_row();
      fence();
      if (has_sc) scores_step<false>(qc, kf, 2, sacc);
      sm.exp_group(0);
      fence();
      if (has_sc) {
        scores_step<false>(qc, kf, 3, sacc);
        qload(min(i + 2, nblk - 1));  // the next step's scores; qc is free from here on
      }
      sm.write_group(row, j, 0);
      sm.exp_group(1);
      fence();
      // key steps 0..7 of block i - 1's p.v, the operands read two steps ahead
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if (has_pv) {
          if (ks == 0) pv_step<true>(vf, ks, phi[0], plo[0], pacc);
          else pv_step<false>(vf, ks, phi[ks & 1], plo[ks & 1], pacc);
          if (ks + 2 < 8) pv_operands(prow, ks + 2, phi[ks & 1], plo[ks & 1]);
        }
        if (ks == 0) sm.write_group(row, j, 1);
        if (ks == 1) sm.exp_group(2);
        if (ks == 2) sm.write_group(row, j, 2);
        if (ks == 3) sm.exp_group(3);
        if (ks == 4) sm.write_group(row, j, 3);
        if (has_sc && ks >= 4) scores_store(sacc[ks - 4], ks - 4, t_lane, nt_sc, wave, lane, a.qscale, Ssc);
        fence();
      }
      store_ml(i, sm.mx, sm.sum_row());
      if constexpr (has_pv) {
        store_o(i - 1, pacc);
      } else if constexpr (BUFST) {
        const f32x4 zeros[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
        store_o(-1, zeros);
      }
      __syncthreads();
    };
    if (masked) mask_v(vf, nt_max, lane);
    {  // block 0's scores
      const int nt0 = nt_tok(0);
      scores_step<true>(qc, kf, 0, sacc);
#pragma unroll
      for (int ds = 1; ds < 4; ++ds) scores_step<false>(qc, kf, ds, sacc);
      if (nblk > 1) qload(1);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) scores_store(sacc[kt], kt, t_lane, nt0, wave, lane, a.qscale, S0);
      __syncthreads();
    }
    // V has arrived before the pipeline starts (a use here; otherwise the
    // compiler would count V's loads as outstanding in every step)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) asm volatile("" ::"v"(vf[ks][dt]));
    constexpr std::true_type T{};
    constexpr std::false_type F{};
    if (nblk == 1) {
      step(F, F, 0, S0, S2, S1);
    } else {
      step(F, T, 0, S0, S2, S1);
      for (int i = 1; i <= nblk - 2;) {
        step(T, T, i, S1, S0, S2);  // i = 1 (mod 3)
        if (++i > nblk - 2) break;
        step(T, T, i, S2, S1, S0);  // i = 2 (mod 3)
        if (++i > nblk - 2) break;
        step(T, T, i, S0, S2, S1);  // i = 0 (mod 3)
        ++i;
      }
      const int i = nblk - 1;
      step(T, F, i, i % 3 == 0 ? S0 : i % 3 == 1 ? S1 : S2, (i - 1) % 3 == 0 ? S0 : (i - 1) % 3 == 1 ? S1 : S2,
           S0);
    }
    {  // the last block's p.v
      const int i = nblk - 1;
      f32x4 acc[2];
      split_pv(vf, i % 3 == 0 ? S0 : i % 3 == 1 ? S1 : S2, nb_of(i), lane, acc);
      store_o(i, acc);
    }
  }
}

// Four consecutive output elements out[at .. at + 3] (at a multiple of 4):
// one 16-byte (fp32) or 8-byte (bf16) store where out's alignment allows it
// (the same for every lane), else four element stores (out need only be
// aligned to its element size).
__device__ __forceinline__ void store_out4(void* out, int64_t at, const float (&r)[4], int out_bf16) {
  if (out_bf16) {
    uint16_t* const p = reinterpret_cast<uint16_t*>(out) + at;
    if ((reinterpret_cast<uintptr_t>(p) & 7) == 0) {
      *reinterpret_cast<u32x2*>(p) =
          u32x2{(uint32_t)f32_to_bf16_rne(r[0]) | ((uint32_t)f32_to_bf16_rne(r[1]) << 16),
                (uint32_t)f32_to_bf16_rne(r[2]) | ((uint32_t)f32_to_bf16_rne(r[3]) << 16)};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = (uint16_t)f32_to_bf16_rne(r[e]);
    }
  } else {
    float* const p = reinterpret_cast<float*>(out) + at;
    if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      *reinterpret_cast<f32x4*>(p) = f32x4{r[0], r[1], r[2], r[3]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = r[e];
    }
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
__global__ __launch_bounds__(128) void decode_combine_kernel(const int32_t* __restrict__ offs, int cap,
                                                              const float* __restrict__ ws_o,
                                                              const float* __restrict__ ws_ml, int hq,
                                                              void* __restrict__ out, int out_bf16) {
  __shared__ float red[2];
  __shared__ float4 po[2][HD / 4];
  __shared__ float pl[2];
  // the heads of one sequence are adjacent in dispatch order, so they read
  // (and write) the sequence's contiguous partials (and output) together
  const int b = blockIdx.x / hq, h = blockIdx.x % hq, tid = threadIdx.x;
  const int pg = tid >> 5, c = tid & 31, wv = tid >> 6;
  // The row's splits [offs[b], offs[b+1]), clamped to the workspace's cap
  // splits so that offsets on the device can never send a read past it.
  const int w1 = min(max(offs[b + 1], 0), cap);
  const int w0 = min(max(offs[b], 0), w1), ns = w1 - w0;
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
    store_out4(out, ((int64_t)b * hq + h) * HD + 4 * c, res, out_bf16);
  }
}

// Combine for prefill rows: one wave per (row, query head), four query
// heads per workgroup. The arithmetic is decode_combine_kernel's, term for
// term -- the same 8 groups (splits s = g, g + 8, ... in increasing order,
// each weighted by 2^(m_s - M) with M the exact max), the same tree
// ((g0 + g1) + (g2 + g3)) + ((g4 + g5) + (g6 + g7)) and the same division --
// so a prefilled token keeps its decode bits. Lane 32 hf + c owns
// o[4c .. 4c + 3] of groups 4 hf .. 4 hf + 3 and adds them as
// (g0 + g1) + (g2 + g3) in registers; the two halves' sums are then added
// across the wave (commutative, so both halves hold the same bits). No LDS
// and no barrier: a row of up to 8 splits (every row of a prompt of up to
// 2048 tokens) takes one memory round trip with all its loads in flight.
__global__ __launch_bounds__(256) void prefill_combine_kernel(const int32_t* __restrict__ offs, int cap,
                                                               const float* __restrict__ ws_o,
                                                               const float* __restrict__ ws_ml, int hq,
                                                               void* __restrict__ out, int out_bf16) {
  // the head groups of one row are adjacent in dispatch order, so they read
  // (and write) the row's contiguous partials (and output) together
  const int b = blockIdx.x / (hq / GQA), lane = threadIdx.x & 63;
  const int h = GQA * (blockIdx.x % (hq / GQA)) + (threadIdx.x >> 6);
  const int hf = lane >> 5, c = lane & 31;
  // the row's splits [offs[b], offs[b+1]), clamped to the workspace's cap
  const int w1 = min(max(offs[b + 1], 0), cap);
  const int w0 = min(max(offs[b], 0), w1), ns = w1 - w0;
  float l[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float4 o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float M;
  auto part = [&](int s, float2& ml, float4& ov) {
    const int64_t ph = (int64_t)(w0 + s) * hq + h;
    ml = *reinterpret_cast<const float2*>(ws_ml + ph * 2);
    ov = *reinterpret_cast<const float4*>(ws_o + ph * HD + 4 * c);
  };
  auto fold = [&](int k, const float2 ml, const float4 ov) {
    const float w = __builtin_amdgcn_exp2f(ml.x - M);
    l[k] = l[k] + w * ml.y;
    o[k].x = o[k].x + w * ov.x;
    o[k].y = o[k].y + w * ov.y;
    o[k].z = o[k].z + w * ov.z;
    o[k].w = o[k].w + w * ov.w;
  };
  if (ns >= 1 && ns <= 8) {
    float2 mls[4];
    float4 ovs[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) part(min(4 * hf + k, ns - 1), mls[k], ovs[k]);
    const float m = fmaxf(fmaxf(mls[0].x, mls[1].x), fmaxf(mls[2].x, mls[3].x));
    M = fmaxf(m, xor_shfl(m, 32));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (4 * hf + k < ns) fold(k, mls[k], ovs[k]);
  } else {
    float m = -INFINITY;
    for (int s = lane; s < ns; s += 64) m = fmaxf(m, ws_ml[((int64_t)(w0 + s) * hq + h) * 2]);
    M = wave_max(m);
    for (int t0 = 0; t0 < ns; t0 += 8) {  // splits t0 .. t0 + 7: one per group, in order
      float2 mls[4];
      float4 ovs[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) part(min(t0 + 4 * hf + k, ns - 1), mls[k], ovs[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (t0 + 4 * hf + k < ns) fold(k, mls[k], ovs[k]);
    }
  }
  auto add = [](float4 x, float4 y) { return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w); };
  const float4 t = add(add(o[0], o[1]), add(o[2], o[3]));
  const float lt = (l[0] + l[1]) + (l[2] + l[3]);
  const float4 os = add(t, make_float4(xor_shfl(t.x, 32), xor_shfl(t.y, 32), xor_shfl(t.z, 32), xor_shfl(t.w, 32)));
  const float ls = lt + xor_shfl(lt, 32);
  if (hf == 0) {
    const float res[4] = {os.x / ls, os.y / ls, os.z / ls, os.w / ls};
    store_out4(out, ((int64_t)b * hq + h) * HD + 4 * c, res, out_bf16);
  }
}

// Scratch of bi_decode_attention_noalloc: the split partials (o, m, l) in a
// file-scope device array instead of a caller's workspace, for callers that
// cannot allocate. Every GPU the library runs on holds its own copy until
// the process ends; all calls on one GPU share it (it keeps the last call's
// partials; every partial a call reads is written earlier in the same call,
// so nothing needs clearing), so calls that overlap on one GPU race. In host
// code the array's name is not a device address: only the pointer from
// hipGetSymbolAddress (decode_scratch) is passed to kernels.
constexpr size_t SCRATCH_BYTES = BI_DECODE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

}  // namespace

size_t decode_scratch_bytes() { return SCRATCH_BYTES; }

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
  static std::mutex mu;
  static void* per_device[256] = {};
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != cur) return hipErrorInvalidDevice;
  }
  if (cur < 0 || cur >= 256) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[cur] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `cur` current
    if (e != hipSuccess) return e;
    per_device[cur] = p;
  }
  *ptr = per_device[cur];
  return hipSuccess;
}

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
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(p.batch * p.num_q_heads)), dim3(128), 0, s,
                     p.split_offsets, (int)p.total_splits, p.ws_o, p.ws_ml, p.num_q_heads, p.out,
                     p.out_bf16 ? 1 : 0);
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
  a.n_rows = (int)p.n_rows;
  a.batch = (int)p.batch;
  a.total_splits = (int)p.total_splits;
  a.hq = p.num_q_heads;
  a.hkv = p.num_kv_heads;
  a.qscale = p.scale * LOG2E;
  a.ws_o = p.ws_o;
  a.ws_ml = p.ws_ml;
  a.ml_off = p.ws_ml - p.ws_o;
  const int64_t ws_bytes = (a.ml_off + p.total_splits * p.num_q_heads * 2) * (int64_t)sizeof(float);
  a.ws_bytes = (uint32_t)min(ws_bytes, (int64_t)INT32_MAX);
  if (ws_bytes < INT32_MAX)
    hipLaunchKernelGGL(prefill_split_kernel<true>, dim3((unsigned)(p.n_work * p.num_kv_heads)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_split_kernel<false>, dim3((unsigned)(p.n_work * p.num_kv_heads)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)(p.n_rows * (p.num_q_heads / GQA))), dim3(256), 0,
                     s, p.q_offsets, (int)p.total_splits, p.ws_o, p.ws_ml, p.num_q_heads, p.out, p.out_bf16 ? 1 : 0);
  return hipGetLastError();
}

int prefill_rows_per_item() { return QB; }

}  // namespace bi
