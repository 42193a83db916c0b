// The GEMM's tile table: which configuration a call of bi_mm / bi_addmm /
// bi_gemm runs, as a function of (m, n, k, layout) -- host code only, shared
// by the launcher (gemm.hip) and the argument checks (api.cpp). Every
// configuration computes each output element with the same chain (one
// v_mfma_f32_32x32x16_bf16 per 16 k, increasing k, fp32 from 0, k padded with
// zeros to a multiple of 64, the same epilogue), so the choice moves work
// between workgroups without changing any bit. Batch invariance gives up
// shape-aware tiling according to the wiki page "Thinking Machines" (section
// on why it is not the main answer, point 3); it is kept here because it
// never touches the reduction.
#include "bi_internal.h"

#include <numeric>

namespace bi {

constexpr int TK = 64;  // k per stage (the kernels' k tile)

// Skinny (M <= 64): one consumer wave (32 rows) when the 32-row strips fit
// in one round over the CUs, else two (64 rows); two producer waves either
// way.
static GemmConfig skinny_config(int64_t m, int64_t strips) {
  if (m <= 32 || ((m + 31) / 32) * strips <= 256) return GemmConfig{32, 32, TK, 3};
  return GemmConfig{64, 32, TK, 4};
}

// The configuration table. Every configuration -- skinny, 64x128, 128x128,
// 256x256, 256x384 -- computes each output element with the same chain (one 32x32x16 MFMA per
// 16 k, increasing k, fp32, k padded to a multiple of 64, the same
// epilogue), so the choice moves work between workgroups without changing
// any bit, and it may depend on M: the result of a row still does not depend
// on how many rows there are. (The batch-dependent selection the pages warn
// about changes the reduction -- split-K, a different instruction -- and
// nothing here does.) Measured on MI355X for the Qwen3-8B projection shapes:
//   * skinny (32 or 64 rows x 32 columns, deep ring) for M <= 64: 2.5-3.6x
//     faster than 128x128 (N = 4096, 6144, K = 4096 and 12288), 1.25-1.6x
//     at N = 24576; at the 151936-wide LM head both stream at ~5.4 TB/s and
//     128x128 is kept; 32 or 64 rows x 96 columns (three consumers across)
//     where that makes one round of tiles out of several (N = 24576);
//   * the same deep ring with a 64x128 tile (2x2 consumer waves of 32x64,
//     two producers, 6 stages) for M > 64 while 128x128 tiles would fill at
//     most half the CUs and the 64x128 ones still fit one round: 6-14 %
//     faster than the 128x128 ring at M = 128-512 for N = 4096 (K = 4096
//     and 12288) and 3-5 % for N = 6144 at M <= 256; four consumer waves
//     (every SIMD issuing MFMAs) instead of two of 64x64: 13-26 % faster at
//     M = 65-512 for N = 4096 and 6144;
//   * the same deep ring with a 128x128 tile (4x2 consumer waves of 32x64)
//     for M > 64 while its tiles fit one round over the CUs: 1.15-1.35x
//     faster than 128x128 or skinny at M = 128-1024, 1.6x than 256x256 at
//     M = 128, N = 24576; eight consumers instead of four of 64x64: 3-7 %
//     faster at M = 384-1024 for N = 4096 and 6144 and at M <= 128 for
//     N = 24576 (K = 12288 at M = 768-1024: ~5 % slower);
//   * 256x384 (8 waves, 128x96 each) where K and N are whole tiles and its
//     tiles make whole rounds over the CUs (gate+up at M in 769..1024,
//     1793..2048, 2817..3072 and 3841..4096; q+kv at M > 3840);
//   * 256x256 (8 waves, 128x64 each) once its tiles fill the chip (M >= 192,
//     at least 192 tiles, rounds of 256 at least 70 % full on average):
//     1.25-1.3x faster than 128x128 at M = 4096 (N = 4096, LM head), 1.1x
//     for the LM head at M = 256, and for the wide N of gate+up at all M;
//   * 128x128 (4 waves, two workgroups per CU) in between.
GemmConfig gemm_config(int64_t m, int64_t n, int64_t k, bool b_is_nk) {
  (void)b_is_nk;
  const int64_t strips = (n + 31) / 32;
  if (m <= 64 && n <= 32768) {
    // 96-column skinny tiles when 32-column strips need more than one round
    // over the CUs and the 96-column ones fill one round at least 3/4 full:
    // a CU then reads the rows' A once for 96 columns instead of once per
    // 32 (gate+up, N = 24576: M = 64 cold 59.8 -> 49.3 us with [N,K]
    // weights, 81.5 -> 45.0 with [K,N]; M = 1 43.4 -> 45.2 and 60.0 -> 41.6)
    const int64_t strips96 = (n + 95) / 96;
    if (strips > 256 && strips96 >= 192 && strips96 <= 256)
      return m <= 32 ? GemmConfig{32, 96, TK, 5} : GemmConfig{64, 96, TK, 8};
    return skinny_config(m, strips);
  }
  const int64_t t128 = ((m + 127) / 128) * ((n + 127) / 128);
  if (m > 64 && t128 <= 128 && ((m + 63) / 64) * ((n + 127) / 128) <= 256) return GemmConfig{64, 128, TK, 6};
  if (m > 64 && t128 <= 256) return GemmConfig{128, 128, TK, 10};
  // 256x384 (8 waves of 128x96) where K is a whole number of k tiles, N of
  // tile columns, and its tiles make whole rounds over the CUs: per flop it
  // reads a fifth fewer LDS bytes than 256x256 and fills LDS with a sixth
  // fewer. Measured against 256x256 (with its column split where taken),
  // warm, [K,N] / [N,K] weights: gate+up (N = 24576) at M = 1024 208 -> 180 /
  // 211 -> 186 us, M = 2048 363 -> 354 / 363 -> 358, M = 3072 556 -> 520 /
  // 566 -> 532, M = 4096 691 -> 671 / 702 -> 687; q+kv (N = 6144) at
  // M = 4096, one round of 256 tiles where 256x256 needs 1.5, 184 -> 167 /
  // 184 -> 169 us. Also with a sparse last row of tiles, whose rows past M
  // it multiplies as zeros: gate+up at M = 769 180 -> 169 us, 832 187 -> 170,
  // 960 190 -> 177; q+kv at M = 3841 185 -> 166 us.
  if (k > 0 && n % 384 == 0 && k % TK == 0) {  // its loads have no k mask: k == 0 (A, B may be NULL) excluded
    const int64_t t384 = ((m + 255) / 256) * (n / 384);
    if (t384 >= 256 && t384 % 256 == 0) return GemmConfig{256, 384, TK, 8};
  }
  const int64_t t256 = ((m + 255) / 256) * ((n + 255) / 256);
  const int64_t rounds = (t256 + 255) / 256;  // one 256x256 workgroup per CU
  if (m >= 192 && t256 >= 192 && 10 * t256 >= 7 * rounds * 256) return GemmConfig{256, 256, TK, 8};
  if (n >= 16384 && n <= 65536 && k <= 8192) return GemmConfig{256, 256, TK, 8};
  return GemmConfig{128, 128, TK, 4};
}

// The fixed-tile mode: one configuration per (N, K, layout), whatever M is
// -- the letter of "one tile config for all M". 256x256 (8 waves) once N
// spans at least 16 tile columns (every projection shape and the LM head),
// 128x128 (4 waves) for narrower N; no column split (where it splits
// depends on M). Its bits are those of gemm_config's table, since every
// configuration runs the same chain; it exists to measure what choosing the
// tile by M gains.
GemmConfig gemm_config_fixed(int64_t n, int64_t k, bool b_is_nk) {
  (void)k;
  (void)b_is_nk;
  if (n >= 16 * 256 - 255) return GemmConfig{256, 256, TK, 8};
  return GemmConfig{128, 128, TK, 4};
}

// Columns of a 256x256 GEMM left to full rounds of 256x256 tiles; the rest
// (if any) goes to 256x128 tiles in a second launch. Whole rounds of 256 CUs
// need tiles_m * n1 to be a multiple of 256. A round of 256x128 tiles takes
// ~0.65 of a 256x256 round (measured, K = 4096); the split is taken only
// when that predicts fewer rounds. Measured on MI355X: q+kv at M = 4096
// (384 tiles, 1.5 rounds) 7-8 % faster, gate+up at M = 1024 4-7 %, the LM
// head at M = 256 (594 tiles) 3-4 %. Both parts compute every element with
// the chain above, so the bits do not change.
// Also gives the plan's predicted time in 256x256 rounds (*cost).
static int64_t full_round_columns(int64_t tiles_m, int64_t tiles_n, int64_t n, double* cost) {
  const double whole = (double)((tiles_m * tiles_n + 255) / 256);
  *cost = whole;
  const int64_t g = 256 / std::gcd(tiles_m, (int64_t)256);  // tiles_m * n1 % 256 == 0 iff g divides n1
  const int64_t n1 = (tiles_n / g) * g;
  if (n1 == 0 || n1 == tiles_n) return tiles_n;
  const int64_t t_tail = tiles_m * ((n - n1 * 256 + 127) / 128);
  const double split = (double)(tiles_m * n1 / 256) + 0.65 * (double)((t_tail + 255) / 256);
  if (split >= whole - 0.05) return tiles_n;
  *cost = split;
  return n1;
}

// Columns of a 256x256 GEMM better taken first by 256x384 tiles, in whole
// rounds over the CUs, the rest staying on 256x256 tiles (a second launch):
// a round of 256x384 tiles takes ~1.45 rounds of 256x256 (measured at
// K = 4096), so for wide N it can cover the columns past the last full
// 256x256 round for less than a part-empty round costs. Returns 0 (no such
// split) or the first launch's width, a multiple of 384 that leaves columns
// to the second; chosen to minimise the predicted rounds, and taken only
// where that beats the 256x256 plan (`cost_256`, in 256x256 rounds) by more
// than 0.05. The 256x384 tile's loads have no k mask, so k must be a
// positive multiple of 64. Only where the last row of tiles is at least 3/4
// full: 256x256 tiles skip the MFMAs of row blocks past M, the 256x384 ones
// multiply them as zeros, so with a sparse last row the round count above
// overstates the 256x256 plan (the LM head at M = 300 508 -> 546 us). Measured
// on MI355X, the LM head (N = 151936, K = 4096), warm, [K,N] weights: M = 200
// 352 -> 321 us, 224 356 -> 329, 256 377 -> 350 ([N,K] 377 -> 361; after a
// read-only flush 372 -> 330), 1000 1150 -> 1117, 1024 1157 -> 1111, 2048
// 2212 -> 2150, 4096 4317 -> 4180; M = 512 even.
static int64_t wide_384_columns(int64_t m, int64_t n, int64_t k, double cost_256) {
  if (k <= 0 || k % TK != 0) return 0;
  const int64_t tiles_m = (m + 255) / 256;
  if (m - (tiles_m - 1) * 256 < 192) return 0;
  const int64_t g = 256 / std::gcd(tiles_m, (int64_t)256);  // tiles_m * c % 256 == 0 iff g divides c
  int64_t best = 0;
  double best_cost = cost_256 - 0.05;
  // widths c * 384 with c a multiple of g leaving columns to the second
  // launch; each step of g adds ~1.45 * tiles_m * g / 256 rounds of 256x384
  // and removes ~1.5 times as many of 256x256, so the best lies near the
  // widest: the 64 widest are tried (all of them for every shape here)
  const int64_t c_max = ((n - 1) / 384 / g) * g;
  for (int64_t c = c_max; c >= g && c > c_max - 64 * g; c -= g) {
    const int64_t rest_tiles = tiles_m * ((n - 384 * c + 255) / 256);
    const double cost = 1.45 * (double)(tiles_m * c / 256) + (double)((rest_tiles + 255) / 256);
    if (cost < best_cost) {
      best_cost = cost;
      best = 384 * c;
    }
  }
  return best;
}

GemmPlan gemm_plan(int64_t m, int64_t n, int64_t k, bool b_is_nk, bool fixed_tile) {
  GemmPlan plan{};
  const GemmConfig cfg = fixed_tile ? gemm_config_fixed(n, k, b_is_nk) : gemm_config(m, n, k, b_is_nk);
  plan.count = 1;
  plan.launch[0] = GemmLaunch{cfg, 0, n};
  if (!fixed_tile && cfg.tile_m == 256 && cfg.tile_n == 256) {
    const int64_t tiles_m = (m + 255) / 256, tiles_n = (n + 255) / 256;
    double cost_256 = 0.0;
    const int64_t n1 = full_round_columns(tiles_m, tiles_n, n, &cost_256);
    const int64_t w384 = wide_384_columns(m, n, k, cost_256);
    if (w384 > 0) {
      plan.count = 2;
      plan.launch[0] = GemmLaunch{GemmConfig{256, 384, TK, 8}, 0, w384};
      plan.launch[1] = GemmLaunch{cfg, w384, n};
    } else if (n1 < tiles_n) {
      plan.count = 2;
      plan.launch[0].n_end = n1 * 256;
      plan.launch[1] = GemmLaunch{GemmConfig{256, 128, TK, 8}, n1 * 256, n};
    }
  }
  return plan;
}

}  // namespace bi
