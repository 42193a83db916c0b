// Batch-invariant bf16 GEMM (mm / addmm) for gfx950.
//
// mm and addmm are two of the four ops listed as supported in
// "thinking-machines-lab/batch_invariant_ops" (catalogue page, section "When
// to avoid"); matmul is the first kernel named as batch-dependent in
// readhandoff.com's agent-run reproducibility pinning, section "What does
// temperature zero actually guarantee?". The fix is a fixed reduction order
// ("How to achieve deterministic LLMs with batch invariant inference",
// "TL;DR"); split-K and shape-aware tiling are the optimisations given up
// (wiki page "Thinking Machines", section on why it is not the main answer,
// point 3).
//
// What fixes the bits of C[i][j]
//   acc = 0; for kc = 0, 16, 32, ... (increasing): acc = MFMA16(A[i][kc..kc+15],
//   B[kc..kc+15][j], acc). One v_mfma_f32_32x32x16_bf16 step per 16 k, fp32
//   accumulator, a single chain per element. Nothing in that chain depends on
//   M, on the row's position, on the other rows or on the tile shape: rows
//   past M and k past K are loaded as zeros, and every tile -- full or
//   partial -- runs the same instruction stream. There is no split-K,
//   stream-K or atomic anywhere.
//
// Which tile configuration runs is chosen from (M, N, K) -- a skinny kernel
// for small M (below), 128x128, 256x256 or 256x384 otherwise; where a
// 256x256 GEMM's final round over the CUs would be part-empty, its leftover
// columns go to 256x128 tiles, or (wide N) its first columns to 256x384
// tiles in whole rounds -- and, because every configuration runs the chain
// above, that choice never changes a bit.
//
// Structure (one workgroup per TM x TN output tile)
//   * global -> LDS directly (buffer_load ... lds, 16 bytes per lane): no
//     register staging and no LDS write instructions. Rows past M or N and k
//     past K read as zero through the buffer range check, so no load needs a
//     branch. The loads of k tile t+1 are issued at the start of tile t into
//     the other of two LDS stages and waited for at the barrier that ends
//     tile t, so they land behind a whole tile of MFMA work;
//   * LDS layout: A (and B stored [N,K]) as rows of 64 bf16 made of eight
//     16-byte chunks whose position is XOR-swizzled by the row, so the MFMA
//     fragment reads (ds_read_b128) are free of bank conflicts; each lane of
//     a direct load fetches the global chunk that belongs at its swizzled
//     LDS position;
//   * B stored [K, N] (N contiguous) goes into LDS as it is, k rows of n
//     with 16-byte chunks XOR-swizzled by row % 4; its MFMA fragments (8
//     consecutive k of one column per lane) come out through gfx950's
//     transposing LDS read, ds_read_b64_tr_b16, two per fragment;
//   * fragments are double-buffered in registers across the four 16-wide k
//     steps of a tile;
//   * epilogue straight from the accumulators: alpha, then + beta * bias in
//     fp32 after the full K loop, one rounding to the output dtype.
//   * workgroup -> tile order is XCD-aware: consecutive workgroup ids land on
//     different XCDs (round robin), so ids are remapped to give each XCD a
//     contiguous band of tiles that share A rows / B columns in its own L2.
//     This only permutes which workgroup computes which tile.
#include "bi_internal.h"
#include "device_common.h"

#include <type_traits>

namespace bi {
namespace {

constexpr int TK = 64;  // k per stage: 8 chunks of 8 bf16

struct GemmArgs {
  const uint16_t* a;
  const uint16_t* b;
  void* c;
  const void* bias;
  int64_t lda, ldb, ldc;
  int m, n, k;
  float alpha, beta;
  int out_bf16;
  int bias_mode;  // 0 none, 1 bf16, 2 fp32
  int tiles_m, tiles_n;
};

// Index (in 16-byte units) of chunk `ch` of LDS row `row`.
__device__ __forceinline__ int swz(int row, int ch) {
  return row * 8 + (ch ^ ((row ^ (row >> 3)) & 7));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Workgroup id -> (tile_m, tile_n). Bijective on [0, tiles).
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int tiles = tiles_m * tiles_n;
  // XCD-aware: ids are dealt round-robin to 8 XCDs; give XCD x the contiguous
  // logical range it would own in a blocked distribution.
  const int x = bid & 7, idx = bid >> 3;
  const int q = tiles >> 3, r = tiles & 7;
  const int logical = x * q + (x < r ? x : r) + idx;
  // Grouped order: bands of GM tile-rows, column-major inside a band. With
  // GM = 4 an XCD's 32 concurrent tiles span 4 tile-rows x 8 tile-columns
  // (measured against 1, 2, 8, 16, 32: gate+up at M = 4096 3-6 % faster than
  // with 8, the other shapes even or better).
  constexpr int GM = 4;
  const int band = logical / (GM * tiles_n);
  const int first = band * GM;
  const int rows = min(tiles_m - first, GM);
  const int in = logical - band * GM * tiles_n;
  tm = first + in % rows;
  tn = in / rows;
}

// Raw buffer loads: an offset at or past the descriptor's byte count reads
// as zero without touching memory, so masked rows/columns and the k tail
// need no branch and the k loop stays one basic block.
constexpr uint32_t OOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane straight into LDS: lane l of the wave writes the 16
// bytes at lds + 16 * l (lds is wave-uniform). Kept as a plain device
// function: called directly inside the kernel template's lambdas, the
// builtin made the host compilation pass drop the kernels' launch stubs.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, const void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

template <int TM, int TN, int WM, int WN, bool B_NK>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(GemmArgs g) {
  constexpr int WTM = TM / WM, WTN = TN / WN;  // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 MFMA tiles per wave
  // LDS stages. A (and B stored [N,K]): rows of 64 bf16 = eight 16-byte
  // chunks, chunk position XOR-swizzled by the row (swz). B stored [K,N]:
  // TK rows of TN bf16, 16-byte chunk c of row r stored at c ^ (4 * (r % 4)),
  // so the four rows one transposing read touches sit on disjoint banks.
  constexpr int NW = WM * WN;
  constexpr int A_I = TM * 8 / 64 / NW;  // 1 KB direct-to-LDS loads per wave per k tile (A)
  constexpr int B_I = TN * 8 / 64 / NW;  // ... (B; TK * TN / 8 == TN * 8 chunks either layout)
  static_assert(A_I * 64 * NW == TM * 8 && B_I * 64 * NW == TN * 8, "tile not evenly split across waves");
  static_assert(FM >= 1 && FN >= 1, "wave tile smaller than one MFMA");
  static_assert(B_NK || TN % 128 == 0, "[K,N] swizzle needs at least 16 chunks per row");
  // FULL (the 256x384 tile): K is a multiple of TK and N of TN, so no load
  // needs a k or n mask; its fragment addresses are recomputed per read and
  // rows past M are multiplied as zeros rather than skipped, which keeps its
  // 192 accumulators and the rest within 256 registers
  constexpr bool FULL = TN == 384;

  // two stages, each its own LDS object
  __shared__ u32x4 As0[TM * 8], As1[TM * 8];
  __shared__ u32x4 Bs0[TN * 8], Bs1[TN * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  int tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * TM, n0 = tn * TN;
  const int M = g.m, N = g.n, K = g.k;
  const int nk = (K + TK - 1) / TK;
  const uint32_t lda2 = (uint32_t)g.lda * 2u, ldb2 = (uint32_t)g.ldb * 2u;

  // A rows past M, and B rows past N ([N,K] layout), lie past the descriptor.
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(g.a + (int64_t)m0 * g.lda, (uint32_t)min(TM, M - m0) * lda2);
  __amdgpu_buffer_rsrc_t bnk_rsrc;
  if constexpr (B_NK) bnk_rsrc = make_rsrc(g.b + (int64_t)n0 * g.ldb, (uint32_t)min(TN, N - n0) * ldb2);

  // Direct-to-LDS loads: lane l of a wave's load writes the 16 bytes at
  // LDS unit base + l, so each lane fetches the global chunk that belongs at
  // that (swizzled) position. Per-lane geometry is fixed over the k loop.
  uint32_t a_off[A_I];
  int a_k[A_I];
#pragma unroll
  for (int i = 0; i < A_I; ++i) {
    const int p = (i * NW + wave) * 64 + lane;
    const int row = p >> 3, ch = (p & 7) ^ ((row ^ (row >> 3)) & 7);
    a_off[i] = (uint32_t)row * lda2 + (uint32_t)ch * 16u;
    a_k[i] = ch * 8;
  }
  uint32_t b_off[B_I];
  int b_k[B_I];  // [N,K]: k of the chunk; [K,N]: n of the chunk, relative to n0
#pragma unroll
  for (int i = 0; i < B_I; ++i) {
    const int p = (i * NW + wave) * 64 + lane;
    if constexpr (B_NK) {
      const int row = p >> 3, ch = (p & 7) ^ ((row ^ (row >> 3)) & 7);
      b_off[i] = (uint32_t)row * ldb2 + (uint32_t)ch * 16u;
      b_k[i] = ch * 8;
    } else {
      const int row = p / (TN / 8), ch = (p % (TN / 8)) ^ (4 * (row & 3));
      b_off[i] = (uint32_t)row * ldb2 + (uint32_t)ch * 16u;
      b_k[i] = ch * 8;
    }
  }

  // global -> LDS stage (as, bs), k tile t; tiles past K read zeros
  auto load = [&](int t, u32x4* as, u32x4* bs) {
    const int k0 = t * TK;
#pragma unroll
    for (int i = 0; i < A_I; ++i)
      lds_load16(a_rsrc, &as[(i * NW + wave) * 64],
                 (FULL || k0 + a_k[i] < K) ? a_off[i] + (uint32_t)k0 * 2u : OOB);
    if constexpr (B_NK) {
#pragma unroll
      for (int i = 0; i < B_I; ++i)
        lds_load16(bnk_rsrc, &bs[(i * NW + wave) * 64],
                   (FULL || k0 + b_k[i] < K) ? b_off[i] + (uint32_t)k0 * 2u : OOB);
    } else {
      // rows of this k tile only: rows past K lie past the descriptor. The
      // base and size are workgroup-uniform; readfirstlane lets the compiler
      // see that (a divergent descriptor would need a waterfall loop).
      const int kr = max(0, min(TK, K - k0));
      const uint64_t base = reinterpret_cast<uint64_t>(g.b + ((int64_t)k0 * g.ldb + n0));
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
      const uint32_t nbytes = __builtin_amdgcn_readfirstlane((uint32_t)kr * ldb2);
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), nbytes);
#pragma unroll
      for (int i = 0; i < B_I; ++i)
        lds_load16(r, &bs[(i * NW + wave) * 64], (FULL || n0 + b_k[i] < N) ? b_off[i] : OOB);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int arow0 = wm * WTM + (lane & 31);
  const int brow0 = wn * WTN + (lane & 31);
  const int khalf = lane >> 5;
  // [K,N] layout: a B fragment (8 consecutive k of one column n per lane) is
  // two ds_read_b64_tr_b16. Within each 16-lane group that instruction hands
  // lane i column i of the 4 x 16 block whose row r, 4-element piece q is
  // addressed by lane 4r + q. Lanes 0..31 take columns n0..n0+31 and k rows
  // 0..7 of the step; lanes 32..63 the same columns, k rows 8..15. Every row
  // a lane touches has row % 4 == tr_l / 4, so its swizzle is fixed per lane.
  const int tr_g = lane >> 4, tr_l = lane & 15;
  const int tr_row = 8 * (tr_g >> 1) + (tr_l >> 2);
  const int tr_sw = 4 * (tr_l >> 2);
  const int tr_lo = 2 * (tr_g & 1) + ((tr_l & 3) >> 1);  // chunk within the 4-chunk group
  const int tr_in = 4 * (tr_l & 1);                      // element within the chunk

  // Fragments of one 16-wide k step from LDS stage d, and the MFMAs that
  // consume them, for the first FMV of the wave's FM 32-row blocks (FMV is a
  // compile-time count, see below). The k loop keeps two fragment sets so the
  // LDS reads of step kk+1 are in flight while the MFMAs of step kk run.
  auto frags = [&](auto FMV, int kk, const u32x4* as, const u32x4* bs, bf16x8* af, bf16x8* bfr) {
    constexpr int fmv = decltype(FMV)::value;
    // FULL: the swizzled addresses are worked out at each read instead of
    // being kept in registers over the loop (an opaque copy of the row index
    // keeps the compiler from hoisting them)
    int ar0 = arow0, br0 = brow0;
    if constexpr (FULL) asm volatile("" : "+v"(ar0), "+v"(br0));
#pragma unroll
    for (int i = 0; i < fmv; ++i) af[i] = __builtin_bit_cast(bf16x8, as[swz(ar0 + i * 32, kk * 2 + khalf)]);
    if constexpr (B_NK) {
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = __builtin_bit_cast(bf16x8, bs[swz(br0 + j * 32, kk * 2 + khalf)]);
    } else {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const __attribute__((address_space(3))) short* bl = (const __attribute__((address_space(3))) short*)bs;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int chunk = (((wn * WTN + j * 32) >> 3) ^ tr_sw) + tr_lo;
        const int e = (kk * 16 + tr_row) * TN + chunk * 8 + tr_in;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(bl + e));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(bl + e + 4 * TN));
        bfr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  auto mma = [&](auto FMV, const bf16x8* af, const bf16x8* bfr) {
#pragma unroll
    for (int i = 0; i < decltype(FMV)::value; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  };

  // The loads of k tile kt+1 go straight into the other stage while tile kt
  // is multiplied; the barrier that ends the tile waits for them (vmcnt) and
  // publishes them to all waves. The stages reach `step` as __restrict__
  // pointers: once inlined, that gives the loads and the fragment reads
  // disjoint alias scopes, so the compiler does not make the reads of one
  // stage wait for the loads still landing in the other. A load past the
  // last tile reads zeros into the unused stage.
  //
  // FMV: how many of the wave's FM 32-row blocks hold rows below M. A block
  // wholly past M is neither read from LDS nor multiplied -- its outputs are
  // never stored, and every stored element still gets the same MFMA chain.
  // Each wave runs the loop copy for its own count (one branch before the
  // loop); all copies load and meet at the barriers alike. Full tiles take
  // the FMV = FM copy, which is the plain loop.
  static_assert(TK / 16 == 4, "the k step pipeline below assumes four 16-wide steps per tile");
  bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto kloop = [&](auto FMV) {
    auto step = [&](int kt, const u32x4* __restrict__ as, const u32x4* __restrict__ bs, u32x4* __restrict__ as_w,
                    u32x4* __restrict__ bs_w) {
      load(kt + 1, as_w, bs_w);
      // keep the loads at the head of the tile: nothing in this block consumes
      // them, and the scheduler would otherwise sink them to the barrier
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(FMV)::value > 0) {
        frags(FMV, 0, as, bs, fa0, fb0);
        frags(FMV, 1, as, bs, fa1, fb1);
        mma(FMV, fa0, fb0);
        frags(FMV, 2, as, bs, fa0, fb0);
        mma(FMV, fa1, fb1);
        frags(FMV, 3, as, bs, fa1, fb1);
        mma(FMV, fa0, fb0);
        mma(FMV, fa1, fb1);
      }
      __syncthreads();
    };
    load(0, As0, Bs0);
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, As0, Bs0, As1, Bs1);
      step(kt + 1, As1, Bs1, As0, Bs0);
    }
    if (kt < nk) step(kt, As0, Bs0, As1, Bs1);
  };
  const int wave_rows = M - m0 - wm * WTM;  // wave-uniform
  const int fmv = wave_rows <= 0 ? 0 : min(FM, (wave_rows + 31) / 32);
  if constexpr (FULL) {
    kloop(std::integral_constant<int, FM>{});
  } else if (fmv == FM) {
    kloop(std::integral_constant<int, FM>{});
  } else {
    static_for<0, FM>([&](auto I) {
      if (fmv == decltype(I)::value) kloop(I);
    });
  }

  // Epilogue: lane holds C[8*(r/4) + 4*(lane/32) + r%4][lane%32] of each
  // 32x32 tile, r = 0..15.
  // Interior fp32 tiles leave as 16-byte row chunks: each wave passes its
  // 32x32 blocks, alpha and bias already applied, through 4 KB of the (now
  // idle) first A stage -- column groups of 4 XOR-swizzled by row -- and
  // stores every row chunk with one 16-byte store. Same values, fewer and
  // wider stores.
  if (!g.out_bf16 && m0 + TM <= M && n0 + TN <= N && (g.ldc & 3) == 0 &&
      (reinterpret_cast<uintptr_t>(g.c) & 15) == 0) {
    static_assert(TM * 8 * 16 >= NW * 4096, "first A stage too small for the epilogue blocks");
    float* blk = reinterpret_cast<float*>(As0) + wave * 1024;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int gn0 = n0 + wn * WTN + j * 32;
      float bterm = 0.0f;
      if (g.bias_mode == 1) {
        bterm = g.beta * __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(g.bias)[gn0 + (lane & 31)]) << 16);
      } else if (g.bias_mode == 2) {
        bterm = g.beta * reinterpret_cast<const float*>(g.bias)[gn0 + (lane & 31)];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          float t = g.alpha * acc[i][j][r];
          if (g.bias_mode != 0) t = t + bterm;
          blk[row * 32 + ((lane & 31) ^ ((row & 7) << 2))] = t;
        }
        const int64_t gm0 = m0 + wm * WTM + i * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = lane + 64 * q;  // 32 rows x 8 chunks of 4 floats
          const int row = ch >> 3, c4 = ch & 7;
          const f32x4 v = *reinterpret_cast<const f32x4*>(blk + row * 32 + 4 * (c4 ^ (row & 7)));
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.c) + (gm0 + row) * g.ldc + gn0 + 4 * c4) = v;
        }
      }
    }
    return;
  }
  const int col_in = lane & 31;
  const int row_in = 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int gn = n0 + wn * WTN + j * 32 + col_in;
    if (gn >= N) continue;
    float bterm = 0.0f;
    if (g.bias_mode == 1) {
      bterm = g.beta * __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(g.bias)[gn]) << 16);
    } else if (g.bias_mode == 2) {
      bterm = g.beta * reinterpret_cast<const float*>(g.bias)[gn];
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + row_in + (r & 3);
        if (gm >= M) continue;
        float t = g.alpha * acc[i][j][r];
        if (g.bias_mode != 0) t = t + bterm;
        const int64_t off = (int64_t)gm * g.ldc + gn;
        if (g.out_bf16)
          reinterpret_cast<uint16_t*>(g.c)[off] = (uint16_t)f32_to_bf16_rne(t);
        else
          reinterpret_cast<float*>(g.c)[off] = t;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Ring kernels for small and medium M. With few rows, a 128-column tile of
// gemm_kernel gives only N / 128 workgroups, and each walks its k loop one
// memory round trip per k tile. gemm_ring_kernel splits a workgroup into C
// consumer waves, each owning a (32 FM) x (32 FN) block of the tile, and P
// producer waves that move its k tiles through an NS-stage LDS ring, up to
// NS - 2 tiles ahead of the MFMAs. The skinny form (one 32x32 block per
// consumer, 32 columns per workgroup) gives N / 32 workgroups for M <= 64,
// its 96-column form (three consumers across) N / 96 where those fill the
// CUs in one round, so a CU reads the rows of A once for 96 columns;
// the 128x128 form (2x2 consumers of 64x64) serves medium M. The
// per-element chain is the one of gemm_kernel: one v_mfma_f32_32x32x16_bf16
// per 16 k, increasing k, fp32 accumulator starting at 0, the same operand
// elements in the same lanes, k padded with zeros to a multiple of 64, the
// same epilogue -- so every output element has the bits the other tiles
// give it, and choosing these kernels by M keeps the result independent of M.
//
// The ring's loads are written as inline assembly (buffer_load_dwordx4 ...
// lds, LDS address in M0, restored afterwards): the compiler then does not
// see them write LDS and does not make every LDS read wait for every load in
// flight. The kernel orders them itself: before a tile is read, each
// producer waits until only the later tiles' loads are outstanding and a
// barrier publishes all parts; a stage is refilled only after the barrier
// that follows the MFMAs that consumed it; all loads have landed before the
// producers end. The instruction writes no register.
// ---------------------------------------------------------------------------

// s_waitcnt immediate waiting for vmcnt <= vm only (expcnt and lgkmcnt at
// their maxima).
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

// Buffer descriptor words from workgroup-uniform values (base, stride 0,
// byte count, format word as in make_rsrc).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffffu,
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// Load with the k offset in the instruction's scalar offset (soffset): the
// per-lane offset stays fixed over the k loop.
__device__ __forceinline__ void ring_load16_k(const u32x4& rsrc, uint32_t lds_byte, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_byte), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

template <int CM, int CN, int FM, int FN, int P, int NS, bool B_NK>
__global__ __launch_bounds__((CM * CN + P) * 64) void gemm_ring_kernel(GemmArgs g) {
  // C = CM x CN consumer waves, each owning a (32 FM) x (32 FN) block of the
  // TM x TN output tile, and P producer waves that only move k tiles into
  // the ring.
  constexpr int C = CM * CN;
  constexpr int WTM = 32 * FM, WTN = 32 * FN;
  constexpr int TM = CM * WTM, TN = CN * WTN;
  // One stage: A as TM rows of 64 k (eight 16-byte chunks, swizzled by swz),
  // then B: [N,K] as TN rows of 64 k (swizzled likewise), or [K,N] as 64 k
  // rows of TN columns (TN / 8 chunks; for TN a multiple of 128 chunk c of
  // row r stored at c ^ 4 (r % 4) as in gemm_kernel, otherwise as they are).
  static_assert(B_NK || TN % 32 == 0, "[K,N] stage layout needs TN a multiple of 32");
  constexpr bool BSW = !B_NK && TN % 128 == 0;
  constexpr int CPR = TN / 8;  // [K,N]: chunks per k row
  constexpr int A_CH = TM * 8, B_CH = TN * 8;
  constexpr int ST = A_CH + B_CH;                          // chunks per stage
  constexpr int A_I = A_CH / 64 / P, B_I = B_CH / 64 / P;  // 1 KB loads per producer per k tile
  constexpr int LPT = A_I + B_I;
  static_assert(A_I * 64 * P == A_CH && B_I * 64 * P == B_CH, "tile not evenly split across producers");
  static_assert(NS >= 4 && (FM * FN > 1 || NS % 2 == 0) && (NS - 2) * LPT < 64, "ring depth");
  static_assert(NS * ST * 16 <= 160 * 1024, "ring larger than LDS");
  __shared__ u32x4 ring[NS * ST];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * TM, n0 = tn * TN;
  const int M = g.m, N = g.n, K = g.k;
  const int nk = (K + TK - 1) / TK;

  // One barrier per k tile in both roles (plus one before the loop). At the
  // barrier of iteration t the producers' loads of tile t + 1 have landed
  // (each producer first waits until only the NS - 3 tiles after it are
  // outstanding), and the consumers have fed every fragment of tile t - 1 to
  // the MFMAs, so its stage may be refilled. No memory fence (it would wait
  // for every load in flight); the signal fences keep the compiler from
  // moving memory operations across.
  auto bar = [&]() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  if (wave >= C) {
    // ---------------- producer ----------------
    const int pw = wave - C;
    const int nk_full = K / TK;  // tiles with no k past K
    const uint32_t lda2 = (uint32_t)g.lda * 2u, ldb2 = (uint32_t)g.ldb * 2u;
    const uint32_t ring_base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(const void*)ring);
    // Rows of A past M (and of B past N, [N,K]) lie past their descriptor.
    const u32x4 a_rsrc = rsrc_words(g.a + (int64_t)m0 * g.lda, (uint32_t)min(TM, M - m0) * lda2);
    u32x4 bnk_rsrc{};
    if constexpr (B_NK) bnk_rsrc = rsrc_words(g.b + (int64_t)n0 * g.ldb, (uint32_t)min(TN, N - n0) * ldb2);
    // Per-lane source of the chunk each lane writes, fixed over the k loop:
    // producer pw's load i writes chunks (i P + pw) 64 + lane of A (of B).
    uint32_t a_off[A_I], b_off[B_I];
    int a_k[A_I], b_k[B_I];  // k of the chunk within the tile (for the tail tile)
#pragma unroll
    for (int i = 0; i < A_I; ++i) {
      const int p = (i * P + pw) * 64 + lane;
      const int row = p >> 3, ch = (p & 7) ^ ((row ^ (row >> 3)) & 7);
      a_off[i] = (uint32_t)row * lda2 + (uint32_t)ch * 16u;
      a_k[i] = ch * 8;
    }
#pragma unroll
    for (int i = 0; i < B_I; ++i) {
      const int p = (i * P + pw) * 64 + lane;
      if constexpr (B_NK) {
        const int row = p >> 3, ch = (p & 7) ^ ((row ^ (row >> 3)) & 7);
        b_off[i] = (uint32_t)row * ldb2 + (uint32_t)ch * 16u;
        b_k[i] = ch * 8;
      } else {
        // [K,N]: k row p / CPR of the tile, the chunk stored at position
        // p % CPR; columns past N read zeros
        const int row = p / CPR, c = p % CPR;
        const int ch = BSW ? (c ^ (4 * (row & 3))) : c;
        b_off[i] = (n0 + ch * 8 < N) ? (uint32_t)row * ldb2 + (uint32_t)ch * 16u : OOB;
        b_k[i] = row;
      }
    }
    // k tile t into stage j. Full tiles put k0 in the scalar offset; the tail
    // tile (and tiles past K, which read zeros) checks every chunk.
    auto load = [&](int t, int j) {
      const int k0 = t * TK;
      const uint32_t sa = ring_base + (uint32_t)(j * ST + pw * 64) * 16u;
      const uint32_t sb = sa + (uint32_t)A_CH * 16u;
      if (t < nk_full) {
#pragma unroll
        for (int i = 0; i < A_I; ++i)
          ring_load16_k(a_rsrc, sa + (uint32_t)(i * P * 64) * 16u, a_off[i], (uint32_t)k0 * 2u);
        if constexpr (B_NK) {
#pragma unroll
          for (int i = 0; i < B_I; ++i)
            ring_load16_k(bnk_rsrc, sb + (uint32_t)(i * P * 64) * 16u, b_off[i], (uint32_t)k0 * 2u);
        } else {
          const u32x4 r = rsrc_words(g.b + ((int64_t)k0 * g.ldb + n0), (uint32_t)TK * ldb2);
#pragma unroll
          for (int i = 0; i < B_I; ++i) ring_load16_k(r, sb + (uint32_t)(i * P * 64) * 16u, b_off[i], 0u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < A_I; ++i)
          ring_load16_k(a_rsrc, sa + (uint32_t)(i * P * 64) * 16u,
                        (k0 + a_k[i] < K) ? a_off[i] + (uint32_t)k0 * 2u : OOB, 0u);
        if constexpr (B_NK) {
#pragma unroll
          for (int i = 0; i < B_I; ++i)
            ring_load16_k(bnk_rsrc, sb + (uint32_t)(i * P * 64) * 16u,
                          (k0 + b_k[i] < K) ? b_off[i] + (uint32_t)k0 * 2u : OOB, 0u);
        } else {
          const u32x4 r =
              rsrc_words(g.b + ((int64_t)min(k0, K) * g.ldb + n0), (uint32_t)max(0, min(TK, K - k0)) * ldb2);
#pragma unroll
          for (int i = 0; i < B_I; ++i) ring_load16_k(r, sb + (uint32_t)(i * P * 64) * 16u, b_off[i], 0u);
        }
      }
    };
    static_for<0, NS - 1>([&](auto J) { load(decltype(J)::value, decltype(J)::value); });
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * LPT));  // tile 0
    bar();
    auto iter = [&](auto J, int t) {
      constexpr int j = decltype(J)::value;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 3) * LPT));  // tile t + 1
      bar();
      load(t + NS - 1, (j + NS - 1) % NS);  // into the stage of tile t - 1
    };
    int t = 0;
    for (; t + NS <= nk; t += NS) static_for<0, NS>([&](auto J) { iter(J, t + decltype(J)::value); });
    static_for<0, NS - 1>([&](auto J) {
      if (t + decltype(J)::value < nk) iter(J, t + decltype(J)::value);
    });
    __builtin_amdgcn_s_waitcnt(0);  // no load may still write LDS when the workgroup ends
    return;
  }

  // ---------------- consumer ----------------
  const int wm = wave / CN, wn = wave % CN;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int arow0 = wm * WTM + (lane & 31);
  const int brow0 = wn * WTN + (lane & 31);
  const int khalf = lane >> 5;
  const int tr_g = lane >> 4, tr_l = lane & 15;
  const int tr_row = 8 * (tr_g >> 1) + (tr_l >> 2);
  const int tr_sw = BSW ? 4 * (tr_l >> 2) : 0;
  const int tr_lo = 2 * (tr_g & 1) + ((tr_l & 3) >> 1);
  const int tr_in = 4 * (tr_l & 1);
  // fragments of k step kk of the tile in stage j
  auto read = [&](int j, int kk, bf16x8 (&af)[FM], bf16x8 (&bfr)[FN]) {
    const u32x4* as = ring + j * ST;
    const u32x4* bs = as + A_CH;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = __builtin_bit_cast(bf16x8, as[swz(arow0 + 32 * i, kk * 2 + khalf)]);
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) {
      if constexpr (B_NK) {
        bfr[jj] = __builtin_bit_cast(bf16x8, bs[swz(brow0 + 32 * jj, kk * 2 + khalf)]);
      } else {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const __attribute__((address_space(3))) short* bl =
            (const __attribute__((address_space(3))) short*)(const void*)bs;
        const int chunk = (((wn * WTN + 32 * jj) >> 3) ^ tr_sw) + tr_lo;
        const int e = (kk * 16 + tr_row) * TN + chunk * 8 + tr_in;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(bl + e));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(bl + e + 4 * TN));
        bfr[jj] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  auto mma = [&](const bf16x8 (&af)[FM], const bf16x8 (&bfr)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FN; ++jj)
        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[jj], acc[i][jj], 0, 0, 0);
  };
  int t = 0;
  if constexpr (FM * FN == 1) {
    // One block per wave: its four MFMAs per tile form a dependent chain, so
    // the next tile's fragments are read while they run (fragment buffers
    // indexed by stage parity; NS is even).
    bf16x8 fa[2][4][1], fb[2][4][1];
    bar();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) read(0, kk, fa[0][kk], fb[0][kk]);
    auto iter = [&](auto J, int) {
      constexpr int j = decltype(J)::value;
      bar();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) read((j + 1) % NS, kk, fa[(j + 1) & 1][kk], fb[(j + 1) & 1][kk]);  // tile t + 1
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) mma(fa[j & 1][kk], fb[j & 1][kk]);
    };
    for (; t + NS <= nk; t += NS) static_for<0, NS>([&](auto J) { iter(J, t + decltype(J)::value); });
    static_for<0, NS - 1>([&](auto J) {
      if (t + decltype(J)::value < nk) iter(J, t + decltype(J)::value);
    });
  } else {
    // Several blocks per wave: the k steps of a tile are pipelined inside it
    // (step kk + 1's fragments read while step kk's MFMAs run).
    bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    bar();
    auto iter = [&](auto J, int) {
      constexpr int j = decltype(J)::value;
      bar();  // tile t is in stage j; every wave is done with tile t - 1
      read(j, 0, fa0, fb0);
      read(j, 1, fa1, fb1);
      mma(fa0, fb0);
      read(j, 2, fa0, fb0);
      mma(fa1, fb1);
      read(j, 3, fa1, fb1);
      mma(fa0, fb0);
      mma(fa1, fb1);
    };
    for (; t + NS <= nk; t += NS) static_for<0, NS>([&](auto J) { iter(J, t + decltype(J)::value); });
    static_for<0, NS - 1>([&](auto J) {
      if (t + decltype(J)::value < nk) iter(J, t + decltype(J)::value);
    });
  }

  // Epilogue (as in gemm_kernel): lane holds C[8 (r / 4) + 4 (lane / 32) +
  // r % 4][lane % 32] of each 32x32 block, r = 0..15.
#pragma unroll
  for (int jj = 0; jj < FN; ++jj) {
    const int gn = n0 + wn * WTN + 32 * jj + (lane & 31);
    if (gn >= N) continue;
    float bterm = 0.0f;
    if (g.bias_mode == 1) {
      bterm = g.beta * __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(g.bias)[gn]) << 16);
    } else if (g.bias_mode == 2) {
      bterm = g.beta * reinterpret_cast<const float*>(g.bias)[gn];
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + wm * WTM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (gm >= M) continue;
        float v = g.alpha * acc[i][jj][r];
        if (g.bias_mode != 0) v = v + bterm;
        const int64_t off = (int64_t)gm * g.ldc + gn;
        if (g.out_bf16)
          reinterpret_cast<uint16_t*>(g.c)[off] = (uint16_t)f32_to_bf16_rne(v);
        else
          reinterpret_cast<float*>(g.c)[off] = v;
      }
    }
  }
}

template <int CM, int CN, int FM, int FN, int P, int NS, bool B_NK>
hipError_t launch_ring(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL((gemm_ring_kernel<CM, CN, FM, FN, P, NS, B_NK>), dim3((unsigned)tiles),
                     dim3((CM * CN + P) * 64), 0, s, a);
  return hipGetLastError();
}

template <int TM, int TN, int WM, int WN, bool B_NK>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL((gemm_kernel<TM, TN, WM, WN, B_NK>), dim3((unsigned)tiles), dim3(WM * WN * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// The tile table (gemm_config, gemm_config_fixed, gemm_plan) is host code in gemm_plan.cpp.

// One launch of the plan: the columns [n0, n1) of the output, with B, C and
// the bias offset to column n0.
static hipError_t launch_part(const GemmParams& p, const GemmLaunch& L, hipStream_t s) {
  const GemmConfig& cfg = L.cfg;
  const int64_t off = L.n_begin;
  GemmArgs a;
  a.a = static_cast<const uint16_t*>(p.a);
  a.b = p.b_is_nk ? static_cast<const uint16_t*>(p.b) + off * p.ldb : static_cast<const uint16_t*>(p.b) + off;
  a.c = p.c_bf16 ? (void*)(static_cast<uint16_t*>(p.c) + off) : (void*)(static_cast<float*>(p.c) + off);
  a.bias = p.bias == nullptr ? nullptr
           : p.bias_bf16     ? (const void*)(static_cast<const uint16_t*>(p.bias) + off)
                             : (const void*)(static_cast<const float*>(p.bias) + off);
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.ldc = p.ldc;
  a.m = (int)p.m;
  a.n = (int)(L.n_end - off);
  a.k = (int)p.k;
  a.alpha = p.alpha;
  a.beta = p.beta;
  a.out_bf16 = p.c_bf16 ? 1 : 0;
  a.bias_mode = p.bias == nullptr ? 0 : (p.bias_bf16 ? 1 : 2);
  a.tiles_m = (int)((p.m + cfg.tile_m - 1) / cfg.tile_m);
  a.tiles_n = (int)((a.n + cfg.tile_n - 1) / cfg.tile_n);
  if (cfg.tile_n == 32) {  // skinny: 16-stage ring with one consumer, 12 with two
    if (cfg.tile_m == 32)
      return p.b_is_nk ? launch_ring<1, 1, 1, 1, 2, 16, true>(a, s) : launch_ring<1, 1, 1, 1, 2, 16, false>(a, s);
    if (cfg.tile_m == 64)
      return p.b_is_nk ? launch_ring<2, 1, 1, 1, 2, 12, true>(a, s) : launch_ring<2, 1, 1, 1, 2, 12, false>(a, s);
    return hipErrorInvalidConfiguration;
  }
  if (cfg.tile_n == 96) {  // 1x3 or 2x3 consumers of 32x32, 8-stage ring
    if (cfg.tile_m == 32)
      return p.b_is_nk ? launch_ring<1, 3, 1, 1, 2, 8, true>(a, s) : launch_ring<1, 3, 1, 1, 2, 8, false>(a, s);
    if (cfg.tile_m == 64)
      return p.b_is_nk ? launch_ring<2, 3, 1, 1, 2, 8, true>(a, s) : launch_ring<2, 3, 1, 1, 2, 8, false>(a, s);
    return hipErrorInvalidConfiguration;
  }
  if (cfg.tile_m == 128 && cfg.tile_n == 128 && cfg.waves == 10)  // 4x2 consumers of 32x64, 4-stage ring
    return p.b_is_nk ? launch_ring<4, 2, 1, 2, 2, 4, true>(a, s) : launch_ring<4, 2, 1, 2, 2, 4, false>(a, s);
  if (cfg.tile_m == 64 && cfg.tile_n == 128)  // 2x2 consumers of 32x64, 6-stage ring
    return p.b_is_nk ? launch_ring<2, 2, 1, 2, 2, 6, true>(a, s) : launch_ring<2, 2, 1, 2, 2, 6, false>(a, s);
#define BI_GEMM_CASE(TM_, TN_, WM_, WN_)                                                          \
  if (cfg.tile_m == TM_ && cfg.tile_n == TN_ && cfg.waves == WM_ * WN_)                            \
    return p.b_is_nk ? launch_cfg<TM_, TN_, WM_, WN_, true>(a, s) : launch_cfg<TM_, TN_, WM_, WN_, false>(a, s);
  BI_GEMM_CASE(128, 128, 2, 2)
  BI_GEMM_CASE(256, 256, 2, 4)
  BI_GEMM_CASE(256, 128, 4, 2)
#undef BI_GEMM_CASE
  // 256x384 assumes whole k tiles and tile columns (no masks); the table
  // picks it only then
  if (cfg.tile_m == 256 && cfg.tile_n == 384 && cfg.waves == 8) {
    if (p.k <= 0 || p.k % 64 != 0 || a.n % 384 != 0) return hipErrorInvalidConfiguration;
    return p.b_is_nk ? launch_cfg<256, 384, 2, 4, true>(a, s) : launch_cfg<256, 384, 2, 4, false>(a, s);
  }
  return hipErrorInvalidConfiguration;
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  const GemmPlan plan = gemm_plan(p.m, p.n, p.k, p.b_is_nk, p.fixed_tile);
  for (int i = 0; i < plan.count; ++i) {
    const hipError_t e = launch_part(p, plan.launch[i], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bi
