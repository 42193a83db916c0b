// Device helpers shared by the kernels: bf16 unpack/pack, fixed-order
// wavefront reductions, 128-bit vector types.
//
// Determinism notes
//  * Every reduction here has a fixed shape: a wave butterfly over xor
//    distances 32,16,8,4,2,1 (or a sub-range), then a fixed-order loop over
//    the waves' partials. In a butterfly each lane combines v[l] with
//    v[l ^ d]; because fp addition is commutative both partners get the same
//    bits, so after every step all lanes of a group hold identical values and
//    the result is independent of which lane reads it.
//  * The code is compiled with -ffp-contract=off; multiply-adds that should
//    fuse are written as explicit fmaf, so the arithmetic of each expression
//    is fixed by the source, not by the optimiser.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Two fp32 -> bf16 RNE conversions in one instruction (gfx950's
// v_cvt_pk_bf16_f32): lo in bits 0..15, hi in 16..31. For every non-NaN
// input it gives f32_to_bf16_rne's bits (checked on MI355X over all 2^32
// patterns, denormals included, in the kernels' default FP mode); a NaN
// stays a NaN, its payload may differ.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Cross-lane read of lane (lane ^ d) within a wavefront (ds_swizzle/bpermute
// chosen by the compiler through __shfl_xor).
__device__ __forceinline__ float xor_shfl(float v, int d) { return __shfl_xor(v, d, 64); }

// Sum over a full 64-lane wave; every lane gets identical bits.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = v + xor_shfl(v, d);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, xor_shfl(v, d));
  return v;
}

// Sum over aligned groups of 16 lanes (xor distances 8,4,2,1).
__device__ __forceinline__ float group16_sum(float v) {
  v = v + xor_shfl(v, 8);
  v = v + xor_shfl(v, 4);
  v = v + xor_shfl(v, 2);
  v = v + xor_shfl(v, 1);
  return v;
}

// Unpack 8 bf16 values (one 128-bit load) to fp32, element order preserved.
__device__ __forceinline__ void unpack8(const u32x4& w, float* f) {
  f[0] = bf16lo(w.x); f[1] = bf16hi(w.x);
  f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
  f[4] = bf16lo(w.z); f[5] = bf16hi(w.z);
  f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
}

}  // namespace bi
