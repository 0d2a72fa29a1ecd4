// Device-side helpers for the gfx950 kernels: bf16 packing, cross-lane
// reductions within a 64-lane wavefront, and float formats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---- bf16 <-> fp32 ------------------------------------------------------
// A dword holding two bf16 values: element 0 in bits 0..15, element 1 in
// bits 16..31.  Widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round fp32 to bf16, nearest with ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 inputs and fp32 accumulation
// (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---- cross-lane ---------------------------------------------------------
// DPP quad permutations: value from lane (lane ^ 1) and (lane ^ 2) within
// each group of four lanes.
__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
// DPP row half-mirror: value from lane 7 - i within each group of eight
// lanes (that is, lane i ^ 7).
__device__ __forceinline__ float octet_mirror(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
}
// Sum over each group of four lanes; every lane of the group gets the sum.
__device__ __forceinline__ float quad_sum(float x) {
  x += quad_xor1(x);
  x += quad_xor2(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  // ds_bpermute: lane reads lane ^ mask
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// Reductions over the full 64-lane wavefront.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, shfl_xor_f(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += shfl_xor_f(x, m);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
