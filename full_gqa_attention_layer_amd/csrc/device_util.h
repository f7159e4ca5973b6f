// Device helpers shared by the gfx950 kernels: bf16 packing, MFMA operand
// types, RoPE angles, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hgqa_internal.h"

namespace hgqa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Two floats to two bf16 (round to nearest even) packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// (cos, sin) of the RoPE angle pos * theta^(-2i/r). The angle is formed in
// half-turns in double and reduced exactly to [-1, 1] before the float
// sincospi, so large positions lose no accuracy.
__device__ __forceinline__ float2 rope_cos_sin(int pos, double freq_over_pi) {
  double h = (double)pos * freq_over_pi;
  double k = rint(h * 0.5);
  float x = (float)(h - 2.0 * k);
  float s, c;
  sincospif(x, &s, &c);
  return make_float2(c, s);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ float sigmoidf_dev(float x) { return 1.0f / (1.0f + __expf(-x)); }

}  // namespace hgqa
