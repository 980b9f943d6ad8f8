// Device helpers shared by the libretention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ret {

// gamma^d for an integer d >= 0 from log2(gamma).  gamma^0 is exactly 1 (also
// for gamma = 0, where 0 * -inf would otherwise give NaN).
__device__ __forceinline__ float gamma_pow(float log2g, int d) {
  return d == 0 ? 1.0f : exp2f(static_cast<float>(d) * log2g);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(static_cast<uint32_t>(u) << 16); }

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// Element access for the two input dtypes: float and raw bf16 bits.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, long i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, long i, float x) { p[i] = x; }
};
template <>
struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, long i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, long i, float x) { p[i] = f32_to_bf16(x); }
};

}  // namespace ret
