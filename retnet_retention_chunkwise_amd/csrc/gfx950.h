// gfx950 building blocks shared by the bf16 MFMA kernels: the 16x16x32 bf16
// MFMA, LDS reads (plain and transposing), LDS-only workgroup barriers and
// raw buffer loads/stores with hardware bounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ret {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, lane j receives element
// (j % 4) of the 4-element row read by lane 4*e + j/4, for e = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 lds_read16(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Workgroup barrier for hand-offs through LDS.  The fences cover LDS only, so
// a wave waits for its own LDS accesses but not for its global loads and
// stores in flight: the K/V/Q loads of later chunks and the Y stores stay
// outstanding across the barrier (a __syncthreads() fence would drain them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads past the end return 0,
// stores past the end are dropped.  0x00020000 is the gfx9 data-format word.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void buffer_store8(rsrc_t r, uint32_t off, u32x2 x) {
  __builtin_amdgcn_raw_buffer_store_b64(x, r, static_cast<int>(off), 0, 0);
}
__device__ __forceinline__ void buffer_store16(rsrc_t r, uint32_t off, u32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, static_cast<int>(off), 0, 0);
}

// Sum of x over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows of
// the wave at one position), in each of them: the gfx950 cross-row swaps
// v_permlane32_swap (rows 0,1 <-> 2,3) and v_permlane16_swap (rows 0 <-> 1,
// 2 <-> 3), VALU operations with no LDS round trip.  The two operands of each
// addition are the same pair in all four lanes, so they agree bit for bit.
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Eight fp32 values as an MFMA bf16 operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16x8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = static_cast<__bf16>(lo[0]);
  r[1] = static_cast<__bf16>(lo[1]);
  r[2] = static_cast<__bf16>(lo[2]);
  r[3] = static_cast<__bf16>(lo[3]);
  r[4] = static_cast<__bf16>(hi[0]);
  r[5] = static_cast<__bf16>(hi[1]);
  r[6] = static_cast<__bf16>(hi[2]);
  r[7] = static_cast<__bf16>(hi[3]);
  return r;
}

}  // namespace ret
