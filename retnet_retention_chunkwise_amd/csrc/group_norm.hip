// Per-head GroupNorm of the retention output.  Multi-scale retention
// normalises its output with GroupNorm, one group per head, because the heads
// (each with its own decay) have different statistics (paperhub page, author
// answer A4 on the GroupNorm of Eq. 8).  For every (b, h, t) the d_v values
// y[b,h,t,:] form one group:
//   mu = mean_c y[c],  var = mean_c (y[c] - mu)^2,
//   out[c] = (y[c] - mu) / sqrt(var + eps) * weight[h,c] + bias[h,c].
// The pass streams y once in and once out, so it is bound by HBM bandwidth:
// each row (token-head) is held by one wave, each lane holding its VEC-element
// pieces in registers (one 16-byte non-temporal load per lane for bf16 rows of
// 512; y is read once and the output is not read back here), mean
// and variance in two passes over the registers with wave-wide sums on DPP
// and cross-row lane swaps, fp32 arithmetic throughout.
#include "common.h"
#include "gfx950.h"
#include "kernels.h"

namespace ret {
namespace {

constexpr int kThreads = 256;  // 4 rows per workgroup
constexpr int kMaxRow = 512;   // longest row (d_v)

template <typename E, int VEC>
struct Vec;
template <>
struct Vec<uint16_t, 8> {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __device__ __forceinline__ static void load(const uint16_t* p, float (&x)[8]) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(v[i] << 16);
      x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store(uint16_t* p, const float (&x)[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  }
};
template <>
struct Vec<float, 4> {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __device__ __forceinline__ static void load(const float* p, float (&x)[4]) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
  }
  __device__ __forceinline__ static void store(float* p, const float (&x)[4]) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
  }
};
template <typename E>
struct Vec<E, 1> {
  __device__ __forceinline__ static void load(const E* p, float (&x)[1]) { x[0] = Elem<E>::load(p, 0); }
  __device__ __forceinline__ static void store(E* p, const float (&x)[1]) { Elem<E>::store(p, 0, x[0]); }
};

// VEC fp32 weights/biases from 16-byte aligned rows (a row of a [H, d_v] fp32
// array starts 16-byte aligned when d_v % 4 == 0, the only case with VEC > 1).
template <int VEC>
__device__ __forceinline__ void load_f32(const float* p, float (&x)[VEC]) {
  if constexpr (VEC % 4 == 0) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * k);
      x[4 * k] = v[0]; x[4 * k + 1] = v[1]; x[4 * k + 2] = v[2]; x[4 * k + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) x[e] = p[e];
  }
}

// Sum over the wave's 64 lanes, the same value in every lane: DPP steps
// inside each 16-lane row (lane pairs xor 1, xor 2, then the row mirror and
// half-row mirror, which pair quads 0+3 with 1+2), then the two cross-row
// swaps of row4_sum.  Every addition has the same two operands in all lanes
// that meet it, so the sums agree bit for bit; all VALU, no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_plus(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_plus<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_plus<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_plus<0x140>(v);  // row_mirror
  v = dpp_plus<0x141>(v);  // row_half_mirror
  return row4_sum(v);
}

// Each wave normalises kRows consecutive rows; lane l holds the pieces that
// start at element VEC * (l + 64 i), i < NI, of every row.  All rows' loads are
// issued before the first reduction and the rows' butterfly sums interleave.
// Consecutive rows are consecutive tokens of one head, so the head's weight
// and bias pieces are loaded once per wave (again only if a row starts a new
// head).  Two rows per wave measured best on the 1.3B-layer output (25.6 us
// for 134 MB with the DPP sums, 27.4 us with ds_bpermute butterflies; one or
// four rows per wave 27.8 and 29.8 us; a persistent grid that loads the next
// pair of rows while normalising the current one 30.7-31.8 us).
constexpr int kRows = 2;

template <typename E, int VEC>
__global__ __launch_bounds__(kThreads) void group_norm_kernel(const E* y, const float* __restrict__ weight,
                                                              const float* __restrict__ bias, float eps, E* out,
                                                              long rows, int H, int T, int dv) {
  constexpr int NI = (kMaxRow + 64 * VEC - 1) / (64 * VEC);
  const int lane = threadIdx.x & 63;
  const long row0 = (static_cast<long>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6)) * kRows;
  if (row0 >= rows) return;  // no barrier in this kernel
  float x[kRows][NI][VEC];
  float s[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    s[r] = 0.0f;
    const long row = row0 + r;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = VEC * (lane + 64 * i);
      if (row < rows && c < dv) Vec<E, VEC>::load(y + row * dv + c, x[r][i]);
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (row0 + r < rows && VEC * (lane + 64 * i) < dv)
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[r] += x[r][i][e];
  const float inv_n = 1.0f / static_cast<float>(dv);
  float mu[kRows], q[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) mu[r] = wave_sum(s[r]) * inv_n;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    q[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (row0 + r < rows && VEC * (lane + 64 * i) < dv)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float d = x[r][i][e] - mu[r];
          q[r] = fmaf(d, d, q[r]);
        }
  }
  float wv[NI][VEC], bv[NI][VEC];
  int hcur = -1;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const long row = row0 + r;
    const float rstd = 1.0f / sqrtf(wave_sum(q[r]) * inv_n + eps);
    if (row >= rows) continue;
    const int h = (static_cast<int>(row) / T) % H;  // rows < 2^31
    if (h != hcur) {  // wave-uniform
      hcur = h;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = VEC * (lane + 64 * i);
        const bool in = c < dv;
        if (weight != nullptr && in)
          load_f32<VEC>(weight + h * dv + c, wv[i]);
        else
#pragma unroll
          for (int e = 0; e < VEC; ++e) wv[i][e] = 1.0f;
        if (bias != nullptr && in)
          load_f32<VEC>(bias + h * dv + c, bv[i]);
        else
#pragma unroll
          for (int e = 0; e < VEC; ++e) bv[i][e] = 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = VEC * (lane + 64 * i);
      if (c < dv) {
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = fmaf((x[r][i][e] - mu[r]) * rstd, wv[i][e], bv[i][e]);
        Vec<E, VEC>::store(out + row * dv + c, o);
      }
    }
  }
}

template <typename E, int VEC>
hipError_t launch_vec(const void* y, const float* w, const float* b, float eps, void* out, long rows, int H, int T,
                      int dv, hipStream_t s) {
  const long per_block = (kThreads / 64) * kRows;
  const long blocks = (rows + per_block - 1) / per_block;
  hipLaunchKernelGGL((group_norm_kernel<E, VEC>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s,
                     static_cast<const E*>(y), w, b, eps, static_cast<E*>(out), rows, H, T, dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_group_norm(const void* y, const float* weight, const float* bias, float eps, void* out, int B,
                             int H, int T, int dv, int dt, hipStream_t s) {
  const long rows = static_cast<long>(B) * H * T;
  if (rows == 0) return hipSuccess;
  if (dt == 1)
    return dv % 8 == 0 ? launch_vec<uint16_t, 8>(y, weight, bias, eps, out, rows, H, T, dv, s)
                       : launch_vec<uint16_t, 1>(y, weight, bias, eps, out, rows, H, T, dv, s);
  return dv % 4 == 0 ? launch_vec<float, 4>(y, weight, bias, eps, out, rows, H, T, dv, s)
                     : launch_vec<float, 1>(y, weight, bias, eps, out, rows, H, T, dv, s);
}

}  // namespace ret
