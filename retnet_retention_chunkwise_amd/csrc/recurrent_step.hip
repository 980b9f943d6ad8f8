// One recurrent (decode) step of retention, in place on an fp32 state:
//   S <- gamma S + k^T v ;  y = q S
// (recurrent form of "Retentive Networks — Microsoft Propone l'Alternativa
// Architetturale ai Transformer", section "Il meccanismo: Multi-Scale Retention").
//
// The step streams the whole d_k x d_v fp32 state once in and once out, so it
// is bound by HBM bandwidth.  Layout of the work:
//   - one workgroup (4 waves) per (batch, head, slice of 64*VEC columns);
//   - lane l of every wave owns VEC consecutive columns, so each wave moves
//     64*VEC*4 contiguous bytes per state row (dwordx4 accesses for VEC = 4);
//   - the 4 waves take interleaved rows, 16 rows in flight per lane, and the
//     state moves with non-temporal loads/stores (it is streamed once per step
//     and is larger than any cache, so it should not displace other lines);
//   - the state row is updated in registers and reused for y without a
//     re-read; the partial y of the 4 waves is summed through LDS;
//   - a workgroup requests its first state rows before it stages q and k.
#include "common.h"
#include "kernels.h"

namespace ret {
namespace {

typedef float vf4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsInFlight = 16;

template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void recurrent_step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                  const T* __restrict__ v, float* __restrict__ S,
                                                                  T* __restrict__ y, HeadDecay gam, int H, int h0,
                                                                  int nh, int dk, int dv) {
  __shared__ float qs[256];
  __shared__ float ks[256];
  __shared__ float red[kWaves][64 * VEC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = blockIdx.y % nh;
  const int b = blockIdx.y / nh;
  const long head = static_cast<long>(b) * H + h0 + hl;
  const float g = gam.log2g[hl] == -INFINITY ? 0.0f : exp2f(gam.log2g[hl]);

  const int c0 = blockIdx.x * 64 * VEC + lane * VEC;
  const bool active = c0 < dv;  // VEC = 4 is only used when dv % 4 == 0
  float* Sh = S + head * static_cast<long>(dk) * dv + c0;
  float s[kRowsInFlight][VEC];
  // rows r0, r0 + 4, ..., r0 + 4 (kRowsInFlight - 1) of this lane's columns
  auto load_rows = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int r = r0 + kWaves * u;
      if (r < dk) {
        if constexpr (VEC == 4) {
          const vf4 t = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(Sh + static_cast<long>(r) * dv));
          s[u][0] = t[0]; s[u][1] = t[1]; s[u][2] = t[2]; s[u][3] = t[3];
        } else {
          s[u][0] = Sh[static_cast<long>(r) * dv];
        }
      }
    }
  };
  // the first rows are requested before the q/k staging and its barrier, so
  // that a starting workgroup's state loads are in flight while it stages
  if (active) load_rows(w);
  for (int i = tid; i < dk; i += kThreads) {
    qs[i] = Elem<T>::load(q, head * dk + i);
    ks[i] = Elem<T>::load(k, head * dk + i);
  }
  float vv[VEC];
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    vv[e] = active ? Elem<T>::load(v, head * dv + c0 + e) : 0.0f;
    acc[e] = 0.0f;
  }
  __syncthreads();

  if (active) {
    for (int r0 = w; r0 < dk; r0 += kWaves * kRowsInFlight) {
      if (r0 != w) load_rows(r0);
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int r = r0 + kWaves * u;
        if (r < dk) {
          const float kr = ks[r];
          const float qr = qs[r];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            s[u][e] = fmaf(g, s[u][e], kr * vv[e]);
            acc[e] = fmaf(qr, s[u][e], acc[e]);
          }
          if constexpr (VEC == 4) {
            __builtin_nontemporal_store(vf4{s[u][0], s[u][1], s[u][2], s[u][3]}, reinterpret_cast<vf4*>(Sh + static_cast<long>(r) * dv));
          } else {
            Sh[static_cast<long>(r) * dv] = s[u][0];
          }
        }
      }
    }
  }

#pragma unroll
  for (int e = 0; e < VEC; ++e) red[w][lane * VEC + e] = acc[e];
  __syncthreads();
  if (w == 0 && active) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float t = red[0][lane * VEC + e];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) t += red[ww][lane * VEC + e];
      Elem<T>::store(y, head * dv + c0 + e, t);
    }
  }
}

template <typename T>
hipError_t launch_t(const void* q, const void* k, const void* v, float* state, void* y, int B, int H, int dk, int dv,
                    const HeadDecay& hd, const HeadGroup& g, hipStream_t s) {
  const bool vec4 = (dv % 4) == 0;
  const int cols = vec4 ? 256 : 64;
  dim3 grid((dv + cols - 1) / cols, B * g.nh);
  const T* qp = static_cast<const T*>(q);
  const T* kp = static_cast<const T*>(k);
  const T* vp = static_cast<const T*>(v);
  T* yp = static_cast<T*>(y);
  if (vec4)
    hipLaunchKernelGGL((recurrent_step_kernel<T, 4>), grid, dim3(kThreads), 0, s, qp, kp, vp, state, yp, hd, H, g.h0,
                       g.nh, dk, dv);
  else
    hipLaunchKernelGGL((recurrent_step_kernel<T, 1>), grid, dim3(kThreads), 0, s, qp, kp, vp, state, yp, hd, H, g.h0,
                       g.nh, dk, dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_recurrent_step(const void* q, const void* k, const void* v, float* state, void* y, int B, int H,
                                 int dk, int dv, int dt, const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  return dt == 0 ? launch_t<float>(q, k, v, state, y, B, H, dk, dv, hd, g, s)
                 : launch_t<uint16_t>(q, k, v, state, y, B, H, dk, dv, hd, g, s);
}

}  // namespace ret
