// Parallel form of retention:
//   Y = ((Q K^T) .* D) V + diag(gamma^(n+1)) Q S_in,  D[n,m] = gamma^(n-m) (n >= m), 0 above
// ("Retentive Networks — Microsoft Propone l'Alternativa Architetturale ai
// Transformer", section "Il meccanismo: Multi-Scale Retention": the whole
// retention matrix at once, like attention).
//
// A plain fp32 VALU kernel: the parallel form costs O(T^2) per head and is
// meant for short sequences and as an independent cross-check of the
// chunkwise kernels.  One workgroup per (batch, head, block of 16 query rows);
// key tiles of 16 rows stream through LDS; every thread owns up to 2 output
// columns for all 16 rows.
#include "common.h"
#include "kernels.h"

namespace ret {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;   // query rows per workgroup
constexpr int kKeys = 16;   // key rows per LDS tile
constexpr int kColsPerThread = 2;

template <typename T>
__global__ __launch_bounds__(kThreads) void parallel_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                const T* __restrict__ v,
                                                                const float* __restrict__ state_in,
                                                                T* __restrict__ y, HeadDecay gam, int H, int h0, int nh,
                                                                int Tn, int dk, int dv) {
  extern __shared__ float smem[];
  float* Qs = smem;                 // [kRows][dk]
  float* Ks = Qs + kRows * dk;      // [kKeys][dk]
  float* Vs = Ks + kKeys * dk;      // [kKeys][dv]
  float* P = Vs + kKeys * dv;       // [kRows][kKeys]

  const int tid = threadIdx.x;
  const int hl = blockIdx.y % nh;
  const int b = blockIdx.y / nh;
  const long head = static_cast<long>(b) * H + h0 + hl;
  const float lg = gam.log2g[hl];
  const int row0 = blockIdx.x * kRows;
  const T* qh = q + head * Tn * dk;
  const T* kh = k + head * Tn * dk;
  const T* vh = v + head * Tn * dv;

  for (int e = tid; e < kRows * dk; e += kThreads) {
    const int i = e / dk, d = e % dk;
    Qs[e] = (row0 + i < Tn) ? Elem<T>::load(qh, static_cast<long>(row0 + i) * dk + d) : 0.0f;
  }

  float acc[kRows][kColsPerThread];
#pragma unroll
  for (int i = 0; i < kRows; ++i)
#pragma unroll
    for (int j = 0; j < kColsPerThread; ++j) acc[i][j] = 0.0f;

  const int last_row = min(Tn, row0 + kRows) - 1;
  for (int m0 = 0; m0 <= last_row; m0 += kKeys) {
    __syncthreads();  // previous tile fully consumed (and Qs written on the first pass)
    for (int e = tid; e < kKeys * dk; e += kThreads) {
      const int j = e / dk, d = e % dk;
      Ks[e] = (m0 + j < Tn) ? Elem<T>::load(kh, static_cast<long>(m0 + j) * dk + d) : 0.0f;
    }
    for (int e = tid; e < kKeys * dv; e += kThreads) {
      const int j = e / dv, c = e % dv;
      Vs[e] = (m0 + j < Tn) ? Elem<T>::load(vh, static_cast<long>(m0 + j) * dv + c) : 0.0f;
    }
    __syncthreads();
    {
      // one score per thread: kRows * kKeys == kThreads
      const int i = tid / kKeys, j = tid % kKeys;
      const int n = row0 + i, m = m0 + j;
      float s = 0.0f;
      if (m <= n && n < Tn) {
        for (int d = 0; d < dk; ++d) s = fmaf(Qs[i * dk + d], Ks[j * dk + d], s);
        s *= gamma_pow(lg, n - m);
      }
      P[i * kKeys + j] = s;
    }
    __syncthreads();
#pragma unroll
    for (int jc = 0; jc < kColsPerThread; ++jc) {
      const int c = tid + jc * kThreads;
      if (c < dv) {
        for (int j = 0; j < kKeys; ++j) {
          const float vj = Vs[j * dv + c];
#pragma unroll
          for (int i = 0; i < kRows; ++i) acc[i][jc] = fmaf(P[i * kKeys + j], vj, acc[i][jc]);
        }
      }
    }
  }

  // contribution of the initial state: gamma^(n+1) Q_n S_in
  if (state_in != nullptr) {
    const float* Sh = state_in + head * static_cast<long>(dk) * dv;
#pragma unroll
    for (int jc = 0; jc < kColsPerThread; ++jc) {
      const int c = tid + jc * kThreads;
      if (c < dv) {
        float t[kRows];
#pragma unroll
        for (int i = 0; i < kRows; ++i) t[i] = 0.0f;
        for (int d = 0; d < dk; ++d) {
          const float sv = Sh[static_cast<long>(d) * dv + c];
#pragma unroll
          for (int i = 0; i < kRows; ++i) t[i] = fmaf(Qs[i * dk + d], sv, t[i]);
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) acc[i][jc] = fmaf(gamma_pow(lg, row0 + i + 1), t[i], acc[i][jc]);
      }
    }
  }

  T* yh = y + head * Tn * dv;
#pragma unroll
  for (int jc = 0; jc < kColsPerThread; ++jc) {
    const int c = tid + jc * kThreads;
    if (c < dv) {
#pragma unroll
      for (int i = 0; i < kRows; ++i)
        if (row0 + i < Tn) Elem<T>::store(yh, static_cast<long>(row0 + i) * dv + c, acc[i][jc]);
    }
  }
}

template <typename T>
hipError_t launch_t(const void* q, const void* k, const void* v, const float* state_in, void* y, int B, int H, int Tn,
                    int dk, int dv, const HeadDecay& hd, const HeadGroup& g, hipStream_t s) {
  const size_t lds = sizeof(float) * (static_cast<size_t>(kRows + kKeys) * dk + static_cast<size_t>(kKeys) * dv +
                                      kRows * kKeys);
  auto kern = parallel_fwd_kernel<T>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  dim3 grid((Tn + kRows - 1) / kRows, B * g.nh);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), state_in, static_cast<T*>(y), hd, H, g.h0, g.nh, Tn, dk, dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_parallel_fwd(const void* q, const void* k, const void* v, const float* state_in, void* y, int B,
                               int H, int T, int dk, int dv, int dt, const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  return dt == 0 ? launch_t<float>(q, k, v, state_in, y, B, H, T, dk, dv, hd, g, s)
                 : launch_t<uint16_t>(q, k, v, state_in, y, B, H, T, dk, dv, hd, g, s);
}

}  // namespace ret
