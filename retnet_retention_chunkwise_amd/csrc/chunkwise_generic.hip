// Chunkwise form of retention, generic fp32-arithmetic VALU kernel.
//
// The chunkwise form of "Retentive Networks — Microsoft Propone l'Alternativa
// Architetturale ai Transformer" (section "Il meccanismo: Multi-Scale
// Retention") runs the parallel form inside chunks of C tokens and the
// recurrence across chunks.  For chunk i (rows j = 0..L-1, carried state R_i):
//   Y_[i]   = ((Q_[i] K_[i]^T) .* D_L) V_[i] + diag(gamma^(j+1)) Q_[i] R_i
//   R_(i+1) = gamma^L R_i + (diag(gamma^(L-1-j)) K_[i])^T V_[i]
//
// This kernel serves fp32 inputs (whose tolerance needs fp32 products) and any
// shape the bf16 MFMA kernel does not take.  One workgroup per (batch, head,
// tile of 32 value columns) walks the chunks in order; the 32 state columns
// (d_k x 32 fp32) stay in LDS for the whole sequence.  d_k is consumed in
// sub-blocks of 32 so that the Q/K staging stays small.
#include "common.h"
#include "kernels.h"

namespace ret {
namespace {

constexpr int kThreads = 256;
constexpr int kTileCols = 32;  // value columns per workgroup
constexpr int kSub = 32;       // d_k sub-block

template <typename T, int CT>
__global__ __launch_bounds__(kThreads) void chunkwise_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* state_in,
    float* state_out, T* __restrict__ y, HeadDecay gam, int H, int h0, int nh, int Tn, int dk, int dv, int C) {
  static_assert(CT * CT % kThreads == 0 || CT * CT < kThreads, "score split");
  constexpr int kScores = (CT * CT + kThreads - 1) / kThreads;  // score entries per thread
  constexpr int kRowsPerThread = CT / 8;                         // output rows per thread (8 row groups)

  extern __shared__ float smem[];
  float* Rs = smem;                   // [dk][kTileCols]  carried state, fp32
  float* Qsub = Rs + dk * kTileCols;  // [CT][kSub]
  float* Ksub = Qsub + CT * kSub;     // [CT][kSub]
  float* Vs = Ksub + CT * kSub;       // [CT][kTileCols]
  float* P = Vs + CT * kTileCols;     // [CT][CT]
  float* zeta = P + CT * CT;          // [CT]  gamma^(L-1-j)

  const int tid = threadIdx.x;
  const int hl = blockIdx.y % nh;
  const int b = blockIdx.y / nh;
  const long head = static_cast<long>(b) * H + h0 + hl;
  const float lg = gam.log2g[hl];
  const int col0 = blockIdx.x * kTileCols;
  const int cl = tid % kTileCols;      // this thread's column inside the tile
  const int rg = tid / kTileCols;      // row group 0..7
  const int c = col0 + cl;
  const bool col_ok = c < dv;

  const T* qh = q + head * Tn * dk;
  const T* kh = k + head * Tn * dk;
  const T* vh = v + head * Tn * dv;
  T* yh = y + head * Tn * dv;
  const long sbase = head * static_cast<long>(dk) * dv;

  // R_0 = state_in (or zeros)
  for (int d = rg; d < dk; d += 8)
    Rs[d * kTileCols + cl] = (state_in != nullptr && col_ok) ? state_in[sbase + static_cast<long>(d) * dv + c] : 0.0f;

  for (int s0 = 0; s0 < Tn; s0 += C) {
    const int L = min(C, Tn - s0);
    __syncthreads();  // previous chunk done with Vs / P / Rs
    for (int e = tid; e < CT * kTileCols; e += kThreads) {
      const int j = e / kTileCols, cc = e % kTileCols;
      Vs[e] = (j < L && col0 + cc < dv) ? Elem<T>::load(vh, static_cast<long>(s0 + j) * dv + col0 + cc) : 0.0f;
    }
    for (int j = tid; j < CT; j += kThreads) zeta[j] = j < L ? gamma_pow(lg, L - 1 - j) : 0.0f;

    float sc[kScores];
#pragma unroll
    for (int r = 0; r < kScores; ++r) sc[r] = 0.0f;
    float xc[kRowsPerThread];
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) xc[r] = 0.0f;

    for (int d0 = 0; d0 < dk; d0 += kSub) {
      const int dn = min(kSub, dk - d0);
      __syncthreads();  // Qsub/Ksub free; Rs rows d0.. final for this chunk's reads
      for (int e = tid; e < CT * kSub; e += kThreads) {
        const int j = e / kSub, d = e % kSub;
        const bool ok = j < L && d < dn;
        Qsub[e] = ok ? Elem<T>::load(qh, static_cast<long>(s0 + j) * dk + d0 + d) : 0.0f;
        Ksub[e] = ok ? Elem<T>::load(kh, static_cast<long>(s0 + j) * dk + d0 + d) : 0.0f;
      }
      __syncthreads();
      // partial scores Q K^T over this sub-block
#pragma unroll
      for (int r = 0; r < kScores; ++r) {
        const int e = tid + r * kThreads;
        if (e < CT * CT) {
          const int i = e / CT, j = e % CT;
          float a = sc[r];
          for (int d = 0; d < kSub; ++d) a = fmaf(Qsub[i * kSub + d], Ksub[j * kSub + d], a);
          sc[r] = a;
        }
      }
      // cross-chunk term with the old state rows d0..d0+31
#pragma unroll
      for (int r = 0; r < kRowsPerThread; ++r) {
        const int i = rg + 8 * r;
        float a = xc[r];
        for (int d = 0; d < dn; ++d) a = fmaf(Qsub[i * kSub + d], Rs[(d0 + d) * kTileCols + cl], a);
        xc[r] = a;
      }
      __syncthreads();  // every thread has read the old rows d0..d0+31
      // state update of rows d0..d0+31: gamma^L R + sum_j K[j][d] zeta_j V[j][c]
      const float gL = gamma_pow(lg, L);
      for (int d = rg; d < dn; d += 8) {
        float a = 0.0f;
        for (int j = 0; j < L; ++j) a = fmaf(Ksub[j * kSub + d] * zeta[j], Vs[j * kTileCols + cl], a);
        float& rr = Rs[(d0 + d) * kTileCols + cl];
        rr = fmaf(gL, rr, a);
      }
    }

    // P = S .* D (causal, chunk-local)
#pragma unroll
    for (int r = 0; r < kScores; ++r) {
      const int e = tid + r * kThreads;
      if (e < CT * CT) {
        const int i = e / CT, j = e % CT;
        P[e] = (j <= i && i < L) ? sc[r] * gamma_pow(lg, i - j) : 0.0f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
      const int i = rg + 8 * r;
      if (i < L && col_ok) {
        float a = 0.0f;
        for (int j = 0; j <= i; ++j) a = fmaf(P[i * CT + j], Vs[j * kTileCols + cl], a);
        a = fmaf(gamma_pow(lg, i + 1), xc[r], a);
        Elem<T>::store(yh, static_cast<long>(s0 + i) * dv + c, a);
      }
    }
  }

  __syncthreads();
  if (state_out != nullptr && col_ok)
    for (int d = rg; d < dk; d += 8) state_out[sbase + static_cast<long>(d) * dv + c] = Rs[d * kTileCols + cl];
}

template <typename T, int CT>
hipError_t launch_ct(const void* q, const void* k, const void* v, const float* state_in, float* state_out, void* y,
                     int B, int H, int Tn, int dk, int dv, int C, const HeadDecay& hd, const HeadGroup& g,
                     hipStream_t s) {
  const size_t lds = sizeof(float) * (static_cast<size_t>(dk) * kTileCols + 2 * CT * kSub + CT * kTileCols +
                                      CT * CT + CT);
  auto kern = chunkwise_generic_kernel<T, CT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  dim3 grid((dv + kTileCols - 1) / kTileCols, B * g.nh);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), state_in, state_out, static_cast<T*>(y), hd, H, g.h0, g.nh, Tn, dk,
                     dv, C);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const void* q, const void* k, const void* v, const float* state_in, float* state_out, void* y,
                    int B, int H, int Tn, int dk, int dv, int C, const HeadDecay& hd, const HeadGroup& g,
                    hipStream_t s) {
  if (C <= 16) return launch_ct<T, 16>(q, k, v, state_in, state_out, y, B, H, Tn, dk, dv, C, hd, g, s);
  if (C <= 32) return launch_ct<T, 32>(q, k, v, state_in, state_out, y, B, H, Tn, dk, dv, C, hd, g, s);
  if (C <= 64) return launch_ct<T, 64>(q, k, v, state_in, state_out, y, B, H, Tn, dk, dv, C, hd, g, s);
  return launch_ct<T, 128>(q, k, v, state_in, state_out, y, B, H, Tn, dk, dv, C, hd, g, s);
}

}  // namespace

hipError_t launch_chunkwise_generic(const void* q, const void* k, const void* v, const float* state_in,
                                    float* state_out, void* y, int B, int H, int T, int dk, int dv, int C, int dt,
                                    const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  return dt == 0 ? launch_t<float>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, C, hd, g, s)
                 : launch_t<uint16_t>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, C, hd, g, s);
}

}  // namespace ret
