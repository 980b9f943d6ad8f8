// Backward of chunkwise retention: gradients of retention_chunkwise_fwd.
//
// The aimpact page ("Retentive Networks — Microsoft Propone l'Alternativa
// Architetturale ai Transformer", section "Il meccanismo: Multi-Scale
// Retention") gives the recurrence S_n = gamma S_(n-1) + K_n^T V_n,
// Y_n = Q_n S_n and says the parallel/chunkwise forms are what training runs;
// it gives no backward pass.  By the chain rule, with G_n = dL/dS_n
// (G_n = Q_n^T dY_n + gamma G_(n+1), G_(T-1) also receiving dS_out):
//   dQ_n = dY_n S_n^T,   dK_n = G_n V_n^T (as a d_k row),   dV_n = K_n G_n,
//   dS_in = gamma G_0.
// Unrolled over chunks, each of the three is one more chunkwise pass of the
// same shape as the forward, with a d_a x (tile of d_x) fp32 state S:
//   forward in time (dQ):    Out_j = gamma^(j+1) A_j S + sum_{j'<=j} gamma^(j-j') (A_j . B_j') X_j'
//                            S <- gamma^L S + sum_j gamma^(L-1-j) B_j^T X_j
//   reverse in time (dK, dV): chunks from last to first,
//                            Out_j = gamma^(L-1-j) A_j S + sum_{j'>=j} gamma^(j'-j) (A_j . B_j') X_j'
//                            S <- gamma^L S + sum_j gamma^(j+1) B_j^T X_j
// with (A, B, X, S_0):
//   dQ: (dY, V, K, S_in^T)   -- S is R^T, d_v x d_k
//   dK: (V, dY, Q, dS_out^T) -- S is G^T (scaled), d_v x d_k
//   dV: (K, Q, dY, dS_out)   -- S is G (scaled), d_k x d_v; its final value is dS_in.
// (The reverse pass's S after chunk i is gamma G at the chunk's first token,
// i.e. the gradient reaching the previous chunk's last state.)
//
// This file holds the generic pass kernel: fp32 arithmetic (bf16 inputs are
// widened), any shape up to d_a = 512, one workgroup per (batch, head, 32 X
// columns), the fp32 state tile in LDS for the whole sequence and 16-token
// chunks (the gradients do not depend on the chunk length beyond rounding).
#include "common.h"
#include "kernels.h"

namespace ret {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 32;     // X / Out columns per workgroup (= state columns)
constexpr int kCT = 16;       // tokens per chunk
constexpr int kMaxDA = 512;   // contraction dim of A . B and A S
constexpr int kALd = kMaxDA + 1;

struct PassArgs {
  const void* a;       // [BH, T, DA]
  const void* b;       // [BH, T, DA]
  const void* x;       // [BH, T, DX]
  void* out;           // [BH, T, DX]
  const float* s0;     // nullable; [BH, DA, DX] (s0_t = 0) or [BH, DX, DA] (s0_t = 1)
  float* s_out;        // nullable; [BH, DA, DX]
  int s0_t;
  int da, dx;
};

template <typename E, bool REV>
__global__ __launch_bounds__(kThreads) void bwd_pass_generic_kernel(PassArgs p, HeadDecay gam, int H, int h0, int nh,
                                                                    int Tn) {
  __shared__ float S[kMaxDA * kCols];   // state tile [a][c]
  __shared__ float As[kCT * kALd];      // A rows of the chunk
  __shared__ float Bs[kCT * kALd];      // B rows of the chunk
  __shared__ float Pm[kCT * kCT];       // masked, decayed scores A_j . B_j'
  __shared__ float Xc[kCT * kCols];     // X tile of the chunk
  __shared__ float wz[2 * kCT];         // weight of A_j S (w) and of B_j^T X_j (z)

  const int tid = threadIdx.x;
  const int DA = p.da, DX = p.dx;
  const int hl = blockIdx.y % nh;
  const int bb = blockIdx.y / nh;
  const long head = static_cast<long>(bb) * H + h0 + hl;
  const float lg = gam.log2g[hl];
  const int c0 = blockIdx.x * kCols;
  const int cl = tid % kCols;
  const int rg = tid / kCols;  // 0..7
  const bool col_ok = c0 + cl < DX;
  const E* A = static_cast<const E*>(p.a) + head * Tn * DA;
  const E* Bm = static_cast<const E*>(p.b) + head * Tn * DA;
  const E* X = static_cast<const E*>(p.x) + head * Tn * DX;
  E* O = static_cast<E*>(p.out) + head * Tn * DX;
  const long sb = head * static_cast<long>(DA) * DX;

  for (int a = rg; a < DA; a += 8) {
    float s = 0.0f;
    if (p.s0 != nullptr && col_ok)
      s = p.s0_t ? p.s0[sb + static_cast<long>(c0 + cl) * DA + a] : p.s0[sb + static_cast<long>(a) * DX + c0 + cl];
    S[a * kCols + cl] = s;
  }

  const int nch = (Tn + kCT - 1) / kCT;
  for (int it = 0; it < nch; ++it) {
    const int ci = REV ? nch - 1 - it : it;
    const int t0 = ci * kCT;
    const int L = min(kCT, Tn - t0);
    __syncthreads();  // previous chunk done with As/Bs/Xc/Pm and S
    for (int e = tid; e < kCT * DA; e += kThreads) {
      const int j = e / DA, a = e - j * DA;
      const bool in = j < L;
      As[j * kALd + a] = in ? Elem<E>::load(A, static_cast<long>(t0 + j) * DA + a) : 0.0f;
      Bs[j * kALd + a] = in ? Elem<E>::load(Bm, static_cast<long>(t0 + j) * DA + a) : 0.0f;
    }
    for (int e = tid; e < kCT * kCols; e += kThreads) {
      const int j = e / kCols, c = e % kCols;
      Xc[e] = (j < L && c0 + c < DX) ? Elem<E>::load(X, static_cast<long>(t0 + j) * DX + c0 + c) : 0.0f;
    }
    if (tid < kCT) {
      const int j = tid;
      const float fwd = gamma_pow(lg, j + 1), bwd = gamma_pow(lg, L - 1 - j);
      wz[j] = j < L ? (REV ? bwd : fwd) : 0.0f;
      wz[kCT + j] = j < L ? (REV ? fwd : bwd) : 0.0f;
    }
    __syncthreads();
    {  // scores: one (j, j') per thread
      const int j = tid / kCT, jp = tid % kCT;
      const bool keep = j < L && jp < L && (REV ? jp >= j : jp <= j);
      float sc = 0.0f;
      if (keep) {
        for (int a = 0; a < DA; ++a) sc = fmaf(As[j * kALd + a], Bs[jp * kALd + a], sc);
        sc *= gamma_pow(lg, REV ? jp - j : j - jp);
      }
      Pm[j * kCT + jp] = sc;
    }
    __syncthreads();
    // Out rows rg and rg + 8 of this column
#pragma unroll
    for (int r = 0; r < kCT / 8; ++r) {
      const int j = rg + 8 * r;
      if (j < L && col_ok) {
        float cross = 0.0f;
        for (int a = 0; a < DA; ++a) cross = fmaf(As[j * kALd + a], S[a * kCols + cl], cross);
        float o = wz[j] * cross;
#pragma unroll
        for (int jp = 0; jp < kCT; ++jp) o = fmaf(Pm[j * kCT + jp], Xc[jp * kCols + cl], o);
        Elem<E>::store(O, static_cast<long>(t0 + j) * DX + c0 + cl, o);
      }
    }
    __syncthreads();  // every read of S for this chunk is done
    const float gL = gamma_pow(lg, L);
    for (int a = rg; a < DA; a += 8) {
      float s = gL * S[a * kCols + cl];
#pragma unroll
      for (int j = 0; j < kCT; ++j) s = fmaf(Bs[j * kALd + a] * wz[kCT + j], Xc[j * kCols + cl], s);
      S[a * kCols + cl] = s;
    }
  }
  if (p.s_out != nullptr && col_ok) {
    // each thread writes only the entries it updated itself (no barrier needed)
    for (int a = rg; a < DA; a += 8) p.s_out[sb + static_cast<long>(a) * DX + c0 + cl] = S[a * kCols + cl];
  }
}

template <typename E>
hipError_t launch_pass(const PassArgs& p, bool rev, int B, int H, int T, const HeadDecay& hd, const HeadGroup& g,
                       hipStream_t s) {
  const dim3 grid((p.dx + kCols - 1) / kCols, B * g.nh);
  if (rev)
    hipLaunchKernelGGL((bwd_pass_generic_kernel<E, true>), grid, dim3(kThreads), 0, s, p, hd, H, g.h0, g.nh, T);
  else
    hipLaunchKernelGGL((bwd_pass_generic_kernel<E, false>), grid, dim3(kThreads), 0, s, p, hd, H, g.h0, g.nh, T);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_all(const BwdArgs& a, int B, int H, int T, int dk, int dv, const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  // dK: reverse pass over (V, dY, Q) from dS_out^T
  PassArgs pk{a.v, a.dy, a.q, a.dk, a.dstate_out, nullptr, 1, dv, dk};
  hipError_t e = launch_pass<E>(pk, true, B, H, T, hd, g, s);
  if (e != hipSuccess) return e;
  // dQ: forward pass over (dY, V, K) from S_in^T
  PassArgs pq{a.dy, a.v, a.k, a.dq, a.state_in, nullptr, 1, dv, dk};
  e = launch_pass<E>(pq, false, B, H, T, hd, g, s);
  if (e != hipSuccess) return e;
  // dV: reverse pass over (K, Q, dY) from dS_out; final state = dS_in.  Last,
  // so that dstate_in may be the dstate_out buffer (the dK pass reads it first).
  PassArgs pv{a.k, a.q, a.dy, a.dv, a.dstate_out, a.dstate_in, 0, dk, dv};
  return launch_pass<E>(pv, true, B, H, T, hd, g, s);
}

}  // namespace

bool chunkwise_bwd_generic_supports(int dk, int dv) { return dk <= kMaxDA && dv <= kMaxDA; }

hipError_t launch_chunkwise_bwd_generic(const BwdArgs& a, int B, int H, int T, int dk, int dv, int dt,
                                        const HeadGroup& g, hipStream_t s) {
  return dt == 0 ? launch_all<float>(a, B, H, T, dk, dv, g, s) : launch_all<uint16_t>(a, B, H, T, dk, dv, g, s);
}

}  // namespace ret
