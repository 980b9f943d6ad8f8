// Chunkwise retention of a block of up to 32 new tokens from a carried state,
// one streaming pass over the state, products on fp32 MFMA
// (v_mfma_f32_16x16x4_f32).  The block is one chunk of L = T tokens of the
// chunkwise form ("Retentive Networks — Microsoft Propone l'Alternativa
// Architetturale ai Transformer", section "Il meccanismo: Multi-Scale
// Retention"); for carried state R:
//   Y_t   = gamma^(t+1) Q_t R + sum_{u<=t} gamma^(t-u) (Q_t . K_u) V_u
//   R_out = gamma^T R + sum_u gamma^(T-1-u) K_u^T V_u
// The fp32 state dominates the bytes (2 x d_k x d_v x 4 per head) and is moved
// once in and once out; with fp32 MFMA the 2T products per state element stay
// under the memory time up to 32 tokens (the VALU streaming kernel becomes
// compute-bound past ~8).
//
// Layout: a workgroup per (batch, head, up to 512 columns), one wave per 64
// columns (4 strips of 16).  q, the decay-weighted k and the T x T intra
// scores of the block sit in LDS in fp32; each lane keeps its v entries in
// registers.  Column n of strip st of a wave is column 4n + st of its 64, so a
// lane's four strips are 4 adjacent columns (16-byte state, v and y accesses,
// 256 contiguous bytes per row and wave).  A wave walks the d_k rows in 16-row
// blocks (the next block's state prefetched): lane (g, l) holds
// R[d0 + 4g + i][4l + strip], the MFMA accumulator layout, so
//   * (Q R)_t accumulates with MFMA i taking R element i as its B operand (k
//     index g = row 4g + i) and one 16-byte LDS read of q_t giving the A
//     operands of all four, and
//   * the new rows gamma^T R + K_w^T V come out of MFMAs in that same layout
//     and are stored where they were read (so state_in may be state_out).
// Finally Y_t = gamma^(t+1) (Q R)_t + (scores V)_t, the intra term as MFMAs
// with the v registers as B operands.  bf16 inputs are widened; all products
// and sums are fp32.
#include "common.h"
#include "gfx950.h"
#include "kernels.h"

namespace ret {
namespace {

constexpr int kMaxDk = 256;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// E: element type of q, k, v, y; NTB: 16-token blocks (T <= 16 NTB)
template <typename E, int NTB>
__global__ __launch_bounds__(512) void short_mfma_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                         const E* __restrict__ v, const float* state_in,
                                                         float* state_out, E* __restrict__ y, HeadDecay gam, int H,
                                                         int h0, int nh, int Tn, int dk, int dv) {
  constexpr int NT = 16 * NTB;
  constexpr int QLD = kMaxDk + 4;  // fp32 row stride of q and k_w (16-byte row reads)
  constexpr int ALD = NT + 4;      // of the scores
  __shared__ __attribute__((aligned(16))) float qs[NT * QLD];
  __shared__ __attribute__((aligned(16))) float kw[NT * QLD];  // k, then gamma^(T-1-t) k
  __shared__ __attribute__((aligned(16))) float As[NT * ALD];  // gamma^(t-u) (q_t . k_u), u <= t < T

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int lr = lane & 15;
  const int hl = blockIdx.y % nh;
  const int b = blockIdx.y / nh;
  const long head = static_cast<long>(b) * H + h0 + hl;
  const float lg = gam.log2g[hl];
  const long qk0 = head * Tn * dk;
  const long v0 = head * Tn * dv;

  for (int i = tid; i < NT * dk; i += nthr) {
    const int t = i / dk, d = i - t * dk;
    const bool in = t < Tn;
    qs[t * QLD + d] = in ? Elem<E>::load(q, qk0 + static_cast<long>(t) * dk + d) : 0.0f;
    kw[t * QLD + d] = in ? Elem<E>::load(k, qk0 + static_cast<long>(t) * dk + d) : 0.0f;
  }
  __syncthreads();
  for (int i = tid; i < NT * NT; i += nthr) {
    const int t = i / NT, u = i - t * NT;
    float a = 0.0f;
    if (u <= t && t < Tn) {
      for (int d = 0; d < dk; ++d) a = fmaf(qs[t * QLD + d], kw[u * QLD + d], a);
      a *= gamma_pow(lg, t - u);
    }
    As[t * ALD + u] = a;
  }
  __syncthreads();
  for (int i = tid; i < NT * dk; i += nthr) {
    const int t = i / dk, d = i - t * dk;
    kw[t * QLD + d] *= t < Tn ? gamma_pow(lg, Tn - 1 - t) : 0.0f;
  }
  __syncthreads();

  const int c0 = blockIdx.x * 512 + 64 * w;  // this wave's 64 columns
  if (c0 >= dv) return;                      // no barrier follows

  // v entries: B operands (k index g of step s = token 4s + g) of strip st,
  // column c0 + 4 lr + st
  const int cl = c0 + 4 * lr;
  float vr[4 * NTB][4];
#pragma unroll
  for (int s = 0; s < 4 * NTB; ++s)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int t = 4 * s + g;
      vr[s][st] = t < Tn ? Elem<E>::load(v, v0 + static_cast<long>(t) * dv + cl + st) : 0.0f;
    }
  f32x4 acc[NTB][4];  // (Q R)[16 tb + 4g + i][c0 + 4 lr + st]
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int st = 0; st < 4; ++st) acc[tb][st] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  if (state_in != nullptr || state_out != nullptr) {
    const float gT = gamma_pow(lg, Tn);
    const long sb = head * static_cast<long>(dk) * dv + cl;
    auto load_blk = [&](int d0, f32x4 (&r)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
        if (state_in != nullptr)
          x = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4*>(state_in + sb + static_cast<long>(d0 + 4 * g + i) * dv));
#pragma unroll
        for (int st = 0; st < 4; ++st) r[st][i] = x[st];
      }
    };
    f32x4 cur[4], nxt[4];
    load_blk(0, cur);
    for (int d0 = 0; d0 < dk; d0 += 16) {
      if (d0 + 16 < dk) load_blk(d0 + 16, nxt);
      // (Q R): A operand q_t[d0 + 4g + i] (row t = 16 tb + lr), B operand R element i
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const f32x4 qa = *reinterpret_cast<const f32x4*>(&qs[(16 * tb + lr) * QLD + d0 + 4 * g]);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tb][st] = mfma4(qa[i], cur[st][i], acc[tb][st]);
      }
      if (state_out != nullptr) {
        // new rows: gamma^T R + K_w^T V, A operand k_w[t = 4s + g][d0 + lr]
        float ka[4 * NTB];
#pragma unroll
        for (int s = 0; s < 4 * NTB; ++s) ka[s] = kw[(4 * s + g) * QLD + d0 + lr];
        f32x4 r[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          r[st] = cur[st] * gT;
#pragma unroll
          for (int s = 0; s < 4 * NTB; ++s) r[st] = mfma4(ka[s], vr[s][st], r[st]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_nontemporal_store(f32x4{r[0][i], r[1][i], r[2][i], r[3][i]},
                                      reinterpret_cast<f32x4*>(state_out + sb + static_cast<long>(d0 + 4 * g + i) * dv));
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) cur[st] = nxt[st];
    }
  }

  // Y_t = gamma^(t+1) (Q R)_t + sum_u scores[t][u] V_u
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    float xi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xi[i] = gamma_pow(lg, 16 * tb + 4 * g + i + 1);
    float sa[4 * NTB];
#pragma unroll
    for (int s = 0; s < 4 * NTB; ++s) sa[s] = As[(16 * tb + lr) * ALD + 4 * s + g];
    f32x4 o[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      o[st] = acc[tb][st];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[st][i] *= xi[i];
#pragma unroll
      for (int s = 0; s < 4 * NTB; ++s) o[st] = mfma4(sa[s], vr[s][st], o[st]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i;
      if (t < Tn)
#pragma unroll
        for (int st = 0; st < 4; ++st) Elem<E>::store(y, v0 + static_cast<long>(t) * dv + cl + st, o[st][i]);
    }
  }
}

template <typename E, int NTB>
hipError_t launch_ntb(const void* q, const void* k, const void* v, const float* state_in, float* state_out, void* y,
                      int B, int H, int T, int dk, int dv, const HeadDecay& hd, const HeadGroup& g, hipStream_t s) {
  const int waves = dv >= 512 ? 8 : dv / 64;
  const dim3 grid((dv + 511) / 512, B * g.nh);
  hipLaunchKernelGGL((short_mfma_kernel<E, NTB>), grid, dim3(64 * waves), 0, s, static_cast<const E*>(q),
                     static_cast<const E*>(k), static_cast<const E*>(v), state_in, state_out, static_cast<E*>(y), hd, H,
                     g.h0, g.nh, T, dk, dv);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const void* q, const void* k, const void* v, const float* state_in, float* state_out, void* y,
                    int B, int H, int T, int dk, int dv, const HeadDecay& hd, const HeadGroup& g, hipStream_t s) {
  if (T <= 16) return launch_ntb<E, 1>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
  return launch_ntb<E, 2>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
}

}  // namespace

bool short_mfma_supports(int T, int dk, int dv) {
  return T >= 1 && T <= kShortMfmaMaxT && dk % 16 == 0 && dk <= kMaxDk && dv % 64 == 0;
}

hipError_t launch_short_mfma(const void* q, const void* k, const void* v, const float* state_in, float* state_out,
                             void* y, int B, int H, int T, int dk, int dv, int dt, const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  return dt == 0 ? launch_e<float>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s)
                 : launch_e<uint16_t>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
}

}  // namespace ret
