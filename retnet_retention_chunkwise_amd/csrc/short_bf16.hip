// Chunkwise retention of a block of up to 64 new bf16 tokens from a carried
// fp32 state, one streaming pass over the state, products on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  The block is one chunk of
// L = T tokens of the chunkwise form ("Retentive Networks — Microsoft Propone
// l'Alternativa Architetturale ai Transformer", section "Il meccanismo:
// Multi-Scale Retention"); for carried state R:
//   Y_t   = gamma^(t+1) Q_t R + sum_{u<=t} gamma^(t-u) (Q_t . K_u) V_u
//   R_out = gamma^T R + sum_u gamma^(T-1-u) K_u^T V_u
// The fp32 state is nearly all of the bytes (2 x d_k x d_v x 4 per head) and
// moves once in and once out.  The operands of the products are bf16, as in
// the long-sequence bf16 kernel: q, k, v exactly, R, gamma^(T-1-u) k and the
// decayed scores rounded to nearest even; sums and the state stay fp32.  With
// 16x16x32 MFMAs the products of 64 tokens stay well under the memory time.
//
// Layout: a workgroup per (batch, head, up to 512 columns), one wave per 64
// columns, in 4 strips of 16: MFMA column n of strip st is column 4n + st, so
// a lane's 4 strips are 4 adjacent columns (16-byte state, 8-byte v and y
// accesses).  A wave walks d_k in steps of 32 rows, the next step's state
// prefetched; lane (g, l) holds R[d0 + 16b + 4g + i][4l + st] for the two
// 16-row blocks b of the step: the accumulator layout of the update's MFMAs,
// which write the new rows back where they were read (state_in may be
// state_out), and, with the k index of the cross term's MFMA taken in the
// order d0 + 16(e/4) + 4g + e%4, the B operand of (Q R) as well.
#include "common.h"
#include "gfx950.h"
#include "kernels.h"

namespace ret {
namespace {

constexpr int kMaxDkS = 256;

// NTB: 16-token blocks (T <= 16 NTB); NKS = ceil(NTB / 2) token steps of 32
template <int NTB>
__global__ __launch_bounds__(512) void short_bf16_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, const float* state_in,
                                                         float* state_out, uint16_t* __restrict__ y, HeadDecay gam,
                                                         int H, int h0, int nh, int Tn, int dk, int dv) {
  constexpr int NT = 16 * NTB;      // token capacity
  constexpr int NKS = (NTB + 1) / 2;
  constexpr int NU = 32 * NKS;      // token capacity rounded up to whole 32-token steps
  constexpr int QLD = kMaxDkS + 8;  // bf16 row stride of q and k (16-byte aligned rows)
  constexpr int TLD = NU + 8;       // bf16 row stride of gamma^(T-1-u) k^T and of the scores
  __shared__ __attribute__((aligned(16))) uint16_t qs[NU * QLD];
  __shared__ __attribute__((aligned(16))) uint16_t ks[NU * QLD];
  __shared__ __attribute__((aligned(16))) uint16_t kwT[kMaxDkS * TLD];  // [d][u]: gamma^(T-1-u) k_u[d]
  __shared__ __attribute__((aligned(16))) uint16_t Ps[NT * TLD];        // [t][u]: gamma^(t-u) (q_t . k_u), u <= t

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nw = nthr >> 6;
  const int g = lane >> 4;
  const int lr = lane & 15;
  const int hl = blockIdx.y % nh;
  const int b = blockIdx.y / nh;
  const long head = static_cast<long>(b) * H + h0 + hl;
  const float lg = gam.log2g[hl];
  const long qk0 = head * Tn * dk;
  const long v0 = head * Tn * dv;

  const int c0 = blockIdx.x * 512 + 64 * w;  // this wave's 64 columns
  const bool wact = c0 < dv;                 // waves past dv only help stage
  const int cl = c0 + 4 * lr;

  // v as B operands: step ks, strip st: tokens 32 ks + 8 g + e, column cl + st
  bf16x8 vb[NKS][4];
#pragma unroll
  for (int ksp = 0; ksp < NKS; ++ksp) {
    uint16_t vv[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = 32 * ksp + 8 * g + e;
      u32x2 x = {0u, 0u};
      if (wact && t < Tn) x = *reinterpret_cast<const u32x2*>(v + v0 + static_cast<long>(t) * dv + cl);
      vv[e][0] = static_cast<uint16_t>(x[0]);
      vv[e][1] = static_cast<uint16_t>(x[0] >> 16);
      vv[e][2] = static_cast<uint16_t>(x[1]);
      vv[e][3] = static_cast<uint16_t>(x[1] >> 16);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      s16x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = static_cast<short>(vv[e][st]);
      vb[ksp][st] = __builtin_bit_cast(bf16x8, p);
    }
  }

  const float gT = gamma_pow(lg, Tn);
  const long sb = head * static_cast<long>(dk) * dv + cl;
  // rows d0 + 16 bk + 4 g + i of a 32-row step; r[bk][i] holds the 4 strips
  auto load_step = [&](int d0, f32x4 (&r)[2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (state_in != nullptr)
          x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
              state_in + sb + static_cast<long>(d0 + 16 * bk + 4 * g + i) * dv));
        r[bk][i] = x;
      }
  };
  f32x4 cur[2][4], nxt[2][4];
  // the first state rows are requested before the staging of q and k, so
  // that they arrive while the workgroup prepares its operands
  if (wact) load_step(0, cur);

  // q and k rows (zero past T), 16 bytes per thread and step
  for (int i = tid; i < NU * (dk / 8); i += nthr) {
    const int t = i / (dk / 8), d8 = i - t * (dk / 8);
    u32x4 qv = {0u, 0u, 0u, 0u}, kv = {0u, 0u, 0u, 0u};
    if (t < Tn) {
      qv = *reinterpret_cast<const u32x4*>(q + qk0 + static_cast<long>(t) * dk + 8 * d8);
      kv = *reinterpret_cast<const u32x4*>(k + qk0 + static_cast<long>(t) * dk + 8 * d8);
    }
    *reinterpret_cast<u32x4*>(&qs[t * QLD + 8 * d8]) = qv;
    *reinterpret_cast<u32x4*>(&ks[t * QLD + 8 * d8]) = kv;
  }
  __syncthreads();
  // gamma^(T-1-u) k_u, transposed (the update's A operand is 8 tokens of one row)
  for (int i = tid; i < dk * NU; i += nthr) {
    const int d = i / NU, u = i - d * NU;
    const float z = u < Tn ? gamma_pow(lg, Tn - 1 - u) : 0.0f;
    kwT[d * TLD + u] = f32_to_bf16(bf16_to_f32(ks[u * QLD + d]) * z);
  }
  // decayed scores: 16x16 blocks (tb, ub), ub <= tb, over d_k in steps of 32;
  // blocks past the diagonal and past NT stay zero
  for (int blk = w; blk < NTB * NKS * 2; blk += nw) {
    const int tb = blk / (2 * NKS), ub = blk - tb * (2 * NKS);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if (ub <= tb) {
      for (int d0 = 0; d0 < dk; d0 += 32) {
        const bf16x8 a = lds_read16(&qs[(16 * tb + lr) * QLD + d0 + 8 * g]);
        const bf16x8 bb = lds_read16(&ks[(16 * ub + lr) * QLD + d0 + 8 * g]);
        s = mfma(a, bb, s);
      }
    }
    // s[i] = S[16 tb + 4 g + i][16 ub + lr]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i, u = 16 * ub + lr;
      const float f = u <= t && t < Tn ? gamma_pow(lg, t - u) : 0.0f;
      Ps[t * TLD + u] = f32_to_bf16(s[i] * f);
    }
  }
  __syncthreads();

  if (!wact) return;  // no barrier follows
  f32x4 acc[NTB][4];  // (Q R)[16 tb + 4 g + i][cl + st]
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int st = 0; st < 4; ++st) acc[tb][st] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (state_in != nullptr || state_out != nullptr) {
    for (int d0 = 0; d0 < dk; d0 += 32) {
      if (d0 + 32 < dk) load_step(d0 + 32, nxt);
      // (Q R): k slot e <-> row d0 + 16 (e/4) + 4 g + e%4
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        f32x8 rf;
#pragma unroll
        for (int e = 0; e < 8; ++e) rf[e] = cur[e >> 2][e & 3][st];
        const bf16x8 rb = __builtin_convertvector(rf, bf16x8);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          const s16x4 lo = *reinterpret_cast<const s16x4*>(&qs[(16 * tb + lr) * QLD + d0 + 4 * g]);
          const s16x4 hi = *reinterpret_cast<const s16x4*>(&qs[(16 * tb + lr) * QLD + d0 + 16 + 4 * g]);
          acc[tb][st] = mfma(join(lo, hi), rb, acc[tb][st]);
        }
      }
      if (state_out != nullptr) {
        // new rows gamma^T R + (gamma^(T-1-u) K)^T V: A operand tokens 32 ks + 8 g .. +7 of row d0 + 16 bk + lr
#pragma unroll
        for (int bk = 0; bk < 2; ++bk) {
          bf16x8 ka[NKS];
#pragma unroll
          for (int ksp = 0; ksp < NKS; ++ksp) ka[ksp] = lds_read16(&kwT[(d0 + 16 * bk + lr) * TLD + 32 * ksp + 8 * g]);
          f32x4 rn[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int i = 0; i < 4; ++i) rn[st][i] = cur[bk][i][st] * gT;
#pragma unroll
            for (int ksp = 0; ksp < NKS; ++ksp) rn[st] = mfma(ka[ksp], vb[ksp][st], rn[st]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __builtin_nontemporal_store(f32x4{rn[0][i], rn[1][i], rn[2][i], rn[3][i]},
                                        reinterpret_cast<f32x4*>(state_out + sb +
                                                                 static_cast<long>(d0 + 16 * bk + 4 * g + i) * dv));
        }
      }
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[bk][i] = nxt[bk][i];
    }
  }

  // Y_t = gamma^(t+1) (Q R)_t + sum_u P[t][u] V_u
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    f32x4 o[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[st][i] = acc[tb][st][i] * gamma_pow(lg, 16 * tb + 4 * g + i + 1);
#pragma unroll
      for (int ksp = 0; ksp < NKS; ++ksp) {
        const bf16x8 pa = lds_read16(&Ps[(16 * tb + lr) * TLD + 32 * ksp + 8 * g]);
        o[st] = mfma(pa, vb[ksp][st], o[st]);
      }
    }
    // o[st][i] = Y[16 tb + 4 g + i][cl + st]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * tb + 4 * g + i;
      if (t < Tn) {
        const bf16x4 ob = __builtin_convertvector(f32x4{o[0][i], o[1][i], o[2][i], o[3][i]}, bf16x4);
        *reinterpret_cast<u32x2*>(y + v0 + static_cast<long>(t) * dv + cl) = __builtin_bit_cast(u32x2, ob);
      }
    }
  }
}

template <int NTB>
hipError_t launch_ntb(const void* q, const void* k, const void* v, const float* state_in, float* state_out, void* y,
                      int B, int H, int T, int dk, int dv, const HeadDecay& hd, const HeadGroup& g, hipStream_t s) {
  const int waves = dv >= 512 ? 8 : dv / 64;
  const dim3 grid((dv + 511) / 512, B * g.nh);
  hipLaunchKernelGGL((short_bf16_kernel<NTB>), grid, dim3(64 * waves), 0, s, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), state_in, state_out,
                     static_cast<uint16_t*>(y), hd, H, g.h0, g.nh, T, dk, dv);
  return hipGetLastError();
}

}  // namespace

bool short_bf16_supports(int T, int dk, int dv, int dt) {
  return dt == 1 && T >= 1 && T <= kShortBf16MaxT && dk % 32 == 0 && dk <= kMaxDkS && dv % 64 == 0;
}

hipError_t launch_short_bf16(const void* q, const void* k, const void* v, const float* state_in, float* state_out,
                             void* y, int B, int H, int T, int dk, int dv, const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  if (T <= 16) return launch_ntb<1>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
  if (T <= 32) return launch_ntb<2>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
  if (T <= 48) return launch_ntb<3>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
  return launch_ntb<4>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
}

}  // namespace ret
