// Chunkwise retention of a short block of new tokens (T <= 16) from a carried
// state, in one streaming pass over that state.  This is the chunkwise form of
// "Retentive Networks — Microsoft Propone l'Alternativa Architetturale ai
// Transformer" (section "Il meccanismo: Multi-Scale Retention") with the whole
// block as one chunk of L = T tokens; for carried state R:
//   Y_t   = gamma^(t+1) Q_t R + sum_{u<=t} gamma^(t-u) (Q_t . K_u) V_u
//   R_out = gamma^T R + sum_u gamma^(T-1-u) K_u^T V_u
// For a few tokens the d_k x d_v fp32 state dominates the bytes, so the work is
// laid out like the recurrent step: it moves the state once in and once out.
//   - one workgroup per (batch, head) and up to 4 waves of 128 value columns;
//     lane l of wave w owns the 2 columns 128 w + 2 l, +1 of the workgroup's
//     range (1 column when d_v is odd, then 64 per wave);
//   - each wave walks all d_k state rows of its columns with a row group
//     prefetched ahead, non-temporal loads and stores (the state is streamed
//     once and is larger than the caches); per row it adds q_t[d] R[d,:] to the
//     T accumulators of Q_t R and forms the new row
//     gamma^T R[d,:] + sum_u (gamma^(T-1-u) k_u[d]) v_u;
//   - q and the decay-weighted k of the block sit in LDS feature-major
//     ([d][t]), so one row needs only broadcast LDS reads;
//   - the T x T intra-block scores gamma^(t-u) (q_t . k_u), u <= t, are formed
//     once per workgroup in LDS before the walk.
// All arithmetic is fp32 (bf16 inputs are widened), the state stays fp32.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ret {
namespace {

typedef float vf2 __attribute__((ext_vector_type(2)));

constexpr int kMaxDk = 256;

template <int VEC>
__device__ __forceinline__ void load_row(float (&s)[VEC], const float* p) {
  if constexpr (VEC == 2) {
    const vf2 x = __builtin_nontemporal_load(reinterpret_cast<const vf2*>(p));
    s[0] = x[0]; s[1] = x[1];
  } else {
    s[0] = __builtin_nontemporal_load(p);
  }
}

template <int VEC>
__device__ __forceinline__ void store_row(float* p, const float (&s)[VEC]) {
  if constexpr (VEC == 2) {
    __builtin_nontemporal_store(vf2{s[0], s[1]}, reinterpret_cast<vf2*>(p));
  } else {
    __builtin_nontemporal_store(s[0], p);
  }
}

// E: element type of q, k, v, y; NT: token capacity (T <= NT); VEC: columns per
// lane (2, or 1 for odd d_v); RG: state rows per prefetch group.
template <typename E, int NT, int VEC, int RG>
__global__ __launch_bounds__(256) void short_chunk_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                          const E* __restrict__ v, const float* state_in,
                                                          float* state_out, E* __restrict__ y, HeadDecay gam,
                                                          int H, int h0, int nh, int Tn, int dk, int dv) {
  __shared__ float qs[kMaxDk * NT];  // q_t[d] at [d * NT + t]
  __shared__ float ks[kMaxDk * NT];  // k_t[d], then gamma^(T-1-t) k_t[d], at [d * NT + t]
  __shared__ float A[NT * NT];       // gamma^(t-u) (q_t . k_u) at [t * NT + u] for u <= t < T, else 0

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = blockIdx.y % nh;
  const int b = blockIdx.y / nh;
  const long head = static_cast<long>(b) * H + h0 + hl;
  const float lg = gam.log2g[hl];
  const long qk0 = head * Tn * dk;  // token t, feature d at qk0 + t * dk + d
  const long v0 = head * Tn * dv;   // token t, column c at v0 + t * dv + c

  // q and k of the block, feature-major; tokens t >= T read as zero
  for (int i = tid; i < dk * NT; i += nthr) {
    const int t = i / dk, d = i - t * dk;  // consecutive threads read consecutive features
    const bool in = t < Tn;
    qs[d * NT + t] = in ? Elem<E>::load(q, qk0 + static_cast<long>(t) * dk + d) : 0.0f;
    ks[d * NT + t] = in ? Elem<E>::load(k, qk0 + static_cast<long>(t) * dk + d) : 0.0f;
  }
  __syncthreads();
  for (int i = tid; i < NT * NT; i += nthr) {
    const int t = i / NT, u = i - t * NT;
    float a = 0.0f;
    if (u <= t && t < Tn) {
      for (int d = 0; d < dk; ++d) a = fmaf(qs[d * NT + t], ks[d * NT + u], a);
      a *= gamma_pow(lg, t - u);
    }
    A[i] = a;
  }
  __syncthreads();
  for (int i = tid; i < dk * NT; i += nthr) {
    const int t = i % NT;
    ks[i] *= t < Tn ? gamma_pow(lg, Tn - 1 - t) : 0.0f;
  }
  __syncthreads();

  const int c0 = blockIdx.x * 64 * VEC * (nthr >> 6) + (w * 64 + lane) * VEC;
  if (c0 >= dv) return;  // no barrier follows
  float vv[NT][VEC];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < VEC; ++e) vv[t][e] = t < Tn ? Elem<E>::load(v, v0 + static_cast<long>(t) * dv + c0 + e) : 0.0f;
  float acc[NT][VEC];  // (Q_t R) at this lane's columns
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[t][e] = 0.0f;

  if (state_in != nullptr || state_out != nullptr) {
    const float gT = gamma_pow(lg, Tn);
    const long sb = head * static_cast<long>(dk) * dv + c0;
    const float* sin = state_in != nullptr ? state_in + sb : nullptr;
    float* sout = state_out != nullptr ? state_out + sb : nullptr;
    float cur[RG][VEC], nxt[RG][VEC];
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int e = 0; e < VEC; ++e) cur[g][e] = nxt[g][e] = 0.0f;
    if (sin != nullptr)
#pragma unroll
      for (int g = 0; g < RG; ++g)
        if (g < dk) load_row<VEC>(cur[g], sin + static_cast<long>(g) * dv);
    for (int r0 = 0; r0 < dk; r0 += RG) {
      // next row group in flight while this one is used (rows of other lanes'
      // columns are never touched, so in-place state_in == state_out is safe)
      if (sin != nullptr)
#pragma unroll
        for (int g = 0; g < RG; ++g)
          if (r0 + RG + g < dk) load_row<VEC>(nxt[g], sin + static_cast<long>(r0 + RG + g) * dv);
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const int r = r0 + g;
        if (r >= dk) break;
        float qr[NT], kr[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          qr[t] = qs[r * NT + t];
          kr[t] = ks[r * NT + t];
        }
        float nw[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          nw[e] = gT * cur[g][e];
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            acc[t][e] = fmaf(qr[t], cur[g][e], acc[t][e]);
            nw[e] = fmaf(kr[t], vv[t][e], nw[e]);
          }
        }
        if (sout != nullptr) store_row<VEC>(sout + static_cast<long>(r) * dv, nw);
      }
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int e = 0; e < VEC; ++e) cur[g][e] = nxt[g][e];
    }
  }

  // (a guard rather than an early exit keeps the token loop fully unrolled, so
  // acc and vv stay in registers)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < Tn) {
      const float xi = gamma_pow(lg, t + 1);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float o = xi * acc[t][e];
#pragma unroll
        for (int u = 0; u <= t; ++u) o = fmaf(A[t * NT + u], vv[u][e], o);
        Elem<E>::store(y, v0 + static_cast<long>(t) * dv + c0 + e, o);
      }
    }
  }
}

// Two columns per lane (a 512-byte row piece per wave) measured faster than
// four at every token count: at 16 tokens four columns need twice the
// accumulator registers, and at 1 to 8 tokens the extra waves hide more of the
// memory latency.  Rows per prefetch group: 8.
constexpr int kShortVec = 2;
constexpr int kShortRowGroup = 8;

template <typename E, int NT>
hipError_t launch_nt(const void* q, const void* k, const void* v, const float* state_in, float* state_out, void* y,
                     int B, int H, int T, int dk, int dv, const HeadDecay& hd, const HeadGroup& g, hipStream_t s) {
  constexpr int RG = kShortRowGroup;
  const E* qp = static_cast<const E*>(q);
  const E* kp = static_cast<const E*>(k);
  const E* vp = static_cast<const E*>(v);
  E* yp = static_cast<E*>(y);
  const auto go = [&](auto vec) {
    constexpr int VEC = decltype(vec)::value;
    const int wcols = 64 * VEC;                                 // columns per wave
    const int waves = std::min(4, (dv + wcols - 1) / wcols);    // per workgroup
    const dim3 grid((dv + wcols * waves - 1) / (wcols * waves), B * g.nh);
    hipLaunchKernelGGL((short_chunk_kernel<E, NT, VEC, RG>), grid, dim3(64 * waves), 0, s, qp, kp, vp, state_in,
                       state_out, yp, hd, H, g.h0, g.nh, T, dk, dv);
  };
  constexpr int V = kShortVec;
  if (dv % V == 0)
    go(std::integral_constant<int, V>{});
  else
    go(std::integral_constant<int, 1>{});
  return hipGetLastError();
}

template <typename E>
hipError_t launch_t(const void* q, const void* k, const void* v, const float* state_in, float* state_out, void* y,
                    int B, int H, int T, int dk, int dv, const HeadDecay& hd, const HeadGroup& g, hipStream_t s) {
  if (T == 1) return launch_nt<E, 1>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
  if (T <= 4) return launch_nt<E, 4>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
  if (T <= 8) return launch_nt<E, 8>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
  return launch_nt<E, kShortChunkMaxT>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
}

}  // namespace

hipError_t launch_short_chunk(const void* q, const void* k, const void* v, const float* state_in, float* state_out,
                              void* y, int B, int H, int T, int dk, int dv, int dt, const HeadGroup& g,
                              hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  return dt == 0 ? launch_t<float>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s)
                 : launch_t<uint16_t>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, hd, g, s);
}

}  // namespace ret
