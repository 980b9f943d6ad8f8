// Chunkwise retention on bf16 MFMA (gfx950, v_mfma_f32_16x16x32_bf16), fp32 state.
//
// Chunkwise form of "Retentive Networks — Microsoft Propone l'Alternativa
// Architetturale ai Transformer" (section "Il meccanismo: Multi-Scale
// Retention"): parallel inside chunks of C tokens, recurrent across chunks.
// For chunk i (rows j = 0..L-1, carried state R_i, decay gamma of the head):
//   Y_[i]   = ((Q_[i] K_[i]^T) .* D_L) V_[i] + diag(gamma^(j+1)) Q_[i] R_i
//   R_(i+1) = gamma^L R_i + K_[i]^T (diag(gamma^(L-1-j)) V_[i])
//
// Work decomposition (one workgroup = 4 waves = 256 threads):
//   * a workgroup owns one (batch, head, tile of 64 value columns) and walks the
//     chunks of the sequence in order; the 8 column tiles of a head are mapped
//     to one XCD so that their shared Q/K reads hit the same L2;
//   * the fp32 state tile R[d_k x 64] lives in MFMA accumulators for the whole
//     sequence: wave w owns rows [w*d_k/4, (w+1)*d_k/4);
//   * per chunk, wave w owns query blocks of 16 rows ({w, 7-w} for 128-token
//     chunks, which balances the causal triangle; {w} for 64-token chunks).
//     Its Q rows are loaded from global memory straight into MFMA operand
//     registers and serve both S^T = K Q^T and the cross term Q R;
//   * S^T stays in registers: its accumulator layout is, up to a permutation of
//     the key index, the A-operand layout that P = S .* D needs for P V, so the
//     decay mask is applied in registers and P never touches LDS;
//   * K and the 64-column V tile are staged in LDS (row-major); the state
//     update contracts over tokens and reads K^T and (gamma^(L-1-j) V) with
//     ds_read_b64_tr_b16, the gfx950 transposing LDS load;
//   * R^T is kept in LDS as bf16 for the cross term's B operand and rewritten
//     after every update;
//   * the next chunk's K/V (and Q) are loaded into registers while the current
//     chunk computes; three barriers per chunk separate the phases.
// Decay factors gamma^d are generated in registers from log2(gamma) (exp2),
// with gamma^0 forced to 1.
#include "common.h"
#include "kernels.h"

namespace ret {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kThreads = 256;
constexpr int kTN = 64;  // value columns per workgroup

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

template <int CT, int DK>
struct Cfg {
  static constexpr int KLD = DK + 8;           // K row stride in LDS (elements)
  static constexpr int VLD = kTN + 8;          // V / zeta*V row stride
  static constexpr int RLD = DK + 8;           // R^T row stride
  static constexpr int NQ = CT / 64;           // query blocks per wave
  static constexpr int RM = DK / 64;           // 16-row state blocks per wave
  static constexpr int KS = DK / 32;           // k-steps over d_k
  static constexpr int KPT = CT * DK / 8 / kThreads;   // 16-byte K pieces per thread
  static constexpr int VPT = CT * kTN / 8 / kThreads;  // 16-byte V pieces per thread
  static_assert(KPT >= 1 && VPT >= 1, "tile too small for the staging split");
};

template <int CT, int DK>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1))) void
chunkwise_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, const float* state_in, float* state_out,
                      uint16_t* __restrict__ y, HeadDecay gam, int H, int h0, int nh, int Tn, int dv, int C,
                      int ntiles) {
  using F = Cfg<CT, DK>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[CT * F::KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[CT * F::VLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vz[CT * F::VLD];
  __shared__ __attribute__((aligned(16))) uint16_t Rt[kTN * F::RLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c16 = lane & 15;
  const int g = lane >> 4;

  // Workgroup -> (batch, head, column tile).  Consecutive linear ids (the
  // column tiles of one head) are placed on one XCD (dispatch is round-robin
  // over the 8 XCDs by workgroup id).
  const int total = gridDim.x;
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int tile = lin % ntiles;
  const int bh = lin / ntiles;
  const int hl = bh % nh;
  const int b = bh / nh;
  const long head = static_cast<long>(b) * H + h0 + hl;
  const int col0 = tile * kTN;
  const float lg = gam.log2g[hl];

  const uint16_t* qh = q + head * Tn * DK;
  const uint16_t* kh = k + head * Tn * DK;
  const uint16_t* vh = v + head * Tn * dv + col0;
  uint16_t* yh = y + head * Tn * dv + col0;
  const long sbase = head * static_cast<long>(DK) * dv + col0;

  int qblk[F::NQ];
  if constexpr (F::NQ == 2) {
    qblk[0] = w;
    qblk[1] = 7 - w;
  } else {
    qblk[0] = w;
  }
  const int dbase = w * (DK / 4);

  // ---- carried state: R_0 = state_in (or zeros), kept as fp32 accumulators
  f32x4 Racc[F::RM][4];
#pragma unroll
  for (int mb = 0; mb < F::RM; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = dbase + 16 * mb + 4 * g + i;
        Racc[mb][nb][i] = state_in != nullptr ? state_in[sbase + static_cast<long>(d) * dv + 16 * nb + c16] : 0.0f;
      }

  auto write_rt = [&]() {
#pragma unroll
    for (int mb = 0; mb < F::RM; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x4 r = __builtin_convertvector(Racc[mb][nb], bf16x4);
        *reinterpret_cast<bf16x4*>(&Rt[(16 * nb + c16) * F::RLD + dbase + 16 * mb + 4 * g]) = r;
      }
  };

  uint4 kreg[F::KPT];
  uint4 vreg[F::VPT];
  bf16x8 Qreg[F::NQ][F::KS];

  auto load_kv = [&](int s1, int Ln) {
#pragma unroll
    for (int r = 0; r < F::KPT; ++r) {
      const int p = tid + kThreads * r;
      const int row = p / (DK / 8), c8 = p % (DK / 8);
      kreg[r] = row < Ln ? *reinterpret_cast<const uint4*>(kh + static_cast<long>(s1 + row) * DK + 8 * c8)
                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < F::VPT; ++r) {
      const int p = tid + kThreads * r;
      const int row = p / (kTN / 8), c8 = p % (kTN / 8);
      vreg[r] = row < Ln ? *reinterpret_cast<const uint4*>(vh + static_cast<long>(s1 + row) * dv + 8 * c8)
                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_kv = [&](int Ln) {
#pragma unroll
    for (int r = 0; r < F::KPT; ++r) {
      const int p = tid + kThreads * r;
      const int row = p / (DK / 8), c8 = p % (DK / 8);
      *reinterpret_cast<uint4*>(&Ks[row * F::KLD + 8 * c8]) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < F::VPT; ++r) {
      const int p = tid + kThreads * r;
      const int row = p / (kTN / 8), c8 = p % (kTN / 8);
      *reinterpret_cast<uint4*>(&Vs[row * F::VLD + 8 * c8]) = vreg[r];
      // zeta_row = gamma^(L-1-row) scales V for the state update (0 past the chunk end)
      const float z = row < Ln ? gamma_pow(lg, Ln - 1 - row) : 0.0f;
      const bf16x8 vb = __builtin_bit_cast(bf16x8, vreg[r]);
      const f32x8 vf = __builtin_convertvector(vb, f32x8) * z;
      *reinterpret_cast<bf16x8*>(&Vz[row * F::VLD + 8 * c8]) = __builtin_convertvector(vf, bf16x8);
    }
  };
  auto load_q = [&](int s1, int Ln) {
#pragma unroll
    for (int qi = 0; qi < F::NQ; ++qi) {
      const int row = 16 * qblk[qi] + c16;
#pragma unroll
      for (int s = 0; s < F::KS; ++s) {
        Qreg[qi][s] = row < Ln ? *reinterpret_cast<const bf16x8*>(qh + static_cast<long>(s1 + row) * DK + 32 * s + 8 * g)
                               : bf16x8{};
      }
    }
  };

  // ---- prologue: chunk 0 into LDS and registers
  {
    const int L0 = min(C, Tn);
    load_kv(0, L0);
    load_q(0, L0);
    write_rt();
    store_kv(L0);
  }
  __syncthreads();

  for (int s0 = 0; s0 < Tn; s0 += C) {
    const int L = min(C, Tn - s0);
    const int s1 = s0 + C;
    const bool has_next = s1 < Tn;
    const int Ln = has_next ? min(C, Tn - s1) : 0;
    if (has_next) load_kv(s1, Ln);

    // ================= phase A: outputs of this chunk =================
    f32x4 Ox[F::NQ][4];
    f32x4 Op[F::NQ][4];
#pragma unroll
    for (int qi = 0; qi < F::NQ; ++qi)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        Ox[qi][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        Op[qi][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    // cross-chunk term Q R_i (B operand = rows of R^T, 16 bytes per lane)
#pragma unroll
    for (int s = 0; s < F::KS; ++s) {
      bf16x8 rb[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) rb[nb] = lds_read16(&Rt[(16 * nb + c16) * F::RLD + 32 * s + 8 * g]);
#pragma unroll
      for (int qi = 0; qi < F::NQ; ++qi)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) Ox[qi][nb] = mfma(Qreg[qi][s], rb[nb], Ox[qi][nb]);
    }
    // intra-chunk term: key steps of 32 keys below the diagonal
    const int qmax = qblk[F::NQ - 1] > qblk[0] ? qblk[F::NQ - 1] : qblk[0];
    for (int sp = 0; 2 * sp <= qmax; ++sp) {
      f32x4 St[F::NQ][2];
#pragma unroll
      for (int qi = 0; qi < F::NQ; ++qi) {
        St[qi][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        St[qi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      bool need0[F::NQ], need1[F::NQ];
#pragma unroll
      for (int qi = 0; qi < F::NQ; ++qi) {
        need0[qi] = qblk[qi] >= 2 * sp;
        need1[qi] = qblk[qi] >= 2 * sp + 1;
      }
#pragma unroll
      for (int s = 0; s < F::KS; ++s) {
        const bf16x8 ka = lds_read16(&Ks[(32 * sp + c16) * F::KLD + 32 * s + 8 * g]);
        const bf16x8 kb = lds_read16(&Ks[(32 * sp + 16 + c16) * F::KLD + 32 * s + 8 * g]);
#pragma unroll
        for (int qi = 0; qi < F::NQ; ++qi) {
          if (need0[qi]) St[qi][0] = mfma(ka, Qreg[qi][s], St[qi][0]);
          if (need1[qi]) St[qi][1] = mfma(kb, Qreg[qi][s], St[qi][1]);
        }
      }
      // V operands (keys 32sp+4g+e and 32sp+16+4g+e), shared by both query blocks
      bf16x8 vb[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = 16 * nb + 4 * (c16 & 3);
        const s16x4 lo = lds_read_tr(&Vs[(32 * sp + 4 * g + (c16 >> 2)) * F::VLD + col]);
        const s16x4 hi = lds_read_tr(&Vs[(32 * sp + 16 + 4 * g + (c16 >> 2)) * F::VLD + col]);
        vb[nb] = join(lo, hi);
      }
#pragma unroll
      for (int qi = 0; qi < F::NQ; ++qi) {
        if (!need0[qi]) continue;
        const int j = 16 * qblk[qi] + c16;  // query row of this lane
        f32x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 32 * sp + 4 * g + (e & 3) + 16 * (e >> 2);
          const int d = j - t;
          const float sv = e < 4 ? St[qi][0][e & 3] : St[qi][1][e & 3];
          p[e] = d > 0 ? sv * exp2f(static_cast<float>(d) * lg) : (d == 0 ? sv : 0.0f);
        }
        const bf16x8 pa = __builtin_convertvector(p, bf16x8);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) Op[qi][nb] = mfma(pa, vb[nb], Op[qi][nb]);
      }
    }
    // combine and store: Y = P V + gamma^(j+1) Q R
#pragma unroll
    for (int qi = 0; qi < F::NQ; ++qi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * qblk[qi] + 4 * g + i;
        const float xi = exp2f(static_cast<float>(row + 1) * lg);
        if (row < L) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            yh[static_cast<long>(s0 + row) * dv + 16 * nb + c16] = f32_to_bf16(fmaf(xi, Ox[qi][nb][i], Op[qi][nb][i]));
        }
      }
    }
    if (has_next) load_q(s1, Ln);
    __syncthreads();  // all waves are done reading R^T, V and K for outputs

    // ================= phase B: state update =================
    {
      const float gL = gamma_pow(lg, L);
#pragma unroll
      for (int mb = 0; mb < F::RM; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) Racc[mb][nb] *= gL;
#pragma unroll
      for (int s = 0; s < CT / 32; ++s) {
        if (32 * s >= L) break;
        bf16x8 zb[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = 16 * nb + 4 * (c16 & 3);
          const s16x4 lo = lds_read_tr(&Vz[(32 * s + 8 * g + (c16 >> 2)) * F::VLD + col]);
          const s16x4 hi = lds_read_tr(&Vz[(32 * s + 8 * g + 4 + (c16 >> 2)) * F::VLD + col]);
          zb[nb] = join(lo, hi);
        }
#pragma unroll
        for (int mb = 0; mb < F::RM; ++mb) {
          const int col = dbase + 16 * mb + 4 * (c16 & 3);
          const s16x4 lo = lds_read_tr(&Ks[(32 * s + 8 * g + (c16 >> 2)) * F::KLD + col]);
          const s16x4 hi = lds_read_tr(&Ks[(32 * s + 8 * g + 4 + (c16 >> 2)) * F::KLD + col]);
          const bf16x8 ka = join(lo, hi);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) Racc[mb][nb] = mfma(ka, zb[nb], Racc[mb][nb]);
        }
      }
      write_rt();
    }
    __syncthreads();  // K and zeta*V fully consumed; R^T rewritten
    if (has_next) {
      store_kv(Ln);
      __syncthreads();
    }
  }

  if (state_out != nullptr) {
#pragma unroll
    for (int mb = 0; mb < F::RM; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = dbase + 16 * mb + 4 * g + i;
          state_out[sbase + static_cast<long>(d) * dv + 16 * nb + c16] = Racc[mb][nb][i];
        }
  }
}

template <int CT, int DK>
hipError_t launch_cfg(const void* q, const void* k, const void* v, const float* state_in, float* state_out, void* y,
                      int B, int H, int Tn, int dv, int C, const HeadDecay& hd, const HeadGroup& g, hipStream_t s) {
  const int ntiles = dv / kTN;
  const int total = B * g.nh * ntiles;
  hipLaunchKernelGGL((chunkwise_mfma_kernel<CT, DK>), dim3(total), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), state_in, state_out, static_cast<uint16_t*>(y), hd, H, g.h0,
                     g.nh, Tn, dv, C, ntiles);
  return hipGetLastError();
}

template <int CT>
hipError_t launch_ct(const void* q, const void* k, const void* v, const float* state_in, float* state_out, void* y,
                     int B, int H, int Tn, int dk, int dv, int C, const HeadDecay& hd, const HeadGroup& g,
                     hipStream_t s) {
  switch (dk) {
    case 64: return launch_cfg<CT, 64>(q, k, v, state_in, state_out, y, B, H, Tn, dv, C, hd, g, s);
    case 128: return launch_cfg<CT, 128>(q, k, v, state_in, state_out, y, B, H, Tn, dv, C, hd, g, s);
    default: return launch_cfg<CT, 256>(q, k, v, state_in, state_out, y, B, H, Tn, dv, C, hd, g, s);
  }
}

}  // namespace

bool chunkwise_mfma_supports(int /*T*/, int dk, int dv, int C, int dt) {
  return dt == 1 && (dk == 64 || dk == 128 || dk == 256) && dv % kTN == 0 && C >= 1 && C <= 128;
}

hipError_t launch_chunkwise_mfma(const void* q, const void* k, const void* v, const float* state_in,
                                 float* state_out, void* y, int B, int H, int T, int dk, int dv, int C,
                                 const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  if (C <= 64) return launch_ct<64>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, C, hd, g, s);
  return launch_ct<128>(q, k, v, state_in, state_out, y, B, H, T, dk, dv, C, hd, g, s);
}

}  // namespace ret
