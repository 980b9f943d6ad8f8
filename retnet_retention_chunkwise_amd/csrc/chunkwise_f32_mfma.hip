// Chunkwise retention passes with fp32 inputs on fp32 MFMA (gfx950,
// v_mfma_f32_16x16x4_f32): fp32 products and accumulation, so fp32 inputs
// keep fp32 accuracy, at matrix-core rate.
//
// One kernel shape serves the forward and the three backward passes of the
// chunkwise form (aimpact page, "Il meccanismo: Multi-Scale Retention"; the
// backward is the chain rule on its recurrence).  Each pass has inputs
// (A, B, X) with A, B of width d_a and X of width d_x, and a d_a x d_x fp32
// state S:
//   forward in time:  Out_j = gamma^(j+1) A_j S + sum_{j'<=j} gamma^(j-j') (A_j . B_j') X_j'
//                     S <- gamma^L S + sum_j gamma^(L-1-j) B_j^T X_j
//   reverse in time:  chunks from last to first,
//                     Out_j = gamma^(L-1-j) A_j S + sum_{j'>=j} gamma^(j'-j) (A_j . B_j') X_j'
//                     S <- gamma^L S + sum_j gamma^(j+1) B_j^T X_j
//   forward: (Q, K, V) from S_in (final S = state_out);  dQ: (dY, V, K) from S_in^T;
//   dK: reverse (V, dY, Q) from dS_out^T;  dV: reverse (K, Q, dY) from dS_out (final S = dS_in).
//
// Work decomposition: a workgroup owns (batch, head, 64 X columns) and walks
// 16-token chunks.  It has 4 column strips of 16 columns times 4 parts of d_a:
// wave (strip, part) keeps the d_a/4 state rows of its part for its strip in
// MFMA accumulator layout (lane: column l%16, rows 4(l/16)+i of a 16-row
// block).  Per chunk:
//   * the waves of part 1 form the 16x16 scores A B^T, each over a quarter of
//     d_a (partial tiles to LDS; the consumers add the four and apply the
//     causal decay mask);
//   * every wave forms its part of the cross term transposed, Out^T = S^T A^T:
//     MFMA i of a 16-row block takes accumulator element i as its A operand,
//     so k index g stands for feature 4g + i, and one 16-byte read of an A row
//     gives the B operands of all four; parts 1..3 hand their partials to
//     part 0 through LDS;
//   * part 0 adds the partials, scales by the row weight, adds X^T P^T and
//     stores (each lane 4 consecutive columns of one token: 16-byte stores);
//   * every wave updates its rows, S <- gamma^L S + B^T (z X), straight into
//     the state registers.
// LDS row strides are padded so that the row reads of A, the column reads of
// B, X and zX, and the score reads hit distinct banks.  Global accesses go
// through buffer resources ending at the sequence's last token (rows past the
// end read as zero, their stores are dropped).
#include "common.h"
#include "gfx950.h"
#include "kernels.h"

namespace ret {
namespace {

constexpr int kCT = 16;        // tokens per chunk
constexpr int kTX = 64;        // X / Out columns per workgroup
constexpr int kParts = 4;      // parts of d_a per column strip
constexpr int kThreads = 1024; // 4 strips x 4 parts

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct FPass {
  const float* a;   // [BH, T, DA]
  const float* b;   // [BH, T, DA]
  const float* x;   // [BH, T, DX]
  float* out;       // [BH, T, DX]
  const float* s0;  // nullable; [BH, DA, DX] (s0_t = 0) or [BH, DX, DA] (s0_t = 1)
  float* s_out;     // nullable; [BH, DA, DX]
  int s0_t;
  int rev;
  int dx;
};
struct FPassSet {
  FPass p[2];
  int npass;  // passes of the launch (same d_a and d_x)
};

template <int DA>
struct FCfg {
  static constexpr int ALD = DA + 4;    // fp32 row stride of the A tile (row reads)
  static constexpr int BLD = DA + 16;   // of the B tile (column reads)
  static constexpr int XLD = kTX + 16;  // of the X and zX tiles (column reads)
  static constexpr int PLD = kCT + 4;   // of the partial score tiles
  static constexpr int RP = DA / kParts;  // state rows per wave
  static constexpr int NAB = RP / 16;     // 16-row blocks per wave
  static constexpr int NP = kCT * DA / 4;                       // 16-byte pieces of the A (and B) tile
  static constexpr int NLD = (NP + kThreads - 1) / kThreads;    // per thread
  static_assert(NAB >= 1, "d_a too small");
};

template <int DA>
__global__ __launch_bounds__(kThreads) void f32_pass_kernel(FPassSet ps, HeadDecay gam, int H, int h0, int nh,
                                                            int Tn) {
  using F = FCfg<DA>;
  __shared__ __attribute__((aligned(16))) float As[kCT * F::ALD];
  __shared__ __attribute__((aligned(16))) float Bs[kCT * F::BLD];
  __shared__ __attribute__((aligned(16))) float Xs[kCT * F::XLD];
  __shared__ __attribute__((aligned(16))) float Zs[kCT * F::XLD];
  __shared__ __attribute__((aligned(16))) float Pp[kParts][kCT * F::PLD];  // partial scores
  __shared__ f32x4 Xch[kParts - 1][4][64];                                 // cross-term partials

  // work item; the column tiles and passes of a head sit on one XCD
  const int nwg = gridDim.x;
  const int lin = blockIdx.x;
  const int item = (nwg % 8 == 0) ? (lin % 8) * (nwg / 8) + lin / 8 : lin;
  const int tiles = ps.p[0].dx / kTX;
  const int tile = item % tiles;
  const int pz = (item / tiles) % ps.npass;
  const int hitem = item / (tiles * ps.npass);
  const FPass p = ps.p[pz];
  const int DX = p.dx;
  const bool rev = p.rev != 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int cs = w & 3;      // column strip
  const int hf = w >> 2;     // part of d_a: rows [hf RP, (hf+1) RP)
  const int g = lane >> 4;
  const int lr = lane & 15;
  const int hl = hitem % nh;
  const int bb = hitem / nh;
  const long head = static_cast<long>(bb) * H + h0 + hl;
  const float lg = gam.log2g[hl];
  const int c0 = tile * kTX;
  const int cw = 16 * cs;

  const rsrc_t ra = make_rsrc(p.a + head * Tn * DA, static_cast<uint32_t>(Tn) * DA * 4);
  const rsrc_t rb = make_rsrc(p.b + head * Tn * DA, static_cast<uint32_t>(Tn) * DA * 4);
  const rsrc_t rx = make_rsrc(p.x + head * Tn * DX, static_cast<uint32_t>(Tn) * DX * 4);
  const rsrc_t ro = make_rsrc(p.out + head * Tn * DX, static_cast<uint32_t>(Tn) * DX * 4);
  const long sb = head * static_cast<long>(DA) * DX;

  // state: S[hf RP + 16 l + 4 g + i][c0 + cw + lr] in Sacc[l][i]
  f32x4 Sacc[F::NAB];
  {
    const int x = c0 + cw + lr;
#pragma unroll
    for (int l = 0; l < F::NAB; ++l) {
      const int a = hf * F::RP + 16 * l + 4 * g;
      f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
      if (p.s0 != nullptr) {
        if (p.s0_t) {
          v = *reinterpret_cast<const f32x4*>(p.s0 + sb + static_cast<long>(x) * DA + a);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = p.s0[sb + static_cast<long>(a + i) * DX + x];
        }
      }
      Sacc[l] = v;
    }
  }

  // staging: A/B piece q = tid + 1024 r (q < NP) = row q / (DA/4), 4 features;
  // X piece of threads 0..255: row tid / 16, columns 4 (tid % 16) .. +3
  constexpr int PPR = DA / 4;
  u32x4 pa[F::NLD], pb[F::NLD], px;
  const bool xthr = tid < kCT * kTX / 4;
  const int xj = (tid >> 4) & (kCT - 1), xc = (tid & 15) * 4;
  auto prefetch = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < F::NLD; ++r) {
      const int q = tid + kThreads * r;
      if (q < F::NP) {
        const uint32_t off = (static_cast<uint32_t>(t0 + q / PPR) * DA + (q % PPR) * 4) * 4;
        pa[r] = buffer_load16(ra, off);
        pb[r] = buffer_load16(rb, off);
      }
    }
    if (xthr) px = buffer_load16(rx, (static_cast<uint32_t>(t0 + xj) * DX + c0 + xc) * 4);
  };

  const int nch = (Tn + kCT - 1) / kCT;
  prefetch((rev ? nch - 1 : 0) * kCT);
  for (int it = 0; it < nch; ++it) {
    const int ci = rev ? nch - 1 - it : it;
    const int t0 = ci * kCT;
    const int L = min(kCT, Tn - t0);
    // ---- stage this chunk (the previous chunk ended with a barrier)
#pragma unroll
    for (int r = 0; r < F::NLD; ++r) {
      const int q = tid + kThreads * r;
      if (q < F::NP) {
        *reinterpret_cast<u32x4*>(&As[(q / PPR) * F::ALD + (q % PPR) * 4]) = pa[r];
        *reinterpret_cast<u32x4*>(&Bs[(q / PPR) * F::BLD + (q % PPR) * 4]) = pb[r];
      }
    }
    if (xthr) {
      *reinterpret_cast<u32x4*>(&Xs[xj * F::XLD + xc]) = px;
      const float z = xj < L ? gamma_pow(lg, rev ? xj + 1 : L - 1 - xj) : 0.0f;
      const f32x4 xv = __builtin_bit_cast(f32x4, px);
      *reinterpret_cast<f32x4*>(&Zs[xj * F::XLD + xc]) = xv * z;
    }
    if (it + 1 < nch) prefetch((rev ? ci - 1 : ci + 1) * kCT);
    lds_barrier();

    // ---- partial scores (part 1): features [cs DA/4, (cs+1) DA/4) of A_j . B_j'
    if (hf == 1) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < DA / 4 / 16; ++s) {
        const int a0 = cs * (DA / 4) + 16 * s + 4 * g;  // k index g of MFMA e = feature a0 + e
        const f32x4 av = *reinterpret_cast<const f32x4*>(&As[lr * F::ALD + a0]);
        const f32x4 bv = *reinterpret_cast<const f32x4*>(&Bs[lr * F::BLD + a0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma4(av[e], bv[e], acc);
      }
      // acc: rows j = 4g + i, column j' = lr
#pragma unroll
      for (int i = 0; i < 4; ++i) Pp[cs][(4 * g + i) * F::PLD + lr] = acc[i];
    }

    // ---- cross term over this wave's part of d_a: Out^T = S^T A^T
    f32x4 O = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int l = 0; l < F::NAB; ++l) {
      const int a0 = hf * F::RP + 16 * l + 4 * g;
      const f32x4 av = *reinterpret_cast<const f32x4*>(&As[lr * F::ALD + a0]);  // A[j = lr][a0 + i]
#pragma unroll
      for (int i = 0; i < 4; ++i) O = mfma4(Sacc[l][i], av[i], O);
    }
    if (hf >= 1) Xch[hf - 1][cs][lane] = O;
    lds_barrier();  // partial scores and cross terms are in LDS

    // ---- outputs (part 0): Out^T = w (sum of partials) + X^T P^T
    if (hf == 0) {
#pragma unroll
      for (int u = 0; u < kParts - 1; ++u) O += Xch[u][cs][lane];
      const int j = lr;
      O *= j < L ? gamma_pow(lg, rev ? L - 1 - j : j + 1) : 0.0f;
#pragma unroll
      for (int s = 0; s < kCT / 4; ++s) {
        const int jp = 4 * s + g;
        const int d = rev ? jp - j : j - jp;
        float pv = 0.0f;
        if (d >= 0) {
          float sc = 0.0f;
#pragma unroll
          for (int u = 0; u < kParts; ++u) sc += Pp[u][j * F::PLD + jp];
          pv = sc * gamma_pow(lg, d);
        }
        O = mfma4(Xs[jp * F::XLD + cw + lr], pv, O);
      }
      // lane: Out[t0 + lr][c0 + cw + 4 g + i]
      buffer_store16(ro, (static_cast<uint32_t>(t0 + lr) * DX + c0 + cw + 4 * g) * 4, __builtin_bit_cast(u32x4, O));
    }

    // ---- state update of this wave's rows: S <- gamma^L S + B^T (z X)
    {
      const float gL = gamma_pow(lg, L);
      float zx[kCT / 4];
#pragma unroll
      for (int s = 0; s < kCT / 4; ++s) zx[s] = Zs[(4 * s + g) * F::XLD + cw + lr];
#pragma unroll
      for (int l = 0; l < F::NAB; ++l) {
        const int a = hf * F::RP + 16 * l + lr;
        f32x4 acc = Sacc[l] * gL;
#pragma unroll
        for (int s = 0; s < kCT / 4; ++s) acc = mfma4(Bs[(4 * s + g) * F::BLD + a], zx[s], acc);
        Sacc[l] = acc;
      }
    }
    lds_barrier();  // every read of this chunk's tiles is done
  }

  if (p.s_out != nullptr) {
    const int x = c0 + cw + lr;
#pragma unroll
    for (int l = 0; l < F::NAB; ++l)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.s_out[sb + static_cast<long>(hf * F::RP + 16 * l + 4 * g + i) * DX + x] = Sacc[l][i];
  }
}

template <int DA>
hipError_t launch_da(const FPassSet& ps, int B, const HeadDecay& hd, int H, const HeadGroup& g, int T,
                     hipStream_t s) {
  const dim3 grid(B * g.nh * ps.npass * (ps.p[0].dx / kTX));
  hipLaunchKernelGGL(f32_pass_kernel<DA>, grid, dim3(kThreads), 0, s, ps, hd, H, g.h0, g.nh, T);
  return hipGetLastError();
}

hipError_t launch_by_da(int da, const FPassSet& ps, int B, const HeadDecay& hd, int H, const HeadGroup& g, int T,
                        hipStream_t s) {
  switch (da) {
    case 64: return launch_da<64>(ps, B, hd, H, g, T, s);
    case 128: return launch_da<128>(ps, B, hd, H, g, T, s);
    case 256: return launch_da<256>(ps, B, hd, H, g, T, s);
    default: return launch_da<512>(ps, B, hd, H, g, T, s);
  }
}

bool d_ok(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

}  // namespace

bool chunkwise_f32_mfma_supports(int dk, int dv, int dt) { return dt == 0 && d_ok(dk) && d_ok(dv); }

hipError_t launch_chunkwise_f32_fwd(const float* q, const float* k, const float* v, const float* state_in,
                                    float* state_out, float* y, int B, int H, int T, int dk, int dv,
                                    const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  FPassSet ps{};
  ps.p[0] = FPass{q, k, v, y, state_in, state_out, 0, 0, dv};
  ps.p[1] = ps.p[0];
  ps.npass = 1;
  return launch_by_da(dk, ps, B, hd, H, g, T, s);
}

hipError_t launch_chunkwise_f32_bwd(const BwdArgs& a, int B, int H, int T, int dk, int dv, const HeadGroup& g,
                                    hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  auto f = [](const void* x) { return static_cast<const float*>(x); };
  FPassSet kq{};
  kq.p[0] = FPass{f(a.v), f(a.dy), f(a.q), static_cast<float*>(a.dk), a.dstate_out, nullptr, 1, 1, dk};
  kq.p[1] = FPass{f(a.dy), f(a.v), f(a.k), static_cast<float*>(a.dq), a.state_in, nullptr, 1, 0, dk};
  kq.npass = 2;
  hipError_t e = launch_by_da(dv, kq, B, hd, H, g, T, s);
  if (e != hipSuccess) return e;
  // dV after dK, so that dstate_in may be the dstate_out buffer
  FPassSet vs{};
  vs.p[0] = FPass{f(a.k), f(a.q), f(a.dy), static_cast<float*>(a.dv), a.dstate_out, a.dstate_in, 0, 1, dv};
  vs.p[1] = vs.p[0];
  vs.npass = 1;
  return launch_by_da(dk, vs, B, hd, H, g, T, s);
}

}  // namespace ret
