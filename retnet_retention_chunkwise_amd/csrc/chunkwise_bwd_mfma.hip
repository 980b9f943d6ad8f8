// Backward passes of chunkwise retention on bf16 MFMA (gfx950), fp32 state.
//
// The gradients of the chunkwise form (aimpact page, "Il meccanismo:
// Multi-Scale Retention"; chain rule on its recurrence) are three chunkwise
// passes of one shape, each with a d_a x d_x fp32 state S:
//   forward in time:  Out_j = gamma^(j+1) A_j S + sum_{j'<=j} gamma^(j-j') (A_j . B_j') X_j'
//                     S <- gamma^L S + sum_j gamma^(L-1-j) B_j^T X_j
//   reverse in time:  chunks from last to first,
//                     Out_j = gamma^(L-1-j) A_j S + sum_{j'>=j} gamma^(j'-j) (A_j . B_j') X_j'
//                     S <- gamma^L S + sum_j gamma^(j+1) B_j^T X_j
//   dQ: forward, (A, B, X) = (dY, V, K), S_0 = S_in^T
//   dK: reverse, (V, dY, Q), S_0 = dS_out^T
//   dV: reverse, (K, Q, dY), S_0 = dS_out; the final S is dS_in.
//
// Work decomposition: a workgroup owns one (batch, head, tile of 64 X
// columns) and walks the 32-token chunks in order.  It has 4 column strips of
// 16 columns times KS parts of d_a (KS = 4, or 2 for d_a = 64): wave (strip,
// part) keeps the d_a/KS state rows of its part for its 16 columns in MFMA
// accumulator layout (lane: column l%16, rows 4(l/16)+i of each 16-row
// block), so no state goes through LDS, and KS waves per SIMD hide each
// other's latency:
//   * the cross term is formed transposed, Out^T = S^T A^T, each wave over its
//     part of d_a: the accumulator layout of S, read as an MFMA A operand,
//     covers the features {32s + 4g + i, 32s + 16 + 4g + i} of lane group g,
//     and the matching B operand is two 8-byte reads of the A rows in LDS (the
//     same feature permutation on both sides of the contraction).  Parts
//     1..KS-1 hand their partial sums to part 0 through LDS (across the
//     barrier that also publishes the scores);
//   * the scores P = (A B^T) .* mask are one 16x16 tile per wave of part 1,
//     written to LDS in bf16; part 0 adds the intra term Out^T += X^T P^T (X^T
//     through the transposing LDS load) and stores;
//   * every wave updates its rows, S <- gamma^L S + B^T (z X), straight into
//     the state registers, B^T and z X through the transposing load.
// Out^T leaves each lane 4 consecutive columns of one token: 8-byte stores.
// In the operands read with the transposing load (X^T, B^T, z X), k index
// 8g + e of lane group g stands for token 4g + (e % 4) + 16 (e / 4) (P^T is
// read with the same order); with the B and X row strides padded to 8 dwords
// mod 64 banks this makes those reads free of bank conflicts.
// The next chunk's A, B and X are loaded into registers while the current
// chunk is computed.  Global accesses go through buffer resources ending at
// the sequence's last token, so rows past the end read as zero and their
// stores are dropped.  dK and dQ (the same d_a) run in one launch; the column
// tiles and passes of a head are placed on one XCD (shared L2).
#include "common.h"
#include "gfx950.h"
#include "kernels.h"

namespace ret {
namespace {

constexpr int kCT = 32;        // tokens per chunk
constexpr int kTX = 64;        // X / Out columns per workgroup (16 per wave pair)

struct MPass {
  const uint16_t* a;  // [BH, T, DA] bf16
  const uint16_t* b;  // [BH, T, DA]
  const uint16_t* x;  // [BH, T, DX]
  uint16_t* out;      // [BH, T, DX]
  const float* s0;    // nullable; [BH, DA, DX] (s0_t = 0) or [BH, DX, DA] (s0_t = 1)
  float* s_out;       // nullable; [BH, DA, DX]
  int s0_t;
  int rev;
  int dx;
  float* ws;       // segmented calls: state slots, slot s at ws + s * ws_stride ([BH, DA, DX])
  long ws_stride;
};
// Sequence segments (for few heads over long sequences): with nseg > 1 a pass
// runs as a state-only launch over every segment but the first in its
// direction (local end states from zero, into the slots), a scan over the
// slots (incoming state of every segment), and the full launch per segment.
struct MPassSet {
  MPass p[2];
  int npass;    // passes of the launch (same d_a and d_x)
  int nseg;     // segments (1: none)
  int seg_len;  // tokens per segment, a multiple of the chunk
  int full;     // 1: outputs and final state; 0: state-only launch
};

template <int DA>
struct BCfg {
  // waves per column strip, each owning DA / KS state rows (a k-step of 32
  // features needs two 16-row blocks per wave)
  static constexpr int KS = DA >= 128 ? 4 : 2;
  static constexpr int NT = 256 * KS;   // threads: 4 column strips x KS parts of d_a
  static constexpr int ALD = DA + 8;    // bf16 row stride of the A tile in LDS
  static constexpr int BLD = DA + 16;   // row stride of the B tile
  static constexpr int XLD = kTX + 16;  // row stride of the X and zX tiles
  static constexpr int PLD = kCT + 8;   // row stride of the score tile
  static constexpr int NABH = DA / 16 / KS;  // 16-row state blocks per wave (its part of d_a)
  static constexpr int NSH = DA / 32 / KS;   // 32-wide k-steps per wave
  static constexpr int NP = kCT * DA / 8;                        // 16-byte pieces of the A (and B) tile
  static constexpr int NLD = (NP + NT - 1) / NT;                 // per thread
};

template <int DA>
__global__ __launch_bounds__(BCfg<DA>::NT) void bwd_pass_mfma_kernel(MPassSet ps, HeadDecay gam, int H, int h0, int nh,
                                                                 int Tn) {
  using F = BCfg<DA>;
  __shared__ __attribute__((aligned(16))) uint16_t As[kCT * F::ALD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kCT * F::BLD];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kCT * F::XLD];
  __shared__ __attribute__((aligned(16))) uint16_t Zs[kCT * F::XLD];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[kCT * F::PLD];
  __shared__ f32x4 Xch[F::KS - 1][4][2][64];  // cross-term partials of parts 1..KS-1

  // Work item.  Workgroup ids are dealt round-robin over the 8 XCDs; the
  // remap gives each XCD a contiguous range of items, so the column tiles and
  // passes of one head (which read the same rows) share one L2.
  const int nwg = gridDim.x;
  const int lin = blockIdx.x;
  const int item = (nwg % 8 == 0) ? (lin % 8) * (nwg / 8) + lin / 8 : lin;
  const int tiles = ps.p[0].dx / kTX;
  const int nsl = ps.full ? ps.nseg : ps.nseg - 1;  // segment launches per (head, pass)
  const int tile = item % tiles;
  const int segl = (item / tiles) % nsl;
  const int pz = (item / (tiles * nsl)) % ps.npass;
  const int hitem = item / (tiles * nsl * ps.npass);
  const MPass p = ps.p[pz];
  const int DX = p.dx;
  const bool rev = p.rev != 0;
  const bool full = ps.full != 0;
  // the state-only launch skips the segment processed first in the pass's direction
  const int seg = (!full && rev) ? segl + 1 : segl;
  const int t_begin = seg * ps.seg_len;
  const int t_end = min(Tn, t_begin + ps.seg_len);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int cs = w & 3;      // column strip
  const int hf = w >> 2;     // d_a part: state rows [hf DA/KS, (hf+1) DA/KS)
  const int g = lane >> 4;   // lane group
  const int lr = lane & 15;  // lane within the group
  const int hl = hitem % nh;
  const int bb = hitem / nh;
  const long head = static_cast<long>(bb) * H + h0 + hl;
  const float lg = gam.log2g[hl];
  const int c0 = tile * kTX;
  const int cw = 16 * cs;  // this wave's columns inside the tile

  const rsrc_t ra = make_rsrc(p.a + head * Tn * DA, static_cast<uint32_t>(Tn) * DA * 2);
  const rsrc_t rb = make_rsrc(p.b + head * Tn * DA, static_cast<uint32_t>(Tn) * DA * 2);
  const rsrc_t rx = make_rsrc(p.x + head * Tn * DX, static_cast<uint32_t>(Tn) * DX * 2);
  const rsrc_t ro = make_rsrc(p.out + head * Tn * DX, static_cast<uint32_t>(Tn) * DX * 2);
  const long sb = head * static_cast<long>(DA) * DX;

  // incoming state: the pass's S_0 (one segment), the scanned slot of this
  // segment, or zero (state-only launch); outgoing: the pass's final state
  // (the segment processed last) or, state-only, the next segment's slot
  const float* init = nullptr;
  bool init_t = false;
  float* endp = nullptr;
  if (ps.nseg == 1) {
    init = p.s0;
    init_t = p.s0_t != 0;
    endp = p.s_out;
  } else if (full) {
    init = p.ws + seg * p.ws_stride;
    if (seg == (rev ? 0 : ps.nseg - 1)) endp = p.s_out;
  } else {
    endp = p.ws + (rev ? seg - 1 : seg + 1) * p.ws_stride;
  }

  // state: S[16 (hf NABH + l) + 4 g + i][c0 + cw + lr] in Sacc[l][i]
  f32x4 Sacc[F::NABH];
  {
    const int x = c0 + cw + lr;
#pragma unroll
    for (int l = 0; l < F::NABH; ++l) {
      const int a = 16 * (hf * F::NABH + l) + 4 * g;
      f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
      if (init != nullptr) {
        if (init_t) {
          v = *reinterpret_cast<const f32x4*>(init + sb + static_cast<long>(x) * DA + a);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = init[sb + static_cast<long>(a + i) * DX + x];
        }
      }
      Sacc[l] = v;
    }
  }

  // staging map: A/B piece q = tid + 512 r (q < NP) = row q / (DA/8), 8 features;
  // X piece of threads 0..255: row tid / 8, columns 8 (tid % 8) .. +7 of the tile
  constexpr int PPR = DA / 8;  // 16-byte pieces per row
  u32x4 pa[F::NLD], pb[F::NLD], px;
  const bool xthr = tid < kCT * kTX / 8;
  const int xj = (tid >> 3) & (kCT - 1), xc = (tid & 7) * 8;
  auto prefetch = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < F::NLD; ++r) {
      const int q = tid + F::NT * r;
      if (q < F::NP) {
        const uint32_t off = (static_cast<uint32_t>(t0 + q / PPR) * DA + (q % PPR) * 8) * 2;
        if (full) pa[r] = buffer_load16(ra, off);  // A feeds only the outputs
        pb[r] = buffer_load16(rb, off);
      }
    }
    if (xthr) px = buffer_load16(rx, (static_cast<uint32_t>(t0 + xj) * DX + c0 + xc) * 2);
  };

  const int nch = (t_end - t_begin + kCT - 1) / kCT;
  const float gL_full = gamma_pow(lg, kCT);
  prefetch(t_begin + (rev ? nch - 1 : 0) * kCT);
  for (int it = 0; it < nch; ++it) {
    const int ci = rev ? nch - 1 - it : it;
    const int t0 = t_begin + ci * kCT;
    const int L = min(kCT, t_end - t0);
    // ---- stage this chunk (the previous chunk ended with a barrier)
#pragma unroll
    for (int r = 0; r < F::NLD; ++r) {
      const int q = tid + F::NT * r;
      if (q < F::NP) {
        if (full) *reinterpret_cast<u32x4*>(&As[(q / PPR) * F::ALD + (q % PPR) * 8]) = pa[r];
        *reinterpret_cast<u32x4*>(&Bs[(q / PPR) * F::BLD + (q % PPR) * 8]) = pb[r];
      }
    }
    if (xthr) {
      *reinterpret_cast<u32x4*>(&Xs[xj * F::XLD + xc]) = px;
      const float z = xj < L ? gamma_pow(lg, rev ? xj + 1 : L - 1 - xj) : 0.0f;
      const bf16x8 xv = __builtin_bit_cast(bf16x8, px);
      bf16x8 zv;
#pragma unroll
      for (int e = 0; e < 8; ++e) zv[e] = static_cast<__bf16>(z * static_cast<float>(xv[e]));
      *reinterpret_cast<bf16x8*>(&Zs[xj * F::XLD + xc]) = zv;
    }
    if (it + 1 < nch) prefetch(t_begin + (rev ? ci - 1 : ci + 1) * kCT);
    lds_barrier();

    // ---- scores (waves of the upper half): tile (jb, jpb) = strip cs, masked
    // and decayed, to LDS in bf16
    if (full && hf == 1) {
      const int jb = cs >> 1, jpb = cs & 1;
      const bool live = rev ? jpb >= jb : jpb <= jb;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if (live) {
#pragma unroll
        for (int s = 0; s < DA / 32; ++s) {
          const bf16x8 av = lds_read16(&As[(16 * jb + lr) * F::ALD + 32 * s + 8 * g]);
          const bf16x8 bv = lds_read16(&Bs[(16 * jpb + lr) * F::BLD + 32 * s + 8 * g]);
          acc = mfma(av, bv, acc);
        }
      }
      const int jp = 16 * jpb + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * jb + 4 * g + i;
        const int d = rev ? jp - j : j - jp;
        const float val = d >= 0 ? acc[i] * gamma_pow(lg, d) : 0.0f;
        Ps[j * F::PLD + jp] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(val));
      }
    }

    // ---- cross term over this wave's half of d_a: Out^T = S^T A^T (partial)
    f32x4 O[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) O[jb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sl = 0; sl < F::NSH; ++sl) {
      if (full) {
        const int s = hf * F::NSH + sl;
        const bf16x8 sv = pack_bf16x8(Sacc[2 * sl], Sacc[2 * sl + 1]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const uint16_t* row = &As[(16 * jb + lr) * F::ALD + 32 * s + 4 * g];
          const bf16x8 av = join(*reinterpret_cast<const s16x4*>(row), *reinterpret_cast<const s16x4*>(row + 16));
          O[jb] = mfma(sv, av, O[jb]);
        }
      }
    }
    if (full && hf >= 1) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) Xch[hf - 1][cs][jb][lane] = O[jb];
    }
    lds_barrier();  // scores and upper partials are in LDS

    // ---- outputs (lower half): add the partner's partial, scale, + X^T P^T
    if (full && hf == 0) {
      const uint16_t* xr = &Xs[(4 * g + (lr >> 2)) * F::XLD + cw + 4 * (lr & 3)];
      const bf16x8 xt = join(lds_read_tr(xr), lds_read_tr(xr + 16 * F::XLD));
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int j = 16 * jb + lr;
        const float wj = j < L ? gamma_pow(lg, rev ? L - 1 - j : j + 1) : 0.0f;
#pragma unroll
        for (int u = 0; u < F::KS - 1; ++u) O[jb] += Xch[u][cs][jb][lane];
        O[jb] *= wj;
        const bf16x8 pv = join(*reinterpret_cast<const s16x4*>(&Ps[j * F::PLD + 4 * g]),
                               *reinterpret_cast<const s16x4*>(&Ps[j * F::PLD + 16 + 4 * g]));
        O[jb] = mfma(xt, pv, O[jb]);
        u32x2 st;
        st[0] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(O[jb][0]))) |
                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(O[jb][1]))) << 16);
        st[1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(O[jb][2]))) |
                (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(O[jb][3]))) << 16);
        buffer_store8(ro, (static_cast<uint32_t>(t0 + j) * DX + c0 + cw + 4 * g) * 2, st);
      }
    }

    // ---- state update of this wave's rows: S <- gamma^L S + B^T (z X)
    {
      const float gL = L == kCT ? gL_full : gamma_pow(lg, L);
      const uint16_t* zr = &Zs[(4 * g + (lr >> 2)) * F::XLD + cw + 4 * (lr & 3)];
      const bf16x8 zx = join(lds_read_tr(zr), lds_read_tr(zr + 16 * F::XLD));
      const uint16_t* br = &Bs[(4 * g + (lr >> 2)) * F::BLD + 4 * (lr & 3) + 16 * hf * F::NABH];
#pragma unroll
      for (int l = 0; l < F::NABH; ++l) {
        const bf16x8 bt = join(lds_read_tr(br + 16 * l), lds_read_tr(br + 16 * l + 16 * F::BLD));
        Sacc[l] = mfma(bt, zx, Sacc[l] * gL);
      }
    }
    lds_barrier();  // every read of this chunk's tiles is done
  }

  if (endp != nullptr) {
    const int x = c0 + cw + lr;
#pragma unroll
    for (int l = 0; l < F::NABH; ++l)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        endp[sb + static_cast<long>(16 * (hf * F::NABH + l) + 4 * g + i) * DX + x] = Sacc[l][i];
  }
}

// Incoming state of every segment of one pass, in place over its slots
// (slot s holds the local end state the state-only launch wrote):
//   forward: slot 0 = S_0, slot s = gamma^seg_len slot(s-1) + slot s;
//   reverse: slot nseg-1 = S_0, slot s = gamma^len(s+1) slot(s+1) + slot s.
// S_0 is read in the pass's layout (transposed for s0_t).
__global__ __launch_bounds__(256) void bwd_segment_scan_kernel(MPass p, int DA, HeadDecay gam, int H, int h0, int nh,
                                                               int B, int Tn, int nseg, int seg_len) {
  const long per_head = static_cast<long>(DA) * p.dx;
  const long n = static_cast<long>(B) * nh * per_head;
  for (long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; idx < n;
       idx += static_cast<long>(gridDim.x) * blockDim.x) {
    const long bh = idx / per_head;
    const long within = idx % per_head;
    const int hl = static_cast<int>(bh % nh);
    const long head = (bh / nh) * H + h0 + hl;
    const long off = head * per_head + within;
    const float lg = gam.log2g[hl];
    float s = 0.0f;
    if (p.s0 != nullptr) {
      const long a = within / p.dx, x = within % p.dx;
      s = p.s0_t ? p.s0[head * per_head + x * DA + a] : p.s0[off];
    }
    if (p.rev) {
      p.ws[(nseg - 1) * p.ws_stride + off] = s;
      for (int sg = nseg - 2; sg >= 0; --sg) {
        const int len = min(seg_len, Tn - (sg + 1) * seg_len);
        s = fmaf(gamma_pow(lg, len), s, p.ws[sg * p.ws_stride + off]);
        p.ws[sg * p.ws_stride + off] = s;
      }
    } else {
      const float gs = gamma_pow(lg, seg_len);
      p.ws[off] = s;
      for (int sg = 1; sg < nseg; ++sg) {
        s = fmaf(gs, s, p.ws[sg * p.ws_stride + off]);
        p.ws[sg * p.ws_stride + off] = s;
      }
    }
  }
}

template <int DA>
hipError_t launch_da(MPassSet ps, int B, const HeadDecay& hd, int H, const HeadGroup& g, int T, hipStream_t s) {
  const int items = B * g.nh * ps.npass * (ps.p[0].dx / kTX);
  if (ps.nseg > 1) {
    ps.full = 0;
    hipLaunchKernelGGL(bwd_pass_mfma_kernel<DA>, dim3(items * (ps.nseg - 1)), dim3(BCfg<DA>::NT), 0, s, ps, hd, H,
                       g.h0, g.nh, T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int i = 0; i < ps.npass; ++i) {
      const long n = static_cast<long>(B) * g.nh * DA * ps.p[i].dx;
      const unsigned blocks = static_cast<unsigned>(min(65536L, (n + 255) / 256));
      hipLaunchKernelGGL(bwd_segment_scan_kernel, dim3(blocks), dim3(256), 0, s, ps.p[i], DA, hd, H, g.h0, g.nh, B,
                         T, ps.nseg, ps.seg_len);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  ps.full = 1;
  hipLaunchKernelGGL(bwd_pass_mfma_kernel<DA>, dim3(items * ps.nseg), dim3(BCfg<DA>::NT), 0, s, ps, hd, H, g.h0,
                     g.nh, T);
  return hipGetLastError();
}

hipError_t launch_by_da(int da, const MPassSet& ps, int B, const HeadDecay& hd, int H, const HeadGroup& g, int T,
                        hipStream_t s) {
  switch (da) {
    case 64: return launch_da<64>(ps, B, hd, H, g, T, s);
    case 128: return launch_da<128>(ps, B, hd, H, g, T, s);
    case 256: return launch_da<256>(ps, B, hd, H, g, T, s);
    default: return launch_da<512>(ps, B, hd, H, g, T, s);
  }
}

bool da_ok(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

}  // namespace

bool chunkwise_bwd_mfma_supports(int dk, int dv, int dt) { return dt == 1 && da_ok(dk) && da_ok(dv); }

// Few (batch, head, column tile) walkers over a long sequence: split into
// segments of at least kMinSegChunks chunks so that the smaller of the two
// launches fills about kTargetWorkgroups workgroups.  A pure function of the
// sizes.
ChunkSegments chunkwise_bwd_segments(int B, int H, int T, int dk, int dv) {
  constexpr long kTargetWorkgroups = 256;  // MI355X compute units
  constexpr int kMinSegChunks = 8;
  ChunkSegments r{T > 0 ? T : 1, 1};
  const long walkers = static_cast<long>(B) * H * min(2 * (dk / kTX), dv / kTX);
  const long nchunks = (static_cast<long>(T) + kCT - 1) / kCT;
  if (walkers < 1 || walkers >= kTargetWorkgroups || nchunks < 2 * kMinSegChunks) return r;
  long want = (kTargetWorkgroups + walkers - 1) / walkers;
  want = min(want, nchunks / kMinSegChunks);
  if (want < 2) return r;
  const long per = (nchunks + want - 1) / want;  // chunks per segment
  r.seg_len = static_cast<int>(per * kCT);
  r.nseg = static_cast<int>((nchunks + per - 1) / per);
  return r;
}

size_t chunkwise_bwd_workspace_floats(int B, int H, int T, int dk, int dv) {
  const ChunkSegments sg = chunkwise_bwd_segments(B, H, T, dk, dv);
  if (sg.nseg <= 1) return 0;
  return static_cast<size_t>(3) * sg.nseg * B * H * dk * dv;  // dV, dK and dQ passes
}

hipError_t launch_chunkwise_bwd_mfma(const BwdArgs& a, int B, int H, int T, int dk, int dv, float* ws,
                                     const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  auto u = [](const void* x) { return static_cast<const uint16_t*>(x); };
  const ChunkSegments sg = chunkwise_bwd_segments(B, H, T, dk, dv);
  const long stride = static_cast<long>(B) * H * dk * dv;  // one slot
  float* wv = sg.nseg > 1 ? ws : nullptr;
  float* wk = sg.nseg > 1 ? ws + sg.nseg * stride : nullptr;
  float* wq = sg.nseg > 1 ? ws + 2 * sg.nseg * stride : nullptr;
  // dK (reverse over V, dY, Q from dS_out^T) and dQ (forward over dY, V, K from
  // S_in^T) share d_a = dv: one launch.  Unsegmented, they run as a pass pair
  // on the forward kernel (64-column tiles of Q and K) where it takes them.
  if (sg.nseg == 1 && T > 0 && chunkwise_mfma_pair_supports(dv, dk, g)) {
    const ChunkPass pk{a.v, a.dy, a.q, a.dstate_out, 1, 1, nullptr, a.dk};
    const ChunkPass pq{a.dy, a.v, a.k, a.state_in, 1, 0, nullptr, a.dq};
    const hipError_t e = launch_chunkwise_mfma_pair(pk, pq, B, H, T, dv, dk, g, s);
    if (e != hipSuccess) return e;
  } else {
    MPassSet kq{};
    kq.p[0] = MPass{u(a.v), u(a.dy), u(a.q), static_cast<uint16_t*>(a.dk), a.dstate_out, nullptr, 1, 1, dk, wk, stride};
    kq.p[1] = MPass{u(a.dy), u(a.v), u(a.k), static_cast<uint16_t*>(a.dq), a.state_in, nullptr, 1, 0, dk, wq, stride};
    kq.npass = 2;
    kq.nseg = sg.nseg;
    kq.seg_len = sg.seg_len;
    const hipError_t e = launch_by_da(dv, kq, B, hd, H, g, T, s);
    if (e != hipSuccess) return e;
  }
  // dV (reverse over K, Q, dY from dS_out); final state = dS_in.  After the dK
  // pass, so that dstate_in may be the dstate_out buffer.  It has the shape of
  // the forward pass (d_a = dk, 64-column tiles of dY), so where the forward
  // kernel's reverse mode takes it (and its segments fit the dV slots) it
  // runs there.
  const ChunkSegments sf = chunkwise_mfma_segments(B, H, T, dv, kRevChunk);
  if (chunkwise_mfma_rev_supports(dk, dv, g) && (sf.nseg == 1 || sf.nseg <= sg.nseg))
    return launch_chunkwise_mfma_rev(a.k, a.q, a.dy, a.dstate_out, a.dstate_in, a.dv, B, H, T, dk, dv, sf, wv, g, s);
  MPassSet vs{};
  vs.p[0] = MPass{u(a.k), u(a.q), u(a.dy), static_cast<uint16_t*>(a.dv), a.dstate_out, a.dstate_in, 0, 1, dv, wv,
                  stride};
  vs.p[1] = vs.p[0];
  vs.npass = 1;
  vs.nseg = sg.nseg;
  vs.seg_len = sg.seg_len;
  return launch_by_da(dk, vs, B, hd, H, g, T, s);
}

}  // namespace ret
