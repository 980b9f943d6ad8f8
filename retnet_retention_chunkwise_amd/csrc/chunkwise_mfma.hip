// Chunkwise retention on bf16 MFMA (gfx950, v_mfma_f32_16x16x32_bf16), fp32 state.
//
// Chunkwise form of "Retentive Networks — Microsoft Propone l'Alternativa
// Architetturale ai Transformer" (section "Il meccanismo: Multi-Scale
// Retention"): parallel inside chunks of C tokens, recurrent across chunks.
// For chunk i (rows j = 0..L-1, carried state R_i, decay gamma of the head):
//   Y_[i]   = ((Q_[i] K_[i]^T) .* D_L) V_[i] + diag(gamma^(j+1)) Q_[i] R_i
//   R_(i+1) = gamma^L R_i + K_[i]^T (diag(gamma^(L-1-j)) V_[i])
//
// Work decomposition.  A workgroup owns one (segment, batch, head, tile of 64
// value columns) and walks the chunks of its segment in order; the 8 column
// tiles of a head are placed on one XCD so that their shared Q/K reads hit
// one L2.  The workgroup has 8 waves in two roles, one of each per SIMD
// (waves w and w+4 share a SIMD):
//   * output waves 0..3 own 16-row query blocks ({w} for 64-token tiles,
//     {w, 7-w} for 128-token tiles, which balances the causal triangle), each
//     with a code path specialised at compile time.  Their Q rows are loaded
//     from global memory straight into MFMA operand registers.  One pass over
//     d_k computes the cross term O^T = R_i^T Q^T (R^T from LDS) and the
//     scores S^T = K Q^T of the key blocks up to the diagonal.  S^T stays in
//     registers: its accumulator layout is, up to a permutation of the key
//     index, the operand layout that P needs for P V, so P is formed in
//     registers and never touches LDS; V^T is read with the same key
//     permutation through ds_read_b64_tr_b16, the gfx950 transposing LDS load.
//     O^T is accumulated, so each lane holds 4 consecutive columns of one
//     query row for the Y stores.
//   * state waves 4..7 own d_k/4 rows of the fp32 state tile R[d_k x 64],
//     kept in MFMA accumulators for the whole segment.  They run the update
//     R <- gamma^L R + K^T (zeta V) (K^T and V through the transposing load),
//     publish R^T to LDS, and stage the K and V tiles of later chunks (global
//     loads into registers one or two chunks ahead, LDS writes after the
//     update).
// 64-token tiles keep two copies of K, V and R^T in LDS, so staging chunk i+1
// overlaps the outputs of chunk i and one barrier per chunk suffices;
// 128-token tiles with d_k = 256 keep one copy: [outputs | update] barrier
// [R^T and next K/V written] barrier.  The barriers fence LDS only.
// Every global access goes through a buffer resource that ends at the
// chunk's last valid row, so rows past the end read as zero / are dropped
// without branches.  Decay factors gamma^d come from log2(gamma) with
// gamma^0 forced to 1.
#include <type_traits>

#include "common.h"
#include "gfx950.h"
#include "kernels.h"

namespace ret {
namespace {

constexpr int kTN = 64;  // value columns per workgroup

template <int CT, int DK, bool kOut>
struct Cfg {
  static constexpr int kThreads = 512;         // 4 output waves + 4 state waves
  static constexpr int kStageThreads = 256;    // the state waves stage K/V
  static constexpr int KLD = DK + 8;           // K row stride in LDS (elements)
  static constexpr int VLD = kTN + 8;          // V row stride
  static constexpr int RLD = DK + 8;           // R^T row stride
  static constexpr int NQ = CT / 64;           // query blocks per output wave
  static constexpr int RM = DK / 64;           // 16-row state blocks per state wave
  static constexpr int KS = DK / 32;           // k-steps over d_k
  static constexpr int KPT = CT * DK / 8 / kStageThreads;   // 16-byte K pieces per staging thread
  static constexpr int VPT = CT * kTN / 8 / kStageThreads;  // 16-byte V pieces per staging thread
  // 64-token tiles fit two copies of K, V and R^T in LDS: the state waves then
  // stage chunk i+1 while the output waves work on chunk i (one barrier per
  // chunk).  128-token tiles keep one copy and two barriers per chunk.  The
  // state-only pass keeps one copy of K and V and no R^T (43 KB at d_k = 256
  // and 64-token tiles), so that several of its workgroups share a CU.
  static constexpr int NBUF = kOut && (2 * (CT * KLD + CT * VLD + kTN * RLD) * 2 <= 160 * 1024) ? 2 : 1;
  static_assert(NQ >= 1 && NQ <= 2 && RM >= 1, "unsupported tile");
  static_assert(KPT >= 1 && VPT >= 1, "tile too small for the staging split");
};

// Sequence segments (long sequences with few heads).  Segment s covers
// positions [s*seg_len, (s+1)*seg_len).  Each pass's ws holds nseg state slots
// of [B,H,dk,dv] fp32: the state-only pass writes the end state of segment s
// (started from zero) into slot s+1, the scan turns slot s into the incoming
// state of segment s, and the full pass starts segment s from slot s.
struct SegArgs {
  int seg_len;     // positions per segment (a multiple of C)
  int nseg;        // segments; 1 = whole sequence, ws unused
  int bnh;         // B * heads of this launch
  long ws_stride;  // elements per slot (B * H * dk * dv)
  int nsub;        // state-only launch: sub-segments per segment (0: none skipped)
};

// Pointers of one pass (the kernel takes one or two; see kDir).
struct PassPtrs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* state_in;  // nullable
  float* state_out;       // nullable
  uint16_t* y;
  int rev;         // reverse direction (kDir = 2)
  int state_in_t;  // state_in stored transposed, [dv x DK] per head (read by the scan when segmented)
  float* ws;       // segment slots (nseg > 1) or null
};

// Per-head GroupNorm fused into the output stores (kGN), the normalisation of
// multi-scale retention (paperhub page, author answer A4: GroupNorm, one group
// per head).  A head's dv outputs of a token are spread over its dv/64
// column-tile workgroups, so each output wave publishes, per token row of its
// query blocks, one 64-bit record: the mean and the sum of squared deviations
// of its tile's 64 rounded outputs.  Records sit at
// rec[segment][batch][head][tile][position in the segment], are filled with
// the all-ones sentinel before the launch (no arithmetic result has that bit
// pattern) and are valid once they differ from it.  A chunk's rounded outputs
// wait GD chunks (in registers or LDS) for the other tiles' records; the tiles
// then combine the records of a row (parallel-variance formula) and store the
// normalised outputs.  The un-normalised outputs never reach memory.
struct GnArgs {
  const float* weight;      // [H_total, dv] or null (ones)
  const float* bias;        // [H_total, dv] or null (zeros)
  float eps;
  unsigned long long* rec;  // records (see above)
  int* err;                 // set to 1 if a wait gave up (spin_limit)
  int B;
  int Htot;
  int spin_limit;
  int items;  // work items of the launch; the grid may be padded past them
  int silent_tile;  // failure-path testing: this column tile publishes no records (-1: none)
};
constexpr unsigned long long kGnEmpty = ~0ull;
constexpr int kGnDelay = 2;  // chunks a rounded output waits for the records

// Sub-segment j (of nsub, sub_len positions each) of a segment reaches every
// later state only through the factor gamma^d, d = (nsub - 1 - j) * sub_len,
// of the segment scan (later segments add further factors <= 1).  With
// gamma^d <= 2^-40 its end state, whose terms are already scaled by gamma^(positions
// to its own end), moves no later state by more than 2^-40 of its own size,
// far below the bf16 rounding of the operands and of y: the state-only pass
// does not walk it and the scan leaves it out.  Both kernels decide with this
// one function, so that they agree bit for bit.  Fast decays leave most of
// the pass (gamma = 1 - 2^-5 ... 1 - 2^-7: every sub-segment of 4096
// positions but the last); gamma = 0 makes every such contribution exactly
// zero (d > 0); d = 0 gives NaN for gamma = 0 and is walked.  The full pass
// still walks every position.
__device__ __forceinline__ bool sub_segment_negligible(float log2g, int nsub, int j, int sub_len) {
  const float d = static_cast<float>(static_cast<long>(nsub - 1 - j) * sub_len);
  return d * -log2g >= 40.0f;
}

// kOut = true: the full kernel (outputs and state, 4 + 4 waves).
// kOut = false: the state-only pass, end states from zero of the segments (or
// sub-segments) given by sg (4 state waves; at d_k <= 256 three of its
// workgroups share a CU).
// kZS = true: V is staged in LDS already scaled by zeta_t = gamma^(L-1-t), once
// per element, and serves both the state update and the outputs.  Since
// gamma^(j-t) V_t = gamma^(j+1) gamma^(-L) zeta_t V_t, the outputs are
//   O_j = gamma^(j+1) (Q R + ((Q K^T) .* causal mask) gamma^(-L) zeta V)_j,
// with one scalar gamma^(-L) per chunk.  zeta >= gamma^(CT-1) and
// gamma^(-L) <= gamma^(-CT) stay within about 2^+-102 when
// gamma^(CT-1) >= 2^-100 (the host checks this for every head of the launch).
// kZS = false keeps V unscaled and applies zeta to the update's operand in
// registers (any gamma in [0, 1]).
// Direction (kDir): 0 = forward in time.  1 = the same pass backwards in time
// with the decay weights shifted by one token, the shape of the gradient
// passes of the chunkwise form (chain rule on the recurrence of the aimpact
// page, "Il meccanismo"): position p counts from the end (token Tn-1-p), and
// for chunk rows j
//   Y_j = gamma^j Q_j R + sum_{t<=j} gamma^(j-t) (Q_j . K_t) V_t
//   R  <- gamma^L R + sum_t gamma^(L-t) K_t^T V_t
// i.e. zeta_t = gamma^(L-t) and gamma^j in place of gamma^(j+1); with
// (Q, K, V, R_0) = (K, Q, dY, dS_out) the outputs are dV and the final state
// is dS_in, with (V, dY, Q, dS_out^T) they are dK.  2 = per pass (PassPtrs::rev),
// for launches that run one or two passes of either direction (dQ forward,
// dK and dV reverse).

template <int CT, int DK, bool kOut, bool kZS, int kDir, bool kGN = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kOut ? 512 : 256, kOut ? 512 : 256),
                          amdgpu_waves_per_eu(kOut ? 2 : (DK <= 256 ? 3 : 1), kOut ? 2 : 4))) void
chunkwise_mfma_kernel(PassPtrs p0, PassPtrs p1, int npass, HeadDecay gam, int H, int h0, int nh, int Tn, int dv,
                      int C, int ntiles, SegArgs sg, GnArgs gn) {
  static_assert(!kGN || (kOut && kDir == 0), "the fused GroupNorm is a forward epilogue");
  using F = Cfg<CT, DK, kOut>;
  constexpr int NSP = CT / 32;  // key (token) steps of 32 per chunk tile
  constexpr int NB = F::NBUF;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NB][CT * F::KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NB][CT * F::VLD];
  __shared__ __attribute__((aligned(16))) uint16_t Rt[NB][kOut ? kTN * F::RLD : 8];
  // With one LDS copy there is room for zeta*V, formed once when V is staged;
  // with two copies zeta is applied to the update's V operand in registers.
  constexpr bool kVz = NB == 1 && !kZS;
  __shared__ __attribute__((aligned(16))) uint16_t Vz[kVz ? CT * F::VLD : 8];
  // Fused GroupNorm: the tile's 64 weights and biases, and with 128-token
  // tiles the rounded outputs waiting for the records (kGnHold chunks of 4
  // waves x 2 query blocks x 4 column blocks x 64 lanes x 8 bytes; two when
  // they fit the LDS beside the K, V and R^T tiles).
  constexpr int kLdsBase = 2 * (NB * CT * F::KLD + NB * CT * F::VLD + NB * kTN * F::RLD + (kVz ? CT * F::VLD : 0));
  constexpr bool kGnLds = kGN && F::NQ == 2;
  constexpr int kGnHold = !kGN ? 1 : !kGnLds ? kGnDelay : (kLdsBase + 2 * 16384 + 512 <= 160 * 1024 ? 2 : 1);
  __shared__ __attribute__((aligned(16))) float Gwb[kGN ? 2 * kTN : 4];
  __shared__ __attribute__((aligned(16))) u32x2 Gh[kGnLds ? kGnHold * 4 * 2 * 4 * 64 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar) by construction
  const int wr = kOut ? (w & 3) : w;                         // index within the role
  const int c16 = lane & 15;
  const int g = lane >> 4;

  // Workgroup -> (segment, batch, head, pass, column tile).  Consecutive
  // linear ids (the column tiles and passes of one head and segment, which
  // read the same rows) are placed on one XCD (dispatch is round-robin over
  // the 8 XCDs by workgroup id).
  const int total = gridDim.x;
  int lin = blockIdx.x;
  if ((total & 7) == 0) lin = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  if (kGN && lin >= gn.items) return;  // padding of a fused-GroupNorm grid (before any barrier)
  const int tile = lin % ntiles;
  const int pz = npass > 1 ? (lin / ntiles) % npass : 0;
  const int bh = (lin / ntiles / npass) % sg.bnh;
  const int seg = lin / ntiles / npass / sg.bnh;
  const PassPtrs P = pz ? p1 : p0;
  const bool rev = kDir == 2 ? P.rev != 0 : kDir == 1;
  const int shift = rev ? 1 : 0;  // decay exponent shift of the reverse direction
  const int hl = bh % nh;
  const int b = bh / nh;
  const long head = static_cast<long>(b) * H + h0 + hl;
  const int col0 = tile * kTN;
  const float lg = gam.log2g[hl];

  const uint16_t* qh = P.q + head * Tn * DK;
  const uint16_t* kh = P.k + head * Tn * DK;
  const uint16_t* vh = P.v + head * Tn * dv + col0;
  uint16_t* yh = P.y + head * Tn * dv + col0;
  const long sbase = head * static_cast<long>(DK) * dv + col0;
  const uint32_t vrow = static_cast<uint32_t>(dv) * 2u;  // bytes per V / Y row
  int t_begin = seg * sg.seg_len;
  const int t_end = min(Tn, t_begin + sg.seg_len);
  if constexpr (!kOut) {
    // State-only pass: position t of a walked sub-segment reaches the next
    // segment's state with weight gamma^e, e = d + (t_end - 1 - t) (d as in
    // sub_segment_negligible); positions with e * -log2(gamma) >= 40 are left
    // out as whole sub-segments are, by starting the walk at the chunk that
    // holds the first position with a larger weight.
    if (sg.nsub > 0 && lg < 0.0f) {
      const float emax = fmaxf(ceilf(40.0f / -lg) - 1.0f, 0.0f);  // largest e kept (e = 0 always)
      const float d = static_cast<float>(static_cast<long>(sg.nsub - 1 - seg % sg.nsub) * sg.seg_len);
      if (emax >= d && emax - d + 1.0f < static_cast<float>(t_end - t_begin)) {
        const int keep = static_cast<int>(emax - d) + 1;  // >= 1
        const int t0 = t_begin + (t_end - keep - t_begin) / C * C;
        if (t0 > t_begin) t_begin = t0;
      }
    }
  }
  const int nchunks = (t_end - t_begin + C - 1) / C;
  // Row addressing of the chunk at position s with L valid rows.  A buffer
  // resource starts at row first_row(s, L) and spans L rows; tile row r sits
  // at row_off(r) in it.  Forward: tokens s..s+L-1 in order.  Reverse: the
  // tokens Tn-s-L..Tn-s-1 read last to first; rows r >= L map past every
  // buffer's end (0x80000000 > any span), so they read as zero and their
  // stores are dropped, as rows past the span do in the forward direction.
  auto first_row = [&](int s, int L) __attribute__((always_inline)) {
    return rev ? max(0, Tn - s - L) : s;
  };
  auto row_off = [&](int r, int L, uint32_t row_bytes) __attribute__((always_inline)) -> uint32_t {
    if (rev) return r < L ? static_cast<uint32_t>(L - 1 - r) * row_bytes : 0x80000000u;
    return static_cast<uint32_t>(r) * row_bytes;
  };

  // fp32 state tile in and out.  init: state_in (one segment), the scanned
  // slot of this segment, or zero (state-only pass); fin: state_out (last
  // segment) or, in the state-only pass, the slot of the next segment.  The
  // [d_k x 64] tile moves through LDS (the K buffers, before the first chunk is
  // staged and after the last one is read), so that global accesses are whole
  // 256-byte rows; SRN rounds of SRR rows, two barriers per round in every wave.
  const float* init = !kOut ? nullptr : (sg.nseg > 1 ? P.ws + seg * sg.ws_stride : P.state_in);
  const bool init_t = sg.nseg == 1 && P.state_in_t != 0;  // init is stored transposed
  float* fin = kOut ? (seg == sg.nseg - 1 ? P.state_out : nullptr) : P.ws + (seg + 1) * sg.ws_stride;
  constexpr int SLD = kTN + 4;                 // fp32 row stride in LDS
  constexpr int kKBytes = NB * CT * F::KLD * 2;  // bytes of the K buffers
  constexpr int SRR = (DK >= 128 && 128 * SLD * 4 <= kKBytes) ? 128
                      : (DK >= 64 && 64 * SLD * 4 <= kKBytes) ? 64
                      : (32 * SLD * 4 <= kKBytes ? 32 : 16);  // rows per round
  constexpr int SRN = DK / SRR;                // rounds
  static_assert(SRR * SLD * 4 <= NB * CT * F::KLD * 2, "state staging does not fit the K buffers");
  float* const Sst = reinterpret_cast<float*>(&Ks[0][0]);

  if constexpr (!kOut) {
    // a negligible sub-segment (see sub_segment_negligible): nothing to walk,
    // its slot is neither written here nor read by the scan
    if (sg.nsub > 0 && sub_segment_negligible(lg, sg.nsub, seg % sg.nsub, sg.seg_len)) return;
  }
  if (!kOut || w >= 4) {
    // =========================== state waves ===========================
    const int st = kOut ? tid - 256 : tid;  // staging thread index 0..255
    const int dbase = wr * (DK / 4);
    f32x4 Racc[F::RM][4];
#pragma unroll
    for (int mb = 0; mb < F::RM; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) Racc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (init != nullptr) {
      for (int rr = 0; rr < SRN; ++rr) {
        const int r0 = rr * SRR;
        if (init_t) {
          // element (row a, column x) of the head's state at x * DK + a: 16-byte
          // reads along a, transposed into the LDS rows
          const float* src = init + head * static_cast<long>(DK) * dv;
#pragma unroll
          for (int p = 0; p < SRR / 16; ++p) {
            const int idx = 256 * p + st;
            const int x = idx / (SRR / 4), a4 = idx % (SRR / 4);
            const u32x4 val = *reinterpret_cast<const u32x4*>(&src[static_cast<long>(col0 + x) * DK + r0 + 4 * a4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) Sst[(4 * a4 + e) * SLD + x] = __uint_as_float(val[e]);
          }
        } else {
          // 16 lanes per 256-byte row, 16 rows per pass of the 256 staging threads
#pragma unroll
          for (int p = 0; p < SRR / 16; ++p) {
            const int row = 16 * p + (st >> 4);
            *reinterpret_cast<u32x4*>(&Sst[row * SLD + 4 * (st & 15)]) =
                *reinterpret_cast<const u32x4*>(&init[sbase + static_cast<long>(r0 + row) * dv + 4 * (st & 15)]);
          }
        }
        lds_barrier();
#pragma unroll
        for (int mb = 0; mb < F::RM; ++mb) {
          const int d0 = dbase + 16 * mb;  // wave-uniform: the block lies in one round
          if (d0 < r0 || d0 >= r0 + SRR) continue;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Racc[mb][nb][i] = Sst[(d0 - r0 + 4 * g + i) * SLD + 16 * nb + c16];
        }
        lds_barrier();
      }
    }
    auto write_rt = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int mb = 0; mb < F::RM; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const bf16x4 r = __builtin_convertvector(Racc[mb][nb], bf16x4);
          *reinterpret_cast<bf16x4*>(&Rt[buf][(16 * nb + c16) * F::RLD + dbase + 16 * mb + 4 * g]) = r;
        }
    };
    // Staging map (16-byte pieces; round r adds r * rows-per-round rows).
    // Rows of 16 or more pieces (d_k >= 128): each 16-lane group moves 256
    // contiguous bytes of one row.  Rows of 8 pieces (d_k = 64, and V): a
    // 16-lane group moves rows x and x+8, which the 144-byte LDS stride places
    // 32 banks apart.  Either way a group's LDS writes hit 64 distinct banks.
    constexpr int KPR = DK / 8;       // pieces per K row
    constexpr int KRR = 256 / KPR;    // K rows per round
    const int prow = (st >> 4 & 7) + 16 * (st >> 7) + 8 * (st >> 3 & 1);  // paired-row map, 32 rows per round
    const int krow = KPR == 8 ? prow : st / KPR;
    const int kc8 = KPR == 8 ? (st & 7) : st % KPR;
    const int vc8 = st & 7;
    // K/V staging registers.  With two LDS copies and zeta-staged V (whose
    // update needs fewer registers) there are two register sets: chunk c+1
    // waits in set c%2 and is loaded two chunks before it is written to LDS,
    // which covers the latency of cold HBM reads.  Otherwise one set holds
    // the chunk after next.
    constexpr int NKV = (NB == 2 && kZS) ? 2 : 1;
    u32x4 kreg[NKV][F::KPT];
    u32x4 vreg[NKV][F::VPT];
    const uint32_t koff = static_cast<uint32_t>(krow * DK + 8 * kc8) * 2u;  // + r * KRR rows
    const uint32_t voff = static_cast<uint32_t>(prow) * vrow + 16u * vc8;   // + r * 32 rows
    // the register set is a compile-time constant (std::integral_constant), so
    // the arrays are indexed statically whether or not the lambdas are inlined
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto load_kv = [&](auto set_c, int s1, int Ln) __attribute__((always_inline)) {
      constexpr int set = decltype(set_c)::value;
      const int r0 = first_row(s1, Ln);
      const rsrc_t rk = make_rsrc(kh + static_cast<long>(r0) * DK, static_cast<uint32_t>(Ln) * DK * 2u);
#pragma unroll
      for (int r = 0; r < F::KPT; ++r)
        kreg[set][r] = buffer_load16(rk, rev ? row_off(krow + r * KRR, Ln, DK * 2u) + 16u * kc8
                                             : koff + static_cast<uint32_t>(r * KRR * DK * 2));
      const rsrc_t rv = make_rsrc(vh + static_cast<long>(r0) * dv,
                                  Ln > 0 ? static_cast<uint32_t>(Ln - 1) * vrow + kTN * 2u : 0u);
#pragma unroll
      for (int r = 0; r < F::VPT; ++r)
        vreg[set][r] = buffer_load16(rv, rev ? row_off(prow + 32 * r, Ln, vrow) + 16u * vc8 : voff + 32u * vrow * r);
    };
    // Ln: length of the chunk being staged (zeta of its rows when kZS)
    auto store_kv = [&](auto set_c, int buf, int Ln) __attribute__((always_inline)) {
      constexpr int set = decltype(set_c)::value;
#pragma unroll
      for (int r = 0; r < F::KPT; ++r)
        *reinterpret_cast<u32x4*>(&Ks[buf][(krow + r * KRR) * F::KLD + 8 * kc8]) = kreg[set][r];
#pragma unroll
      for (int r = 0; r < F::VPT; ++r) {
        const int row = prow + 32 * r;
        if constexpr (kZS) {
          const float z = row < Ln ? gamma_pow(lg, Ln - 1 - row + shift) : 0.0f;
          const f32x8 vf = __builtin_convertvector(__builtin_bit_cast(bf16x8, vreg[set][r]), f32x8) * z;
          *reinterpret_cast<bf16x8*>(&Vs[buf][row * F::VLD + 8 * vc8]) = __builtin_convertvector(vf, bf16x8);
        } else {
          *reinterpret_cast<u32x4*>(&Vs[buf][row * F::VLD + 8 * vc8]) = vreg[set][r];
        }
      }
    };
    // zeta*V for the one-copy layout: zeta_row = gamma^(L-1-row), 0 past the chunk end
    auto store_vz = [&](int Ln) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < F::VPT; ++r) {
        const int row = prow + 32 * r;
        const float z = row < Ln ? gamma_pow(lg, Ln - 1 - row + shift) : 0.0f;
        const f32x8 vf = __builtin_convertvector(__builtin_bit_cast(bf16x8, vreg[0][r]), f32x8) * z;
        *reinterpret_cast<bf16x8*>(&Vz[row * F::VLD + 8 * vc8]) = __builtin_convertvector(vf, bf16x8);
      }
    };
    // zeta_t = gamma^(L-1-t) (gamma^(L-t) in reverse) for the tokens
    // t = 32s + 8g + 2(e%4) + e/4 this lane holds in the update's B operand;
    // for chunks that fill the tile (L = CT), zeta = zbase[s] * zc[e] with
    // zbase[s] = gamma^(CT-8-32s-8g (+1)) and zc[e] = gamma^(7-2(e%4)-e/4)
    // (both exponents >= 0).
    float zbase[NSP], zc[8];
#pragma unroll
    for (int s = 0; s < NSP; ++s) zbase[s] = gamma_pow(lg, CT - 8 - 32 * s - 8 * g + shift);
#pragma unroll
    for (int e = 0; e < 8; ++e) zc[e] = gamma_pow(lg, 7 - 2 * (e & 3) - (e >> 2));

    // R <- gamma^L R + K^T (zeta V) on LDS buffer `buf`.  The token contraction
    // uses k-slot e of lane group g <-> token 32s + 8g + 2(e%4) + e/4 for both
    // operands: each transposing read then touches rows {0,2,..,14} or
    // {1,3,..,15} (+16), which the padded row strides place in disjoint banks.
    auto update = [&](int buf, int L) __attribute__((always_inline)) {
      const float gL = L == C ? gamma_pow(lg, C) : gamma_pow(lg, L);
#pragma unroll
      for (int mb = 0; mb < F::RM; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) Racc[mb][nb] *= gL;
      // With two LDS copies (64-token tiles) the operands of step s+1 are read
      // before the MFMAs of step s; 128-token tiles hold the K/V staging
      // registers of a full tile and read each step just before use.
      constexpr int PB = NB == 2 ? 2 : 1;
      bf16x8 zb[PB][4], ka[PB][F::RM];
      auto read_step = [&](int s, int slot) __attribute__((always_inline)) {
        const uint16_t* vsrc = kVz ? Vz : Vs[buf];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = 16 * nb + 4 * (c16 & 3);
          const s16x4 lo = lds_read_tr(&vsrc[(32 * s + 8 * g + 2 * (c16 >> 2)) * F::VLD + col]);
          const s16x4 hi = lds_read_tr(&vsrc[(32 * s + 8 * g + 2 * (c16 >> 2) + 1) * F::VLD + col]);
          zb[slot][nb] = join(lo, hi);
        }
#pragma unroll
        for (int mb = 0; mb < F::RM; ++mb) {
          const int col = dbase + 16 * mb + 4 * (c16 & 3);
          const s16x4 lo = lds_read_tr(&Ks[buf][(32 * s + 8 * g + 2 * (c16 >> 2)) * F::KLD + col]);
          const s16x4 hi = lds_read_tr(&Ks[buf][(32 * s + 8 * g + 2 * (c16 >> 2) + 1) * F::KLD + col]);
          ka[slot][mb] = join(lo, hi);
        }
      };
      if constexpr (PB == 2) read_step(0, 0);
#pragma unroll
      for (int s = 0; s < NSP; ++s) {
        if (32 * s >= L) break;
        const int slot = PB == 2 ? (s & 1) : 0;
        if constexpr (PB == 2) {
          if (s + 1 < NSP && 32 * (s + 1) < L) read_step(s + 1, (s + 1) & 1);
        } else {
          read_step(s, 0);
        }
        // zeta-scale the V operand of step s (in place)
        if constexpr (!kVz && !kZS) {
        float z[8];
        if (L == CT) {  // a full tile: every token group lies inside the chunk
#pragma unroll
          for (int e = 0; e < 8; ++e) z[e] = zbase[s] * zc[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = 32 * s + 8 * g + 2 * (e & 3) + (e >> 2);
            z[e] = t < L ? gamma_pow(lg, L - 1 - t + shift) : 0.0f;
          }
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          f32x8 vf = __builtin_convertvector(zb[slot][nb], f32x8);
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[e] *= z[e];
          zb[slot][nb] = __builtin_convertvector(vf, bf16x8);
        }
        }
#pragma unroll
        for (int mb = 0; mb < F::RM; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) Racc[mb][nb] = mfma(ka[slot][mb], zb[slot][nb], Racc[mb][nb]);
      }
    };

    // length of the chunk starting at token s (0 past the segment end); loads
    // of such empty chunks are issued anyway (they read zeros) so that the
    // wait counts stay exact
    auto clen = [&](int s) __attribute__((always_inline)) { return s < t_end ? min(C, t_end - s) : 0; };
    {
      const int L0 = clen(t_begin);
      load_kv(I0(), t_begin, L0);
      if constexpr (kOut) write_rt(0);
      store_kv(I0(), 0, L0);
      if constexpr (kVz) store_vz(L0);
      if constexpr (NB == 2) load_kv(I0(), t_begin + C, clen(t_begin + C));            // chunk 1 into set 0
      if constexpr (NKV == 2) load_kv(I1(), t_begin + 2 * C, clen(t_begin + 2 * C));  // chunk 2 into set 1
    }
    lds_barrier();  // chunk 0 staged, R_0 published

    // one chunk with two LDS copies: chunk ci+1 waits in register set SET
    // (ci%2 with two sets)
    auto iter2 = [&](int ci, auto set_c) __attribute__((always_inline)) {
      using SET = std::integral_constant<int, NKV == 2 ? decltype(set_c)::value : 0>;
      const int s0 = t_begin + ci * C;
      const int L = min(C, t_end - s0);
      const int Ln = clen(s0 + C);
      const int X = ci & 1;
      update(X, L);
      if constexpr (kOut) write_rt(X ^ 1);      // R_(i+1) into the other copy
      if (Ln > 0) store_kv(SET(), X ^ 1, Ln);   // chunk i+1
      const int sn = s0 + (NKV + 1) * C;        // chunk i+3 (two sets) or i+2 into the freed set
      load_kv(SET(), sn, clen(sn));
      lds_barrier();
    };
    if constexpr (NB == 2) {
      for (int ci = 0; ci < nchunks; ci += 2) {
        iter2(ci, I0());
        if (ci + 1 < nchunks) iter2(ci + 1, I1());
      }
    } else {
      for (int ci = 0; ci < nchunks; ++ci) {
        const int s0 = t_begin + ci * C;
        const int L = min(C, t_end - s0);
        const int s1 = s0 + C;
        const int Ln = clen(s1);
        // next chunk's K/V, written after the barrier (d_k = 512: issued after
        // the update, whose state and operand registers leave no room for them)
        if constexpr (DK <= 256) load_kv(I0(), s1, Ln);
        update(0, L);
        if constexpr (DK > 256) load_kv(I0(), s1, Ln);
        lds_barrier();  // output waves are done with R^T, K and V of this chunk
        if constexpr (kOut) write_rt(0);
        if (Ln > 0) {
          store_kv(I0(), 0, Ln);
          if constexpr (kVz) store_vz(Ln);
        }
        lds_barrier();  // R_(i+1) and the next chunk's K/V are in LDS
      }
    }

    // final state (all K reads ended with the last chunk's barrier)
    if (fin != nullptr) {
      for (int rr = 0; rr < SRN; ++rr) {
        const int r0 = rr * SRR;
#pragma unroll
        for (int mb = 0; mb < F::RM; ++mb) {
          const int d0 = dbase + 16 * mb;
          if (d0 < r0 || d0 >= r0 + SRR) continue;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sst[(d0 - r0 + 4 * g + i) * SLD + 16 * nb + c16] = Racc[mb][nb][i];
        }
        lds_barrier();
#pragma unroll
        for (int p = 0; p < SRR / 16; ++p) {
          const int row = 16 * p + (st >> 4);
          *reinterpret_cast<u32x4*>(&fin[sbase + static_cast<long>(r0 + row) * dv + 4 * (st & 15)]) =
              *reinterpret_cast<const u32x4*>(&Sst[row * SLD + 4 * (st & 15)]);
        }
        lds_barrier();
      }
    }
  } else if constexpr (kOut) {
    // =========================== output waves ===========================
    // (the state tile's staging rounds: the same barriers as the state waves)
    if (init != nullptr)
      for (int rr = 0; rr < 2 * SRN; ++rr) lds_barrier();
    // One code path per output wave: its query blocks ({W} for 64-token tiles,
    // {W, 7-W} for 128-token tiles, which balances the causal triangle) are
    // compile-time constants, so the causal block structure needs no branches.
    auto out_role = [&](auto w_c) __attribute__((always_inline)) {
    constexpr int W = decltype(w_c)::value;
    constexpr int QB1 = F::NQ == 2 ? 7 - W : W;
    constexpr int QMAX = QB1 > W ? QB1 : W;  // last query block of the wave
    // Decay factors (positions are chunk-relative, so these do not depend on
    // the chunk).  Off-diagonal key block kb < qb:
    //   gamma^(j-t) = gamma^(16(qb-kb) + c16 - 4g - 3) * cst[t % 4],  cst[e] = gamma^(3-e)
    // (both exponents >= 0: no overflow for any gamma in [0,1]); diagonal key
    // block: Ddg[e] = gamma^(c16 - 4g - e) on or below the diagonal, else 0.
    float cst[4], Ddg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cst[e] = gamma_pow(lg, 3 - e);
      const int d = c16 - 4 * g - e;
      Ddg[e] = d >= 0 ? gamma_pow(lg, d) : 0.0f;
    }
    const int lane_off = c16 - 4 * g - 3;
    // Q operand registers.  With one query block per wave there is room for
    // two copies: the next chunk's Q is loaded at the start of a chunk, a
    // whole chunk ahead of its use; otherwise it is loaded after the d_k pass.
    constexpr bool kQ2 = F::NQ == 1 && DK <= 256;
    typedef bf16x8 QTile[F::NQ][F::KS];
    QTile Qa, Qb;
    auto load_q = [&](QTile& Qd, int s1, int Ln) __attribute__((always_inline)) {
      const rsrc_t rq = make_rsrc(qh + static_cast<long>(first_row(s1, Ln)) * DK, static_cast<uint32_t>(Ln) * DK * 2u);
#pragma unroll
      for (int qi = 0; qi < F::NQ; ++qi) {
        const uint32_t rowoff = row_off(16 * (qi == 0 ? W : QB1) + c16, Ln, DK * 2u) + 16u * g;
#pragma unroll
        for (int s = 0; s < F::KS; ++s) Qd[qi][s] = __builtin_bit_cast(bf16x8, buffer_load16(rq, rowoff + 64u * s));
      }
    };

    // ---- fused GroupNorm (kGN) ----
    // Lane (g, c16) holds row c16 of each query block; it reads the records of
    // tiles g and g+4 for those rows.  The records of chunk ci - GD are loaded
    // at the start of chunk ci, before the chunk's Q prefetch, so that waiting
    // for them at its end does not wait for that prefetch; no load or store of
    // this path sits in a branch of the common case (rows past the chunk,
    // tiles past ntiles and chunks before the first get an offset past the
    // buffer: reads give 0, writes are dropped), so the compiler's wait counts
    // stay exact.  Records are written with device-scope stores.  The first
    // read of a record is a workgroup-scope load: the tiles of a head share an
    // XCD (the host pads the grid to a multiple of 8 tiles per head and
    // workgroups go round-robin over the 8 XCDs), so it is served by the L2
    // the store passed through.  A record seen as the sentinel (read before
    // its store, or from a stale line) is read again with device-scope loads
    // until it is valid or spin_limit polls have passed.
    constexpr int GQ = kGN ? F::NQ : 1;
    constexpr int GD = kGnHold;
    // 128-token tiles with two LDS hold slots normalise chunk ci - 2 inside
    // the d_k pass of chunk ci (its records were loaded at the end of chunk
    // ci - 1), where the normalisation's VALU work overlaps the pass's MFMAs;
    // otherwise chunk ci - GD is normalised at the end of chunk ci.
    constexpr bool kGnLate = kGnLds && GD == 2;
    static_assert(!kGN || kGnLds || GD == 2, "register holds alternate two slots");
    typedef u32x2 Held[GQ][4];
    Held held[kGN && !kGnLds ? GD : 1];
    unsigned long long grec[GQ][2];
    // after a wave has given up once, its later waits poll once only: a head
    // whose tiles cannot all be resident then fails fast (error word set)
    // instead of waiting out the spin limit at every chunk
    int spin_limit = gn.spin_limit;
    constexpr uint32_t kOutside = 0x80000000u;
    rsrc_t rrs = make_rsrc(nullptr, 0u);
    if constexpr (kGN) {
#pragma unroll
      for (int d = 0; d < (kGnLds ? 1 : GD); ++d)
#pragma unroll
        for (int qi = 0; qi < GQ; ++qi)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) held[d][qi][nb] = u32x2{0u, 0u};
      const long item = (static_cast<long>(seg) * gn.B + b) * gn.Htot + h0 + hl;
      rrs = make_rsrc(gn.rec + item * ntiles * static_cast<long>(sg.seg_len),
                      static_cast<uint32_t>(ntiles) * static_cast<uint32_t>(sg.seg_len) * 8u);
      if constexpr (W == 0) {
        // the tile's weights and biases (null: ones and zeros)
        const long hoff = static_cast<long>(h0 + hl) * dv + col0;
        Gwb[lane] = gn.weight != nullptr ? gn.weight[hoff + lane] : 1.0f;
        Gwb[kTN + lane] = gn.bias != nullptr ? gn.bias[hoff + lane] : 0.0f;
      }
    }
    auto row_of = [&](int qi) __attribute__((always_inline)) { return 16 * (qi == 0 ? W : QB1) + c16; };
    auto chunk_len = [&](int cj) __attribute__((always_inline)) {
      return cj >= 0 ? min(C, t_end - (t_begin + cj * C)) : 0;
    };
    auto rec_off = [&](int t, int cj, int qi) __attribute__((always_inline)) -> uint32_t {
      return row_of(qi) < chunk_len(cj) && t < ntiles
                 ? static_cast<uint32_t>(t * sg.seg_len + cj * C + row_of(qi)) * 8u
                 : kOutside;
    };
    using kFirst = std::integral_constant<bool, true>;
    using kRetry = std::integral_constant<bool, false>;
    auto gn_load = [&](int cj, auto first_c) __attribute__((always_inline)) {
      constexpr int aux = decltype(first_c)::value ? 1 : 16;  // sc0 : sc1
#pragma unroll
      for (int qi = 0; qi < GQ; ++qi)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          grec[qi][i] = __builtin_bit_cast(unsigned long long,
                                           __builtin_amdgcn_raw_buffer_load_b64(rrs, rec_off(g + 4 * i, cj, qi), 0, aux));
    };
    auto gn_valid = [&]() __attribute__((always_inline)) {
      bool ok = true;
#pragma unroll
      for (int qi = 0; qi < GQ; ++qi)
#pragma unroll
        for (int i = 0; i < 2; ++i) ok = ok && grec[qi][i] != kGnEmpty;
      return __all(ok) != 0;
    };
    // combine the records of chunk cj, normalise its held outputs and store them
    auto gn_finish = [&](int cj, auto hold) __attribute__((always_inline)) {
      if (__builtin_expect(!gn_valid(), 0)) {
        int spin = 0;
        bool ok;
        do {
          __builtin_amdgcn_s_sleep(2);
          gn_load(cj, kRetry());
          ok = gn_valid();
        } while (!ok && ++spin < spin_limit);
        // the error word (device scope), written by lane 0 of a wave that gave up
        if (!ok) {
          __builtin_amdgcn_raw_buffer_store_b32(1, make_rsrc(gn.err, 4u), lane == 0 ? 0u : kOutside, 0, 16);
          spin_limit = 1;
        }
      }
      const int L = chunk_len(cj);
      const rsrc_t ry = make_rsrc(yh + static_cast<long>(L > 0 ? first_row(t_begin + cj * C, L) : 0) * dv,
                                  L > 0 ? static_cast<uint32_t>(L - 1) * vrow + kTN * 2u : 0u);
      const float inv_t = 1.0f / static_cast<float>(ntiles);
      const float inv_n = 1.0f / static_cast<float>(dv);
#pragma unroll
      for (int qi = 0; qi < GQ; ++qi) {
        float m[2], q[2];
        bool in[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          in[i] = g + 4 * i < ntiles;
          m[i] = __uint_as_float(static_cast<uint32_t>(grec[qi][i]));
          q[i] = __uint_as_float(static_cast<uint32_t>(grec[qi][i] >> 32));
        }
        // mean of the tile means (every tile holds 64 columns), then the sum
        // of squared deviations: sum_t (M2_t + 64 (mean_t - mean)^2)
        float ms = (in[0] ? m[0] : 0.0f) + (in[1] ? m[1] : 0.0f);
        ms = row4_sum(ms);
        const float mean = ms * inv_t;
        float qs = 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float d = m[i] - mean;
          qs += in[i] ? fmaf(static_cast<float>(kTN) * d, d, q[i]) : 0.0f;
        }
        qs = row4_sum(qs);
        const float rstd = 1.0f / sqrtf(qs * inv_n + gn.eps);
        const uint32_t roff = row_off(row_of(qi), L, vrow) + 8u * g;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const f32x4 x = __builtin_convertvector(__builtin_bit_cast(bf16x4, hold(qi, nb)), f32x4);
          const f32x4 wv = *reinterpret_cast<const f32x4*>(&Gwb[16 * nb + 4 * g]);
          const f32x4 bv = *reinterpret_cast<const f32x4*>(&Gwb[kTN + 16 * nb + 4 * g]);
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = fmaf((x[e] - mean) * rstd, wv[e], bv[e]);
          buffer_store8(ry, roff + 32u * nb, __builtin_bit_cast(u32x2, __builtin_convertvector(o, bf16x4)));
        }
      }
    };
    // LDS hold slot of chunk cj (128-token tiles), this lane's entry
    auto gh_at = [&](int cj, int qi, int nb) __attribute__((always_inline)) -> u32x2& {
      return Gh[(((cj % GD) * 4 + W) * 2 * 4 + qi * 4 + nb) * 64 + lane];
    };

    load_q(Qa, t_begin, min(C, t_end - t_begin));
    lds_barrier();  // chunk 0 staged, R_0 published

    // one chunk with Q in Qreg; Qnext receives the next chunk's Q (kQ2);
    // slot_c: register hold slot of the chunk (fused GroupNorm)
    auto chunk = [&](int ci, QTile& Qreg, QTile& Qnext, auto slot_c) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
      const int s0 = t_begin + ci * C;
      const int L = min(C, t_end - s0);
      const int s1 = s0 + C;
      const int Ln = s1 < t_end ? min(C, t_end - s1) : 0;
      const int X = NB == 2 ? (ci & 1) : 0;
      const uint16_t* Kx = Ks[X];
      const uint16_t* Vx = Vs[X];
      const uint16_t* Rx = Rt[X];
      if constexpr (kGN && !kGnLate) gn_load(ci - GD, kFirst());
      if constexpr (kQ2) load_q(Qnext, s1, Ln);

      // cross-chunk term O^T = (R_i^T Q^T) diag(gamma^(j+1)); V^T P^T
      // accumulates on top.  O^T[16nb + 4g + i][query c16] sits in lane
      // (g, c16): four consecutive value columns of one query row.
      f32x4 O[F::NQ][4];
      // The cross term and the scores share one pass over d_k: each step's Q
      // operand feeds the cross-term products (4 per query block) and the
      // score products of the key blocks up to the diagonal; the LDS reads
      // of a step are issued one step ahead.
      f32x4 St[F::NQ][NSP][2];
      // V^T operands of key step sp (keys 32sp+4g+e and 32sp+16+4g+e), in
      // the key order of the S^T accumulators
      auto read_v = [&](int sp, bf16x8 (&vb)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = 16 * nb + 4 * (c16 & 3);
          const s16x4 lo = lds_read_tr(&Vx[(32 * sp + 4 * g + (c16 >> 2)) * F::VLD + col]);
          const s16x4 hi = lds_read_tr(&Vx[(32 * sp + 16 + 4 * g + (c16 >> 2)) * F::VLD + col]);
          vb[nb] = join(lo, hi);
        }
      };
      // 64-token tiles: the V operands are read before the d_k pass, so that
      // they arrive while it runs (128-token tiles read them per key step)
      constexpr bool kVpre = F::NQ == 1;
      bf16x8 vpre[kVpre ? NSP : 1][4];
      if constexpr (kVpre) {
#pragma unroll
        for (int sp = 0; sp < NSP; ++sp)
          if (2 * sp <= W) read_v(sp, vpre[sp]);
      }
      {
        // key blocks 0..QMAX are read once per step and serve both query blocks
        constexpr int KB = QMAX + 1;
        bf16x8 rb[2][4], kk[2][KB];
        auto rd = [&](int s, int slot) __attribute__((always_inline)) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) rb[slot][nb] = lds_read16(&Rx[(16 * nb + c16) * F::RLD + 32 * s + 8 * g]);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) kk[slot][kb] = lds_read16(&Kx[(16 * kb + c16) * F::KLD + 32 * s + 8 * g]);
        };
        rd(0, 0);
#pragma unroll
        for (int s = 0; s < F::KS; ++s) {
          if constexpr (kGnLate) {
            // after the first step (later steps keep more registers live and
            // spill; measured 354 against 367 us per layer6p7b call at the
            // first step, 434 us with spills halfway); chunk ci - 2 holds the
            // slot of chunk ci
            if (s == 1) gn_finish(ci - 2, [&](int qi, int nb) { return gh_at(ci, qi, nb); });
          }
          if (s + 1 < F::KS) rd(s + 1, (s + 1) & 1);
          const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int qi = 0; qi < F::NQ; ++qi)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) O[qi][nb] = mfma(rb[s & 1][nb], Qreg[qi][s], s == 0 ? z4 : O[qi][nb]);
#pragma unroll
          for (int qi = 0; qi < F::NQ; ++qi)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              if (kb <= (qi == 0 ? W : QB1))
                St[qi][kb / 2][kb % 2] = mfma(kk[s & 1][kb], Qreg[qi][s], s == 0 ? z4 : St[qi][kb / 2][kb % 2]);
        }
      }
      // gamma^(j+1) of this lane's query rows j.  Without kZS it scales the
      // cross term here; with kZS it is factored out of both terms,
      //   O = gamma^(j+1) (Q R + (S .* mask) gamma^(-L) zeta V),
      // and applied when O is converted for the store, so the cross-term and
      // P V products accumulate without a pass over O in between.
      float xi[F::NQ];
#pragma unroll
      for (int qi = 0; qi < F::NQ; ++qi) {
        xi[qi] = gamma_pow(lg, 16 * (qi == 0 ? W : QB1) + c16 + 1 - shift);
        if constexpr (!kZS) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) O[qi][nb] *= xi[qi];
        }
      }
      const float ginvL = kZS ? exp2f(-static_cast<float>(L) * lg) : 1.0f;  // gamma^(-L)

      // intra-chunk term: P V per key step of 32 keys on or below the diagonal
      auto pv = [&](int sp) __attribute__((always_inline)) {
        const int slot = sp;
        bf16x8 vb[4];
        if constexpr (kVpre) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) vb[nb] = vpre[sp][nb];
        } else {
          read_v(sp, vb);
        }
#pragma unroll
        for (int qi = 0; qi < F::NQ; ++qi) {
          if ((qi == 0 ? W : QB1) < 2 * sp) continue;
          f32x8 p;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int m = (qi == 0 ? W : QB1) - (2 * sp + h);  // wave-uniform
            if constexpr (kZS) {
              // P'' = (S .* causal mask) gamma^(-L)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                p[4 * h + e] = (m > 0 || (m == 0 && 4 * g + e <= c16)) ? St[qi][slot][h][e] * ginvL : 0.0f;
            } else {
              const float boff = m > 0 ? exp2f(static_cast<float>(16 * m + lane_off) * lg) : 0.0f;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float f;
                if (m > 0) f = boff * cst[e];
                else if (m == 0) f = Ddg[e];
                else f = 0.0f;
                p[4 * h + e] = m >= 0 ? St[qi][slot][h][e] * f : 0.0f;
              }
            }
          }
          const bf16x8 pa = __builtin_convertvector(p, bf16x8);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) O[qi][nb] = mfma(vb[nb], pa, O[qi][nb]);
        }
      };
      if constexpr (!kQ2) load_q(Qreg, s1, Ln);  // the Q operand registers are free now
#pragma unroll
      for (int sp = 0; sp < NSP; ++sp)
        if (2 * sp <= QMAX) pv(sp);
      if constexpr (NB == 1) lds_barrier();  // this chunk's K, V and R^T are no longer read
      if constexpr (kGN) {
        // round to the output dtype; this tile's record of each of the lane's
        // rows: mean and sum of squared deviations over the tile's 64 columns
        Held hn;
        float gm[GQ], gq[GQ];
#pragma unroll
        for (int qi = 0; qi < GQ; ++qi) {
          float x[16];
          float sm = 0.0f;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const bf16x4 o = __builtin_convertvector(kZS ? O[qi][nb] * xi[qi] : O[qi][nb], bf16x4);
            hn[qi][nb] = __builtin_bit_cast(u32x2, o);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[4 * nb + e] = static_cast<float>(o[e]);
              sm += x[4 * nb + e];
            }
          }
          sm = row4_sum(sm);
          const float mt = sm * (1.0f / kTN);
          float q2 = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float d = x[j] - mt;
            q2 = fmaf(d, d, q2);
          }
          q2 = row4_sum(q2);
          gm[qi] = mt;
          gq[qi] = q2;
        }
        if constexpr (kGnLate) {
          // the records of chunk ci - 1, for its normalisation in chunk ci + 1
          // (loaded before this chunk's record stores, so that waiting for
          // them does not wait for those stores)
          gn_load(ci - 1, kFirst());
        }
        // publish (lane group 0) with a device-scope store, which passes the
        // XCD's L2 on its way to memory.  (A plain store beside it, meant to
        // keep the line in L2 for the first reads, measured slower: 138 us
        // against 102 us per layer1p3b call with inputs read from HBM.)
#pragma unroll
        for (int qi = 0; qi < GQ; ++qi) {
          const u32x2 r = {__float_as_uint(gm[qi]), __float_as_uint(gq[qi])};
          const uint32_t off = g == 0 && tile != gn.silent_tile ? rec_off(tile, ci, qi) : kOutside;
          __builtin_amdgcn_raw_buffer_store_b64(r, rrs, off, 0, 16);
        }
        if constexpr (kGnLate) {
          // hold this chunk's outputs (chunk ci - 2, normalised halfway
          // through this chunk's d_k pass, freed the slot)
#pragma unroll
          for (int qi = 0; qi < GQ; ++qi)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) gh_at(ci, qi, nb) = hn[qi][nb];
        } else {
          // normalise chunk ci - GD (its records were loaded at the start of
          // this chunk), then hold this chunk's outputs in the freed slot.
          // No instruction moves across this point: the records' validity
          // check would otherwise be hoisted to the start of the chunk and
          // wait there for loads issued just before.
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kGnLds) {
            // (chunk ci - GD holds the slot that chunk ci takes)
            gn_finish(ci - GD, [&](int qi, int nb) { return gh_at(ci, qi, nb); });
#pragma unroll
            for (int qi = 0; qi < GQ; ++qi)
#pragma unroll
              for (int nb = 0; nb < 4; ++nb) gh_at(ci, qi, nb) = hn[qi][nb];
          } else {
            gn_finish(ci - GD, [&](int qi, int nb) { return held[slot][qi][nb]; });
#pragma unroll
            for (int qi = 0; qi < GQ; ++qi)
#pragma unroll
              for (int nb = 0; nb < 4; ++nb) held[slot][qi][nb] = hn[qi][nb];
          }
        }
      } else {
        // store Y rows, 4 columns (8 bytes) per lane and block (rows past the
        // chunk end fall outside the buffer and are dropped)
        const rsrc_t ry = make_rsrc(yh + static_cast<long>(first_row(s0, L)) * dv,
                                    static_cast<uint32_t>(L - 1) * vrow + kTN * 2u);
#pragma unroll
        for (int qi = 0; qi < F::NQ; ++qi) {
          const uint32_t roff = row_off(16 * (qi == 0 ? W : QB1) + c16, L, vrow) + 8u * g;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const bf16x4 o = __builtin_convertvector(kZS ? O[qi][nb] * xi[qi] : O[qi][nb], bf16x4);
            buffer_store8(ry, roff + 32u * nb, __builtin_bit_cast(u32x2, o));
          }
        }
      }
      lds_barrier();  // the next chunk's R^T, K and V are in LDS
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    for (int ci = 0; ci < nchunks; ci += 2) {
      if constexpr (kQ2) {
        chunk(ci, Qa, Qb, I0());
        if (ci + 1 < nchunks) chunk(ci + 1, Qb, Qa, I1());
      } else {
        chunk(ci, Qa, Qa, I0());
        if (ci + 1 < nchunks) chunk(ci + 1, Qa, Qa, I1());
      }
    }
    if constexpr (kGnLate) {
      // the chunks still waiting: nchunks - 2 (its records were loaded at the
      // end of the last chunk) and nchunks - 1
      if (nchunks >= 2) gn_finish(nchunks - 2, [&](int qi, int nb) { return gh_at(nchunks - 2, qi, nb); });
      gn_load(nchunks - 1, kFirst());
      gn_finish(nchunks - 1, [&](int qi, int nb) { return gh_at(nchunks - 1, qi, nb); });
    } else if constexpr (kGN) {
      // the chunks still waiting: nchunks - GD .. nchunks - 1
      for (int cj = max(0, nchunks - GD); cj < nchunks; ++cj) {
        gn_load(cj, kFirst());
        if constexpr (kGnLds) {
          gn_finish(cj, [&](int qi, int nb) { return gh_at(cj, qi, nb); });
        } else if ((cj & 1) == 0) {
          gn_finish(cj, [&](int qi, int nb) { return held[0][qi][nb]; });
        } else {
          gn_finish(cj, [&](int qi, int nb) { return held[1][qi][nb]; });
        }
      }
    }
    };
    switch (wr) {
      case 0: out_role(std::integral_constant<int, 0>()); break;
      case 1: out_role(std::integral_constant<int, 1>()); break;
      case 2: out_role(std::integral_constant<int, 2>()); break;
      default: out_role(std::integral_constant<int, 3>()); break;
    }
    if (fin != nullptr)
      for (int rr = 0; rr < 2 * SRN; ++rr) lds_barrier();
  }
}

// Incoming state of every segment.  ws: main slots 0..nseg-1, then the
// sub-segment slots (nsub per segment of all but the last, in order), each
// holding that sub-segment's end state from zero.  Main slot 0 = state_in (or
// 0); main slot m = the state after segments 0..m-1, composed sub-segment by
// sub-segment: S <- gamma^sub_len S + local.  state_in_t: state_in holds each
// head's [da x dx] state transposed.
// VEC = 4: four consecutive elements of one head per thread (16-byte
// accesses; per_head % 4 == 0 and state_in not transposed); VEC = 1: one.
template <int VEC>
__global__ __launch_bounds__(256) void segment_scan_kernel(float* __restrict__ ws, const float* state_in,
                                                           int state_in_t, int dx, HeadDecay gam, int H, int h0,
                                                           int nh, int B, long per_head, int nseg, int nsub,
                                                           int sub_len, long stride) {
  typedef float vec_t __attribute__((ext_vector_type(VEC)));
  const long n = static_cast<long>(B) * nh * per_head / VEC;
  const float* sub = ws + nseg * stride;
  for (long iv = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; iv < n;
       iv += static_cast<long>(gridDim.x) * blockDim.x) {
    const long idx = VEC * iv;
    const long bh = idx / per_head;
    const long within = idx % per_head;
    const int hl = static_cast<int>(bh % nh);
    const long head = (bh / nh) * H + h0 + hl;
    const long off = head * per_head + within;
    const float gs = gamma_pow(gam.log2g[hl], sub_len);
    vec_t s;
    if constexpr (VEC == 1) {
      const long src = state_in_t ? head * per_head + (within % dx) * (per_head / dx) + within / dx : off;
      s = state_in != nullptr ? state_in[src] : 0.0f;
    } else {
      s = state_in != nullptr ? *reinterpret_cast<const vec_t*>(&state_in[off]) : vec_t(0.0f);
    }
    *reinterpret_cast<vec_t*>(&ws[off]) = s;
    // sub-segments 0..j0-1 of every segment are negligible (the test is
    // monotone in j, and j = nsub - 1 never is): they were not walked, and
    // their slots are not read
    int j0 = 0;
    while (j0 < nsub - 1 && sub_segment_negligible(gam.log2g[hl], nsub, j0, sub_len)) ++j0;
    const float gskip = gamma_pow(gam.log2g[hl], j0 * sub_len);
    for (int m = 1; m < nseg; ++m) {
      if (j0 > 0) s *= gskip;
      // the sub-slot loads do not depend on s: unrolled, several are in flight
#pragma unroll 4
      for (int j = j0; j < nsub; ++j) {
        const vec_t x = *reinterpret_cast<const vec_t*>(&sub[((m - 1) * nsub + j) * stride + off]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[e] = fmaf(gs, s[e], x[e]);
      }
      *reinterpret_cast<vec_t*>(&ws[m * stride + off]) = s;
    }
  }
}

// One launch sequence of the kernel.  With segments: the state-only launch
// over the sub-segments of segments 0..nseg-2 (64-token chunks when the
// sub-segment length allows, else the call's own tile and chunk), the scan of
// every pass, then the full launch.
template <int CT, int DK, bool kZS, int kDir, bool kGN = false>
hipError_t launch_cfg(const PassPtrs (&pp)[2], int npass, int B, int H, int Tn, int dx, int C, const HeadDecay& hd,
                      const HeadGroup& g, const ChunkSegments& segs, hipStream_t s, const GnArgs& gn = GnArgs{}) {
  const int ntiles = dx / kTN;
  const int bnh = B * g.nh;
  const long stride = static_cast<long>(B) * H * DK * dx;
  const int items = bnh * ntiles * npass;
  if (segs.nseg > 1) {
    const int sub_len = segs.seg_len / segs.nsub;
    const int nsubs = segs.nsub * (segs.nseg - 1);  // sub-segments before the last segment
    // the state-only kernel writes sub-segment i's end state to "slot i + 1"
    // of its ws, i.e. to the sub-segment slots
    PassPtrs pre[2] = {pp[0], pp[1]};
    for (auto& p : pre) p.ws = p.ws + (segs.nseg - 1) * stride;
    const SegArgs sp{sub_len, nsubs + 1, bnh, stride, segs.nsub};
    if (sub_len % 64 == 0)
      hipLaunchKernelGGL((chunkwise_mfma_kernel<64, DK, false, kZS, kDir>), dim3(items * nsubs), dim3(256), 0, s,
                         pre[0], pre[1], npass, hd, H, g.h0, g.nh, Tn, dx, 64, ntiles, sp, GnArgs{});
    else
      hipLaunchKernelGGL((chunkwise_mfma_kernel<CT, DK, false, kZS, kDir>), dim3(items * nsubs), dim3(256), 0, s,
                         pre[0], pre[1], npass, hd, H, g.h0, g.nh, Tn, dx, C, ntiles, sp, GnArgs{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long per_head = static_cast<long>(DK) * dx;
    const long n = static_cast<long>(bnh) * per_head;
    const unsigned blocks = static_cast<unsigned>(min(65536L, (n + 255) / 256));
    for (int i = 0; i < npass; ++i) {
      if (!pp[i].state_in_t && per_head % 4 == 0) {
        const unsigned b4 = static_cast<unsigned>(min(65536L, (n / 4 + 255) / 256));
        hipLaunchKernelGGL(segment_scan_kernel<4>, dim3(b4), dim3(256), 0, s, pp[i].ws, pp[i].state_in, 0, dx, hd, H,
                           g.h0, g.nh, B, per_head, segs.nseg, segs.nsub, sub_len, stride);
      } else {
        hipLaunchKernelGGL(segment_scan_kernel<1>, dim3(blocks), dim3(256), 0, s, pp[i].ws, pp[i].state_in,
                           pp[i].state_in_t, dx, hd, H, g.h0, g.nh, B, per_head, segs.nseg, segs.nsub, sub_len,
                           stride);
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const SegArgs sg{segs.seg_len, segs.nseg, bnh, stride, 0};
  GnArgs ga = gn;
  unsigned grid = static_cast<unsigned>(items * segs.nseg);
  if (kGN) {
    // a multiple of 8 * ntiles, so that the tiles of a head share an XCD
    ga.items = static_cast<int>(grid);
    const unsigned m = 8u * static_cast<unsigned>(ntiles);
    grid = (grid + m - 1) / m * m;
  }
  hipLaunchKernelGGL((chunkwise_mfma_kernel<CT, DK, true, kZS, kDir, kGN>), dim3(grid), dim3(512), 0, s, pp[0], pp[1],
                     npass, hd, H, g.h0, g.nh, Tn, dx, C, ntiles, sg, ga);
  return hipGetLastError();
}

template <int CT, bool kZS, bool kGN = false>
hipError_t launch_fwd_ct(const PassPtrs (&pp)[2], int B, int H, int Tn, int dk, int dv, int C, const HeadDecay& hd,
                         const HeadGroup& g, const ChunkSegments& segs, hipStream_t s, const GnArgs& gn = GnArgs{}) {
  switch (dk) {
    case 64: return launch_cfg<CT, 64, kZS, 0, kGN>(pp, 1, B, H, Tn, dv, C, hd, g, segs, s, gn);
    case 128: return launch_cfg<CT, 128, kZS, 0, kGN>(pp, 1, B, H, Tn, dv, C, hd, g, segs, s, gn);
    default: return launch_cfg<CT, 256, kZS, 0, kGN>(pp, 1, B, H, Tn, dv, C, hd, g, segs, s, gn);
  }
}

// One pass backwards in time (dV) at d_a <= 256: the direction fixed at compile
// time, which measured 7% faster than the per-pass direction of kDir = 2.
template <bool kZS>
hipError_t launch_passes_rev1(const PassPtrs (&pp)[2], int B, int H, int Tn, int da, int dx, const HeadDecay& hd,
                              const HeadGroup& g, const ChunkSegments& segs, hipStream_t s) {
  constexpr int C = kPassChunk;
  switch (da) {
    case 64: return launch_cfg<C, 64, kZS, 1>(pp, 1, B, H, Tn, dx, C, hd, g, segs, s);
    case 128: return launch_cfg<C, 128, kZS, 1>(pp, 1, B, H, Tn, dx, C, hd, g, segs, s);
    default: return launch_cfg<C, 256, kZS, 1>(pp, 1, B, H, Tn, dx, C, hd, g, segs, s);
  }
}

template <bool kZS>
hipError_t launch_passes_zs(const PassPtrs (&pp)[2], int npass, int B, int H, int Tn, int da, int dx,
                            const HeadDecay& hd, const HeadGroup& g, const ChunkSegments& segs, hipStream_t s) {
  constexpr int C = kPassChunk;
  switch (da) {
    case 64: return launch_cfg<C, 64, kZS, 2>(pp, npass, B, H, Tn, dx, C, hd, g, segs, s);
    case 128: return launch_cfg<C, 128, kZS, 2>(pp, npass, B, H, Tn, dx, C, hd, g, segs, s);
    case 256: return launch_cfg<C, 256, kZS, 2>(pp, npass, B, H, Tn, dx, C, hd, g, segs, s);
    default: return launch_cfg<C, 512, kZS, 2>(pp, npass, B, H, Tn, dx, C, hd, g, segs, s);
  }
}

// zeta-staged V when every head's zeta and gamma^(-L) stay within 2^+-100:
// gamma^e >= 2^-100 for the largest zeta exponent e
bool zeta_staged(const HeadDecay& hd, int nh, int e) {
  bool zs = true;
  for (int i = 0; i < nh; ++i) zs = zs && static_cast<double>(e) * hd.log2g[i] >= -100.0;
  return zs;
}

}  // namespace

bool chunkwise_mfma_supports(int /*T*/, int dk, int dv, int C, int dt) {
  return dt == 1 && (dk == 64 || dk == 128 || dk == 256) && dv % kTN == 0 && C >= 1 && C <= 128;
}

// Sub-segments of the state-only launch: about kPreWorkgroups work items
// (several of its 4-wave workgroups share a CU), each sub-segment a multiple
// of 64 positions and at least kMinSubChunks chunks of 64; 1 when the segment
// length allows no such split.
int state_pass_split(long items_per_sub, int nseg, int seg_len) {
  constexpr long kPreWorkgroups = 3 * 256;
  constexpr int kMinSubChunks = 4;
  if (nseg <= 1 || items_per_sub < 1) return 1;
  const long want = (kPreWorkgroups + items_per_sub * (nseg - 1) - 1) / (items_per_sub * (nseg - 1));
  int best = 1;
  for (int n = 2; n <= want && n <= 64; ++n)
    if (seg_len % (n * 64) == 0 && seg_len / n >= kMinSubChunks * 64) best = n;
  return best;
}

// A call whose (batch, head, column tile) walkers fill fewer than
// kTargetWorkgroups compute units is split into sequence segments (each at
// least kMinSegChunks chunks long) so that the walkers cover the device.
ChunkSegments chunkwise_mfma_segments(int B, int H, int T, int dv, int C) {
  constexpr long kTargetWorkgroups = 256;  // MI355X compute units
  constexpr int kMinSegChunks = 8;
  ChunkSegments r{T > 0 ? T : 1, 1, 1};
  const long walkers = static_cast<long>(B) * H * (dv / kTN);
  const long nchunks = (static_cast<long>(T) + C - 1) / C;
  if (walkers < 1 || walkers >= kTargetWorkgroups || nchunks < 2 * kMinSegChunks) return r;
  long want = (kTargetWorkgroups + walkers - 1) / walkers;
  want = min(want, nchunks / kMinSegChunks);
  if (want < 2) return r;
  const long per = (nchunks + want - 1) / want;  // chunks per segment
  r.seg_len = static_cast<int>(per * C);
  r.nseg = static_cast<int>((nchunks + per - 1) / per);
  r.nsub = state_pass_split(walkers, r.nseg, r.seg_len);
  return r;
}

size_t chunkwise_segment_slots(const ChunkSegments& sg) {
  return sg.nseg <= 1 ? 0 : static_cast<size_t>(sg.nseg) + static_cast<size_t>(sg.nsub) * (sg.nseg - 1);
}

hipError_t launch_chunkwise_mfma(const void* q, const void* k, const void* v, const float* state_in,
                                 float* state_out, void* y, int B, int H, int T, int dk, int dv, int C,
                                 const ChunkSegments& segs, float* ws, const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  const PassPtrs p{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                   state_in, state_out, static_cast<uint16_t*>(y), 0, 0, ws};
  const PassPtrs pp[2] = {p, p};
  const int ct = C <= 64 ? 64 : 128;
  const bool zs = zeta_staged(hd, g.nh, ct - 1);
  if (C <= 64) {
    if (zs) return launch_fwd_ct<64, true>(pp, B, H, T, dk, dv, C, hd, g, segs, s);
    return launch_fwd_ct<64, false>(pp, B, H, T, dk, dv, C, hd, g, segs, s);
  }
  if (zs) return launch_fwd_ct<128, true>(pp, B, H, T, dk, dv, C, hd, g, segs, s);
  return launch_fwd_ct<128, false>(pp, B, H, T, dk, dv, C, hd, g, segs, s);
}

size_t chunkwise_gn_record_bytes(int B, int H, int T, int dv, int C) {
  const ChunkSegments sg = chunkwise_mfma_segments(B, H, T, dv, C);
  return static_cast<size_t>(sg.nseg) * B * H * (dv / kTN) * static_cast<size_t>(sg.seg_len) * 8u;
}

bool chunkwise_gn_supports(int B, int H, int T, int dv, int C) {
  const ChunkSegments sg = chunkwise_mfma_segments(B, H, T, dv, C);
  // 8 tiles at most (two records per lane); one head's records within the
  // 32-bit offsets of a buffer resource
  return dv / kTN <= 8 && static_cast<long>(dv / kTN) * sg.seg_len * 8 < (1L << 31);
}

hipError_t launch_chunkwise_mfma_gn(const void* q, const void* k, const void* v, const float* state_in,
                                    float* state_out, void* y, int B, int H, int T, int dk, int dv, int C,
                                    const ChunkSegments& segs, float* ws, const GnLaunch& gl, const HeadGroup& g,
                                    hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  const PassPtrs p{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                   state_in, state_out, static_cast<uint16_t*>(y), 0, 0, ws};
  const PassPtrs pp[2] = {p, p};
  const GnArgs gn{gl.weight, gl.bias, gl.eps, static_cast<unsigned long long*>(gl.records), gl.err, B, H,
                  gl.spin_limit, 0, gl.silent_tile};
  const int ct = C <= 64 ? 64 : 128;
  const bool zs = zeta_staged(hd, g.nh, ct - 1);
  if (C <= 64) {
    if (zs) return launch_fwd_ct<64, true, true>(pp, B, H, T, dk, dv, C, hd, g, segs, s, gn);
    return launch_fwd_ct<64, false, true>(pp, B, H, T, dk, dv, C, hd, g, segs, s, gn);
  }
  if (zs) return launch_fwd_ct<128, true, true>(pp, B, H, T, dk, dv, C, hd, g, segs, s, gn);
  return launch_fwd_ct<128, false, true>(pp, B, H, T, dk, dv, C, hd, g, segs, s, gn);
}

bool chunkwise_mfma_pass_supports(int da, int dx) {
  return (da == 64 || da == 128 || da == 256 || da == 512) && dx % kTN == 0;
}

hipError_t launch_chunkwise_mfma_passes(const ChunkPass* p, int npass, int B, int H, int T, int da, int dx,
                                        const ChunkSegments& segs, const HeadGroup& g, hipStream_t s) {
  const HeadDecay hd = make_head_decay(g);
  PassPtrs pp[2];
  for (int i = 0; i < 2; ++i) {
    const ChunkPass& c = p[i < npass ? i : 0];
    pp[i] = PassPtrs{static_cast<const uint16_t*>(c.q), static_cast<const uint16_t*>(c.k),
                     static_cast<const uint16_t*>(c.v), c.state_in, c.state_out, static_cast<uint16_t*>(c.y), c.rev,
                     c.state_in_t, c.ws};
  }
  if (npass == 1 && p[0].rev && da <= 256) {
    if (zeta_staged(hd, g.nh, kPassChunk)) return launch_passes_rev1<true>(pp, B, H, T, da, dx, hd, g, segs, s);
    return launch_passes_rev1<false>(pp, B, H, T, da, dx, hd, g, segs, s);
  }
  // reverse passes weight by up to gamma^C: the stricter bound for both directions
  if (zeta_staged(hd, g.nh, kPassChunk)) return launch_passes_zs<true>(pp, npass, B, H, T, da, dx, hd, g, segs, s);
  return launch_passes_zs<false>(pp, npass, B, H, T, da, dx, hd, g, segs, s);
}

}  // namespace ret
