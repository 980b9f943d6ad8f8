// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
// Arguments are validated by the caller; these functions only enqueue work.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace ret {

// Per-launch head decay table, passed by value as a kernel argument.  A launch
// covers at most kHeadsPerLaunch heads; the host splits larger H into groups.
constexpr int kHeadsPerLaunch = 128;
struct HeadDecay {
  float log2g[kHeadsPerLaunch];  // log2(gamma_h); -inf for gamma_h = 0
};

struct HeadGroup {
  int h0;              // first head of this launch
  int nh;              // number of heads in this launch (<= 128)
  const float* gamma;  // host, gamma of head h0 + i at gamma[i]
};

// log2(gamma) of the group's heads, computed in double on the host.
HeadDecay make_head_decay(const HeadGroup& g);

// dt: 0 = fp32, 1 = bf16 (raw bits).
hipError_t launch_recurrent_step(const void* q, const void* k, const void* v, float* state, void* y, int B,
                                 int H, int dk, int dv, int dt, const HeadGroup& g, hipStream_t s);

hipError_t launch_parallel_fwd(const void* q, const void* k, const void* v, const float* state_in, void* y,
                               int B, int H, int T, int dk, int dv, int dt, const HeadGroup& g, hipStream_t s);

// Generic VALU chunkwise kernel (any supported shape, fp32 or bf16 inputs).
hipError_t launch_chunkwise_generic(const void* q, const void* k, const void* v, const float* state_in,
                                    float* state_out, void* y, int B, int H, int T, int dk, int dv, int C,
                                    int dt, const HeadGroup& g, hipStream_t s);

// bf16 MFMA chunkwise kernel; chunkwise_mfma_supports() says whether it takes a shape.
bool chunkwise_mfma_supports(int T, int dk, int dv, int C, int dt);
// Sequence segmentation of an MFMA call: nseg segments of seg_len tokens
// (nseg = 1: no segmentation, no workspace); the state-only launch splits each
// segment but the last into nsub sub-segments.  A pure function of the sizes.
struct ChunkSegments {
  int seg_len;
  int nseg;
  int nsub;
};
ChunkSegments chunkwise_mfma_segments(int B, int H, int T, int dv, int C);
// State slots of one pass: nseg + nsub * (nseg - 1) (0 when nseg = 1).
size_t chunkwise_segment_slots(const ChunkSegments& sg);
// Sub-segments for a state-only launch of items_per_sub work items per sub-segment.
int state_pass_split(long items_per_sub, int nseg, int seg_len);
// ws: chunkwise_segment_slots(segs) * B*H*dk*dv fp32 when segs.nseg > 1 (else unused)
hipError_t launch_chunkwise_mfma(const void* q, const void* k, const void* v, const float* state_in,
                                 float* state_out, void* y, int B, int H, int T, int dk, int dv, int C,
                                 const ChunkSegments& segs, float* ws, const HeadGroup& g, hipStream_t s);

// The same forward with the per-head GroupNorm fused into the output stores
// (y receives the normalised outputs).  records: chunkwise_gn_record_bytes()
// bytes filled with 0xFF before the launch; err: one int set to 1 if a wait
// for another tile's records gave up after spin_limit polls.
struct GnLaunch {
  const float* weight;  // [H, dv] or null
  const float* bias;    // [H, dv] or null
  float eps;
  void* records;
  int* err;
  int spin_limit;   // polls before a wait for another tile's records gives up
  int silent_tile;  // failure-path testing: a column tile that publishes no records (-1: none)
};
bool chunkwise_gn_supports(int B, int H, int T, int dv, int C);
size_t chunkwise_gn_record_bytes(int B, int H, int T, int dv, int C);
hipError_t launch_chunkwise_mfma_gn(const void* q, const void* k, const void* v, const float* state_in,
                                    float* state_out, void* y, int B, int H, int T, int dk, int dv, int C,
                                    const ChunkSegments& segs, float* ws, const GnLaunch& gl, const HeadGroup& g,
                                    hipStream_t s);

// Passes of the same kernel for the gradients, in chunks of kPassChunk
// positions: each pass runs forward in time or backwards with the decay
// weights shifted by one token (rev = 1; position p = T-1-n for token n, chunk
// rows j):
//   Y_j = gamma^j Q_j R + sum_{t<=j} gamma^(j-t) (Q_j . K_t) V_t,
//   R <- gamma^L R + sum_t gamma^(L-t) K_t^T V_t.
// One launch runs one or two passes of one d_a (Q and K width, in {64, 128,
// 256, 512}) and X width dx (V and Y, a multiple of 64), bf16, T >= 1.  The
// initial state may be stored transposed ([dx, da] per head).  With
// segments (segs.nseg > 1, seg_len a multiple of kPassChunk) each pass needs
// ws: nseg slots of B*H*da*dx fp32.
//   dQ: forward over (dY, V, K) from S_in^T;  dK: reverse over (V, dY, Q)
//   from dS_out^T;  dV: reverse over (K, Q, dY) from dS_out, final state dS_in.
constexpr int kPassChunk = 64;
struct ChunkPass {
  const void* q;
  const void* k;
  const void* v;
  const float* state_in;  // nullable
  int state_in_t;
  int rev;
  float* state_out;  // nullable
  void* y;
  float* ws;  // segment slots (segmented launches)
};
bool chunkwise_mfma_pass_supports(int da, int dx);
hipError_t launch_chunkwise_mfma_passes(const ChunkPass* p, int npass, int B, int H, int T, int da, int dx,
                                        const ChunkSegments& segs, const HeadGroup& g, hipStream_t s);

// Streaming chunkwise kernel for a short block of tokens from a carried state
// (1 <= T <= kShortChunkMaxT, fp32 or bf16 inputs, any supported dk and dv):
// the whole block is one chunk, and the state is read and written once.
constexpr int kShortChunkMaxT = 16;
hipError_t launch_short_chunk(const void* q, const void* k, const void* v, const float* state_in, float* state_out,
                              void* y, int B, int H, int T, int dk, int dv, int dt, const HeadGroup& g,
                              hipStream_t s);

// Backward of the chunkwise form (gradients of retention_chunkwise_fwd).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* state_in;    // nullable
  const void* dy;
  const float* dstate_out;  // nullable
  void* dq;
  void* dk;
  void* dv;
  float* dstate_in;         // nullable; may be dstate_out
};
// Generic fp32-arithmetic passes (any dtype, dk and dv up to 512).
bool chunkwise_bwd_generic_supports(int dk, int dv);
hipError_t launch_chunkwise_bwd_generic(const BwdArgs& a, int B, int H, int T, int dk, int dv, int dt,
                                        const HeadGroup& g, hipStream_t s);
// bf16 MFMA passes (the chunkwise kernel's gradient passes): bf16 inputs with
// dk, dv in {64, 128, 256, 512}.
bool chunkwise_bwd_mfma_supports(int dk, int dv, int dt);
// Sequence segments of a backward call on the MFMA passes, and the fp32
// workspace they need (0: none); pure functions of the sizes.
ChunkSegments chunkwise_bwd_segments(int B, int H, int T, int dk, int dv);
size_t chunkwise_bwd_workspace_floats(int B, int H, int T, int dk, int dv);
// ws: chunkwise_bwd_workspace_floats(...) fp32 (unused when 0)
hipError_t launch_chunkwise_bwd_mfma(const BwdArgs& a, int B, int H, int T, int dk, int dv, float* ws,
                                     const HeadGroup& g, hipStream_t s);

// fp32 inputs on fp32 MFMA (dk, dv in {64, 128, 256, 512}): the forward and
// the backward passes of the chunkwise form at fp32 accuracy.
bool chunkwise_f32_mfma_supports(int dk, int dv, int dt);
hipError_t launch_chunkwise_f32_fwd(const float* q, const float* k, const float* v, const float* state_in,
                                    float* state_out, float* y, int B, int H, int T, int dk, int dv,
                                    const HeadGroup& g, hipStream_t s);
hipError_t launch_chunkwise_f32_bwd(const BwdArgs& a, int B, int H, int T, int dk, int dv, const HeadGroup& g,
                                    hipStream_t s);

// Per-head GroupNorm of a [B,H,T,dv] output (dt: 0 = fp32, 1 = bf16); out may be y.
hipError_t launch_group_norm(const void* y, const float* weight, const float* bias, float eps, void* out, int B,
                             int H, int T, int dv, int dt, hipStream_t s);

// The same on fp32 MFMA for 1 <= T <= kShortMfmaMaxT (dk % 16 == 0, dv % 64 == 0).
constexpr int kShortMfmaMaxT = 32;
constexpr int kShortMfmaMinT = 1;  // below this the VALU streaming kernel is used
bool short_mfma_supports(int T, int dk, int dv);
hipError_t launch_short_mfma(const void* q, const void* k, const void* v, const float* state_in, float* state_out,
                             void* y, int B, int H, int T, int dk, int dv, int dt, const HeadGroup& g, hipStream_t s);

// bf16 inputs, 1 <= T <= kShortBf16MaxT, dk % 32 == 0, dv % 64 == 0: the same
// one-chunk streaming pass with bf16 MFMA products.
constexpr int kShortBf16MaxT = 64;
bool short_bf16_supports(int T, int dk, int dv, int dt);
hipError_t launch_short_bf16(const void* q, const void* k, const void* v, const float* state_in, float* state_out,
                             void* y, int B, int H, int T, int dk, int dv, const HeadGroup& g, hipStream_t s);

// Copies state_in (or zeros when null) into state_out: the T = 0 case.
hipError_t launch_state_copy(const float* state_in, float* state_out, size_t n, hipStream_t s);

// Sets n 32-bit words to val, and *word to word_val when word is not null (a
// kernel, so that it can sit in a captured graph).
hipError_t launch_fill_u32(void* p, size_t n, unsigned int val, hipStream_t s, unsigned int* word = nullptr,
                           unsigned int word_val = 0);

}  // namespace ret
