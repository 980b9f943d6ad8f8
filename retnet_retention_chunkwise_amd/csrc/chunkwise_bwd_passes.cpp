// Backward of the chunkwise form on bf16 MFMA: the three gradient passes on
// the chunkwise kernel (chunkwise_mfma.hip).
//
// The gradients of the chunkwise form (aimpact page, "Il meccanismo:
// Multi-Scale Retention"; chain rule on its recurrence) are three chunkwise
// passes of the forward's shape, each with a d_a x d_x fp32 state S:
//   dQ: forward in time over (A, B, X) = (dY, V, K) from S_0 = S_in^T,
//   dK: backwards in time over (V, dY, Q) from dS_out^T,
//   dV: backwards in time over (K, Q, dY) from dS_out; its final S is dS_in,
// where a pass backwards in time is, in positions counted from the end, the
// forward pass with the decay exponents shifted by one token.  dQ and dK
// (d_a = dv, X width dk) run as one launch of two passes, whose column tiles
// of one head share an XCD (dY and V are read by both); dV (d_a = dk, X width
// dv) follows, so that dS_in may be the dS_out buffer.  Few (batch, head,
// column-tile) walkers over a long sequence run in sequence segments
// (state-only launch, scan, full launch), each pass in its own slots of the
// caller's workspace.
#include <algorithm>

#include "kernels.h"

namespace ret {
namespace {

bool da_ok(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

}  // namespace

bool chunkwise_bwd_mfma_supports(int dk, int dv, int dt) { return dt == 1 && da_ok(dk) && da_ok(dv); }

// Few walkers in the smaller launch over a long sequence: segments of at least
// kMinSegChunks chunks of kPassChunk positions, so that the smaller launch
// fills about kTargetWorkgroups workgroups, and sub-segments for the
// state-only launches.  A pure function of the sizes.
ChunkSegments chunkwise_bwd_segments(int B, int H, int T, int dk, int dv) {
  constexpr long kTargetWorkgroups = 256;  // MI355X compute units
  constexpr int kMinSegChunks = 8;
  ChunkSegments r{T > 0 ? T : 1, 1, 1};
  const long walkers = static_cast<long>(B) * H * std::min(2 * (dk / 64), dv / 64);
  const long nchunks = (static_cast<long>(T) + kPassChunk - 1) / kPassChunk;
  if (walkers < 1 || walkers >= kTargetWorkgroups || nchunks < 2 * kMinSegChunks) return r;
  long want = (kTargetWorkgroups + walkers - 1) / walkers;
  want = std::min(want, nchunks / kMinSegChunks);
  if (want < 2) return r;
  const long per = (nchunks + want - 1) / want;  // chunks per segment
  r.seg_len = static_cast<int>(per * kPassChunk);
  r.nseg = static_cast<int>((nchunks + per - 1) / per);
  r.nsub = state_pass_split(walkers, r.nseg, r.seg_len);
  return r;
}

size_t chunkwise_bwd_workspace_floats(int B, int H, int T, int dk, int dv) {
  const ChunkSegments sg = chunkwise_bwd_segments(B, H, T, dk, dv);
  return 3 * chunkwise_segment_slots(sg) * B * H * dk * dv;  // dV, dK and dQ slots
}

hipError_t launch_chunkwise_bwd_mfma(const BwdArgs& a, int B, int H, int T, int dk, int dv, float* ws,
                                     const HeadGroup& g, hipStream_t s) {
  const ChunkSegments sg = chunkwise_bwd_segments(B, H, T, dk, dv);
  const long slot = static_cast<long>(B) * H * dk * dv;
  const long per_pass = static_cast<long>(chunkwise_segment_slots(sg)) * slot;
  float* wv = sg.nseg > 1 ? ws : nullptr;
  float* wk = sg.nseg > 1 ? ws + per_pass : nullptr;
  float* wq = sg.nseg > 1 ? ws + 2 * per_pass : nullptr;
  const ChunkPass kq[2] = {
      {a.v, a.dy, a.q, a.dstate_out, 1, 1, nullptr, a.dk, wk},  // dK
      {a.dy, a.v, a.k, a.state_in, 1, 0, nullptr, a.dq, wq},    // dQ
  };
  const hipError_t e = launch_chunkwise_mfma_passes(kq, 2, B, H, T, dv, dk, sg, g, s);
  if (e != hipSuccess) return e;
  const ChunkPass pv{a.k, a.q, a.dy, a.dstate_out, 0, 1, a.dstate_in, a.dv, wv};  // dV, dS_in
  return launch_chunkwise_mfma_passes(&pv, 1, B, H, T, dk, dv, sg, g, s);
}

}  // namespace ret
