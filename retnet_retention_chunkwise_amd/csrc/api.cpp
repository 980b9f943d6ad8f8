// C-ABI layer of libretention: argument validation, per-head decay tables,
// kernel choice and launch.  Every check happens before the first HIP call, so
// a rejected call enqueues nothing and touches no output.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "abi_internal.h"
#include "kernels.h"
#include "libretention.h"

namespace {

thread_local std::string g_last_error;

ret_status fail(ret_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ret_status ok() {
  g_last_error.clear();
  return RET_OK;
}

ret_status hip_fail(const char* fn, hipError_t e) {
  return fail(RET_ERR_HIP, "%s: HIP error %d (%s)", fn, static_cast<int>(e), hipGetErrorString(e));
}

constexpr long long kMaxElems = (1LL << 31) - 1;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Shared checks of sizes, dtype and gamma.
ret_status check_common(const char* fn, int B, int H, int T, int dk, int dv, ret_dtype dt, const float* gamma) {
  if (B < 1 || H < 1) return fail(RET_ERR_INVALID_ARG, "%s: B=%d and H=%d must be >= 1", fn, B, H);
  if (T < 0) return fail(RET_ERR_INVALID_ARG, "%s: T=%d must be >= 0", fn, T);
  if (dk < 1 || dv < 1) return fail(RET_ERR_INVALID_ARG, "%s: dk=%d and dv=%d must be >= 1", fn, dk, dv);
  if (dt != RET_F32 && dt != RET_BF16) return fail(RET_ERR_UNSUPPORTED, "%s: dtype %d is not RET_F32 or RET_BF16", fn, static_cast<int>(dt));
  if (gamma == nullptr) return fail(RET_ERR_INVALID_ARG, "%s: gamma (host array of H floats) is null", fn);
  for (int h = 0; h < H; ++h) {
    const float g = gamma[h];
    if (!std::isfinite(g) || g < 0.0f || g > 1.0f)
      return fail(RET_ERR_INVALID_ARG, "%s: gamma[%d] = %g is not a decay in [0, 1]", fn, h, static_cast<double>(g));
  }
  if (dk > RET_MAX_DK || dv > RET_MAX_DV)
    return fail(RET_ERR_UNSUPPORTED, "%s: dk=%d, dv=%d exceed the built limits (dk <= %d, dv <= %d)", fn, dk, dv,
                RET_MAX_DK, RET_MAX_DV);
  const long long bh = static_cast<long long>(B) * H;
  if (bh * T * dk > kMaxElems || bh * T * dv > kMaxElems || bh * dk * dv > kMaxElems)
    return fail(RET_ERR_UNSUPPORTED, "%s: a tensor has 2^31 or more elements", fn);
  return RET_OK;
}

size_t dsize(ret_dtype dt) { return dt == RET_F32 ? 4 : 2; }

template <typename F>
ret_status for_head_groups(const char* fn, int H, const float* gamma, F&& launch) {
  for (int h0 = 0; h0 < H; h0 += ret::kHeadsPerLaunch) {
    ret::HeadGroup g{h0, H - h0 < ret::kHeadsPerLaunch ? H - h0 : ret::kHeadsPerLaunch, gamma + h0};
    const hipError_t e = launch(g);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  return ok();
}

}  // namespace

namespace ret {
HeadDecay make_head_decay(const HeadGroup& g) {
  HeadDecay hd;
  for (int i = 0; i < kHeadsPerLaunch; ++i) {
    const double gm = i < g.nh ? static_cast<double>(g.gamma[i]) : 1.0;
    hd.log2g[i] = gm > 0.0 ? static_cast<float>(std::log2(gm)) : -INFINITY;
  }
  return hd;
}
}  // namespace ret

namespace ret {

void set_last_error(const char* text) { g_last_error = text; }

// Validation of a chunkwise forward call: sizes, pointers, aliasing and (when
// check_ws) the caller's workspace.  Makes no HIP call.
ret_status chunkwise_fwd_check(const ChunkwiseFwdArgs& a, const void* workspace, size_t workspace_bytes,
                               bool check_ws, const char* fn) {
  const int B = a.B, H = a.H, T = a.T, dk = a.dk, dv = a.dv, C = a.C;
  const ret_dtype dt = static_cast<ret_dtype>(a.dt);
  ret_status st = check_common(fn, B, H, T, dk, dv, dt, a.gamma);
  if (st != RET_OK) return st;
  if (C < 1) return fail(RET_ERR_INVALID_ARG, "%s: chunk length C=%d must be >= 1", fn, C);
  if (C > RET_MAX_CHUNK) return fail(RET_ERR_UNSUPPORTED, "%s: chunk length C=%d exceeds %d", fn, C, RET_MAX_CHUNK);
  if (T > 0 && (!a.q || !a.k || !a.v || !a.y)) return fail(RET_ERR_INVALID_ARG, "%s: q, k, v and y are required", fn);
  if (misaligned(a.q) || misaligned(a.k) || misaligned(a.v) || misaligned(a.y) || misaligned(a.state_in) ||
      misaligned(a.state_out) || (check_ws && misaligned(workspace)))
    return fail(RET_ERR_UNSUPPORTED, "%s: tensor pointers must be 16-byte aligned", fn);
  const size_t es = dsize(dt);
  const size_t bht = static_cast<size_t>(B) * H * T;
  const size_t ny = bht * dv * es;
  const size_t ns = static_cast<size_t>(B) * H * dk * dv * 4;
  if (overlap(a.y, ny, a.q, bht * dk * es) || overlap(a.y, ny, a.k, bht * dk * es) || overlap(a.y, ny, a.v, ny) ||
      overlap(a.y, ny, a.state_in, ns) || overlap(a.y, ny, a.state_out, ns))
    return fail(RET_ERR_INVALID_ARG, "%s: y overlaps an input or a state buffer", fn);
  if (a.state_in != a.state_out && overlap(a.state_in, ns, a.state_out, ns))
    return fail(RET_ERR_INVALID_ARG, "%s: state_in and state_out overlap without being the same buffer", fn);
  if (a.state_out != nullptr && (overlap(a.state_out, ns, a.q, bht * dk * es) ||
                                 overlap(a.state_out, ns, a.k, bht * dk * es) || overlap(a.state_out, ns, a.v, ny)))
    return fail(RET_ERR_INVALID_ARG, "%s: state_out overlaps an input", fn);
  if (!check_ws) return RET_OK;
  const size_t need = retention_chunkwise_workspace_bytes(B, H, T, dk, dv, C, dt);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(RET_ERR_INVALID_ARG, "%s: workspace of %zu bytes required, %zu given", fn, need, workspace_bytes);
  if (need > 0 && (overlap(workspace, need, a.y, ny) || overlap(workspace, need, a.q, bht * dk * es) ||
                   overlap(workspace, need, a.k, bht * dk * es) || overlap(workspace, need, a.v, ny) ||
                   overlap(workspace, need, a.state_in, ns) || overlap(workspace, need, a.state_out, ns)))
    return fail(RET_ERR_INVALID_ARG, "%s: workspace overlaps another argument", fn);
  return RET_OK;
}

// Kernel choice and launch of a validated chunkwise forward call; workspace
// holds retention_chunkwise_workspace_bytes() bytes when that is non-zero.
ret_status chunkwise_fwd_run(const ChunkwiseFwdArgs& a, void* workspace, void* stream) {
  const char* fn = "retention_chunkwise_fwd";
  const void *q = a.q, *k = a.k, *v = a.v;
  const float* state_in = a.state_in;
  float* state_out = a.state_out;
  void* y = a.y;
  const int B = a.B, H = a.H, T = a.T, dk = a.dk, dv = a.dv, C = a.C, dt = a.dt;
  const size_t ns = static_cast<size_t>(B) * H * dk * dv * 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    if (state_out == nullptr || state_out == state_in) return ok();
    const hipError_t e = launch_state_copy(state_in, state_out, ns / 4, s);
    return e == hipSuccess ? ok() : hip_fail(fn, e);
  }
  if (T == 1 && state_in != nullptr && state_in == state_out) {
    // one token continued in place: exactly the recurrent step
    return for_head_groups(fn, H, a.gamma, [&](const HeadGroup& g) {
      return launch_recurrent_step(q, k, v, state_out, y, B, H, dk, dv, dt, g, s);
    });
  }
  if (short_bf16_supports(T, dk, dv, dt)) {
    // one chunk of T tokens on bf16 MFMA (the same result as any C up to rounding)
    return for_head_groups(fn, H, a.gamma, [&](const HeadGroup& g) {
      return launch_short_bf16(q, k, v, state_in, state_out, y, B, H, T, dk, dv, g, s);
    });
  }
  if (T >= kShortMfmaMinT && short_mfma_supports(T, dk, dv)) {
    // one chunk of T tokens on fp32 MFMA (the same result as any C up to rounding order)
    return for_head_groups(fn, H, a.gamma, [&](const HeadGroup& g) {
      return launch_short_mfma(q, k, v, state_in, state_out, y, B, H, T, dk, dv, dt, g, s);
    });
  }
  if (T <= kShortChunkMaxT) {
    // one chunk of T tokens (the same result as any C up to rounding order)
    return for_head_groups(fn, H, a.gamma, [&](const HeadGroup& g) {
      return launch_short_chunk(q, k, v, state_in, state_out, y, B, H, T, dk, dv, dt, g, s);
    });
  }
  const bool mfma = chunkwise_mfma_supports(T, dk, dv, C, dt);
  const bool f32 = chunkwise_f32_mfma_supports(dk, dv, dt);
  const ChunkSegments segs = mfma ? chunkwise_mfma_segments(B, H, T, dv, C) : ChunkSegments{T, 1, 1};
  float* ws = static_cast<float*>(workspace);
  return for_head_groups(fn, H, a.gamma, [&](const HeadGroup& g) {
    if (mfma) return launch_chunkwise_mfma(q, k, v, state_in, state_out, y, B, H, T, dk, dv, C, segs, ws, g, s);
    if (f32)
      return launch_chunkwise_f32_fwd(static_cast<const float*>(q), static_cast<const float*>(k),
                                      static_cast<const float*>(v), state_in, state_out, static_cast<float*>(y), B,
                                      H, T, dk, dv, g, s);
    return launch_chunkwise_generic(q, k, v, state_in, state_out, y, B, H, T, dk, dv, C, dt, g, s);
  });
}

// The fused GroupNorm runs inside the bf16 MFMA kernel.  Calls that take
// another kernel (blocks of up to 64 tokens, fp32, other shapes) run the
// forward and then the standalone GroupNorm on y in place.
bool gn_fused(int B, int H, int T, int dk, int dv, int C, int dt) {
  return T > kShortBf16MaxT && chunkwise_mfma_supports(T, dk, dv, C, dt) && chunkwise_gn_supports(B, H, T, dv, C);
}

// Workspace of the fused call: [error word | 256 B][segment slots][records].
constexpr size_t kGnHead = 256;
// a wait for another tile's records gives up after 2^16 device-scope polls
// (about 0.1 s), sets the error word and goes on
constexpr int kGnSpinLimit = 1 << 16;
size_t gn_slot_bytes(int B, int H, int T, int dk, int dv, int C) {
  const size_t b = chunkwise_segment_slots(chunkwise_mfma_segments(B, H, T, dv, C)) * B * H * dk * dv * sizeof(float);
  return (b + 255) / 256 * 256;
}

// Waits of the fused kernel: polls before giving up, and a column tile whose
// records are never published (-1: none).  Process-wide; changed only by
// retention_testing_gn_wait.
int g_gn_spin_limit = kGnSpinLimit;
int g_gn_silent_tile = -1;

}  // namespace ret

extern "C" {

const char* retention_last_error(void) { return g_last_error.c_str(); }

int retention_version(void) { return 100; }

ret_status retention_recurrent_step(const void* q, const void* k, const void* v, const float* gamma, float* state,
                                    void* y, int B, int H, int dk, int dv, ret_dtype dt, void* stream) {
  const char* fn = "retention_recurrent_step";
  ret_status st = check_common(fn, B, H, 1, dk, dv, dt, gamma);
  if (st != RET_OK) return st;
  if (!q || !k || !v || !state || !y) return fail(RET_ERR_INVALID_ARG, "%s: q, k, v, state and y are required", fn);
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(state) || misaligned(y))
    return fail(RET_ERR_UNSUPPORTED, "%s: tensor pointers must be 16-byte aligned", fn);
  const size_t es = dsize(dt);
  const size_t bh = static_cast<size_t>(B) * H;
  const size_t ny = bh * dv * es;
  if (overlap(y, ny, q, bh * dk * es) || overlap(y, ny, k, bh * dk * es) || overlap(y, ny, v, ny) ||
      overlap(y, ny, state, bh * dk * dv * 4))
    return fail(RET_ERR_INVALID_ARG, "%s: y overlaps an input or the state", fn);
  // the state is rewritten while other workgroups still read q, k and v
  const size_t ns = bh * dk * dv * 4;
  if (overlap(state, ns, q, bh * dk * es) || overlap(state, ns, k, bh * dk * es) || overlap(state, ns, v, ny))
    return fail(RET_ERR_INVALID_ARG, "%s: the state overlaps q, k or v", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return for_head_groups(fn, H, gamma, [&](const ret::HeadGroup& g) {
    return ret::launch_recurrent_step(q, k, v, state, y, B, H, dk, dv, static_cast<int>(dt), g, s);
  });
}

ret_status retention_parallel_fwd(const void* q, const void* k, const void* v, const float* gamma,
                                  const float* state_in, void* y, int B, int H, int T, int dk, int dv, ret_dtype dt,
                                  void* stream) {
  const char* fn = "retention_parallel_fwd";
  ret_status st = check_common(fn, B, H, T, dk, dv, dt, gamma);
  if (st != RET_OK) return st;
  if (T > 0 && (!q || !k || !v || !y)) return fail(RET_ERR_INVALID_ARG, "%s: q, k, v and y are required", fn);
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(y) || misaligned(state_in))
    return fail(RET_ERR_UNSUPPORTED, "%s: tensor pointers must be 16-byte aligned", fn);
  const size_t es = dsize(dt);
  const size_t bht = static_cast<size_t>(B) * H * T;
  const size_t ny = bht * dv * es;
  if (overlap(y, ny, q, bht * dk * es) || overlap(y, ny, k, bht * dk * es) || overlap(y, ny, v, ny) ||
      overlap(y, ny, state_in, static_cast<size_t>(B) * H * dk * dv * 4))
    return fail(RET_ERR_INVALID_ARG, "%s: y overlaps an input", fn);
  if (T == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  return for_head_groups(fn, H, gamma, [&](const ret::HeadGroup& g) {
    return ret::launch_parallel_fwd(q, k, v, state_in, y, B, H, T, dk, dv, static_cast<int>(dt), g, s);
  });
}

size_t retention_chunkwise_workspace_bytes(int B, int H, int T, int dk, int dv, int C, ret_dtype dt) {
  if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1 || C < 1) return static_cast<size_t>(-1);
  if (dk > RET_MAX_DK || dv > RET_MAX_DV || C > RET_MAX_CHUNK) return static_cast<size_t>(-1);
  if (dt != RET_F32 && dt != RET_BF16) return static_cast<size_t>(-1);
  if (T <= ret::kShortChunkMaxT || !ret::chunkwise_mfma_supports(T, dk, dv, C, static_cast<int>(dt))) return 0;
  if (ret::short_bf16_supports(T, dk, dv, static_cast<int>(dt))) return 0;
  if (T <= ret::kShortMfmaMaxT && T >= ret::kShortMfmaMinT && ret::short_mfma_supports(T, dk, dv)) return 0;
  const ret::ChunkSegments segs = ret::chunkwise_mfma_segments(B, H, T, dv, C);
  return ret::chunkwise_segment_slots(segs) * B * H * dk * dv * sizeof(float);
}

ret_status retention_chunkwise_fwd(const void* q, const void* k, const void* v, const float* gamma,
                                   const float* state_in, float* state_out, void* y, int B, int H, int T, int dk,
                                   int dv, int C, ret_dtype dt, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  const ret::ChunkwiseFwdArgs a{q, k, v, gamma, state_in, state_out, y, B, H, T, dk, dv, C, static_cast<int>(dt)};
  const ret_status st = ret::chunkwise_fwd_check(a, workspace, workspace_bytes, true, "retention_chunkwise_fwd");
  if (st != RET_OK) return st;
  return ret::chunkwise_fwd_run(a, workspace, stream);
}

size_t retention_chunkwise_fwd_group_norm_workspace_bytes(int B, int H, int T, int dk, int dv, int C, ret_dtype dt) {
  const size_t fwd = retention_chunkwise_workspace_bytes(B, H, T, dk, dv, C, dt);
  if (fwd == static_cast<size_t>(-1)) return fwd;
  if (!ret::gn_fused(B, H, T, dk, dv, C, static_cast<int>(dt))) return fwd;
  return ret::kGnHead + ret::gn_slot_bytes(B, H, T, dk, dv, C) + ret::chunkwise_gn_record_bytes(B, H, T, dv, C);
}

ret_status retention_chunkwise_fwd_group_norm(const void* q, const void* k, const void* v, const float* gamma,
                                              const float* state_in, float* state_out, const float* weight,
                                              const float* bias, float eps, void* y, int B, int H, int T, int dk,
                                              int dv, int C, ret_dtype dt, void* workspace, size_t workspace_bytes,
                                              void* stream) {
  const char* fn = "retention_chunkwise_fwd_group_norm";
  const ret::ChunkwiseFwdArgs a{q, k, v, gamma, state_in, state_out, y, B, H, T, dk, dv, C, static_cast<int>(dt)};
  ret_status st = ret::chunkwise_fwd_check(a, nullptr, 0, false, fn);
  if (st != RET_OK) return st;
  if (!std::isfinite(eps) || eps < 0.0f)
    return fail(RET_ERR_INVALID_ARG, "%s: eps = %g must be finite and >= 0", fn, static_cast<double>(eps));
  if (misaligned(weight) || misaligned(bias) || misaligned(workspace))
    return fail(RET_ERR_UNSUPPORTED, "%s: tensor pointers must be 16-byte aligned", fn);
  const size_t es = dsize(dt);
  const size_t bht = static_cast<size_t>(B) * H * T;
  const size_t ny = bht * dv * es, nk = bht * dk * es;
  const size_t ns = static_cast<size_t>(B) * H * dk * dv * 4;
  const size_t nw = static_cast<size_t>(H) * dv * 4;
  if (overlap(y, ny, weight, nw) || overlap(y, ny, bias, nw))
    return fail(RET_ERR_INVALID_ARG, "%s: y overlaps weight or bias", fn);
  if (state_out != nullptr && (overlap(state_out, ns, weight, nw) || overlap(state_out, ns, bias, nw)))
    return fail(RET_ERR_INVALID_ARG, "%s: state_out overlaps weight or bias", fn);
  const size_t need = retention_chunkwise_fwd_group_norm_workspace_bytes(B, H, T, dk, dv, C, dt);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(RET_ERR_INVALID_ARG, "%s: workspace of %zu bytes required, %zu given", fn, need, workspace_bytes);
  if (need > 0 && (overlap(workspace, need, y, ny) || overlap(workspace, need, q, nk) ||
                   overlap(workspace, need, k, nk) || overlap(workspace, need, v, ny) ||
                   overlap(workspace, need, state_in, ns) || overlap(workspace, need, state_out, ns) ||
                   overlap(workspace, need, weight, nw) || overlap(workspace, need, bias, nw)))
    return fail(RET_ERR_INVALID_ARG, "%s: workspace overlaps another argument", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!ret::gn_fused(B, H, T, dk, dv, C, static_cast<int>(dt))) {
    st = ret::chunkwise_fwd_run(a, workspace, stream);
    if (st != RET_OK || T == 0) return st;
    const hipError_t e = ret::launch_group_norm(y, weight, bias, eps, y, B, H, T, dv, static_cast<int>(dt), s);
    return e == hipSuccess ? ok() : hip_fail(fn, e);
  }
  char* base = static_cast<char*>(workspace);
  int* err = reinterpret_cast<int*>(base);
  float* slots = reinterpret_cast<float*>(base + ret::kGnHead);
  void* records = base + ret::kGnHead + ret::gn_slot_bytes(B, H, T, dk, dv, C);
  const size_t rec_bytes = ret::chunkwise_gn_record_bytes(B, H, T, dv, C);
  // records to the sentinel and the error word to 0, in one launch
  hipError_t e = ret::launch_fill_u32(records, rec_bytes / 4, 0xFFFFFFFFu, s, reinterpret_cast<unsigned*>(err), 0u);
  if (e != hipSuccess) return hip_fail(fn, e);
  const ret::ChunkSegments segs = ret::chunkwise_mfma_segments(B, H, T, dv, C);
  const ret::GnLaunch gl{weight, bias, eps, records, err, ret::g_gn_spin_limit, ret::g_gn_silent_tile};
  return for_head_groups(fn, H, gamma, [&](const ret::HeadGroup& g) {
    return ret::launch_chunkwise_mfma_gn(q, k, v, state_in, state_out, y, B, H, T, dk, dv, C, segs, slots, gl, g, s);
  });
}

ret_status retention_testing_gn_wait(int spin_limit, int silent_tile) {
  const char* fn = "retention_testing_gn_wait";
  if (spin_limit < 1) return fail(RET_ERR_INVALID_ARG, "%s: spin_limit = %d must be >= 1", fn, spin_limit);
  if (silent_tile < -1) return fail(RET_ERR_INVALID_ARG, "%s: silent_tile = %d must be >= -1", fn, silent_tile);
  ret::g_gn_spin_limit = spin_limit;
  ret::g_gn_silent_tile = silent_tile;
  return ok();
}

size_t retention_chunkwise_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C, ret_dtype dt) {
  if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1 || C < 1) return static_cast<size_t>(-1);
  if (dk > RET_MAX_DK || dv > RET_MAX_DV || C > RET_MAX_CHUNK) return static_cast<size_t>(-1);
  if (dt != RET_F32 && dt != RET_BF16) return static_cast<size_t>(-1);
  if (T == 0 || !ret::chunkwise_bwd_mfma_supports(dk, dv, static_cast<int>(dt))) return 0;
  return ret::chunkwise_bwd_workspace_floats(B, H, T, dk, dv) * sizeof(float);
}

ret_status retention_chunkwise_bwd(const void* q, const void* k, const void* v, const float* gamma,
                                   const float* state_in, const void* grad_y, const float* grad_state_out,
                                   void* grad_q, void* grad_k, void* grad_v, float* grad_state_in, int B, int H,
                                   int T, int dk, int dv, int C, ret_dtype dt, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const char* fn = "retention_chunkwise_bwd";
  ret_status st = check_common(fn, B, H, T, dk, dv, dt, gamma);
  if (st != RET_OK) return st;
  if (C < 1) return fail(RET_ERR_INVALID_ARG, "%s: chunk length C=%d must be >= 1", fn, C);
  if (C > RET_MAX_CHUNK) return fail(RET_ERR_UNSUPPORTED, "%s: chunk length C=%d exceeds %d", fn, C, RET_MAX_CHUNK);
  if (T > 0 && (!q || !k || !v || !grad_y || !grad_q || !grad_k || !grad_v))
    return fail(RET_ERR_INVALID_ARG, "%s: q, k, v, grad_y, grad_q, grad_k and grad_v are required", fn);
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(state_in) || misaligned(grad_y) ||
      misaligned(grad_state_out) || misaligned(grad_q) || misaligned(grad_k) || misaligned(grad_v) ||
      misaligned(grad_state_in) || misaligned(workspace))
    return fail(RET_ERR_UNSUPPORTED, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!ret::chunkwise_bwd_generic_supports(dk, dv))
    return fail(RET_ERR_UNSUPPORTED, "%s: dk=%d, dv=%d not supported", fn, dk, dv);
  const size_t es = dsize(dt);
  const size_t bht = static_cast<size_t>(B) * H * T;
  const size_t nk = bht * dk * es, nv = bht * dv * es;
  const size_t ns = static_cast<size_t>(B) * H * dk * dv * 4;
  struct Buf {
    const void* p;
    size_t n;
  };
  const size_t need = retention_chunkwise_bwd_workspace_bytes(B, H, T, dk, dv, C, dt);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(RET_ERR_INVALID_ARG, "%s: workspace of %zu bytes required, %zu given", fn, need, workspace_bytes);
  const Buf ins[] = {{q, nk}, {k, nk}, {v, nv}, {grad_y, nv}, {state_in, ns}, {grad_state_out, ns}};
  const Buf outs[] = {{grad_q, nk}, {grad_k, nk}, {grad_v, nv}, {grad_state_in, ns}};
  if (need > 0) {
    for (const Buf& b : ins)
      if (overlap(workspace, need, b.p, b.n)) return fail(RET_ERR_INVALID_ARG, "%s: workspace overlaps another argument", fn);
    for (const Buf& b : outs)
      if (overlap(workspace, need, b.p, b.n)) return fail(RET_ERR_INVALID_ARG, "%s: workspace overlaps another argument", fn);
  }
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j) {
      const bool in_place = i == 3 && j == 5 && outs[i].p == ins[j].p;
      if (!in_place && overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n))
        return fail(RET_ERR_INVALID_ARG, "%s: a gradient output overlaps an input", fn);
    }
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(RET_ERR_INVALID_ARG, "%s: gradient outputs overlap", fn);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    if (grad_state_in == nullptr || grad_state_in == grad_state_out) return ok();
    const hipError_t e = ret::launch_state_copy(grad_state_out, grad_state_in, ns / 4, s);
    return e == hipSuccess ? ok() : hip_fail(fn, e);
  }
  const ret::BwdArgs a{q, k, v, state_in, grad_y, grad_state_out, grad_q, grad_k, grad_v, grad_state_in};
  const bool mfma = ret::chunkwise_bwd_mfma_supports(dk, dv, static_cast<int>(dt));
  const bool f32 = ret::chunkwise_f32_mfma_supports(dk, dv, static_cast<int>(dt));
  return for_head_groups(fn, H, gamma, [&](const ret::HeadGroup& g) {
    if (mfma) return ret::launch_chunkwise_bwd_mfma(a, B, H, T, dk, dv, static_cast<float*>(workspace), g, s);
    if (f32) return ret::launch_chunkwise_f32_bwd(a, B, H, T, dk, dv, g, s);
    return ret::launch_chunkwise_bwd_generic(a, B, H, T, dk, dv, static_cast<int>(dt), g, s);
  });
}

ret_status retention_group_norm(const void* y, const float* weight, const float* bias, float eps, void* out, int B,
                                int H, int T, int dv, ret_dtype dt, void* stream) {
  const char* fn = "retention_group_norm";
  if (B < 1 || H < 1) return fail(RET_ERR_INVALID_ARG, "%s: B=%d and H=%d must be >= 1", fn, B, H);
  if (T < 0) return fail(RET_ERR_INVALID_ARG, "%s: T=%d must be >= 0", fn, T);
  if (dv < 1) return fail(RET_ERR_INVALID_ARG, "%s: dv=%d must be >= 1", fn, dv);
  if (dt != RET_F32 && dt != RET_BF16)
    return fail(RET_ERR_UNSUPPORTED, "%s: dtype %d is not RET_F32 or RET_BF16", fn, static_cast<int>(dt));
  if (dv > RET_MAX_DV) return fail(RET_ERR_UNSUPPORTED, "%s: dv=%d exceeds %d", fn, dv, RET_MAX_DV);
  if (!std::isfinite(eps) || eps < 0.0f)
    return fail(RET_ERR_INVALID_ARG, "%s: eps = %g must be finite and >= 0", fn, static_cast<double>(eps));
  const long long n = static_cast<long long>(B) * H * T * dv;
  if (n > kMaxElems) return fail(RET_ERR_UNSUPPORTED, "%s: y has 2^31 or more elements", fn);
  if (T > 0 && (y == nullptr || out == nullptr)) return fail(RET_ERR_INVALID_ARG, "%s: y and out are required", fn);
  if (misaligned(y) || misaligned(out) || misaligned(weight) || misaligned(bias))
    return fail(RET_ERR_UNSUPPORTED, "%s: tensor pointers must be 16-byte aligned", fn);
  const size_t ny = static_cast<size_t>(n) * dsize(dt);
  const size_t nw = static_cast<size_t>(H) * dv * 4;
  if (out != y && overlap(out, ny, y, ny))
    return fail(RET_ERR_INVALID_ARG, "%s: out overlaps y without being the same buffer", fn);
  if (overlap(out, ny, weight, nw) || overlap(out, ny, bias, nw))
    return fail(RET_ERR_INVALID_ARG, "%s: out overlaps weight or bias", fn);
  if (T == 0) return ok();
  const hipError_t e = ret::launch_group_norm(y, weight, bias, eps, out, B, H, T, dv, static_cast<int>(dt),
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(fn, e);
}

}  // extern "C"
