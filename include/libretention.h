/*
 * libretention — multi-scale retention on AMD Instinct MI355X (gfx950).
 *
 * The operator, per batch b and head h with decay gamma_h in [0, 1]:
 *
 *   Y_n = sum_{m <= n} gamma^(n-m) (Q_n . K_m) V_m  +  gamma^(n+1) Q_n S_in
 *
 * The first term is the retention definition of "Retentive Networks — Microsoft
 * Propone l'Alternativa Architetturale ai Transformer" (aimpact.prandi.net),
 * section "Il meccanismo: Multi-Scale Retention", which also gives the
 * recurrent form S_n = gamma S_(n-1) + K_n^T V_n, Y_n = Q_n S_n, names the
 * parallel and chunkwise forms as equivalent, and makes gamma a per-head
 * hyperparameter.  The second term is the contribution of an initial state
 * S_in (zero when none is passed).  No softmax, scale, clamp or denominator is
 * applied (author answers to Q2 and Q3 on the paperhub.cn page "Retentive
 * Network: A Successor to Transformer for Large Language Models"); the state
 * has shape d_k x d_v (answer to Q1 on inference cost there).
 *
 * Conventions shared by every entry point
 *   - Layouts (row-major, contiguous):
 *       q, k : [B, H, T, dk]      v, y : [B, H, T, dv]
 *       state: [B, H, dk, dv] fp32 (always fp32, whatever the input dtype)
 *     decode step: q, k [B, H, dk]; v, y [B, H, dv]; state as above.
 *   - q, k, v and y share one dtype (RET_F32 or RET_BF16); arithmetic and
 *     accumulation are fp32; y is rounded to the dtype (round to nearest even).
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device,
 *     owned by the caller; the library keeps no pointer after the call and
 *     allocates no device memory.  Tensor pointers must be 16-byte aligned.
 *   - gamma is a HOST array of H floats, read during the call only.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; no call synchronises the device.
 *   - Validation happens before any HIP call.  On error nothing is enqueued,
 *     no output is touched, and retention_last_error() describes the problem.
 *   - Thread safety: calls from different host threads are independent;
 *     the error text is thread-local.
 */
#ifndef LIBRETENTION_H_
#define LIBRETENTION_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RET_F32 = 0, RET_BF16 = 1 } ret_dtype;

typedef enum {
  RET_OK = 0,
  RET_ERR_INVALID_ARG = 1, /* null required pointer, negative size, gamma not finite or outside [0,1] */
  RET_ERR_UNSUPPORTED = 2, /* valid but outside what is built (see the limits below) */
  RET_ERR_HIP = 3          /* a HIP launch failed; the text carries hipGetErrorString */
} ret_status;

/* Limits of this build: 1 <= dk <= 256, 1 <= dv <= 512, 1 <= C <= 128,
 * B, H >= 1, T >= 0, B*H*T and every tensor's element count below 2^31. */
#define RET_MAX_DK 256
#define RET_MAX_DV 512
#define RET_MAX_CHUNK 128

/*
 * Parallel form: Y = ((Q K^T) .* D) V + diag(gamma^(n+1)) Q S_in, with the causal
 * decay mask D[n,m] = gamma^(n-m) for n >= m (D[n,n] = 1, also for gamma = 0)
 * and 0 above the diagonal.  The aimpact page ("Il meccanismo") describes this
 * form as computing the whole retention matrix at once, like attention; the
 * baulab page "Retention Networks Explained" ("Methodology and Architecture")
 * calls it the representation used for training.
 *   state_in : nullable; fp32 [B,H,dk,dv].
 *   y        : written, [B,H,T,dv] in dt.  Must not alias an input.
 * O(T^2) work per head: meant for short sequences and as a cross-check.
 */
ret_status retention_parallel_fwd(const void* q, const void* k, const void* v, const float* gamma,
                                  const float* state_in, void* y, int B, int H, int T, int dk, int dv,
                                  ret_dtype dt, void* stream);

/*
 * Chunkwise form with chunk length C: the sequence is cut into chunks of C
 * tokens (the last may be shorter); inside a chunk the parallel form runs, and
 * a d_k x d_v state carries the past across chunks (aimpact page, "Il
 * meccanismo").  For chunk i with rows j = 0..L-1 and carried state R_i:
 *   Y_[i]   = ((Q_[i] K_[i]^T) .* D_L) V_[i] + diag(gamma^(j+1)) Q_[i] R_i
 *   R_(i+1) = gamma^L R_i + (diag(gamma^(L-1-j)) K_[i])^T V_[i],  R_0 = S_in.
 *   state_in  : nullable (zeros); fp32 [B,H,dk,dv].
 *   state_out : nullable; receives R after the last token, fp32 [B,H,dk,dv].
 *               May alias state_in exactly (in-place continuation).
 *   y         : written, [B,H,T,dv] in dt; must not alias an input.
 *   workspace : device scratch of at least retention_chunkwise_workspace_bytes()
 *               bytes for the same arguments (may be NULL when that is 0), owned
 *               by the caller, 16-byte aligned, overlapping no other argument;
 *               its contents on entry are ignored and on return undefined.  A
 *               missing or short workspace is RET_ERR_INVALID_ARG.
 * T = 0 is valid: y is untouched and state_out receives state_in (or zeros).
 * The result does not depend on C beyond rounding.  A segmented call (see
 * retention_chunkwise_workspace_bytes) leaves out of the segments' incoming
 * states every sub-segment, and every leading run of positions of one, that
 * reaches them only through a weight gamma^d <= 2^-40, far below the rounding
 * of the bf16 operands; every position's output is still computed.  Kernels, in the order the
 * call picks them: T = 1 with state_out == state_in runs the recurrent step;
 * bf16 blocks of 1 <= T <= 64 tokens with dk % 32 == 0 and dv % 64 == 0 run
 * as one chunk in a single streaming pass over the state on bf16 MFMA; other
 * blocks of 1 <= T <= 32 tokens with dk % 16 == 0 and dv % 64 == 0 (either
 * dtype) the same way on fp32 MFMA; other blocks of T <= 16 tokens the same
 * way on fp32 VALU arithmetic; bf16 inputs with dk in {64,128,256} and
 * dv % 64 == 0 run on bf16 MFMA with chunks of C; fp32 inputs with dk in
 * {64,128,256} and dv in {64,128,256,512} run on fp32 MFMA with 16-token
 * chunks; every other case runs on fp32 VALU arithmetic with chunks of C.
 * State and accumulators are fp32 throughout.
 */
ret_status retention_chunkwise_fwd(const void* q, const void* k, const void* v, const float* gamma,
                                   const float* state_in, float* state_out, void* y, int B, int H, int T,
                                   int dk, int dv, int C, ret_dtype dt, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Workspace size for retention_chunkwise_fwd with these arguments (0 when the
 * chosen kernel needs none).  bf16 calls whose (batch, head, 64-column tile)
 * count is below the device's 256 compute units and whose sequence has at
 * least 16 chunks run in sequence segments; they need one fp32 state slot per
 * segment and per sub-segment of the pass that finds the segments' incoming
 * states: (nseg + nsub * (nseg - 1)) * B * H * dk * dv * 4 bytes.  A pure
 * function of the sizes.  Returns (size_t)-1 for arguments the call would
 * reject. */
size_t retention_chunkwise_workspace_bytes(int B, int H, int T, int dk, int dv, int C, ret_dtype dt);

/*
 * retention_chunkwise_fwd without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments, results, validation and
 * kernels are those of retention_chunkwise_fwd.  A call that needs a workspace
 * (retention_chunkwise_workspace_bytes() > 0: the segmented calls) uses a
 * static device array of RET_NOALLOC_SCRATCH_BYTES bytes inside the library
 * instead; each GPU the library runs on holds its own copy until the process
 * ends.  A call whose workspace would exceed it returns RET_ERR_UNSUPPORTED
 * (the long-context workload B1 H8 T65536 dk256 dv512 C128 needs exactly
 * 64 MiB and fits).  Nothing is allocated: no hipMalloc, hipFree or allocating
 * library routine is called.  All calls on one GPU share that GPU's array:
 * calls ordered on one stream are safe, but calls that overlap in time on one
 * GPU (several streams, or several host threads) race on it and give
 * undefined results.  Its contents on entry are ignored (every slot a call
 * reads was written earlier in the same call).
 */
#define RET_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ret_status retention_chunkwise_fwd_noalloc(const void* q, const void* k, const void* v, const float* gamma,
                                           const float* state_in, float* state_out, void* y, int B, int H,
                                           int T, int dk, int dv, int C, ret_dtype dt, void* stream);

/*
 * Backward of the chunkwise form: the gradients of retention_chunkwise_fwd for
 * the loss L = sum <grad_y, y> + <grad_state_out, state_out>.  The aimpact page
 * ("Il meccanismo") says the parallel form is the one run in parallel for
 * training; the gradients are the chain rule applied to its recurrence
 * S_n = gamma S_(n-1) + K_n^T V_n, Y_n = Q_n S_n, S_(-1) = state_in.  With
 * G_n = dL/dS_n = Q_n^T dY_n + gamma G_(n+1) (G_(T-1) also receives
 * grad_state_out):
 *   grad_q[n] = dY_n S_n^T     grad_k[n] = G_n V_n^T     grad_v[n] = K_n G_n
 *   grad_state_in = gamma G_0  (grad_state_out, or zeros, when T = 0)
 * gamma (host) and the dtype dt are those of the forward call; q, k, v and
 * state_in are the forward inputs (state_in nullable: zeros).
 *   grad_y         : [B,H,T,dv] in dt.
 *   grad_state_out : nullable (zeros); fp32 [B,H,dk,dv].
 *   grad_q, grad_k : written, [B,H,T,dk] in dt.   grad_v : written, [B,H,T,dv] in dt.
 *   grad_state_in  : nullable; written, fp32 [B,H,dk,dv].  May be the
 *                    grad_state_out buffer exactly (in place).
 *   workspace      : device scratch of at least retention_chunkwise_bwd_workspace_bytes()
 *                    bytes (may be NULL when that is 0), owned by the caller,
 *                    16-byte aligned, overlapping no other argument; contents
 *                    on entry ignored, on return undefined.  A missing or
 *                    short workspace is RET_ERR_INVALID_ARG.
 * The written gradients must not overlap each other or any input (apart from
 * that in-place case).  C is the chunk length of the forward call (validated
 * like there); the gradients do not depend on it beyond rounding, and the
 * kernels choose their own chunking.  State and accumulators are fp32; bf16
 * inputs with dk in {64, 128, 256} and dv in {64, 128, 256, 512} take bf16
 * MFMA products (as the forward does), fp32 inputs with those dk and dv fp32
 * MFMA products, every other case (dk <= 256, dv <= 512) fp32 VALU arithmetic.
 */
ret_status retention_chunkwise_bwd(const void* q, const void* k, const void* v, const float* gamma,
                                   const float* state_in, const void* grad_y, const float* grad_state_out,
                                   void* grad_q, void* grad_k, void* grad_v, float* grad_state_in, int B, int H,
                                   int T, int dk, int dv, int C, ret_dtype dt, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Workspace size for retention_chunkwise_bwd with these arguments (0 when the
 * call needs none: fp32 inputs, or enough (batch, head, column) walkers to fill
 * the device).  Few heads over a long sequence are split into sequence
 * segments whose incoming states are found by a scan; the workspace holds one
 * fp32 state per segment and sub-segment and pass:
 * 3 * (nseg + nsub * (nseg - 1)) * B*H*dk*dv * 4 bytes.  Returns (size_t)-1
 * for arguments the call would reject. */
size_t retention_chunkwise_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C, ret_dtype dt);

/*
 * Per-head GroupNorm of a retention output: every head is one group (the
 * paperhub page, author answer A4: GroupNorm rather than LayerNorm because the
 * heads have different statistics).  For each (b, h, t), over c = 0..dv-1:
 *   mu = mean_c y, var = mean_c (y - mu)^2 (biased),
 *   out[c] = (y[c] - mu) / sqrt(var + eps) * weight[h][c] + bias[h][c].
 * The gate that follows it in a retention layer is not part of this call.
 *   y      : [B,H,T,dv] in dt (the layout retention_*_fwd write).
 *   weight : nullable (ones); device fp32 [H,dv].  bias : nullable (zeros); device fp32 [H,dv].
 *   eps    : finite, >= 0.
 *   out    : written, [B,H,T,dv] in dt; may be y exactly (in place), must not
 *            overlap it otherwise, nor weight or bias.
 * fp32 arithmetic; the output is rounded to dt.
 */
ret_status retention_group_norm(const void* y, const float* weight, const float* bias, float eps, void* out, int B,
                                int H, int T, int dv, ret_dtype dt, void* stream);

/*
 * The chunkwise forward followed by the per-head GroupNorm of its output, in
 * one pass: y receives retention_group_norm(retention_chunkwise_fwd(...)) and
 * the un-normalised output is never written to memory.  The paperhub page
 * (author answer A4) names GroupNorm per head as the normalisation of
 * multi-scale retention; the closing list there names retention and group
 * normalization together.  Arguments are those of retention_chunkwise_fwd
 * plus weight, bias and eps of retention_group_norm (weight/bias nullable,
 * device fp32 [H,dv]; eps finite, >= 0); state_out receives the carried state
 * as there.  The outputs are rounded to dt before they are normalised, as the
 * two separate calls do; the statistics are fp32.
 * bf16 calls on the bf16 MFMA kernel (dk in {64,128,256}, dv % 64 == 0,
 * dv <= 512, T > 64) normalise inside that kernel: the dv/64 column-tile
 * workgroups of a head exchange per-row partial statistics through the
 * workspace.  Every other call runs the forward and then
 * retention_group_norm on y in place.
 *   workspace : at least retention_chunkwise_fwd_group_norm_workspace_bytes()
 *               bytes (may be NULL when that is 0), 16-byte aligned, owned by
 *               the caller, overlapping no other argument.  For the fused
 *               kernel its first 32-bit word is 0 after the call, or 1 if a
 *               workgroup gave up waiting for another tile's statistics
 *               (possible only if the tiles of a head cannot all be resident
 *               on the device at once; y is then wrong).
 * Errors as retention_chunkwise_fwd; y must not overlap weight or bias.
 */
ret_status retention_chunkwise_fwd_group_norm(const void* q, const void* k, const void* v, const float* gamma,
                                              const float* state_in, float* state_out, const float* weight,
                                              const float* bias, float eps, void* y, int B, int H, int T, int dk,
                                              int dv, int C, ret_dtype dt, void* workspace, size_t workspace_bytes,
                                              void* stream);

/* Workspace size for retention_chunkwise_fwd_group_norm (0 when the call
 * needs none).  Fused calls: 256 bytes + the segment slots of
 * retention_chunkwise_workspace_bytes (rounded up to 256 bytes) + 8 bytes per
 * row and column tile, nseg * B * H * (dv/64) * seg_len * 8, where seg_len is
 * the segment length (T without segments).  Other calls: the forward's
 * workspace.  Returns (size_t)-1 for arguments the call would reject. */
size_t retention_chunkwise_fwd_group_norm_workspace_bytes(int B, int H, int T, int dk, int dv, int C, ret_dtype dt);

/*
 * Testing hook for the fused call's failure path (not for production use):
 * sets, process-wide, the number of polls after which a wait for another
 * tile's statistics gives up (default 65536, >= 1) and a column tile whose
 * statistics are never published (-1, the default: none).  With a silent
 * tile every wait of that head gives up, so the error word of
 * retention_chunkwise_fwd_group_norm becomes 1 and y is wrong, while every
 * workgroup still finishes.  retention_testing_gn_wait(65536, -1) restores
 * the defaults.  Not thread-safe: no fused call may run concurrently.
 * Errors: RET_ERR_INVALID_ARG for spin_limit < 1 or silent_tile < -1.
 */
ret_status retention_testing_gn_wait(int spin_limit, int silent_tile);

/*
 * One recurrent (decode) step, in place on the state: S <- gamma S + k^T v,
 * then y = q S (the new state, so the current token is included).  This is the
 * recurrent form of the aimpact page ("Il meccanismo"); the baulab page
 * ("Methodology and Architecture") calls it the O(1)-per-token inference
 * representation.
 *   q, k  : [B,H,dk] in dt.   v : [B,H,dv] in dt.
 *   state : in/out, fp32 [B,H,dk,dv]; required; must not overlap q, k or v.
 *   y     : written, [B,H,dv] in dt; must not alias the other arguments.
 */
ret_status retention_recurrent_step(const void* q, const void* k, const void* v, const float* gamma,
                                    float* state, void* y, int B, int H, int dk, int dv, ret_dtype dt,
                                    void* stream);

/* Text of the last error on this host thread ("" after a successful call).
 * Valid until the next libretention call on the same thread. */
const char* retention_last_error(void);

/* Library version as 10000*major + 100*minor + patch. */
int retention_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBRETENTION_H_ */
