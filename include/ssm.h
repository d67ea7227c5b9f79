/*
 * libssm: selective scan and scalar-decay chunked SSD forward on AMD MI355X
 * (gfx950).  Plain C ABI: device pointers, sizes, a HIP stream; no torch types.
 *
 * Sources of the definitions (page titles, then the section):
 *   [Mamba on Trainium]  "We brought Mamba to Trainium - and mapped where
 *                        custom kernels actually help"
 *   [Mamba-3 NKI]        "Mamba-3 NKI Kernels for AWS Neuron"
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; scratch memory ("workspace") is
 *     passed in by the caller through the dims struct.
 *   - Every tensor is dense, row-major, with the last listed index contiguous.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *     A kernel fault surfaces at the caller's next synchronisation.
 *   - All argument checks run on the host before any HIP call.  A call that
 *     fails a check returns a negative ssm_status_t, launches nothing and
 *     writes nothing; ssm_last_error() then holds a one-line reason (per
 *     host thread).  SSM_ERR_HIP is returned when a launch itself fails.
 *   - Pointers must be aligned to their element size (4 bytes for float32,
 *     2 for bfloat16), and more where an entry point says so; otherwise
 *     SSM_ERR_ALIGN.
 *   - Unsupported sizes return SSM_ERR_UNSUPPORTED; there is no fallback path.
 *   - Indices and offsets are 64-bit throughout.
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point is exported from libssm.so; nothing else is. */
#define SSM_API __attribute__((visibility("default")))

/* Storage dtypes. Arithmetic is float32 in every kernel. */
typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = -1,        /* a required pointer is NULL                    */
  SSM_ERR_SHAPE = -2,       /* negative size, ngroups does not divide, ...   */
  SSM_ERR_DTYPE = -3,       /* dtype code is not an ssm_dtype_t              */
  SSM_ERR_ALIGN = -4,       /* pointer not aligned to its element size       */
  SSM_ERR_UNSUPPORTED = -5, /* valid but not implemented (e.g. dstate = 12)  */
  SSM_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required    */
  SSM_ERR_HIP = -7          /* a HIP launch failed                           */
} ssm_status_t;

/*
 * dims.flags bits; every other bit must be 0.
 *   SSM_DT_SOFTPLUS: the delta (dt) argument holds raw values and every kernel
 *     steps with softplus(delta + dt_bias), softplus(v) = log(1 + exp(v)),
 *     dt_bias being the per-channel (per-head) float32 vector named in the
 *     dims (zero when NULL; it must be NULL without this flag).  Steps past
 *     the end of a sequence still count as zero steps.
 *     [Mamba-3 NKI], "How it works", Phase 0: dt_softplus = softplus(dt + dt_bias).
 *   SSM_LAM_SIGMOID (ssd_trap_chunked_fwd only): lam holds raw values and the
 *     recurrence uses sigmoid(lam) = 1 / (1 + exp(-lam)).
 *     [Mamba-3 NKI], "How it works", Phase 0: lam_sigmoid = sigmoid(lam).
 */
enum { SSM_DT_SOFTPLUS = 1, SSM_LAM_SIGMOID = 2 };

/* ------------------------------------------------------------------------ */
/* Selective scan                                                            */
/* ------------------------------------------------------------------------ */

/*
 * Sizes of one selective-scan call.
 *   batch, dim (channels), dstate (N), seqlen (L), ngroups (G; G divides dim,
 *   channel d reads the B/C of group d / (dim / G)).
 *   in_dtype : storage dtype of u, delta, B, C, z.
 *   out_dtype: storage dtype of y.  A, D and h_last are always float32.
 *   n_chunks : 0 = the library picks; 1 = one sequential pass per channel;
 *              k > 1 = split L into chunks of len = 32 * ceil(ceil(L / k) / 32)
 *              steps (ceil(L / len) <= k chunks) that run in parallel, joined
 *              by the (decay product, state) carry.
 *   flags    : 0 or SSM_DT_SOFTPLUS.
 *   workspace, workspace_bytes: caller-owned device scratch of at least
 *              ssm_scan_workspace_size() bytes (may be NULL when that is 0).
 *   dt_bias  : (dim) float32, nullable; read only with SSM_DT_SOFTPLUS.
 * Supported: dstate in {1, 2, 4, 8, 16, 32, 64}; any batch, dim, seqlen >= 0.
 */
typedef struct {
  int64_t batch, dim, dstate, seqlen, ngroups;
  int32_t in_dtype, out_dtype;
  int32_t n_chunks;
  int32_t flags;
  void *workspace;
  size_t workspace_bytes;
  const float *dt_bias;
} ssm_scan_dims_t;

/*
 * Workspace the scan needs for `dims` (with n_chunks resolved as the call
 * would resolve it).  Writes *bytes; returns SSM_OK or a check failure.
 * The chunked carry keeps, per (batch, channel, chunk but the last, state),
 * the chunk's decay product and its local end state: 8 * batch * dim *
 * (chunks - 1) * dstate bytes.  One pass (a single chunk) needs none.
 */
SSM_API int ssm_scan_workspace_size(const ssm_scan_dims_t *dims, size_t *bytes);

/* The chunk count ssm_scan_fwd uses for `dims` (resolves n_chunks = 0). */
SSM_API int ssm_scan_resolved_chunks(const ssm_scan_dims_t *dims, int32_t *n_chunks);

/*
 * The same workspace size as the return value: the bytes ssm_scan_fwd needs
 * for `dims`, or SIZE_MAX when `dims` fails a check (ssm_last_error_message()
 * then says why).
 */
SSM_API size_t ssm_scan_workspace_bytes(const ssm_scan_dims_t *dims);

/*
 * Selective-scan forward.
 *
 * For every batch b and channel d (state h in R^N; before t = 0 it is
 * h0[b,d,:], or zero when h0 is NULL):
 *   h_t[n] = exp(delta_t * A[d,n]) * h_{t-1}[n] + delta_t * B_t[n] * u_t
 *   y_t    = (sum_n C_t[n] * h_t[n] + D[d] * u_t) * silu(z_t)
 * with silu(z) = z / (1 + exp(-z)); the D term is dropped when D is NULL and
 * the gate when z is NULL.  h_last receives h after the last step.
 *   [Mamba on Trainium], "Mamba: bringing an unsupported model to the chip":
 *     the state update h_t = Abar_t h_{t-1} + Bbar_t x_t and readout
 *     y_t = sum_n C_t h_t, walked along the sequence.
 *   [Mamba-3 NKI], "How it works", Phase 0: decay alpha = exp(dt * A) and
 *     input weight gamma = lam * dt, here with lam = 1 (so Bbar x = dt B x);
 *     Phase 5: the D skip connection, then the silu gate.
 *   [Mamba on Trainium], "We built the parallel scan": the recurrence is
 *     associative, which the chunked carry (n_chunks > 1) relies on.
 *
 * Layouts (in_dtype unless noted):
 *   u, delta, z : (batch, dim, seqlen)         z nullable
 *   A           : (dim, dstate) float32
 *   B, C        : (batch, ngroups, dstate, seqlen)
 *   D           : (dim) float32                nullable
 *   h0          : (batch, dim, dstate) float32  nullable (initial state)
 *   y           : (batch, dim, seqlen) out_dtype
 *   h_last      : (batch, dim, dstate) float32  nullable
 * y and h_last must not overlap any input, with one exception: h_last may be
 * exactly h0 (the state updated in place, as when a prefill continues from a
 * cache) when the call runs as one pass (ssm_scan_resolved_chunks() == 1).
 * With h0 = the h_last of a call on steps [0, L1), a call on [L1, L) continues
 * that sequence.  bfloat16 y is rounded to nearest even from the float32
 * result.
 */
SSM_API int ssm_scan_fwd(const void *u, const void *delta, const float *A, const void *B,
                 const void *C, const float *D, const void *z, const float *h0, void *y,
                 float *h_last, const ssm_scan_dims_t *dims, void *stream);

/*
 * Allocation-free selective-scan forward, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, math,
 * supported sizes and checks as ssm_scan_fwd; dims->workspace and
 * dims->workspace_bytes are ignored.  The chunked carry (needed only when
 * ssm_scan_resolved_chunks() > 1: 8 * batch * dim * (chunks - 1) * dstate
 * bytes) lives instead in a static device array of 16 MiB that the library
 * holds on each GPU it runs on until the process ends; a call whose carry
 * would exceed it returns SSM_ERR_WORKSPACE and launches nothing.  The call
 * allocates and frees nothing (its first call on a device looks up that
 * device's copy of the array).  Every chunk's carry is written before it is
 * read within one call, so nothing in the array needs clearing; but all calls
 * on one GPU share the array, so calls that may overlap in time on one GPU
 * (on different streams, or from several host threads) race and must be
 * serialised by the caller.
 */
SSM_API int ssm_scan_fwd_noalloc(const void *u, const void *delta, const float *A, const void *B,
                         const void *C, const float *D, const void *z, const float *h0, void *y,
                         float *h_last, const ssm_scan_dims_t *dims, void *stream);

/*
 * Workspace ssm_scan_bwd needs for `dims` (n_chunks is ignored), 4 bytes per
 * float: the forward state every 16 steps, batch * dim * dstate *
 * ceil(seqlen / 16) floats; the dB and dC terms of every tile of
 * 256 / dstate channels, 2 * batch * ngroups * ceil(dim / ngroups /
 * (256 / dstate)) * dstate * seqlen floats; and per-batch dA and dD terms,
 * batch * dim * (dstate + 1) floats.
 */
SSM_API int ssm_scan_bwd_workspace_size(const ssm_scan_dims_t *dims, size_t *bytes);

/*
 * Selective-scan backward: gradients of a loss L with respect to every input
 * of ssm_scan_fwd, given dy = dL/dy and dh_last = dL/dh_last.
 *
 * The chain rule on the forward above (the pages report gradient checks,
 * [Mamba-3 NKI] "Correctness", backward parity, but print no backward).  With
 * yhat = C.h + D u the output before the gate and lambda_t = dL/dh_t, walked
 * from the last step to the first (lambda after the last step = dh_last):
 *   dyhat_t  = dy_t silu(z_t),  dz_t = dy_t yhat_t silu'(z_t)
 *   lambda_t = dyhat_t C_t + exp(delta_{t+1} A) lambda_{t+1}
 *   du_t     = dyhat_t D + sum_n lambda_t delta_t B_t
 *   ddelta_t = sum_n lambda_t (B_t u_t + A exp(delta_t A) h_{t-1})
 *   dB_t     = sum over the group's channels of lambda_t delta_t u_t
 *   dC_t     = sum over the group's channels of dyhat_t h_t
 *   dA       = sum over batch and steps of lambda_t delta_t exp(delta_t A) h_{t-1}
 *   dD       = sum over batch and steps of dyhat_t u_t;   dh0 = exp(delta_0 A) lambda_0
 * The forward is recomputed (from h0, checkpointed every 16 steps in the
 * workspace); nothing from the forward call is needed.
 *
 * Inputs: as ssm_scan_fwd (dims, u, delta, A, B, C, D, z, h0), plus
 *   dy      : (batch, dim, seqlen) out_dtype
 *   dh_last : (batch, dim, dstate) float32, nullable (zero)
 * Outputs (overwritten):
 *   du, ddelta : (batch, dim, seqlen) in_dtype
 *   dz         : (batch, dim, seqlen) in_dtype, required when z is given
 *   dA         : (dim, dstate) float32
 *   dB, dC     : (batch, ngroups, dstate, seqlen) float32
 *   dD         : (dim) float32, required when D is given (ignored otherwise)
 *   dh0        : (batch, dim, dstate) float32, nullable
 * No output may overlap an input, another output or the workspace.  The sums
 * over channels (dB, dC) and over batch rows (dA, dD) are formed per channel
 * tile or batch row in the workspace and then added in a fixed order, so every
 * output is deterministic.  Supported sizes are those of ssm_scan_fwd.
 * With SSM_DT_SOFTPLUS the recurrence runs on softplus(delta + dt_bias) and
 * ddelta is the gradient with respect to the raw delta (the softplus chain
 * applied, i.e. times sigmoid(delta + dt_bias)); the gradient of dt_bias is
 * the sum of ddelta over batch and steps.
 */
SSM_API int ssm_scan_bwd(const void *u, const void *delta, const float *A, const void *B,
                 const void *C, const float *D, const void *z, const float *h0, const void *dy,
                 const float *dh_last, void *du, void *ddelta, float *dA, float *dB, float *dC,
                 float *dD, void *dz, float *dh0, const ssm_scan_dims_t *dims, void *stream);

/* ------------------------------------------------------------------------ */
/* Scalar-decay chunked SSD                                                  */
/* ------------------------------------------------------------------------ */

/*
 * Sizes of one SSD call.
 *   batch, seqlen (L), nheads (H), headdim (P), dstate (N), ngroups (G; G
 *   divides H, head h reads group h / (H / G)), chunk (Q).
 *   in_dtype must be SSM_BF16 (the intra-chunk contractions run on bf16
 *   matrix cores with float32 accumulation); out_dtype is SSM_BF16 or SSM_F32.
 *   flags: 0, SSM_DT_SOFTPLUS, and (ssd_trap_chunked_fwd) SSM_LAM_SIGMOID.
 *   dt_bias: (nheads) float32, nullable; read only with SSM_DT_SOFTPLUS.
 * Supported: headdim = 64, dstate in {64, 128}, chunk = 64, any seqlen >= 0
 * (a ragged last chunk is masked); nheads * headdim and ngroups * dstate below
 * 2^25 (a chunk's rows are addressed with 32-bit offsets), else
 * SSM_ERR_UNSUPPORTED.
 * Alignment: x, z, B, C, h0 and h_last must be 16-byte aligned (they are read
 * and written as 16-byte vectors); dt and y need their element alignment.
 */
typedef struct {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
  int32_t in_dtype, out_dtype;
  int32_t flags;
  int32_t reserved;
  void *workspace;
  size_t workspace_bytes;
  const float *dt_bias;
} ssd_dims_t;

/* Workspace the SSD needs for `dims` (currently always 0). */
SSM_API int ssd_workspace_size(const ssd_dims_t *dims, size_t *bytes);

/* The same as the return value, or SIZE_MAX when `dims` fails a check. */
SSM_API size_t ssd_workspace_bytes(const ssd_dims_t *dims);

/*
 * Scalar-decay SSD forward: the selective scan with one decay per (batch,
 * time, head), shared by the head's headdim x dstate states, computed chunk by
 * chunk with matrix-core contractions.
 *
 * For every batch b and head h (state S in R^{P x N}; before t = 0 it is
 * h0[b,h,:,:], or zero when h0 is NULL):
 *   S_t   = exp(dt_t * A[h]) * S_{t-1} + dt_t * x_t B_t^T
 *   y_t   = (S_t C_t + D[h] * x_t) * silu(z_t)
 *   [Mamba-3 NKI], "Kernel details", mamba3_siso_ssd_kernel: a chunked SSD
 *     with the Mamba-2 structure and chunk size 64 (the trapezoidal and
 *     rotary Mamba-3 terms are not part of this call);
 *   [Mamba-3 NKI], "Repository layout": segsum and causal masks;
 *   [Mamba-3 NKI], "How it works", Phase 0 (alpha = exp(dt * A)) and Phase 5
 *     (D skip, silu gate);
 *   [Mamba on Trainium], "We built the parallel scan": the state passes from
 *     chunk to chunk by the associative (decay, state) combine.
 *
 * Layouts:
 *   x, z    : (batch, seqlen, nheads, headdim) bf16    z nullable
 *   dt      : (batch, seqlen, nheads) bf16  (the step; with SSM_DT_SOFTPLUS
 *             the raw value, and the step is softplus(dt + dt_bias[h]))
 *   A, D    : (nheads) float32                          D nullable
 *   B, C    : (batch, seqlen, ngroups, dstate) bf16
 *   h0      : (batch, nheads, headdim, dstate) float32  nullable (initial state)
 *   y       : (batch, seqlen, nheads, headdim) out_dtype
 *   h_last  : (batch, nheads, headdim, dstate) float32  nullable
 * h0 and h_last must be 16-byte aligned; h_last may be exactly h0 (updated in
 * place), any other overlap with an input is rejected.
 */
SSM_API int ssd_chunked_fwd(const void *x, const void *dt, const float *A, const void *B,
                    const void *C, const float *D, const void *z, const float *h0, void *y,
                    float *h_last, const ssd_dims_t *dims, void *stream);

/*
 * Trapezoidal (Mamba-3 SISO) form of the SSD, chunked.  Per token
 *   alpha_t = exp(dt_t A[h]),  gamma_t = lam_t dt_t,  beta_t = (dt_t - gamma_t) alpha_t
 *   S_t = alpha_t S_{t-1} + beta_t x_{t-1} B_{t-1}^T + gamma_t x_t B_t^T
 *   y_t = (S_t C_t + D[h] x_t) * silu(z_t)
 * with the previous-token term zero before the first token.
 *   [Mamba-3 NKI], "How it works", Phase 0: alpha, gamma = lam dt and
 *     beta = (dt - gamma) alpha (lam after its sigmoid, dt after its
 *     softplus: applied by the caller, or by the kernel with the flags
 *     SSM_LAM_SIGMOID and SSM_DT_SOFTPLUS); the step form is its Eq. 9;
 *   [Mamba-3 NKI], "Kernel details", mamba3_siso_ssd_kernel: chunked in the
 *     single-SSD form, the input of step s weighted by scale_s = gamma_s +
 *     dt_{s+1} (1 - lam_{s+1}) at later steps, plus a diagonal correction
 *     (weight gamma_s at its own step), chunk 64.
 * Arguments, layouts and supported sizes are those of ssd_chunked_fwd, plus
 *   lam    : (batch, seqlen, nheads) bf16, 2-byte aligned;
 *   x_prev : (batch, nheads, headdim) bf16, 16-byte aligned, nullable;
 *   B_prev : (batch, ngroups, dstate) bf16, 16-byte aligned, nullable;
 * x_prev and B_prev are the token before the sequence (given together or not
 * at all): the first token's previous-token term is beta_0 x_prev B_prev^T,
 * or zero when they are NULL.  h0 is the state S before the first token and
 * h_last is S after the last token, so a call on steps [L1, L) with h0 = the
 * h_last of a call on [0, L1) and x_prev, B_prev = x and B of step L1 - 1
 * continues that sequence exactly (and ssd_trap_step continues it token by
 * token the same way).
 * The rotary and normalisation steps that precede the SSD core in Mamba-3
 * are not part of this call.
 */
SSM_API int ssd_trap_chunked_fwd(const void *x, const void *dt, const void *lam, const float *A,
                         const void *B, const void *C, const float *D, const void *z,
                         const float *h0, const void *x_prev, const void *B_prev, void *y,
                         float *h_last, const ssd_dims_t *dims, void *stream);

/*
 * The SSD with the rotary step on B and C fused in (Mamba-3's complex-valued
 * state): the same result as ssm_rope_bc (per-head rotated B and C, bf16)
 * followed by ssd_chunked_fwd on them, without the rotated B and C ever being
 * stored.  For every batch b, head h and state pair k < N/2
 *   phi_t[k] = angle0[b,h,k] - sum_{s <= t} dt_s theta_s[b,h',k]
 *   (B_rot[k], B_rot[k + N/2]) = (B[k] cos phi - B[k + N/2] sin phi,
 *                                 B[k] sin phi + B[k + N/2] cos phi),  C alike,
 * and the SSD of ssd_chunked_fwd runs on B_rot, C_rot (rounded to bf16) of
 * head h.
 *   [Mamba-3 NKI], "How it works", Phase 1 (the rotation) then Phase 2 (the
 *     chunked SSD); the pairing (k, k + N/2) and the direction are this
 *     library's reading, as for ssm_rope_bc.
 * Arguments, layouts and supported sizes are those of ssd_chunked_fwd, plus
 *   theta       : (batch, seqlen, theta_heads, dstate / 2) bf16, 16-byte
 *                 aligned; theta_heads is 1 (shared by every head, h' = 0)
 *                 or nheads (h' = h);
 *   angle0      : (batch, nheads, dstate / 2) float32, nullable (zero);
 *   angle_last  : (batch, nheads, dstate / 2) float32, nullable; the angle
 *                 after the last step reduced to [-pi, pi]; may be exactly
 *                 angle0 (updated in place);
 *   B_last      : (batch, nheads, dstate) bf16, 16-byte aligned, nullable:
 *                 the rotated B of the last step (the previous-token input of
 *                 a trapezoidal continuation); untouched when seqlen is 0.
 * The angle is carried from chunk to chunk in float64 and summed within a
 * chunk in float32, in revolutions.  The SSD (dt_softplus included) is
 * computed as in ssd_chunked_fwd; with SSM_DT_SOFTPLUS the angles use the
 * mapped step.  Outputs must not overlap inputs or each other (angle_last ==
 * angle0, h_last == h0 excepted).
 */
SSM_API int ssd_rope_chunked_fwd(const void *x, const void *dt, const float *A, const void *B, const void *C,
                                 const void *theta, int64_t theta_heads, const float *angle0, const float *D,
                                 const void *z, const float *h0, void *y, float *h_last, float *angle_last,
                                 void *B_last, const ssd_dims_t *dims, void *stream);

/*
 * The trapezoidal form of ssd_rope_chunked_fwd: ssm_rope_bc followed by
 * ssd_trap_chunked_fwd on the per-head rotated B and C, fused.
 *   [Mamba-3 NKI], "How it works", Phases 0-2, and "Kernel details",
 *     mamba3_siso_ssd_kernel (the single-SSD form, as ssd_trap_chunked_fwd).
 * Arguments as ssd_rope_chunked_fwd plus lam, x_prev and B_prev as
 * ssd_trap_chunked_fwd, except that B_prev is per head, (batch, nheads,
 * dstate) bf16, and already rotated (the B_last of the call before, or the
 * rotated B that ssm_rope_bc gave for the previous token).
 */
SSM_API int ssd_rope_trap_chunked_fwd(const void *x, const void *dt, const void *lam, const float *A,
                                      const void *B, const void *C, const void *theta, int64_t theta_heads,
                                      const float *angle0, const float *D, const void *z, const float *h0,
                                      const void *x_prev, const void *B_prev, void *y, float *h_last,
                                      float *angle_last, void *B_last, const ssd_dims_t *dims, void *stream);

/*
 * Workspace ssd_bwd and ssd_trap_bwd need for `dims`.  With K =
 * ceil(seqlen / 64) chunks and the chunk kernel's hpw heads per workgroup (a
 * function of the sizes, up to 8): two bf16 state matrices per (batch, head,
 * chunk) (2 * batch * nheads * K * headdim * dstate * 2 bytes), two floats
 * per (batch, head, chunk), two float32 (batch, seqlen, nheads / hpw,
 * dstate) arrays of dB and dC terms, three floats per (batch, step, head),
 * one per (batch, head) and (batch, nheads, dstate) floats; each region
 * rounded up to 256 bytes.
 */
SSM_API int ssd_bwd_workspace_size(const ssd_dims_t *dims, size_t *bytes);

/*
 * Backward of the scalar-decay SSD (ssd_chunked_fwd): gradients of a loss L
 * with respect to every input, given dy = dL/dy and dh_last = dL/dh_last.
 *
 * The chain rule on the chunked form of ssd_chunked_fwd ([Mamba-3 NKI],
 * "Kernel details", the chunk-64 SSD; "Correctness" reports backward parity
 * of the SSD and prints no formulas).  With yhat = S C + D x, dyhat = dy
 * silu(z) and Lam_t = dL/dS_t (Lam after the last step = dh_last):
 *   dx_t  = dt_t Lam_t B_t + D dyhat_t,        dz_t = dy_t yhat_t silu'(z_t)
 *   ddt_t = sum_{p,n} Lam_t (x_t B_t^T + A exp(dt_t A) S_{t-1})
 *   dB_t  = sum over the group's heads of dt_t Lam_t^T x_t
 *   dC_t  = sum over the group's heads of S_t^T dyhat_t
 *   dA    = sum over batch and steps of dt_t sum Lam_t exp(dt_t A) S_{t-1}
 *   dD    = sum over batch and steps of dyhat_t . x_t;   dh0 = exp(dt_0 A) Lam_0
 * computed chunk by chunk: a forward pass rebuilds the state entering every
 * chunk from h0, a reverse pass the gradient leaving every chunk from
 * dh_last, and every chunk's gradients then follow from matrix products over
 * the chunk (bf16 operands, float32 accumulation, as the forward).  Nothing
 * from the forward call is needed.
 *
 * Inputs: as ssd_chunked_fwd (dims, x, dt, A, B, C, D, z, h0), plus
 *   dy      : (batch, seqlen, nheads, headdim) out_dtype
 *   dh_last : (batch, nheads, headdim, dstate) float32, nullable (zero)
 * Outputs (overwritten):
 *   dx, dz  : (batch, seqlen, nheads, headdim) bf16; dz required with z
 *   ddt     : (batch, seqlen, nheads) bf16 (with SSM_DT_SOFTPLUS: the
 *             gradient of the raw dt, i.e. times sigmoid(dt + dt_bias[h]))
 *   dA, dD  : (nheads) float32; dD required with D
 *   dB, dC  : (batch, seqlen, ngroups, dstate) float32
 *   dh0     : (batch, nheads, headdim, dstate) float32, nullable
 * The sums over heads (dB, dC) and over batch rows (dA, dD) run in a fixed
 * order, so every output is deterministic.  No output may overlap an input,
 * another output or the workspace (dims->workspace, at least
 * ssd_bwd_workspace_size() bytes, 16-byte aligned).  x, z, B, C, dy, h0,
 * dh_last and dh0 must be 16-byte aligned, the other pointers element
 * aligned.  Supported sizes are those of ssd_chunked_fwd; flags 0 or
 * SSM_DT_SOFTPLUS.
 */
SSM_API int ssd_bwd(const void *x, const void *dt, const float *A, const void *B, const void *C,
            const float *D, const void *z, const float *h0, const void *dy, const float *dh_last,
            void *dx, void *ddt, float *dA, float *dB, float *dC, float *dD, void *dz, float *dh0,
            const ssd_dims_t *dims, void *stream);

/*
 * Backward of the trapezoidal SSD (ssd_trap_chunked_fwd): gradients of a loss
 * L with respect to every input, given dy = dL/dy and dh_last = dL/dh_last.
 *
 * The chain rule on the three-term recurrence of ssd_trap_chunked_fwd
 * ([Mamba-3 NKI], "How it works": Eq. 9, H_t = alpha_t H_{t-1} +
 * beta_t B_{t-1} x_{t-1} + gamma_t B_t x_t with alpha = exp(dt A),
 * beta = dt (1 - lam) alpha, gamma = lam dt; "Correctness" reports backward
 * parity and prints no formulas).  With Lam_t = dL/dH_t:
 *   Lam_t  = dyhat_t C_t^T + alpha_{t+1} Lam_{t+1},   dQ_t = gamma_t Lam_t + beta_{t+1} Lam_{t+1}
 *   dx_t   = dQ_t B_t + D dyhat_t,   dB_t = sum over heads of dQ_t^T x_t,   dC_t as ssd_bwd
 *   ddt, dlam and dA through alpha, beta and gamma (the chain rule on each);
 *   dx_prev, dB_prev: the token before the sequence, through beta_0.
 * computed chunk by chunk as ssd_bwd, the input of step s weighted by
 * scale_s = gamma_s + dt_{s+1} (1 - lam_{s+1}) where it reaches a later step
 * and by gamma_s at its own step, as in the forward.
 *
 * Inputs: as ssd_trap_chunked_fwd (dims, x, dt, lam, A, B, C, D, z, h0,
 * x_prev, B_prev), plus dy and dh_last as ssd_bwd.
 * Outputs (overwritten): as ssd_bwd, plus
 *   dlam    : (batch, seqlen, nheads) bf16 (with SSM_LAM_SIGMOID: the gradient
 *             of the raw lam, i.e. times s (1 - s), s = sigmoid(lam))
 *   dx_prev : (batch, nheads, headdim) bf16 and dB_prev : (batch, ngroups,
 *             dstate) float32, required with x_prev and B_prev (ignored
 *             without them).
 * Workspace: ssd_bwd_workspace_size() bytes (one size serves both forms).
 * Flags: SSM_DT_SOFTPLUS and SSM_LAM_SIGMOID.  Alignment, overlap and size
 * rules as ssd_bwd; x_prev, B_prev and dx_prev element aligned.
 */
SSM_API int ssd_trap_bwd(const void *x, const void *dt, const void *lam, const float *A, const void *B,
                 const void *C, const float *D, const void *z, const float *h0, const void *x_prev,
                 const void *B_prev, const void *dy, const float *dh_last, void *dx, void *ddt, void *dlam,
                 float *dA, float *dB, float *dC, float *dD, void *dz, float *dh0, void *dx_prev,
                 float *dB_prev, const ssd_dims_t *dims, void *stream);

/* ------------------------------------------------------------------------ */
/* Rotary step on B and C (Mamba-3 complex-valued state)                     */
/* ------------------------------------------------------------------------ */

/*
 * Sizes of one rotary step.
 *   batch, seqlen (L), nheads (H), ngroups (G divides H; head h reads group
 *   h / (H / G)), dstate (N: a power of two from 2 to 256),
 *   theta_heads: 1 (one set of angles for every head) or nheads;
 *   in_dtype: dt, theta, B, C; out_dtype: B_rot, C_rot;
 *   flags: 0 or SSM_DT_SOFTPLUS (dt_bias: (nheads) float32, nullable);
 *   reserved: must be 0.
 */
typedef struct {
  int64_t batch, seqlen, nheads, ngroups, dstate, theta_heads;
  int32_t in_dtype, out_dtype;
  int32_t flags;
  int32_t reserved;
  const float *dt_bias;
} ssm_rope_dims_t;

/*
 * Rotary step on B and C: for every batch row b, head h and state pair
 * k < N/2 (states k and k + N/2, read as the complex number B[k] + i B[k+N/2])
 *   phi_t[k]   = angle0[b,h,k] - sum_{s <= t} dt_s[b,h] * theta_s[b,h',k]
 *   B_rot_t[k] = B_t[k] cos phi_t[k] - B_t[k + N/2] sin phi_t[k]
 *   B_rot_t[k + N/2] = B_t[k] sin phi_t[k] + B_t[k + N/2] cos phi_t[k]
 * and C alike with the same angle (h' = h, or 0 when theta_heads = 1).
 *   [Mamba-3 NKI], "How it works", Phase 1: the angles are the negated
 *     running sum of dt * theta, and B and C are rotated by them; the page's
 *     list of Mamba-3 features names this a complex-valued state driven by
 *     data-dependent RoPE.  The page gives no formula for the rotation; the
 *     pairing (k, k + N/2) and the direction are this library's reading.
 * The rotated B and C feed ssd_chunked_fwd / ssd_trap_chunked_fwd with
 * ngroups = nheads; chained over a sequence split in pieces (prefill then
 * decode), angle_last of one call is angle0 of the next.
 *
 * Layouts:
 *   dt         : (batch, seqlen, nheads) in_dtype (the step; with
 *                SSM_DT_SOFTPLUS the raw value, the step being
 *                softplus(dt + dt_bias[h]))
 *   theta      : (batch, seqlen, theta_heads, dstate / 2) in_dtype
 *   B, C       : (batch, seqlen, ngroups, dstate) in_dtype
 *   angle0     : (batch, nheads, dstate / 2) float32, nullable (zero)
 *   B_rot, C_rot: (batch, seqlen, nheads, dstate) out_dtype
 *   angle_last : (batch, nheads, dstate / 2) float32, nullable; may be
 *                exactly angle0 (updated in place)
 * The running angle is summed in float64 inside the call; angle0 and
 * angle_last are float32.  angle_last is the final angle reduced modulo 2 pi
 * to [-pi, pi] (in float64, before the float32 rounding), which is all a
 * later call starting from it needs; it equals angle0 - sum dt theta up to a
 * multiple of 2 pi.  theta, B, C, B_rot and C_rot must be 16-byte
 * aligned (they are accessed as vectors of up to four pairs' halves); dt,
 * angle0 and angle_last need their element alignment.  Outputs must not
 * overlap inputs or each other (angle_last == angle0 excepted).
 * Supported: any batch, seqlen >= 0 with batch * nheads < 2^31.
 */
SSM_API int ssm_rope_bc(const void *dt, const void *theta, const void *B, const void *C,
                        const float *angle0, void *B_rot, void *C_rot, float *angle_last,
                        const ssm_rope_dims_t *dims, void *stream);

/*
 * Workspace ssm_rope_bc_bwd needs for `dims`: two float32 arrays of
 * (batch, nheads, ceil(seqlen / T), dstate / 2), where T, the steps of one
 * tile, is 8 for dstate >= 64, 16 for 32, 32 for 16 and 64 below; and for
 * dstate 128 or 256 one float32 array of (batch, seqlen, nheads, P) with
 * P = 2 or 4 (the parts of ddt).  Each is rounded up to 256 bytes.
 */
SSM_API int ssm_rope_bc_bwd_workspace_size(const ssm_rope_dims_t *dims, size_t *bytes);

/*
 * Backward of the rotary step (ssm_rope_bc): gradients of a loss with respect
 * to dt, theta, B, C and angle0, given dB_rot = dL/dB_rot, dC_rot = dL/dC_rot
 * and dangle_last = dL/dangle_last.  The chain rule on the forward's formula
 * ([Mamba-3 NKI], "How it works", Phase 1, as read above; the page prints no
 * backward): with c, s = cos, sin phi_t[k] and the pair (g1, g2) of dB_rot
 * (states k, k + N/2),
 *   dB_t[k] += g1 c + g2 s,   dB_t[k + N/2] += -g1 s + g2 c   (C alike),
 *   dphi_t[k] = B_rot x dB_rot + C_rot x dC_rot   (x: the 2-D cross
 *               product r1 g2 - r2 g1),
 *   R_t[k]    = dangle_last[k] + sum_{s >= t} dphi_s[k],
 *   dtheta_t[k] += -dt_t R_t[k],   ddt_t = -sum_k theta_t[k] R_t[k],
 *   dangle0[k] = R_0[k]   (dangle_last when seqlen = 0),
 * summed over the heads of a group for dB and dC and over the heads for
 * dtheta when theta_heads = 1.
 *
 * Inputs: dims, dt, theta, B, C, angle0 as ssm_rope_bc (the same forward
 *   call), and
 *   dB_rot, dC_rot : (batch, seqlen, nheads, dstate) in dims->out_dtype (the
 *                    forward's B_rot dtype; float32 as ssd_bwd writes dB, dC)
 *   dangle_last    : (batch, nheads, dstate / 2) float32, nullable (zero)
 * Outputs (overwritten, all float32):
 *   ddt     : (batch, seqlen, nheads) (with SSM_DT_SOFTPLUS the gradient of
 *             the raw dt, i.e. times sigmoid(dt + dt_bias[h]))
 *   dtheta  : (batch, seqlen, theta_heads, dstate / 2)
 *   dB, dC  : (batch, seqlen, ngroups, dstate)
 *   dangle0 : (batch, nheads, dstate / 2), nullable
 * Workspace: caller-owned device memory of at least
 * ssm_rope_bc_bwd_workspace_size() bytes, 16-byte aligned (NULL when that is
 * 0).  The angle before every tile of T steps is rebuilt in float64 as in the
 * forward, the angles within a tile and the rotations are float32, and R is
 * summed in float32 within a tile and in float64 across tiles.  Every sum
 * runs in a fixed order, so every output is deterministic.  theta, B, C, dB_rot, dC_rot, dtheta, dB
 * and dC must be 16-byte aligned, ddt and the angle arrays 4-byte aligned,
 * dt element aligned.  No output may overlap an input, another output or the
 * workspace.  Supported sizes: those of ssm_rope_bc, with
 * batch * seqlen / 4 < 2^31 - 1 (the grids of the tiled kernels).
 */
SSM_API int ssm_rope_bc_bwd(const void *dt, const void *theta, const void *B, const void *C,
                            const float *angle0, const void *dB_rot, const void *dC_rot,
                            const float *dangle_last, float *ddt, float *dtheta, float *dB, float *dC,
                            float *dangle0, void *workspace, size_t workspace_bytes,
                            const ssm_rope_dims_t *dims, void *stream);

/* ------------------------------------------------------------------------ */
/* Single-token decode steps (state cache updated in place)                  */
/* ------------------------------------------------------------------------ */

/*
 * Sizes of one selective-scan decode step.
 *   batch, dim (channels), dstate (N), ngroups (G divides dim);
 *   in_dtype: u, delta, B, C, z; out_dtype: y.  flags: 0 or SSM_DT_SOFTPLUS
 *   (dt_bias: (dim) float32, nullable); reserved: must be 0.
 * Supported: dstate a power of two up to 256; any batch, dim >= 0.
 */
typedef struct {
  int64_t batch, dim, dstate, ngroups;
  int32_t in_dtype, out_dtype;
  int32_t flags, reserved;
  const float *dt_bias;
} ssm_step_dims_t;

/*
 * One decode step of the selective scan: the recurrence of ssm_scan_fwd at a
 * single token, continuing from the cached state.  For every (b, d):
 *   state[n] <- exp(delta * A[d,n]) * state[n] + delta * B[n] * u
 *   y        = (sum_n C[n] * state[n] + D[d] * u) * silu(z)
 *   [Mamba-3 NKI], "How it works": decode through step() is the direct
 *     recurrence h_t = alpha h_{t-1} + beta prev_Bx + gamma B_t x_t with
 *     output C_t^T h_t; here beta = 0 and gamma = delta (lam = 1);
 *   [Mamba-3 NKI], "Kernel details", mamba3_siso_decode_state_kernel: the
 *     state update and the output contraction in one kernel.
 * Layouts: u, delta, z, y (batch, dim); A (dim, dstate) float32;
 *   B, C (batch, ngroups, dstate); D (dim) float32 nullable; z nullable;
 *   state (batch, dim, dstate) float32, read and written in place, 16-byte
 *   aligned when dstate >= 4.  y and the state must not overlap any input.
 * Equal to ssm_scan_fwd with seqlen 1, h0 = h_last = state.
 */
SSM_API int ssm_scan_step(const void *u, const void *delta, const float *A, const void *B,
                  const void *C, const float *D, const void *z, float *state, void *y,
                  const ssm_step_dims_t *dims, void *stream);

/*
 * Sizes of one SSD decode step: batch, nheads (H), headdim (P), dstate (N),
 * ngroups (G divides H); in_dtype: x, dt, B, C, z; out_dtype: y; flags: 0 or
 * SSM_DT_SOFTPLUS (dt_bias: (nheads) float32, nullable); reserved: must be 0.
 * Supported: any headdim >= 1, dstate a power of two up to 256.
 */
typedef struct {
  int64_t batch, nheads, headdim, dstate, ngroups;
  int32_t in_dtype, out_dtype;
  int32_t flags, reserved;
  const float *dt_bias;
} ssd_step_dims_t;

/*
 * One decode step of the scalar-decay SSD: for every (b, h, p),
 *   state[p][n] <- exp(dt[b,h] * A[h]) * state[p][n] + dt[b,h] * x[p] * B[n]
 *   y[p]        = (sum_n C[n] * state[p][n] + D[h] * x[p]) * silu(z[p])
 *   [Mamba-3 NKI], "Kernel details", mamba3_siso_decode_state_kernel: the
 *     per-head state update alpha h + gamma B (x) x and y = C^T h, batched
 *     over the heads (beta = 0, gamma = dt here).
 * Layouts: x, z, y (batch, nheads, headdim); dt (batch, nheads);
 *   A, D (nheads) float32 (D nullable); B, C (batch, ngroups, dstate);
 *   state (batch, nheads, headdim, dstate) float32, read and written in place,
 *   16-byte aligned when dstate >= 4.
 * Equal to ssd_chunked_fwd with seqlen 1, h0 = h_last = state.
 */
SSM_API int ssd_step(const void *x, const void *dt, const float *A, const void *B, const void *C,
             const float *D, const void *z, float *state, void *y, const ssd_step_dims_t *dims,
             void *stream);

/*
 * One decode step of the trapezoidal (Mamba-3 SISO) SSD: for every (b, h, p),
 * with alpha = exp(dt[b,h] A[h]), gamma = lam[b,h] dt[b,h] and
 * beta = (dt[b,h] - gamma) alpha,
 *   state[p][n] <- alpha state[p][n] + beta x_prev[p] B_prev[n] + gamma x[p] B[n]
 *   y[p]        = (sum_n C[n] state[p][n] + D[h] x[p]) * silu(z[p])
 *   [Mamba-3 NKI], "How it works": decode through step() is this direct
 *     recurrence (its Eq. 9), h_t = alpha h_{t-1} + beta prev_Bx +
 *     gamma B_t x_t with output C_t^T h_t; Phase 0 gives alpha, beta, gamma
 *     (lam after its sigmoid: applied by the caller, or by the kernel with
 *     SSM_LAM_SIGMOID; dt likewise with SSM_DT_SOFTPLUS);
 *   [Mamba-3 NKI], "Kernel details", mamba3_siso_decode_state_kernel.
 * x_prev, B_prev: the previous token's x (batch, nheads, headdim) and B
 *   (batch, ngroups, dstate), in_dtype, given together or not at all (NULL:
 *   the term is zero, as for the first token of a sequence).  After a
 *   prefill by ssd_trap_chunked_fwd, pass its last token's x and B (or the
 *   rotated B); each later step passes the previous step's x and B.  They are
 *   read only; the caller keeps them.
 * lam: (batch, nheads) in_dtype.  Other layouts, alignment, flags (plus
 *   SSM_LAM_SIGMOID) and sizes as ssd_step; no input may overlap y or state.
 * Equal to ssd_trap_chunked_fwd with seqlen 1, h0 = h_last = state and the
 * same x_prev, B_prev.
 */
SSM_API int ssd_trap_step(const void *x, const void *dt, const void *lam, const float *A, const void *B,
                  const void *C, const float *D, const void *z, const void *x_prev,
                  const void *B_prev, float *state, void *y, const ssd_step_dims_t *dims,
                  void *stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                               */
/* ------------------------------------------------------------------------ */

/* Static name of a status code ("SSM_OK", "SSM_ERR_SHAPE", ...). */
SSM_API const char *ssm_status_string(int status);

/* Reason for the last failure on the calling host thread ("" if none).
 * The pointer stays valid until the next libssm call on that thread. */
SSM_API const char *ssm_last_error(void);

/* The same string as ssm_last_error(). */
SSM_API const char *ssm_last_error_message(void);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
SSM_API int ssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
