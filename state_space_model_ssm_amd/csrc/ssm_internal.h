// Internal declarations of libssm: kernel parameter blocks and the launchers
// that ssm_api.hip calls after validating a request.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

// softplus(v) = log(1 + exp(v)), the step-size map of SSM_DT_SOFTPLUS: v itself
// above 20 (where log(1 + exp(v)) rounds to v in float32), else log1p(exp(v)).
__device__ __forceinline__ float dt_softplus(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// One selective-scan launch (see ssm_scan_fwd in include/ssm.h for the math).
struct ScanParams {
  const void *u, *delta, *B, *C, *z;  // in_dtype
  const float *A, *D;                 // float32; D nullable
  const float *h0;                    // nullable initial state [batch][dim][dstate]
  void *y;                            // out_dtype
  float *h_last;                      // nullable
  float *carry;                       // chunked path: [batch][dim][n_chunks-1][2][dstate]
  const float *dt_bias;               // nullable (dim); read when dt_softplus
  int32_t dt_softplus;                // step with softplus(delta + dt_bias)
  int64_t batch, dim, seqlen, ngroups, dim_per_group;
  int64_t chunk_len;                  // time steps per chunk
  int64_t tiles_per_group;            // channel tiles per (batch, group)
  int32_t n_chunks;                   // resolved chunk count (>= 1)
  int32_t dstate;
  int32_t vec_ok;                     // u, delta, B, C rows start 16-byte aligned
};

// Chunks start on multiples of this many steps (the scan's time tile).
constexpr int64_t kScanChunkAlign = 32;

// The backward pass keeps the forward state every kScanCkptStep steps.
constexpr int64_t kScanCkptStep = 16;

// Channel tile of one workgroup for a given dstate: 256 threads, one state per
// thread, so 256 / dstate channels.
int scan_channels_per_block(int dstate);

// Storage elements per 16-byte vector load of the scan inputs.
int scan_vector_elems(int in_bf16);

// Launch the chunk-summary pass (chunks 0 .. n_chunks-2) when n_chunks > 1,
// then the sweep that writes y and h_last.  Returns a hipError_t.
hipError_t launch_scan(const ScanParams &p, int in_bf16, int out_bf16, hipStream_t stream);

// Forward pass of one chunk (p.n_chunks == 1) from h0 that stores the state
// at every kScanCkptStep-step boundary t into
// p.carry[(batch*dim + d) * ceil(L / kScanCkptStep) + t / kScanCkptStep][n].
hipError_t launch_scan_ckpt(const ScanParams &p, int in_bf16, hipStream_t stream);

// The selective-scan backward (see ssm_scan_bwd in include/ssm.h): the
// checkpoint pass stores the forward state every kScanCkptStep steps into
// ckpt; the backward kernel walks 16-step tiles from the last to the first.
struct ScanBwdParams {
  const void *u, *delta, *B, *C, *z;  // in_dtype
  const float *A, *D;                 // float32; D nullable
  const void *dy;                     // out_dtype
  const float *dh_last;               // nullable
  void *du, *ddelta, *dz;             // in_dtype; dz only with z
  float *dA, *dB, *dC, *dD, *dh0;     // float32; dD only with D; dh0 nullable
  const float *ckpt;                  // [batch][dim][ceil(L / kScanCkptStep)][dstate]
  const float *dt_bias;               // nullable (dim); read when dt_softplus
  int32_t dt_softplus;                // step with softplus(delta + dt_bias); ddelta is then d/d(raw delta)
  // Workspace for the sums: per channel tile, dB and dC terms
  // [batch][ngroups][tiles_per_group][dstate][L]; per batch row, dA terms
  // [batch][dim][dstate] and dD terms [batch][dim].
  float *part_dB, *part_dC, *part_dA, *part_dD;
  int64_t batch, dim, seqlen, ngroups, dim_per_group, tiles_per_group;
  int32_t dstate;
};

// Run the backward kernel (the checkpoint pass must have run on the same
// stream), then reduce its per-tile and per-batch terms into dB, dC, dA, dD.
hipError_t launch_scan_bwd(const ScanBwdParams &p, int in_bf16, int out_bf16, hipStream_t stream);

// One chunked-SSD launch (see ssd_chunked_fwd in include/ssm.h).
struct SsdParams {
  const void *x, *dt, *B, *C, *z;     // bf16
  const void *lam;                    // bf16 (batch, seqlen, nheads); non-null = trapezoidal form
  const void *x_prev, *B_prev;        // trapezoid: the token before the sequence, bf16
                                      // (batch, nheads, headdim) and (batch, ngroups, dstate); nullable
  const float *A, *D;                 // float32; D nullable
  const float *h0;                    // nullable initial state [batch][nheads][headdim][dstate]
  void *y;                            // out dtype
  float *h_last;                      // nullable
  const float *dt_bias;               // nullable (nheads); read when dt_softplus
  int32_t dt_softplus, lam_sigmoid;   // dt = softplus(dt + dt_bias); lam = sigmoid(lam)
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
};

hipError_t launch_ssd(const SsdParams &p, int out_bf16, hipStream_t stream);

// The chunked SSD with the rotary step on B and C fused in (see
// ssd_rope_chunked_fwd in include/ssm.h): one workgroup per (batch, head).
// ssd.B_prev is per head here (batch, nheads, dstate), already rotated.
struct SsdRopeParams {
  SsdParams ssd;
  const void *theta;                  // bf16 (batch, seqlen, theta_heads, dstate / 2)
  const float *angle0;                // nullable (batch, nheads, dstate / 2)
  float *angle_last;                  // nullable; may be angle0 itself
  void *B_last;                       // nullable: bf16 (batch, nheads, dstate), the last step's rotated B
  int64_t theta_heads;                // 1 or nheads
};

hipError_t launch_ssd_rope(const SsdRopeParams &p, int out_bf16, hipStream_t stream);
// Heads one SSD workgroup takes (1, 2 or 4, at most max_hpb; they share a
// group), and the grid size below which fewer heads per workgroup are taken
// (the CU count).
constexpr int64_t kSsdMinBlocks = 256;
int ssd_heads_per_block(int64_t batch, int64_t nheads, int64_t ngroups, int max_hpb);

// The SSD backward (see ssd_bwd in include/ssm.h): a forward and a reverse
// state pass per (batch, head), then a kernel per (batch, chunk, block of hpw
// heads) and the sums over head blocks, batch rows and chunks.
struct SsdBwdParams {
  const void *x, *dt, *B, *C, *z;     // bf16
  const void *dy;                     // bf16 or float32 (the forward's out dtype)
  const float *A, *D, *h0, *dh_last;  // float32; D, h0, dh_last nullable
  const float *dt_bias;               // nullable (nheads); read when dt_softplus
  int32_t dt_softplus;
  void *dx, *ddt, *dz;                // bf16; dz only with z
  float *dA, *dB, *dC, *dD, *dh0;     // float32; dD only with D; dh0 nullable
  // Workspace, per (batch, head, chunk): the chunk's entering state S_in
  // (ws_Sp) and the gradient of its leaving state (ws_dSp), headdim x dstate
  // bf16 in the state passes' lane-blocked order; the dA and dD terms
  // (float32).  Per (batch, step,
  // head block), the dB and dC terms [batch][seqlen][nheads / hpw][dstate].
  uint16_t *ws_Sp, *ws_dSp;
  float *ws_dApart, *ws_dDpart, *ws_dBp, *ws_dCp;
  // Trapezoidal form (lam non-null): lam (batch, seqlen, nheads) and the
  // token before the sequence x_prev (batch, nheads, headdim), B_prev (batch,
  // ngroups, dstate), bf16, nullable together; outputs dlam (bf16), dx_prev
  // (bf16) and dB_prev (float32) with them.  Workspace per (batch, step,
  // head): the gradients of the step's two input weights (scale_s and
  // gamma_s) and the suffix sum of the log-decay gradient; per (batch, head)
  // the gradient of the previous-token weight and the dB_prev terms.
  const void *lam, *x_prev, *B_prev;
  int32_t lam_sigmoid;
  void *dlam, *dx_prev;
  float *dB_prev;
  float *ws_dsc, *ws_dga, *ws_rc, *ws_dw0, *ws_dBpp;
  int64_t batch, seqlen, nheads, ngroups, dstate, nchunks;
  int32_t hpw;                        // heads per chunk-kernel workgroup
};

// The chunk kernel takes hpw heads of a group per workgroup: the most (up to
// 8) that keep its grid at kSsdBwdMinBlocks workgroups or more.
constexpr int64_t kSsdBwdMinBlocks = 1024;
int ssd_bwd_heads_per_block(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups);

hipError_t launch_ssd_bwd(const SsdBwdParams &p, int dy_bf16, hipStream_t stream);

// One decode step (see ssm_scan_step and ssd_step in include/ssm.h).  The
// SSD step is the scan step over channels d = (head, p) with A, dt and D
// taken per head (headdim channels per head); the scan step has headdim 1.
struct StepParams {
  const void *u, *delta, *B, *C, *z;  // in_dtype
  const void *lam;                    // trapezoidal SSD step: (batch, nheads) in_dtype; else null
  const void *x_prev, *B_prev;        // trapezoid: the previous token's x (batch, dim) and B
                                      // (batch, ngroups, dstate), in_dtype; nullable (zero term)
  const float *A, *D;                 // float32; D nullable
  float *state;                       // [batch][dim][dstate], updated in place
  void *y;                            // out_dtype
  const float *dt_bias;               // nullable (per dt element's channel or head); read when dt_softplus
  int32_t dt_softplus, lam_sigmoid;
  int64_t batch, dim, ngroups, headdim;
  int32_t dstate;
};

hipError_t launch_step(const StepParams &p, int per_head, int in_bf16, int out_bf16, hipStream_t stream);

// Rotary step on B and C (Mamba-3 Phase 1).
struct RopeParams {
  const void *dt, *theta, *B, *C;     // in_dtype
  const float *angle0, *dt_bias;      // nullable
  void *B_rot, *C_rot;                // out_dtype
  float *angle_last;                  // nullable; may be angle0 itself
  int32_t dt_softplus;
  int32_t dstate;
  int64_t batch, seqlen, nheads, ngroups, theta_heads;
};

hipError_t launch_rope(const RopeParams &p, int in_bf16, int out_bf16, hipStream_t stream);

// Backward of the rotary step (ssm_rope_bc_bwd): tiles of tile_len steps, a
// workgroup per (batch row, tile) holding every head of the tile in `slots`
// head slots, a row's pairs split over ws_parts wavefronts.  Workspace: the
// angle before every tile and the tiles' sums of the angle gradient,
// (batch, nheads, ntile, dstate / 2) float32 each, and with ws_parts > 1 the
// parts of ddt, (batch, seqlen, nheads, ws_parts) float32.
struct RopeBwdParams {
  const void *dt, *theta, *B, *C;     // in_dtype
  const void *dB_rot, *dC_rot;        // g_dtype (the forward's out_dtype)
  const float *angle0, *dangle_last;  // nullable
  const float *dt_bias;               // nullable
  float *ddt, *dtheta, *dB, *dC;      // float32 outputs
  float *dangle0;                     // nullable
  float *ws_ang, *ws_tot, *ws_ddt;
  int32_t dt_softplus;
  int32_t dstate;
  int32_t tile_len, slots, ws_parts;
  int64_t ntile;
  int64_t batch, seqlen, nheads, ngroups, theta_heads;
};

// Tiling of the rotary backward for `dstate`, nheads and ngroups (it must
// match the tile kernel's layout): threads per step tpr = max(1, dstate / 8)
// split over parts = 4, 2 or 1 wavefronts as tpr >= 32, >= 16 or less; steps
// per tile = 64 * parts / tpr; head slots: up to 8 / parts, a power of two
// that divides nheads and divides or is a multiple of the heads per group.
struct RopeBwdTilingCfg {
  int32_t tile_len, slots, parts;
};
inline RopeBwdTilingCfg rope_bwd_tiling(int64_t dstate, int64_t nheads, int64_t ngroups) {
  const int64_t kp = dstate / 2, tpr = kp < 4 ? 1 : kp / 4;
  const int64_t parts = tpr >= 32 ? 4 : (tpr >= 16 ? 2 : 1);
  const int64_t hpg = nheads / ngroups;
  int64_t use = 8 / parts;
  while (use > 1 && (nheads % use != 0 || (use % hpg != 0 && hpg % use != 0))) use /= 2;
  RopeBwdTilingCfg c;
  c.tile_len = static_cast<int32_t>(64 * parts / tpr);
  c.slots = static_cast<int32_t>(use);
  c.parts = static_cast<int32_t>(parts);
  return c;
}

hipError_t launch_rope_bwd(const RopeBwdParams &p, int in_bf16, int g_bf16, hipStream_t stream);

}  // namespace ssm
