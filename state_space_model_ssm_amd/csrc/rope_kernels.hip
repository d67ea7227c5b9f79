// Rotary step on B and C for gfx950: the data-dependent rotation that gives
// Mamba-3 its complex-valued state.
//
// Math ("Mamba-3 NKI Kernels for AWS Neuron", section "How it works", Phase 1:
// the angles are the negated running sum of dt * theta, and B and C are
// rotated by them; the page's Mamba-3 feature list calls the result a
// complex-valued state).  Per batch row b, head h and state pair k < N/2:
//   phi_t = angle0 - sum_{s <= t} dt_s theta_s[k]
//   (B_rot[k], B_rot[k + N/2]) = (B[k] cos phi - B[k + N/2] sin phi,
//                                 B[k] sin phi + B[k + N/2] cos phi),  C alike.
//
// The work is a prefix sum over time followed by an elementwise rotation: it
// is bound by HBM (the rotated B and C are written per head).  One workgroup
// per (b, h): lane k of a KP = N/2 lane group owns pair k, and the NSEG groups
// of the workgroup own consecutive time segments.  Each segment first sums its
// dt * theta, the segment totals are combined through LDS, and then every
// segment walks its steps from its own starting angle.  The running angle is
// kept in float64 (a float32 sum over thousands of steps would drift by more
// than the result's tolerance); it is reduced to [-pi, pi] in float64 and the
// rotation itself is float32.
#include "ssm_internal.h"

namespace ssm {
namespace {

__device__ __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t *p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ void st(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t *p, int64_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // round to nearest even
}

constexpr double kTwoPi = 6.283185307179586476925;
constexpr double kInvTwoPi = 0.15915494309189533576888;

// Time segments per workgroup for KP pair lanes (at most 512 threads, at
// least one wavefront).
template <int KP>
constexpr int rope_segments() { return KP >= 8 ? 512 / KP : 64; }

template <typename Tin, typename Tout, int KP>
__global__ void __launch_bounds__(512) rope_bc_kernel(const RopeParams p) {
  constexpr int NSEG = rope_segments<KP>();
  constexpr int N = 2 * KP;
  __shared__ double sPart[NSEG * KP];
  const Tin *__restrict__ gdt = static_cast<const Tin *>(p.dt);
  const Tin *__restrict__ gth = static_cast<const Tin *>(p.theta);
  const Tin *__restrict__ gB = static_cast<const Tin *>(p.B);
  const Tin *__restrict__ gC = static_cast<const Tin *>(p.C);
  Tout *__restrict__ gBr = static_cast<Tout *>(p.B_rot);
  Tout *__restrict__ gCr = static_cast<Tout *>(p.C_rot);

  const int seg = threadIdx.x / KP;
  const int k = threadIdx.x % KP;
  const int64_t H = p.nheads, L = p.seqlen;
  const int64_t b = blockIdx.x / H, h = blockIdx.x % H;
  const int64_t g = h / (H / p.ngroups);
  const int64_t th = p.theta_heads == 1 ? 0 : h;
  const int64_t seglen = (L + NSEG - 1) / NSEG;
  const int64_t t0 = min(L, seg * seglen), t1 = min(L, t0 + seglen);
  const float bias = (p.dt_softplus && p.dt_bias != nullptr) ? p.dt_bias[h] : 0.0f;
  auto turn = [&](int64_t t) __attribute__((always_inline)) {  // dt_t * theta_t[k]
    float dt = ld(gdt, (b * L + t) * H + h);
    if (p.dt_softplus) dt = dt_softplus(dt + bias);
    return static_cast<double>(dt) * static_cast<double>(ld(gth, ((b * L + t) * p.theta_heads + th) * KP + k));
  };

  // The starting angle is read before the barrier, so angle_last may be
  // angle0 itself (it is written after the barrier).
  const int64_t ai = (b * H + h) * KP + k;
  double phi = p.angle0 != nullptr ? static_cast<double>(p.angle0[ai]) : 0.0;
  double part = 0.0;
  for (int64_t t = t0; t < t1; ++t) part += turn(t);
  sPart[seg * KP + k] = part;
  __syncthreads();
  for (int j = 0; j < seg; ++j) phi -= sPart[j * KP + k];
  if (seg == NSEG - 1 && p.angle_last != nullptr) p.angle_last[ai] = static_cast<float>(phi - part);

#pragma unroll 4
  for (int64_t t = t0; t < t1; ++t) {
    phi -= turn(t);
    const float r = static_cast<float>(phi - kTwoPi * rint(phi * kInvTwoPi));
    float sn, cs;
    sincosf(r, &sn, &cs);
    const int64_t src = ((b * L + t) * p.ngroups + g) * N + k;
    const int64_t dst = ((b * L + t) * H + h) * N + k;
    const float b1 = ld(gB, src), b2 = ld(gB, src + KP);
    const float c1 = ld(gC, src), c2 = ld(gC, src + KP);
    st(gBr, dst, b1 * cs - b2 * sn);
    st(gBr, dst + KP, b1 * sn + b2 * cs);
    st(gCr, dst, c1 * cs - c2 * sn);
    st(gCr, dst + KP, c1 * sn + c2 * cs);
  }
}

template <typename Tin, typename Tout, int KP>
hipError_t launch_kp(const RopeParams &p, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(p.batch * p.nheads));
  hipLaunchKernelGGL((rope_bc_kernel<Tin, Tout, KP>), grid, dim3(KP * rope_segments<KP>()), 0, stream, p);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const RopeParams &p, hipStream_t stream) {
  switch (p.dstate) {
    case 2: return launch_kp<Tin, Tout, 1>(p, stream);
    case 4: return launch_kp<Tin, Tout, 2>(p, stream);
    case 8: return launch_kp<Tin, Tout, 4>(p, stream);
    case 16: return launch_kp<Tin, Tout, 8>(p, stream);
    case 32: return launch_kp<Tin, Tout, 16>(p, stream);
    case 64: return launch_kp<Tin, Tout, 32>(p, stream);
    case 128: return launch_kp<Tin, Tout, 64>(p, stream);
    case 256: return launch_kp<Tin, Tout, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rope(const RopeParams &p, int in_bf16, int out_bf16, hipStream_t stream) {
  if (p.batch * p.nheads == 0) return hipSuccess;
  if (!in_bf16 && !out_bf16) return launch_typed<float, float>(p, stream);
  if (!in_bf16 && out_bf16) return launch_typed<float, uint16_t>(p, stream);
  if (in_bf16 && !out_bf16) return launch_typed<uint16_t, float>(p, stream);
  return launch_typed<uint16_t, uint16_t>(p, stream);
}

}  // namespace ssm
