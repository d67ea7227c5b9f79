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
// per (b, h): each thread owns four consecutive pairs (all of them when
// N / 2 < 4), a group of threads covers a row's N / 2 pairs, and the NSEG
// groups of the workgroup own consecutive time segments.  Each segment first sums its
// dt * theta, the segment totals are combined through LDS, and then every
// segment walks its steps from its own starting angle.  The running angle is
// summed in float64 (a float32 sum over thousands of steps would drift by more
// than the result's tolerance), in revolutions, reduced to
// [-1/2, 1/2] in float64, and the sine, cosine and rotation are float32 (the
// hardware v_sin_f32 / v_cos_f32, which take revolutions; the outputs then
// differ from the float64 oracle by ~1.4e-7 of their largest magnitude).
#include "ssm_internal.h"

namespace ssm {
namespace {

__device__ __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t *p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

constexpr double kInvTwoPi = 0.15915494309189533576888;
constexpr double kTwoPi = 6.28318530717958647692529;
// Steps whose loads are issued together: 2 per rotation batch and 4 per
// batch of the angle sums (1 rotation step per batch measured 7% slower; 4 or
// 8 no faster).
constexpr int kBatch = 2;
constexpr int kSumBatch = 4;

// Vector loads and stores of V consecutive elements (V * element size bytes,
// aligned to that size).
template <int BYTES> struct RawT;
template <> struct RawT<2> { typedef uint16_t T; };
template <> struct RawT<4> { typedef uint32_t T; };
template <> struct RawT<8> { typedef uint2 T; };
template <> struct RawT<16> { typedef uint4 T; };

template <int V>
__device__ __forceinline__ void vload(const float *p, float (&v)[V]) {
  const auto r = *reinterpret_cast<const typename RawT<4 * V>::T *>(p);
  static_assert(sizeof(r) == sizeof(v), "vector width");
  __builtin_memcpy(v, &r, sizeof(v));
}
template <int V>
__device__ __forceinline__ void vload(const uint16_t *p, float (&v)[V]) {
  const auto r = *reinterpret_cast<const typename RawT<2 * V>::T *>(p);
  uint16_t e[V];
  static_assert(sizeof(r) == sizeof(e), "vector width");
  __builtin_memcpy(e, &r, sizeof(e));
#pragma unroll
  for (int j = 0; j < V; ++j) v[j] = __uint_as_float(static_cast<uint32_t>(e[j]) << 16);
}
template <int V>
__device__ __forceinline__ void vstore(float *p, const float (&v)[V]) {
  typename RawT<4 * V>::T r;
  __builtin_memcpy(&r, v, sizeof(v));
  *reinterpret_cast<typename RawT<4 * V>::T *>(p) = r;
}
template <int V>
__device__ __forceinline__ void vstore(uint16_t *p, const float (&v)[V]) {
  uint16_t e[V];
#pragma unroll
  for (int j = 0; j < V; ++j) e[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[j]));  // round to nearest even
  typename RawT<2 * V>::T r;
  __builtin_memcpy(&r, e, sizeof(e));
  *reinterpret_cast<typename RawT<2 * V>::T *>(p) = r;
}

// Pairs per thread (consecutive k), threads per (batch, time, head) row, and
// time segments per workgroup (at most 512 threads, at least one wavefront).
// Four pairs per thread (8-byte bf16 or 16-byte float32 accesses per row
// half) measured 36 us on 32 x 256 x 32 heads x 128 states against 49 us
// with one pair per thread and 42 us with eight (more registers, fewer
// wavefronts).
template <int KP>
struct RopeCfg {
  static constexpr int VEC = KP < 4 ? KP : 4;
  static constexpr int TPR = KP / VEC;
  static constexpr int NSEG = 512 / TPR < 64 ? 512 / TPR : 64;
  static constexpr int THREADS = TPR * NSEG;
};

// Registers held to six wavefronts per SIMD (at most 80 per lane, no spills):
// three 512-thread workgroups per CU instead of two measured 4% faster;
// eight wavefronts (64 registers) spill and run 2% slower than two.
template <typename Tin, typename Tout, int KP>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(6))) rope_bc_kernel(const RopeParams p) {
  using Cfg = RopeCfg<KP>;
  constexpr int VEC = Cfg::VEC, TPR = Cfg::TPR, NSEG = Cfg::NSEG;
  constexpr int N = 2 * KP;
  __shared__ double sPart[NSEG * KP];

  const int seg = threadIdx.x / TPR;
  const int k0 = (threadIdx.x % TPR) * VEC;
  const int64_t H = p.nheads, L = p.seqlen;
  // The heads of a batch row read the same theta (when shared), B and C.
  // Consecutive workgroup ids are dealt round-robin to the 8 XCDs, so remap
  // ids to give each XCD a contiguous run of (b, h) and keep a batch row's
  // shared rows in one L2 (without it every XCD fetches them: 8x the reads).
  const int64_t nblk = p.batch * H;
  int64_t id = blockIdx.x;
  if (nblk % 8 == 0) id = (id % 8) * (nblk / 8) + id / 8;
  const int64_t b = id / H, h = id % H;
  const int64_t g = h / (H / p.ngroups);
  const int64_t th = p.theta_heads == 1 ? 0 : h;
  const int64_t seglen = (L + NSEG - 1) / NSEG;
  const int64_t t0 = min(L, seg * seglen), t1 = min(L, t0 + seglen);
  const int n = static_cast<int>(t1 - t0);  // steps of this segment
  const float bias = (p.dt_softplus && p.dt_bias != nullptr) ? p.dt_bias[h] : 0.0f;

  // Pointers at step t0 of this thread's rows, and their per-step strides.
  const int64_t row0 = b * L + t0;
  const Tin *dtp = static_cast<const Tin *>(p.dt) + row0 * H + h;
  const Tin *thp = static_cast<const Tin *>(p.theta) + (row0 * p.theta_heads + th) * KP + k0;
  const Tin *bp = static_cast<const Tin *>(p.B) + (row0 * p.ngroups + g) * N + k0;
  const Tin *cp = static_cast<const Tin *>(p.C) + (row0 * p.ngroups + g) * N + k0;
  Tout *brp = static_cast<Tout *>(p.B_rot) + (row0 * H + h) * N + k0;
  Tout *crp = static_cast<Tout *>(p.C_rot) + (row0 * H + h) * N + k0;
  const int64_t s_dt = H, s_th = p.theta_heads * KP, s_bc = p.ngroups * N, s_out = H * N;
  auto step = [&](int i) __attribute__((always_inline)) {
    const float dt = ld(dtp, i * s_dt);
    return p.dt_softplus ? dt_softplus(dt + bias) : dt;
  };

  // The starting angles are read before the barrier, so angle_last may be
  // angle0 itself (it is written after the barrier).
  const int64_t ai = (b * H + h) * KP + k0;
  double phi[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) phi[j] = p.angle0 != nullptr ? static_cast<double>(p.angle0[ai + j]) : 0.0;

  // Steps go in batches whose loads are all issued before any of them is
  // used; steps past the segment's end load the segment's last step
  // (branch-free) and are not used.
  double part[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) part[j] = 0.0;
  for (int i0 = 0; i0 < n; i0 += kSumBatch) {
    float dv[kSumBatch], tv[kSumBatch][VEC];
#pragma unroll
    for (int q = 0; q < kSumBatch; ++q) {
      const int i = min(i0 + q, n - 1);
      dv[q] = step(i);
      vload<VEC>(thp + i * s_th, tv[q]);
    }
#pragma unroll
    for (int q = 0; q < kSumBatch; ++q)
      if (i0 + q < n) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) part[j] += static_cast<double>(dv[q]) * static_cast<double>(tv[q][j]);
      }
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) sPart[seg * KP + k0 + j] = part[j];
  __syncthreads();
  for (int s = 0; s < seg; ++s) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) phi[j] -= sPart[s * KP + k0 + j];
  }
  // angle_last is the final angle reduced to [-pi, pi] in float64 before it
  // is rounded to float32: only the angle modulo 2 pi matters to a later call
  // that starts from it, and a float32 of the unreduced running angle would
  // lose its low bits once the angle has grown (at 1e4 rad one float32 ulp is
  // 1e-3 rad).
  if (seg == NSEG - 1 && p.angle_last != nullptr) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const double r = (phi[j] - part[j]) * kInvTwoPi;
      p.angle_last[ai + j] = static_cast<float>((r - rint(r)) * kTwoPi);
    }
  }

  // The running angles in revolutions, reduced to [-1/2, 1/2] for the
  // hardware sine and cosine (which take revolutions).
  double rev[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) rev[j] = phi[j] * kInvTwoPi;
  for (int i0 = 0; i0 < n; i0 += kBatch) {
    float dv[kBatch], tv[kBatch][VEC], b1[kBatch][VEC], b2[kBatch][VEC], c1[kBatch][VEC], c2[kBatch][VEC];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = min(i0 + q, n - 1);
      dv[q] = step(i);
      vload<VEC>(thp + i * s_th, tv[q]);
      vload<VEC>(bp + i * s_bc, b1[q]);
      vload<VEC>(bp + i * s_bc + KP, b2[q]);
      vload<VEC>(cp + i * s_bc, c1[q]);
      vload<VEC>(cp + i * s_bc + KP, c2[q]);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (i0 + q < n) {
        float ob1[VEC], ob2[VEC], oc1[VEC], oc2[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          rev[j] -= static_cast<double>(dv[q]) * static_cast<double>(tv[q][j]) * kInvTwoPi;
          const float fr = static_cast<float>(rev[j] - rint(rev[j]));
          const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
          ob1[j] = b1[q][j] * cs - b2[q][j] * sn;
          ob2[j] = b1[q][j] * sn + b2[q][j] * cs;
          oc1[j] = c1[q][j] * cs - c2[q][j] * sn;
          oc2[j] = c1[q][j] * sn + c2[q][j] * cs;
        }
        const int64_t o = (i0 + q) * s_out;
        vstore<VEC>(brp + o, ob1);
        vstore<VEC>(brp + o + KP, ob2);
        vstore<VEC>(crp + o, oc1);
        vstore<VEC>(crp + o + KP, oc2);
      }
    }
  }
}

template <typename Tin, typename Tout, int KP>
hipError_t launch_kp(const RopeParams &p, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(p.batch * p.nheads));
  hipLaunchKernelGGL((rope_bc_kernel<Tin, Tout, KP>), grid, dim3(RopeCfg<KP>::THREADS), 0, stream, p);
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

// ---------------------------------------------------------------------------
// Backward of the rotary step.
//
// Writing the rotation of a pair v as r = (v1 c - v2 s, v1 s + v2 c) with
// c = cos phi_t and s = sin phi_t, the chain rule for an upstream gradient
// g = (g1, g2) of r gives
//   dv     = (g1 c + g2 s, -g1 s + g2 c)        the rotation undone,
//   dphi_t = r1 g2 - r2 g1 = v1 dv2 - v2 dv1     (rotations keep the 2-D cross
//                                                product), summed over B and C,
// and, phi_t being angle0 minus the running sum of dt theta, with
// R_t = dangle_last + sum_{s >= t} dphi_s:
//   dtheta_t[k] = -dt_t R_t[k],   ddt_t = -sum_k theta_t[k] R_t[k],   dangle0 = R_0.
//
// One workgroup per (b, h) in the forward's layout.  Pass 1 sums each time
// segment's dt theta and combines the sums through LDS, which gives every
// segment its starting angle (as the forward does).  Pass 2 walks each
// segment backwards from its last angle: it undoes the rotation (per-head dB
// and dC), sums dphi from the segment's end (R local to the segment, float64),
// and writes dtheta and ddt as if nothing came after the segment.  The
// segment totals of dphi are combined through LDS, and pass 3 adds what the
// later segments and dangle_last contribute (R_end, constant over the
// segment): -dt_t R_end to dtheta and -theta_t . R_end to ddt.  Pass 3 reads
// only dt and theta again, and the dtheta and ddt values the same thread
// wrote in pass 2.  Every output element is written by one thread, so the
// result does not depend on timing; sums over the heads that share a group
// (dB, dC) or theta (dtheta) run afterwards in rope_bwd_reduce_kernel.

// Sum over the TPR consecutive lanes that hold one row's pairs (every lane of
// the row is active wherever this is called: lanes of a row share their
// segment and so every branch).
template <int TPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Steps per batch of loads in the backward's rotation pass.
#ifndef SSM_ROPE_BWD_BATCH
#define SSM_ROPE_BWD_BATCH 1
#endif
#ifndef SSM_ROPE_BWD_WAVES
#define SSM_ROPE_BWD_WAVES 4
#endif
constexpr int kBwdBatch = SSM_ROPE_BWD_BATCH;

template <typename Tin, typename Tg, int KP>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(SSM_ROPE_BWD_WAVES))) rope_bc_bwd_kernel(const RopeBwdParams p) {
  using Cfg = RopeCfg<KP>;
  constexpr int VEC = Cfg::VEC, TPR = Cfg::TPR, NSEG = Cfg::NSEG;
  constexpr int N = 2 * KP;
  __shared__ double sPart[NSEG * KP];
  __shared__ double sTot[NSEG * KP];

  const int seg = threadIdx.x / TPR;
  const int k0 = (threadIdx.x % TPR) * VEC;
  const int64_t H = p.nheads, L = p.seqlen;
  const int64_t nblk = p.batch * H;
  int64_t id = blockIdx.x;
  if (nblk % 8 == 0) id = (id % 8) * (nblk / 8) + id / 8;  // a batch row's heads on one XCD (shared B, C, theta)
  const int64_t b = id / H, h = id % H;
  const int64_t g = h / (H / p.ngroups);
  const int64_t th = p.theta_heads == 1 ? 0 : h;
  const int64_t seglen = (L + NSEG - 1) / NSEG;
  const int64_t t0 = min(L, seg * seglen), t1 = min(L, t0 + seglen);
  const int n = static_cast<int>(t1 - t0);
  const float bias = (p.dt_softplus && p.dt_bias != nullptr) ? p.dt_bias[h] : 0.0f;

  const int64_t row0 = b * L + t0;
  const Tin *dtp = static_cast<const Tin *>(p.dt) + row0 * H + h;
  const Tin *thp = static_cast<const Tin *>(p.theta) + (row0 * p.theta_heads + th) * KP + k0;
  const Tin *bp = static_cast<const Tin *>(p.B) + (row0 * p.ngroups + g) * N + k0;
  const Tin *cp = static_cast<const Tin *>(p.C) + (row0 * p.ngroups + g) * N + k0;
  const Tg *gbp = static_cast<const Tg *>(p.dB_rot) + (row0 * H + h) * N + k0;
  const Tg *gcp = static_cast<const Tg *>(p.dC_rot) + (row0 * H + h) * N + k0;
  float *dbp = (p.ngroups == H ? p.dB : p.ws_dB) + (row0 * H + h) * N + k0;
  float *dcp = (p.ngroups == H ? p.dC : p.ws_dC) + (row0 * H + h) * N + k0;
  float *dthp = (p.theta_heads == H ? p.dtheta : p.ws_dth) + (row0 * H + h) * KP + k0;
  float *ddtp = p.ddt + row0 * H + h;
  const int64_t s_dt = H, s_th = p.theta_heads * KP, s_bc = p.ngroups * N, s_g = H * N, s_dth = H * KP;
  auto step = [&](int i) __attribute__((always_inline)) {
    const float dt = ld(dtp, i * s_dt);
    return p.dt_softplus ? dt_softplus(dt + bias) : dt;
  };

  // Pass 1: the angle before this segment's first step.
  const int64_t ai = (b * H + h) * KP + k0;
  double phi[VEC], part[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    phi[j] = p.angle0 != nullptr ? static_cast<double>(p.angle0[ai + j]) : 0.0;
    part[j] = 0.0;
  }
  for (int i0 = 0; i0 < n; i0 += kSumBatch) {
    float dv[kSumBatch], tv[kSumBatch][VEC];
#pragma unroll
    for (int q = 0; q < kSumBatch; ++q) {
      const int i = min(i0 + q, n - 1);
      dv[q] = step(i);
      vload<VEC>(thp + i * s_th, tv[q]);
    }
#pragma unroll
    for (int q = 0; q < kSumBatch; ++q)
      if (i0 + q < n) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) part[j] += static_cast<double>(dv[q]) * static_cast<double>(tv[q][j]);
      }
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) sPart[seg * KP + k0 + j] = part[j];
  __syncthreads();
  for (int s = 0; s < seg; ++s) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) phi[j] -= sPart[s * KP + k0 + j];
  }

  // Pass 2: backwards over the segment, from the angle after its last step
  // (in revolutions; each step then adds its dt theta back).
  double rev[VEC], R[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    rev[j] = (phi[j] - part[j]) * kInvTwoPi;
    R[j] = 0.0;
  }
  for (int i0 = n - 1; i0 >= 0; i0 -= kBwdBatch) {
    float dv[kBwdBatch], tv[kBwdBatch][VEC], b1[kBwdBatch][VEC], b2[kBwdBatch][VEC], c1[kBwdBatch][VEC],
        c2[kBwdBatch][VEC];
    float gb1[kBwdBatch][VEC], gb2[kBwdBatch][VEC], gc1[kBwdBatch][VEC], gc2[kBwdBatch][VEC];
#pragma unroll
    for (int q = 0; q < kBwdBatch; ++q) {
      const int i = max(i0 - q, 0);
      dv[q] = step(i);
      vload<VEC>(thp + i * s_th, tv[q]);
      vload<VEC>(bp + i * s_bc, b1[q]);
      vload<VEC>(bp + i * s_bc + KP, b2[q]);
      vload<VEC>(cp + i * s_bc, c1[q]);
      vload<VEC>(cp + i * s_bc + KP, c2[q]);
      vload<VEC>(gbp + i * s_g, gb1[q]);
      vload<VEC>(gbp + i * s_g + KP, gb2[q]);
      vload<VEC>(gcp + i * s_g, gc1[q]);
      vload<VEC>(gcp + i * s_g + KP, gc2[q]);
    }
#pragma unroll
    for (int q = 0; q < kBwdBatch; ++q) {
      if (i0 - q >= 0) {
        const int i = i0 - q;
        float db1[VEC], db2[VEC], dc1[VEC], dc2[VEC], dth[VEC];
        float dd = 0.0f;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const float fr = static_cast<float>(rev[j] - rint(rev[j]));
          const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
          db1[j] = gb1[q][j] * cs + gb2[q][j] * sn;
          db2[j] = gb2[q][j] * cs - gb1[q][j] * sn;
          dc1[j] = gc1[q][j] * cs + gc2[q][j] * sn;
          dc2[j] = gc2[q][j] * cs - gc1[q][j] * sn;
          R[j] += static_cast<double>(b1[q][j] * db2[j] - b2[q][j] * db1[j] + c1[q][j] * dc2[j] - c2[q][j] * dc1[j]);
          const float rf = static_cast<float>(R[j]);
          dth[j] = -dv[q] * rf;
          dd += tv[q][j] * rf;
          rev[j] += static_cast<double>(dv[q]) * static_cast<double>(tv[q][j]) * kInvTwoPi;
        }
        dd = row_sum<TPR>(dd);
        vstore<VEC>(dbp + i * s_g, db1);
        vstore<VEC>(dbp + i * s_g + KP, db2);
        vstore<VEC>(dcp + i * s_g, dc1);
        vstore<VEC>(dcp + i * s_g + KP, dc2);
        vstore<VEC>(dthp + i * s_dth, dth);
        if (k0 == 0) ddtp[i * s_dt] = -dd;
      }
    }
  }

  // The later segments' dphi and dangle_last: R_end of this segment.
#pragma unroll
  for (int j = 0; j < VEC; ++j) sTot[seg * KP + k0 + j] = R[j];
  __syncthreads();
  double rend[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) rend[j] = p.dangle_last != nullptr ? static_cast<double>(p.dangle_last[ai + j]) : 0.0;
  for (int s = seg + 1; s < NSEG; ++s) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) rend[j] += sTot[s * KP + k0 + j];
  }
  if (seg == 0 && p.dangle0 != nullptr) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) p.dangle0[ai + j] = static_cast<float>(rend[j] + R[j]);
  }

  // Pass 3: R_end's share of dtheta and ddt, and the chain rule through the
  // step's softplus (d softplus(v) / dv = sigmoid(v) = 1 - exp(-softplus(v))).
  float re[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) re[j] = static_cast<float>(rend[j]);
  for (int i0 = 0; i0 < n; i0 += kSumBatch) {
    float dv[kSumBatch], tv[kSumBatch][VEC], old[kSumBatch][VEC];
#pragma unroll
    for (int q = 0; q < kSumBatch; ++q) {
      const int i = min(i0 + q, n - 1);
      dv[q] = step(i);
      vload<VEC>(thp + i * s_th, tv[q]);
      vload<VEC>(dthp + i * s_dth, old[q]);
    }
#pragma unroll
    for (int q = 0; q < kSumBatch; ++q)
      if (i0 + q < n) {
        const int i = i0 + q;
        float dth[VEC];
        float dd = 0.0f;
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          dth[j] = old[q][j] - dv[q] * re[j];
          dd += tv[q][j] * re[j];
        }
        vstore<VEC>(dthp + i * s_dth, dth);
        dd = row_sum<TPR>(dd);
        if (k0 == 0) {
          float v = ddtp[i * s_dt] - dd;
          if (p.dt_softplus) v *= 1.0f - expf(-dv[q]);
          ddtp[i * s_dt] = v;
        }
      }
  }
}

// Sums of per-head terms over heads, in head order: for job j,
//   out[r][c] = sum_{i < cnt} in[(r / per) * nheads + (r % per) * cnt + i][c]
// over rows r < rows and columns c < width (blockIdx.y picks the job).
struct RopeReduceJob {
  const float *in;
  float *out;
  int64_t rows, per, cnt, width;
};
struct RopeReduceJobs {
  RopeReduceJob job[3];
  int64_t nheads;
};

template <int W>
__device__ __forceinline__ void reduce_unit(const RopeReduceJob &jb, int64_t H, int64_t u) {
  const int64_t wu = jb.width / W;
  const int64_t r = u / wu, c = (u % wu) * W;
  const float *src = jb.in + ((r / jb.per) * H + (r % jb.per) * jb.cnt) * jb.width + c;
  float acc[W];
  vload<W>(src, acc);
  for (int64_t i = 1; i < jb.cnt; ++i) {
    float v[W];
    vload<W>(src + i * jb.width, v);
#pragma unroll
    for (int e = 0; e < W; ++e) acc[e] += v[e];
  }
  vstore<W>(jb.out + r * jb.width + c, acc);
}

__global__ void __launch_bounds__(256) rope_bwd_reduce_kernel(const RopeReduceJobs jobs) {
  const RopeReduceJob jb = blockIdx.y == 0 ? jobs.job[0] : (blockIdx.y == 1 ? jobs.job[1] : jobs.job[2]);
  if (jb.out == nullptr) return;
  const int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (jb.width % 4 == 0) {
    if (u < jb.rows * (jb.width / 4)) reduce_unit<4>(jb, jobs.nheads, u);
  } else {
    if (u < jb.rows * jb.width) reduce_unit<1>(jb, jobs.nheads, u);
  }
}

template <typename Tin, typename Tg, int KP>
hipError_t launch_bwd_kp(const RopeBwdParams &p, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(p.batch * p.nheads));
  hipLaunchKernelGGL((rope_bc_bwd_kernel<Tin, Tg, KP>), grid, dim3(RopeCfg<KP>::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <typename Tin, typename Tg>
hipError_t launch_bwd_typed(const RopeBwdParams &p, hipStream_t stream) {
  switch (p.dstate) {
    case 2: return launch_bwd_kp<Tin, Tg, 1>(p, stream);
    case 4: return launch_bwd_kp<Tin, Tg, 2>(p, stream);
    case 8: return launch_bwd_kp<Tin, Tg, 4>(p, stream);
    case 16: return launch_bwd_kp<Tin, Tg, 8>(p, stream);
    case 32: return launch_bwd_kp<Tin, Tg, 16>(p, stream);
    case 64: return launch_bwd_kp<Tin, Tg, 32>(p, stream);
    case 128: return launch_bwd_kp<Tin, Tg, 64>(p, stream);
    case 256: return launch_bwd_kp<Tin, Tg, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rope_bwd(const RopeBwdParams &p, int in_bf16, int g_bf16, hipStream_t stream) {
  if (p.batch * p.nheads == 0) return hipSuccess;
  hipError_t e;
  if (!in_bf16 && !g_bf16) e = launch_bwd_typed<float, float>(p, stream);
  else if (!in_bf16 && g_bf16) e = launch_bwd_typed<float, uint16_t>(p, stream);
  else if (in_bf16 && !g_bf16) e = launch_bwd_typed<uint16_t, float>(p, stream);
  else e = launch_bwd_typed<uint16_t, uint16_t>(p, stream);
  if (e != hipSuccess) return e;
  // Head sums of the per-head terms that went to the workspace.
  const int64_t H = p.nheads, half = p.dstate / 2, bl = p.batch * p.seqlen;
  RopeReduceJobs jobs{};
  jobs.nheads = H;
  int64_t units = 0;
  if (p.ngroups < H && bl > 0) {
    const int64_t rows = bl * p.ngroups;
    jobs.job[0] = RopeReduceJob{p.ws_dB, p.dB, rows, p.ngroups, H / p.ngroups, p.dstate};
    jobs.job[1] = RopeReduceJob{p.ws_dC, p.dC, rows, p.ngroups, H / p.ngroups, p.dstate};
    units = max(units, rows * p.dstate / (p.dstate % 4 == 0 ? 4 : 1));
  }
  if (p.theta_heads < H && bl > 0) {
    jobs.job[2] = RopeReduceJob{p.ws_dth, p.dtheta, bl, 1, H, half};
    units = max(units, bl * half / (half % 4 == 0 ? 4 : 1));
  }
  if (units == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((units + 255) / 256), 3);
  hipLaunchKernelGGL(rope_bwd_reduce_kernel, grid, dim3(256), 0, stream, jobs);
  return hipGetLastError();
}

hipError_t launch_rope(const RopeParams &p, int in_bf16, int out_bf16, hipStream_t stream) {
  if (p.batch * p.nheads == 0) return hipSuccess;
  if (!in_bf16 && !out_bf16) return launch_typed<float, float>(p, stream);
  if (!in_bf16 && out_bf16) return launch_typed<float, uint16_t>(p, stream);
  if (in_bf16 && !out_bf16) return launch_typed<uint16_t, float>(p, stream);
  return launch_typed<uint16_t, uint16_t>(p, stream);
}

}  // namespace ssm
