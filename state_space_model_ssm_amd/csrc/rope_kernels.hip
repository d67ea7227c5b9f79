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
// dB and dC sum over the heads that share a group, and dtheta over all heads
// when they share theta, so the work is tiled over time with every head of a
// tile in one workgroup and the head sums kept in registers:
//   1. rope_bwd_angle_kernel, per (b, h): the angle before each tile of T
//      steps (float64 running sum as in the forward; stored as float32
//      revolutions reduced to [-1/2, 1/2]).
//   2. rope_bwd_tile_kernel, per (b, tile): each wavefront holds the tile's T
//      steps (rows) for one part of the pairs and one head slot, and loops
//      over its slot's heads.  Per head, a scan over the rows gives the angle
//      within the tile (float32 revolutions, reduced after every addition)
//      and a reverse scan the sum of dphi from the tile's end (R local to the
//      tile); both stay inside the wavefront (lane shuffles), so the head
//      loop has no barrier.  The undone rotations add into registers and
//      are summed over slots through LDS when a group ends.  It writes dB,
//      dC, the local parts of dtheta and ddt, and each (head, tile)'s total
//      of dphi.
//   3. rope_bwd_suffix_kernel, per (b, h): R at each tile's end (dangle_last
//      plus the later tiles' totals, float64) and dangle0.
//   4. rope_bwd_fix_kernel, per step: adds R_end's share, -dt R_end to dtheta
//      and -theta . R_end to ddt, then the chain rule through the step's
//      softplus.
// Every output element is written by one thread and every sum runs in a
// fixed order, so results do not depend on timing.

constexpr int kBwdThreads = 512;
// Tile kernel layout for N / 2 = KP pairs: a row (one step) takes TPR
// threads of VEC pairs (as the forward), split over KS wavefronts of TPRW
// (at most 8) lanes each; a wavefront holds T = 64 / TPRW rows; the 8
// wavefronts are HS = 8 / KS head slots.  T is 8 from KP = 32 up.  (Two
// pairs per thread, with fewer registers but twice the head rounds, measured
// 10% slower on 32 x 256 x 32 heads x 128 states.)
template <int KP>
struct BwdCfg {
  static constexpr int VEC = RopeCfg<KP>::VEC;
  static constexpr int TPR = RopeCfg<KP>::TPR;
  static constexpr int KS = TPR >= 32 ? 4 : (TPR >= 16 ? 2 : 1);
  static constexpr int TPRW = TPR / KS;
  static constexpr int T = 64 / TPRW;
  static constexpr int HS = 8 / KS;
  static_assert(T * TPRW == 64 && HS * KS == 8, "rows tile a wavefront");
};
// Fix-up kernel layout: rows (steps) of TPR threads of VEC pairs.
template <int KP>
struct FixCfg {
  static constexpr int VEC = RopeCfg<KP>::VEC;
  static constexpr int TPR = RopeCfg<KP>::TPR;
  static constexpr int ROWS = kBwdThreads / 4 / TPR;  // steps per workgroup
};

// Sum over the W consecutive lanes that hold one row's pairs.  Called by
// every lane of the wavefront (no enclosing branch).
template <int W>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ float wrap_rev(float v) { return v - rintf(v); }

// Pass 1: the angle before every tile.  The forward's layout (segments of
// consecutive steps, combined through LDS) with half its segments per
// workgroup (256 threads), so that every workgroup of the SSD-sized problems
// is resident at once.
template <int KP>
struct AngleCfg {
  static constexpr int VEC = RopeCfg<KP>::VEC;
  static constexpr int TPR = RopeCfg<KP>::TPR;
  static constexpr int NSEG = 256 / TPR < 64 ? 256 / TPR : 64;
  static constexpr int THREADS = TPR * NSEG;
};

template <typename Tin, int KP>
__global__ void __launch_bounds__(256) rope_bwd_angle_kernel(const RopeBwdParams p) {
  using Cfg = AngleCfg<KP>;
  constexpr int VEC = Cfg::VEC, TPR = Cfg::TPR, NSEG = Cfg::NSEG;
  constexpr int NB = 8;                // steps whose loads are issued together
  constexpr int T = BwdCfg<KP>::T;     // steps per tile, a power of two
  constexpr bool kShort = T <= 8;      // segments of up to two tiles in one pass
  __shared__ double sPart[NSEG * KP];

  const int seg = threadIdx.x / TPR;
  const int k0 = (threadIdx.x % TPR) * VEC;
  const int64_t H = p.nheads, L = p.seqlen;
  const int64_t nblk = p.batch * H;
  int64_t id = blockIdx.x;
  if (nblk % 8 == 0) id = (id % 8) * (nblk / 8) + id / 8;  // a batch row's heads on one XCD (shared theta)
  const int64_t b = id / H, h = id % H;
  const int64_t th = p.theta_heads == 1 ? 0 : h;
  // Segments of whole tiles.
  const int64_t seglen = ((L + NSEG - 1) / NSEG + T - 1) / T * T;
  const int64_t t0 = min(L, seg * seglen), t1 = min(L, t0 + seglen);
  const int n = static_cast<int>(t1 - t0);
  const float bias = (p.dt_softplus && p.dt_bias != nullptr) ? p.dt_bias[h] : 0.0f;
  const int64_t row0 = b * L + t0;
  const Tin *dtp = static_cast<const Tin *>(p.dt) + row0 * H + h;
  const Tin *thp = static_cast<const Tin *>(p.theta) + (row0 * p.theta_heads + th) * KP + k0;
  const int64_t s_dt = H, s_th = p.theta_heads * KP;
  auto step = [&](int i) __attribute__((always_inline)) {
    const float dt = ld(dtp, i * s_dt);
    return p.dt_softplus ? dt_softplus(dt + bias) : dt;
  };
  const int64_t ai = (b * H + h) * KP + k0;
  float *angp = p.ws_ang + ((b * H + h) * p.ntile + t0 / T) * KP + k0;
  double phi[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) phi[j] = p.angle0 != nullptr ? static_cast<double>(p.angle0[ai + j]) : 0.0;
  auto combine = [&](const double (&part)[VEC]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) sPart[seg * KP + k0 + j] = part[j];
    __syncthreads();
    for (int s = 0; s < seg; ++s) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) phi[j] -= sPart[s * KP + k0 + j];
    }
  };
  auto store_angle = [&](int tile_in_seg, const double (&a)[VEC]) __attribute__((always_inline)) {
    float v[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const double r = a[j] * kInvTwoPi;
      v[j] = static_cast<float>(r - rint(r));
    }
    vstore<VEC>(angp + tile_in_seg * KP, v);
  };

  if (kShort && seglen <= 2 * T) {
    // The segment's (at most two) tiles summed apart, one tile's loads at a
    // time, so the tile angles follow from the segment's start.
    double ts[2][VEC];
#pragma unroll 1
    for (int u = 0; u < 2; ++u) {
      float dv[T], tv[T][VEC];
#pragma unroll
      for (int q = 0; q < T; ++q) {
        dv[q] = 0.0f;
#pragma unroll
        for (int j = 0; j < VEC; ++j) tv[q][j] = 0.0f;
        if (u * T + q < n) {
          dv[q] = step(u * T + q);
          vload<VEC>(thp + (u * T + q) * s_th, tv[q]);
        }
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        double a = 0.0;
#pragma unroll
        for (int q = 0; q < T; ++q) a += static_cast<double>(dv[q]) * static_cast<double>(tv[q][j]);
        if (u == 0) ts[0][j] = a;
        else ts[1][j] = a;
      }
    }
    double part[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) part[j] = ts[0][j] + ts[1][j];
    combine(part);
    if (n > 0) store_angle(0, phi);
    if (n > T) {
      double a1[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) a1[j] = phi[j] - ts[0][j];
      store_angle(1, a1);
    }
    return;
  }

  // Longer segments: sum, combine, then walk the segment again.
  double part[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) part[j] = 0.0;
  for (int i0 = 0; i0 < n; i0 += NB) {
    float dv[NB], tv[NB][VEC];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = min(i0 + q, n - 1);
      dv[q] = step(i);
      vload<VEC>(thp + i * s_th, tv[q]);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (i0 + q < n) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) part[j] += static_cast<double>(dv[q]) * static_cast<double>(tv[q][j]);
      }
  }
  combine(part);
  for (int i0 = 0; i0 < n; i0 += NB) {
    float dv[NB], tv[NB][VEC];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int i = min(i0 + q, n - 1);
      dv[q] = step(i);
      vload<VEC>(thp + i * s_th, tv[q]);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (i0 + q < n) {
        const int i = i0 + q;  // t0 is a multiple of T
        if ((i & (T - 1)) == 0) store_angle(i / T, phi);
#pragma unroll
        for (int j = 0; j < VEC; ++j) phi[j] -= static_cast<double>(dv[q]) * static_cast<double>(tv[q][j]);
      }
  }
}

// Pass 2: one tile of T steps of one batch row, every head (see above).
// Wavefront w: pair part ks = w % KS, head slot w / KS; lane: row (step) r =
// lane / TPRW, pairs k0 .. k0 + VEC - 1 of part ks.
// Registers held to 128 (two workgroups per CU; a few spill): unbounded
// (~140 registers, one workgroup per CU) measured 16% slower, and loading the
// next head's operands a round ahead (160 registers) slower still.
template <typename Tin, typename Tg, int KP>
__global__ void __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(4)))
rope_bwd_tile_kernel(const RopeBwdParams p) {
  using Cfg = BwdCfg<KP>;
  constexpr int VEC = Cfg::VEC, TPRW = Cfg::TPRW, T = Cfg::T, KS = Cfg::KS;
  constexpr int N = 2 * KP;
  constexpr int NACC = 4 * VEC;
  __shared__ float sRed[NACC * kBwdThreads];  // [component][thread]: lanes consecutive

  const int tid = threadIdx.x;
  const int lane = tid % 64, wave = tid / 64;
  const int ks = wave % KS, slot = wave / KS;
  const int r = lane / TPRW;
  const int k0 = (ks * TPRW + lane % TPRW) * VEC;
  const int64_t H = p.nheads, L = p.seqlen, G = p.ngroups, hpg = H / G;
  const int US = p.slots;                    // slots in use
  const int64_t b = blockIdx.x / p.ntile, tile = blockIdx.x % p.ntile;
  const int64_t t = tile * T + r;
  const bool act_t = t < L;
  const int64_t bt = b * L + (act_t ? t : 0);
  const int rounds = static_cast<int>((H + US - 1) / US);
  const int64_t span = hpg < US ? hpg : US;  // slots that share a group in one round

  const Tin *dtp = static_cast<const Tin *>(p.dt) + bt * H;
  const Tin *thp = static_cast<const Tin *>(p.theta) + bt * p.theta_heads * KP + k0;
  const Tg *gbp = static_cast<const Tg *>(p.dB_rot) + bt * H * N + k0;
  const Tg *gcp = static_cast<const Tg *>(p.dC_rot) + bt * H * N + k0;
  const bool shared_theta = p.theta_heads == 1 && H > 1;
  float th[VEC], aTh[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) th[j] = aTh[j] = 0.0f;
  if (act_t && p.theta_heads == 1) vload<VEC>(thp, th);
  float b1[VEC], b2[VEC], c1[VEC], c2[VEC], acc[NACC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) b1[j] = b2[j] = c1[j] = c2[j] = 0.0f;
#pragma unroll
  for (int q = 0; q < NACC; ++q) acc[q] = 0.0f;
  int64_t gcur = -1;

  for (int it = 0; it < rounds; ++it) {
    const int64_t hh = static_cast<int64_t>(it) * US + slot;
    const bool hv = slot < US && hh < H;  // wavefront-uniform
    const bool act = act_t && hv;
    const int64_t h = hv ? hh : 0;
    const int64_t g = h / hpg;
    if (hv && g != gcur) {
      gcur = g;
      if (act_t) {
        const Tin *bp = static_cast<const Tin *>(p.B) + (bt * G + g) * N + k0;
        const Tin *cp = static_cast<const Tin *>(p.C) + (bt * G + g) * N + k0;
        vload<VEC>(bp, b1);
        vload<VEC>(bp + KP, b2);
        vload<VEC>(cp, c1);
        vload<VEC>(cp + KP, c2);
      }
    }
    float dv = 0.0f, a0[VEC], gb1[VEC], gb2[VEC], gc1[VEC], gc2[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) a0[j] = gb1[j] = gb2[j] = gc1[j] = gc2[j] = 0.0f;
    if (hv) vload<VEC>(p.ws_ang + ((b * H + h) * p.ntile + tile) * KP + k0, a0);
    if (act) {
      const float raw = ld(dtp, h);
      dv = p.dt_softplus ? dt_softplus(raw + (p.dt_bias != nullptr ? p.dt_bias[h] : 0.0f)) : raw;
      if (p.theta_heads != 1) vload<VEC>(thp + h * KP, th);
      vload<VEC>(gbp + h * N, gb1);
      vload<VEC>(gbp + h * N + KP, gb2);
      vload<VEC>(gcp + h * N, gc1);
      vload<VEC>(gcp + h * N + KP, gc2);
    }
    // The angle within the tile: inclusive prefix over the rows of dt theta
    // in revolutions (each term formed in float64 and reduced, then the
    // float32 partial sums reduced after every addition).
    float pre[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const double a = static_cast<double>(dv) * static_cast<double>(th[j]) * kInvTwoPi;
      pre[j] = act ? static_cast<float>(a - rint(a)) : 0.0f;
    }
#pragma unroll
    for (int d = 1; d < T; d <<= 1) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float u = __shfl_up(pre[j], d * TPRW);
        if (r >= d) pre[j] = wrap_rev(pre[j] + u);
      }
    }
    // Undo the rotation; dphi.
    float R[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const float fr = wrap_rev(a0[j] - pre[j]);
      const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
      const float db1 = gb1[j] * cs + gb2[j] * sn, db2 = gb2[j] * cs - gb1[j] * sn;
      const float dc1 = gc1[j] * cs + gc2[j] * sn, dc2 = gc2[j] * cs - gc1[j] * sn;
      acc[j] += db1;
      acc[VEC + j] += db2;
      acc[2 * VEC + j] += dc1;
      acc[3 * VEC + j] += dc2;
      R[j] = b1[j] * db2 - b2[j] * db1 + c1[j] * dc2 - c2[j] * dc1;
    }
    // R local to the tile: inclusive suffix over the rows.
#pragma unroll
    for (int d = 1; d < T; d <<= 1) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float u = __shfl_down(R[j], d * TPRW);
        if (r + d < T) R[j] += u;
      }
    }
    if (r == 0 && hv) vstore<VEC>(p.ws_tot + ((b * H + h) * p.ntile + tile) * KP + k0, R);
    float dd = 0.0f;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      dd += th[j] * R[j];
      if (shared_theta) aTh[j] -= dv * R[j];
    }
    if (act && !shared_theta) {
      float o[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) o[j] = -dv * R[j];
      vstore<VEC>(p.dtheta + (bt * H + h) * KP + k0, o);
    }
    dd = row_sum<TPRW>(dd);
    if (act && lane % TPRW == 0) {
      if (KS == 1) p.ddt[bt * H + h] = -dd;
      else p.ws_ddt[(bt * H + h) * KS + ks] = -dd;
    }

    // A group ends with this round: its slots' sums of dB, dC, added in slot
    // order by the first slot of the group.
    if (((static_cast<int64_t>(it) + 1) * US) % hpg == 0 || it == rounds - 1) {
      if (span == 1) {
        if (act) {
          float *dbp = p.dB + (bt * G + g) * N + k0;
          float *dcp = p.dC + (bt * G + g) * N + k0;
          vstore<VEC>(dbp, *reinterpret_cast<float(*)[VEC]>(&acc[0]));
          vstore<VEC>(dbp + KP, *reinterpret_cast<float(*)[VEC]>(&acc[VEC]));
          vstore<VEC>(dcp, *reinterpret_cast<float(*)[VEC]>(&acc[2 * VEC]));
          vstore<VEC>(dcp + KP, *reinterpret_cast<float(*)[VEC]>(&acc[3 * VEC]));
        }
      } else {
#pragma unroll
        for (int q = 0; q < NACC; ++q) sRed[q * kBwdThreads + tid] = acc[q];
        __syncthreads();
        if (act && slot % span == 0) {
          for (int s = 1; s < span; ++s) {
            const int src = tid + s * KS * 64;  // same part and lane, slot + s
#pragma unroll
            for (int q = 0; q < NACC; ++q) acc[q] += sRed[q * kBwdThreads + src];
          }
          float *dbp = p.dB + (bt * G + g) * N + k0;
          float *dcp = p.dC + (bt * G + g) * N + k0;
          vstore<VEC>(dbp, *reinterpret_cast<float(*)[VEC]>(&acc[0]));
          vstore<VEC>(dbp + KP, *reinterpret_cast<float(*)[VEC]>(&acc[VEC]));
          vstore<VEC>(dcp, *reinterpret_cast<float(*)[VEC]>(&acc[2 * VEC]));
          vstore<VEC>(dcp + KP, *reinterpret_cast<float(*)[VEC]>(&acc[3 * VEC]));
        }
        __syncthreads();
      }
#pragma unroll
      for (int q = 0; q < NACC; ++q) acc[q] = 0.0f;
    }
  }

  // The local dtheta of a theta shared by all heads: the slots' sums.
  if (shared_theta) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) sRed[j * kBwdThreads + tid] = aTh[j];
    __syncthreads();
    if (slot == 0 && act_t) {
      for (int s = 1; s < US; ++s) {
        const int src = tid + s * KS * 64;
#pragma unroll
        for (int j = 0; j < VEC; ++j) aTh[j] += sRed[j * kBwdThreads + src];
      }
      vstore<VEC>(p.dtheta + bt * KP + k0, aTh);
    }
  }
}

// Pass 3: R at the end of every tile (in place of the tile totals) and
// dangle0.  One workgroup per (b, h): threads (pair k, segment of tiles),
// segment sums combined through LDS.
template <int KP>
__global__ void __launch_bounds__(256) rope_bwd_suffix_kernel(const RopeBwdParams p) {
  constexpr int NS = 256 / KP < 1 ? 1 : 256 / KP;  // segments (KP <= 128: at least 2)
  constexpr int NB = 8;
  __shared__ double sSeg[NS * KP];
  const int k = threadIdx.x % KP, seg = threadIdx.x / KP;
  const int64_t bh = blockIdx.x;
  const int64_t nt = p.ntile, per = (nt + NS - 1) / NS;
  const int64_t i0 = min(nt, seg * per), i1 = min(nt, i0 + per);
  float *tot = p.ws_tot + bh * nt * KP + k;
  double s = 0.0;
  for (int64_t a = i0; a < i1; a += NB) {
    float v[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) v[q] = a + q < i1 ? tot[(a + q) * KP] : 0.0f;
#pragma unroll
    for (int q = 0; q < NB; ++q) s += static_cast<double>(v[q]);
  }
  sSeg[seg * KP + k] = s;
  __syncthreads();
  double R = p.dangle_last != nullptr ? static_cast<double>(p.dangle_last[bh * KP + k]) : 0.0;
  for (int q = seg + 1; q < NS; ++q) R += sSeg[q * KP + k];
  if (seg == 0 && p.dangle0 != nullptr) p.dangle0[bh * KP + k] = static_cast<float>(R + s);
  // Walk the segment from its end; every load of a batch precedes its stores.
  for (int64_t e = i1; e > i0; e -= NB) {
    float v[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) v[q] = e - 1 - q >= i0 ? tot[(e - 1 - q) * KP] : 0.0f;
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (e - 1 - q >= i0) {
        tot[(e - 1 - q) * KP] = static_cast<float>(R);
        R += static_cast<double>(v[q]);
      }
  }
}

// Pass 4: R_end's share of dtheta and ddt.  A row (one step) takes TPR
// threads of VEC pairs in each of NHG head groups (128 threads per group);
// group g takes heads in blocks of HB, g * HB + NHG * HB * i + q, whose loads
// are issued together (HB = 8 with a theta shared by all heads, whose dtheta
// is one row per step; 4 with theta per head, which also reads and writes a
// dtheta row per head).  With a shared theta the groups' sums of -dt R_end
// are added in group order through LDS.
template <typename Tin, int KP, bool SHARED>
__global__ void __launch_bounds__(kBwdThreads) rope_bwd_fix_kernel(const RopeBwdParams p) {
  using Cfg = FixCfg<KP>;
  constexpr int VEC = Cfg::VEC, TPR = Cfg::TPR, KS = BwdCfg<KP>::KS;
  constexpr int NHG = 4, GT = kBwdThreads / NHG, HB = SHARED ? 8 : 4;
  constexpr int NTH = SHARED ? 1 : HB;  // theta rows held
  constexpr int RPG = GT / TPR;  // rows (steps) per workgroup
  __shared__ float sAcc[SHARED ? VEC * kBwdThreads : 1];
  const int hg = threadIdx.x / GT, tl = threadIdx.x % GT;
  const int kb = tl % TPR, k0 = kb * VEC;
  const int64_t H = p.nheads, L = p.seqlen;
  const int64_t flat = static_cast<int64_t>(blockIdx.x) * RPG + tl / TPR;  // (b, t)
  const bool act = flat < p.batch * L;
  const int64_t bt = act ? flat : 0;
  const int64_t b = bt / L, t = bt % L, tile = t / BwdCfg<KP>::T;
  const Tin *dtp = static_cast<const Tin *>(p.dt) + bt * H;
  const Tin *thp = static_cast<const Tin *>(p.theta) + bt * p.theta_heads * KP + k0;
  const float *rep = p.ws_tot + (b * H * p.ntile + tile) * KP + k0;
  const int64_t s_re = p.ntile * KP;
  float th[NTH][VEC], acc[VEC], thold[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] = thold[j] = 0.0f;
#pragma unroll
  for (int q = 0; q < NTH; ++q)
#pragma unroll
    for (int j = 0; j < VEC; ++j) th[q][j] = 0.0f;
  // Loads that precede every store (a load after a store waits for it).
  if (act && SHARED) {
    vload<VEC>(thp, th[0]);
    if (hg == 0) vload<VEC>(p.dtheta + bt * KP + k0, thold);
  }
  for (int64_t h0 = static_cast<int64_t>(hg) * HB; h0 < H; h0 += NHG * HB) {
    float re[HB][VEC], dv[HB], part[HB], old[SHARED ? 1 : HB][VEC];
#pragma unroll
    for (int q = 0; q < HB; ++q) {
      const int64_t h = min(h0 + q, H - 1);
      dv[q] = part[q] = 0.0f;
#pragma unroll
      for (int j = 0; j < VEC; ++j) re[q][j] = 0.0f;
      if (!SHARED) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) old[SHARED ? 0 : q][j] = 0.0f;
      }
      if (act) {
        vload<VEC>(rep + h * s_re, re[q]);
        const float raw = ld(dtp, h);
        dv[q] = p.dt_softplus ? dt_softplus(raw + (p.dt_bias != nullptr ? p.dt_bias[h] : 0.0f)) : raw;
        if (!SHARED) {
          vload<VEC>(thp + (p.theta_heads != 1 ? h * KP : 0), th[SHARED ? 0 : q]);
          vload<VEC>(p.dtheta + (bt * H + h) * KP + k0, old[SHARED ? 0 : q]);
        }
        if (kb == 0) {
          if (KS == 1) {
            part[q] = p.ddt[bt * H + h];
          } else {
#pragma unroll
            for (int s = 0; s < KS; ++s) part[q] += p.ws_ddt[(bt * H + h) * KS + s];
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < HB; ++q) {
      const int64_t h = h0 + q;
      const int tq = SHARED ? 0 : q;
      float dd = 0.0f;
#pragma unroll
      for (int j = 0; j < VEC; ++j) dd += th[tq][j] * re[q][j];
      dd = row_sum<TPR>(dd);
      if (h < H) {
        if (SHARED) {
#pragma unroll
          for (int j = 0; j < VEC; ++j) acc[j] -= dv[q] * re[q][j];
        } else if (act) {
          float o[VEC];
#pragma unroll
          for (int j = 0; j < VEC; ++j) o[j] = old[tq][j] - dv[q] * re[q][j];
          vstore<VEC>(p.dtheta + (bt * H + h) * KP + k0, o);
        }
        if (act && kb == 0) {
          float v = part[q] - dd;
          if (p.dt_softplus) v *= 1.0f - expf(-dv[q]);  // d softplus(x) / dx = sigmoid(x) = 1 - exp(-softplus(x))
          p.ddt[bt * H + h] = v;
        }
      }
    }
  }
  if (SHARED) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) sAcc[j * kBwdThreads + threadIdx.x] = acc[j];
    __syncthreads();
    if (hg == 0 && act) {
      for (int g = 1; g < NHG; ++g) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[j] += sAcc[j * kBwdThreads + g * GT + tl];
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) thold[j] += acc[j];
      vstore<VEC>(p.dtheta + bt * KP + k0, thold);
    }
  }
}

template <typename Tin, typename Tg, int KP>
hipError_t launch_bwd_kp(const RopeBwdParams &p, hipStream_t stream) {
  using Cfg = BwdCfg<KP>;
  if (p.tile_len != Cfg::T || p.slots < 1 || p.slots > Cfg::HS || p.ws_parts != Cfg::KS) return hipErrorInvalidValue;
  const int64_t bl = p.batch * p.seqlen;
  if (bl > 0) {
    hipLaunchKernelGGL((rope_bwd_angle_kernel<Tin, KP>), dim3(static_cast<uint32_t>(p.batch * p.nheads)),
                       dim3(AngleCfg<KP>::THREADS), 0, stream, p);
    hipLaunchKernelGGL((rope_bwd_tile_kernel<Tin, Tg, KP>), dim3(static_cast<uint32_t>(p.batch * p.ntile)),
                       dim3(kBwdThreads), 0, stream, p);
  }
  hipLaunchKernelGGL((rope_bwd_suffix_kernel<KP>), dim3(static_cast<uint32_t>(p.batch * p.nheads)), dim3(256), 0,
                     stream, p);
  if (bl > 0) {
    const dim3 grid(static_cast<uint32_t>((bl + FixCfg<KP>::ROWS - 1) / FixCfg<KP>::ROWS));
    if (p.theta_heads == 1 && p.nheads > 1)
      hipLaunchKernelGGL((rope_bwd_fix_kernel<Tin, KP, true>), grid, dim3(kBwdThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((rope_bwd_fix_kernel<Tin, KP, false>), grid, dim3(kBwdThreads), 0, stream, p);
  }
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
  if (!in_bf16 && !g_bf16) return launch_bwd_typed<float, float>(p, stream);
  if (!in_bf16 && g_bf16) return launch_bwd_typed<float, uint16_t>(p, stream);
  if (in_bf16 && !g_bf16) return launch_bwd_typed<uint16_t, float>(p, stream);
  return launch_bwd_typed<uint16_t, uint16_t>(p, stream);
}

hipError_t launch_rope(const RopeParams &p, int in_bf16, int out_bf16, hipStream_t stream) {
  if (p.batch * p.nheads == 0) return hipSuccess;
  if (!in_bf16 && !out_bf16) return launch_typed<float, float>(p, stream);
  if (!in_bf16 && out_bf16) return launch_typed<float, uint16_t>(p, stream);
  if (in_bf16 && !out_bf16) return launch_typed<uint16_t, float>(p, stream);
  return launch_typed<uint16_t, uint16_t>(p, stream);
}

}  // namespace ssm
