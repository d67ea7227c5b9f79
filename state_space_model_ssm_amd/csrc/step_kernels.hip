// Single-token decode step for gfx950: one recurrence step from a cached
// state, updated in place.
//
// Math ("Mamba-3 NKI Kernels for AWS Neuron", section "How it works": decode
// through step() is the direct recurrence, and section "Kernel details",
// mamba3_siso_decode_state_kernel: state update plus output contraction; here
// with beta = 0 and gamma = dt, i.e. the selective-scan step):
//   h[n] <- exp(dt A[n]) h[n] + dt B[n] u
//   y     = (sum_n C[n] h[n] + D u) * silu(z)
// Per channel (scan step: A is (dim, N), dt is per channel) or per head (SSD
// step: channel d = (head, p), A and dt are per head, D too).
//
// TRAP (SSD step only): the trapezoidal three-term step of the same section
// (its Eq. 9), with alpha = exp(dt A), gamma = lam dt, beta = (dt - gamma) alpha:
//   h[n] <- alpha h[n] + beta x_prev B_prev[n] + gamma x B[n]
// where x_prev, B_prev are the previous token's inputs (zero when absent).
//
// The step reads and writes the whole state once, so it is bound by HBM:
// every thread owns K = 8 consecutive states of one channel (two 16-byte
// loads and stores in flight per thread: 5.9 TB/s on a 33.6 MB state, against
// 4.6 TB/s with K = 4 and 4.2 TB/s with K = 16), the N / K threads of a
// channel are adjacent lanes, and the readout is a butterfly over those lanes.
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t *p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ void st(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t *p, int64_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // round to nearest even
}

// States per thread (two 16-byte state loads and stores in flight); 4 and 16
// measured slower.
constexpr int kStepStates = 8;

template <typename Tin, typename Tout, int N, bool HEAD, bool HAS_Z, bool TRAP>
__global__ void __launch_bounds__(256) step_kernel(const StepParams p) {
  static_assert(!TRAP || HEAD, "the trapezoidal step is per head");
  constexpr int K = N < kStepStates ? N : kStepStates;  // states per thread
  constexpr int TPC = N / K;              // threads per channel (adjacent lanes)
  const Tin *__restrict__ gu = static_cast<const Tin *>(p.u);
  const Tin *__restrict__ gdt = static_cast<const Tin *>(p.delta);
  const Tin *__restrict__ gB = static_cast<const Tin *>(p.B);
  const Tin *__restrict__ gC = static_cast<const Tin *>(p.C);
  const Tin *__restrict__ gz = static_cast<const Tin *>(p.z);
  Tout *__restrict__ gy = static_cast<Tout *>(p.y);

  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t chan = gid / TPC;                 // (batch, channel) row
  const int j = static_cast<int>(gid % TPC);      // state group of this thread
  const bool live = chan < p.batch * p.dim;
  const int64_t cc = live ? chan : 0;             // a valid row for every lane
  const int64_t b = cc / p.dim;
  const int64_t d = cc % p.dim;
  const int64_t g = d / (p.dim / p.ngroups);
  const int64_t hd = HEAD ? d / p.headdim : d;    // per-head quantities live here

  const float u = ld(gu, cc);
  float dt = HEAD ? ld(gdt, b * (p.dim / p.headdim) + hd) : ld(gdt, cc);
  if (p.dt_softplus) dt = dt_softplus(dt + (p.dt_bias != nullptr ? p.dt_bias[hd] : 0.0f));
  float *st_row = p.state + cc * N + j * K;
  const int64_t bc = (b * p.ngroups + g) * N + j * K;

  float h[K], part = 0.0f;
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int k = 0; k < K; k += 4) {
      const float4 h4 = *reinterpret_cast<const float4 *>(st_row + k);
      h[k] = h4.x; h[k + 1] = h4.y; h[k + 2] = h4.z; h[k + 3] = h4.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) h[k] = st_row[k];
  }
  if constexpr (TRAP) {
    const Tin *__restrict__ glam = static_cast<const Tin *>(p.lam);
    float lam = ld(glam, b * (p.dim / p.headdim) + hd);
    if (p.lam_sigmoid) lam = 1.0f / (1.0f + expf(-lam));
    const float gam = lam * dt;
    const float decay = __builtin_amdgcn_exp2f(dt * p.A[hd] * kLog2e);
    const float gu = gam * u;
    // beta x_prev = (dt - gamma) alpha x_prev; zero without a previous token.
    const float bxp = p.x_prev != nullptr ? (dt - gam) * decay * ld(static_cast<const Tin *>(p.x_prev), cc) : 0.0f;
    const Tin *gBp = static_cast<const Tin *>(p.x_prev != nullptr ? p.B_prev : p.B);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      h[k] = fmaf(decay, h[k], fmaf(bxp, ld(gBp, bc + k), gu * ld(gB, bc + k)));
      part = fmaf(ld(gC, bc + k), h[k], part);
    }
  } else {
    const float dtu = dt * u;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float a = HEAD ? p.A[hd] : p.A[d * N + j * K + k];
      const float decay = __builtin_amdgcn_exp2f(dt * a * kLog2e);
      h[k] = fmaf(decay, h[k], dtu * ld(gB, bc + k));
      part = fmaf(ld(gC, bc + k), h[k], part);
    }
  }
  if (live) {
    if constexpr (K % 4 == 0) {
#pragma unroll
      for (int k = 0; k < K; k += 4)
        *reinterpret_cast<float4 *>(st_row + k) = make_float4(h[k], h[k + 1], h[k + 2], h[k + 3]);
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) st_row[k] = h[k];
    }
  }
  // Sum over the TPC adjacent lanes of the channel (TPC is a power of two
  // <= 64 and channels start on multiples of TPC, so groups never straddle).
#pragma unroll
  for (int m = 1; m < TPC; m <<= 1) part += __shfl_xor(part, m);
  if (live && j == 0) {
    float y = part;
    if (p.D != nullptr) y = fmaf(p.D[hd], u, y);
    if constexpr (HAS_Z) {
      const float zv = ld(gz, cc);
      y *= zv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * kLog2e));
    }
    st(gy, cc, y);
  }
}

template <typename Tin, typename Tout, int N, bool HEAD>
hipError_t launch_n(const StepParams &p, hipStream_t stream) {
  constexpr int TPC = N < kStepStates ? 1 : N / kStepStates;
  const int64_t threads = p.batch * p.dim * TPC;
  if (threads == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((threads + 255) / 256));
  const bool trap = HEAD && p.lam != nullptr;
  if (trap) {
    if constexpr (HEAD) {
      if (p.z != nullptr)
        hipLaunchKernelGGL((step_kernel<Tin, Tout, N, HEAD, true, true>), grid, dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL((step_kernel<Tin, Tout, N, HEAD, false, true>), grid, dim3(256), 0, stream, p);
    }
  } else if (p.z != nullptr) {
    hipLaunchKernelGGL((step_kernel<Tin, Tout, N, HEAD, true, false>), grid, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((step_kernel<Tin, Tout, N, HEAD, false, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename Tin, typename Tout, bool HEAD>
hipError_t launch_typed(const StepParams &p, hipStream_t stream) {
  switch (p.dstate) {
    case 1: return launch_n<Tin, Tout, 1, HEAD>(p, stream);
    case 2: return launch_n<Tin, Tout, 2, HEAD>(p, stream);
    case 4: return launch_n<Tin, Tout, 4, HEAD>(p, stream);
    case 8: return launch_n<Tin, Tout, 8, HEAD>(p, stream);
    case 16: return launch_n<Tin, Tout, 16, HEAD>(p, stream);
    case 32: return launch_n<Tin, Tout, 32, HEAD>(p, stream);
    case 64: return launch_n<Tin, Tout, 64, HEAD>(p, stream);
    case 128: return launch_n<Tin, Tout, 128, HEAD>(p, stream);
    case 256: return launch_n<Tin, Tout, 256, HEAD>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool HEAD>
hipError_t launch_mode(const StepParams &p, int in_bf16, int out_bf16, hipStream_t stream) {
  if (!in_bf16 && !out_bf16) return launch_typed<float, float, HEAD>(p, stream);
  if (!in_bf16 && out_bf16) return launch_typed<float, uint16_t, HEAD>(p, stream);
  if (in_bf16 && !out_bf16) return launch_typed<uint16_t, float, HEAD>(p, stream);
  return launch_typed<uint16_t, uint16_t, HEAD>(p, stream);
}

}  // namespace

hipError_t launch_step(const StepParams &p, int per_head, int in_bf16, int out_bf16, hipStream_t stream) {
  return per_head ? launch_mode<true>(p, in_bf16, out_bf16, stream)
                  : launch_mode<false>(p, in_bf16, out_bf16, stream);
}

}  // namespace ssm
