// Backward of the scalar-decay SSD for gfx950: gradients of x, dt, A, B, C,
// D, z and h0 for upstream gradients dy and dh_last.
//
// Math (the chain rule on the SSD recurrence; "Mamba-3 NKI Kernels for AWS
// Neuron", section "Correctness", reports backward parity of the SSD but
// prints no formulas).  Per batch b and head h, with S_t the (P x N) state,
// yhat_t = S_t C_t + D x_t, dyhat_t = dy_t silu(z_t) and Lam_t = dL/dS_t:
//   Lam_t  = dyhat_t C_t^T + alpha_{t+1} Lam_{t+1}      (Lam_{L-1} + dh_last)
//   dx_t   = dt_t Lam_t B_t + D dyhat_t,   dB_t += dt_t Lam_t^T x_t,   dC_t += S_t^T dyhat_t
//   dz_t   = dy_t yhat_t silu'(z_t),       dD  += dyhat_t . x_t,       dh0 = alpha_0 Lam_0
//   g_t    = <Lam_t, alpha_t S_{t-1}>,     ddt_t = x_t^T Lam_t B_t + A g_t,   dA += dt_t g_t
//
// Two walks per (b, h), one workgroup each:
//   * forward walk: rebuilds S_t from h0 and writes dz, the per-head dC terms
//     S_t^T dyhat_t, u_t = dyhat_t . Y_t (Y_t = S_t C_t) and <dh_last, S_{L-1}>;
//   * reverse walk: carries Lam from dh_last and writes dx, ddt, dh0 and the
//     per-head dB terms.  g_t needs S_{t-1}, which this walk does not have; it
//     follows instead from phi_t = <Lam_t, S_t>, which obeys
//       g_t = phi_t - dt_t x_t^T Lam_t B_t,   phi_{t-1} = g_t + u_{t-1},
//       phi_{L-1} = <dh_last, S_{L-1}> + u_{L-1}
//     (both identities follow from S_t = alpha_t S_{t-1} + dt_t x_t B_t^T and
//     the Lam recurrence above), so only the scalars u_t cross from one walk
//     to the other.
// A reduction kernel then sums the per-head dB, dC terms over the heads of
// each group and the per-(b, h) dA, dD terms over batch rows, in a fixed
// order (no atomics: two calls give equal gradients).
//
// Work split inside a walk: 256 threads; thread (pg = tid / 16, ng = tid % 16)
// holds a 4 x (N / 16) block of the state (headdim rows 4 pg .. 4 pg + 3,
// dstate columns (N / 16) ng ..).  Sums over n (Y_t, Lam_t B_t) run inside the
// thread and then across the 16 lanes of a DPP row (rotations); sums over p
// (dC, dB terms) and over the whole head go through LDS, a tile of kTT steps
// at a time.  Steps are staged in LDS per tile (float32), and steps past the
// end of the sequence are zero steps (dt = 0, x = dy = 0), so they change
// nothing.
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kP = 64;   // headdim
constexpr int kTT = 4;   // steps per tile
constexpr int kPB = 4;   // headdim rows per thread

__device__ __forceinline__ float ldf(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const uint16_t *p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ void stf(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void stf(uint16_t *p, int64_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // round to nearest even
}

// Sum over the 16 lanes of this lane's DPP row, in every lane of the row.
template <int R>
__device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + R, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}

__device__ __forceinline__ float sigm(float z) { return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e)); }

// Steps [t0, t0 + kTT) of one head staged in LDS (float32; zero past the end).
template <int N>
struct Stage {
  float x[kTT][kP], dy[kTT][kP], z[kTT][kP];
  float B[kTT][N], C[kTT][N];
  float dt[kTT];
};

template <typename Tdy, int N, bool HAS_Z>
__device__ __forceinline__ void stage_tile(Stage<N> &s, const SsdBwdParams &p, int64_t b, int64_t h, int64_t g,
                                           int64_t t0, float bias) {
  const uint16_t *gx = static_cast<const uint16_t *>(p.x);
  const uint16_t *gz = static_cast<const uint16_t *>(p.z);
  const uint16_t *gB = static_cast<const uint16_t *>(p.B);
  const uint16_t *gC = static_cast<const uint16_t *>(p.C);
  const uint16_t *gdt = static_cast<const uint16_t *>(p.dt);
  const Tdy *gdy = static_cast<const Tdy *>(p.dy);
  const int64_t L = p.seqlen, H = p.nheads, G = p.ngroups;
  const int tid = threadIdx.x;
  for (int e = tid; e < kTT * kP; e += 256) {
    const int i = e / kP, q = e % kP;
    const int64_t t = t0 + i;
    const bool in = t < L;
    const int64_t o = ((b * L + (in ? t : 0)) * H + h) * kP + q;
    s.x[i][q] = in ? ldf(gx, o) : 0.0f;
    s.dy[i][q] = in ? ldf(gdy, o) : 0.0f;
    if constexpr (HAS_Z) s.z[i][q] = in ? ldf(gz, o) : 0.0f;
  }
  for (int e = tid; e < kTT * N; e += 256) {
    const int i = e / N, n = e % N;
    const int64_t t = t0 + i;
    const bool in = t < L;
    const int64_t o = ((b * L + (in ? t : 0)) * G + g) * N + n;
    s.B[i][n] = in ? ldf(gB, o) : 0.0f;
    s.C[i][n] = in ? ldf(gC, o) : 0.0f;
  }
  if (tid < kTT) {
    const int64_t t = t0 + tid;
    const bool in = t < L;
    const float raw = in ? ldf(gdt, (b * L + t) * H + h) : 0.0f;
    s.dt[tid] = in ? (p.dt_softplus ? dt_softplus(raw + bias) : raw) : 0.0f;
  }
}

// ---- forward walk -------------------------------------------------------------
template <typename Tdy, int N, bool HAS_Z>
__global__ void __launch_bounds__(256) ssd_bwd_fwd_kernel(const SsdBwdParams p) {
  constexpr int NB = N / 16;
  __shared__ Stage<N> st;
  __shared__ float sDC[kTT][16][N];   // per-pg partial dC terms of a tile
  __shared__ float sU[kTT][16];       // per-pg partial u of a tile
  __shared__ float sRed[2][4];        // per-wavefront sums of dD and <dh_last, S>

  const int tid = threadIdx.x, pg = tid / 16, ng = tid % 16;
  const int64_t H = p.nheads, L = p.seqlen;
  const int64_t bh = blockIdx.x, b = bh / H, h = bh % H, g = h / (H / p.ngroups);
  const float Ah = p.A[h] * kLog2e, Dh = p.D ? p.D[h] : 0.0f;
  const float bias = (p.dt_softplus && p.dt_bias) ? p.dt_bias[h] : 0.0f;
  uint16_t *gdz = static_cast<uint16_t *>(p.dz);

  float S[kPB][NB];
  const int64_t sbase = (bh * kP + kPB * pg) * N + NB * ng;
#pragma unroll
  for (int a = 0; a < kPB; ++a)
#pragma unroll
    for (int k = 0; k < NB; ++k) S[a][k] = p.h0 ? p.h0[sbase + a * N + k] : 0.0f;
  float dD_acc = 0.0f;

  auto reduce_tile = [&](int64_t t0) __attribute__((always_inline)) {
    for (int e = tid; e < kTT * N; e += 256) {
      const int i = e / N, n = e % N;
      const int64_t t = t0 + i;
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) v += sDC[i][q][n];
      if (t < L) p.ws_dCh[((b * L + t) * H + h) * N + n] = v;
    }
    if (tid < kTT && t0 + tid < L) {
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) v += sU[tid][q];
      p.ws_u[(b * L + t0 + tid) * H + h] = v;
    }
  };

  for (int64_t t0 = 0; t0 < L; t0 += kTT) {
    stage_tile<Tdy, N, HAS_Z>(st, p, b, h, g, t0, bias);
    if (t0 > 0) reduce_tile(t0 - kTT);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTT; ++i) {
      const float dl = st.dt[i];
      const float al = __builtin_amdgcn_exp2f(dl * Ah);
      float xv[kPB], bv[NB], cv[NB];
#pragma unroll
      for (int a = 0; a < kPB; ++a) xv[a] = st.x[i][kPB * pg + a];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        bv[k] = st.B[i][NB * ng + k];
        cv[k] = st.C[i][NB * ng + k];
      }
      float Y[kPB];
#pragma unroll
      for (int a = 0; a < kPB; ++a) {
        const float dx = dl * xv[a];
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          S[a][k] = fmaf(al, S[a][k], dx * bv[k]);
          acc = fmaf(S[a][k], cv[k], acc);
        }
        Y[a] = row_sum(acc);
      }
      float dyh[kPB], up = 0.0f, dDp = 0.0f;
#pragma unroll
      for (int a = 0; a < kPB; ++a) {
        const float dyv = st.dy[i][kPB * pg + a];
        if constexpr (HAS_Z) {
          const float zv = st.z[i][kPB * pg + a];
          const float sg = sigm(zv);
          const float yh = fmaf(Dh, xv[a], Y[a]);
          dyh[a] = dyv * zv * sg;
          if (ng == a && t0 + i < L)
            stf(gdz, ((b * L + t0 + i) * H + h) * kP + kPB * pg + a, dyv * yh * sg * (1.0f + zv * (1.0f - sg)));
        } else {
          dyh[a] = dyv;
        }
        up = fmaf(dyh[a], Y[a], up);
        dDp = fmaf(dyh[a], xv[a], dDp);
      }
      if (ng == 0) {
        sU[i][pg] = up;
        dD_acc += dDp;
      }
      float dcp[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        float v = 0.0f;
#pragma unroll
        for (int a = 0; a < kPB; ++a) v = fmaf(S[a][k], dyh[a], v);
        dcp[k] = v;
      }
#pragma unroll
      for (int k = 0; k < NB; k += 4)
        *reinterpret_cast<float4 *>(&sDC[i][pg][NB * ng + k]) = make_float4(dcp[k], dcp[k + 1], dcp[k + 2], dcp[k + 3]);
    }
    __syncthreads();
  }
  if (L > 0) reduce_tile(((L - 1) / kTT) * kTT);

  // <dh_last, S_{L-1}> and the head's dD term, summed over the workgroup.
  float ph = 0.0f;
  if (p.dh_last) {
#pragma unroll
    for (int a = 0; a < kPB; ++a)
#pragma unroll
      for (int k = 0; k < NB; ++k) ph = fmaf(p.dh_last[sbase + a * N + k], S[a][k], ph);
  }
  for (int m = 32; m >= 1; m >>= 1) {
    ph += __shfl_xor(ph, m);
    dD_acc += __shfl_xor(dD_acc, m);
  }
  if (tid % 64 == 0) {
    sRed[0][tid / 64] = ph;
    sRed[1][tid / 64] = dD_acc;
  }
  __syncthreads();
  if (tid == 0) {
    p.ws_phi0[bh] = (sRed[0][0] + sRed[0][1]) + (sRed[0][2] + sRed[0][3]);
    p.ws_dDpart[bh] = (sRed[1][0] + sRed[1][1]) + (sRed[1][2] + sRed[1][3]);
  }
}

// ---- reverse walk -------------------------------------------------------------
template <typename Tdy, int N, bool HAS_Z>
__global__ void __launch_bounds__(256) ssd_bwd_rev_kernel(const SsdBwdParams p) {
  constexpr int NB = N / 16;
  __shared__ Stage<N> st;
  __shared__ float sR[kTT][16][N];    // per-pg partial Lam^T x terms of a tile
  __shared__ float sS[kTT][16];       // per-pg partial x^T Lam B of a tile
  __shared__ float sDt[kTT];          // the tile's steps, kept for its reduction

  const int tid = threadIdx.x, pg = tid / 16, ng = tid % 16;
  const int64_t H = p.nheads, L = p.seqlen;
  const int64_t bh = blockIdx.x, b = bh / H, h = bh % H, g = h / (H / p.ngroups);
  const float A = p.A[h], Ah = A * kLog2e, Dh = p.D ? p.D[h] : 0.0f;
  const float bias = (p.dt_softplus && p.dt_bias) ? p.dt_bias[h] : 0.0f;
  uint16_t *gdx = static_cast<uint16_t *>(p.dx);
  uint16_t *gddt = static_cast<uint16_t *>(p.ddt);

  float lam[kPB][NB];
  const int64_t sbase = (bh * kP + kPB * pg) * N + NB * ng;
#pragma unroll
  for (int a = 0; a < kPB; ++a)
#pragma unroll
    for (int k = 0; k < NB; ++k) lam[a][k] = p.dh_last ? p.dh_last[sbase + a * N + k] : 0.0f;
  // Thread 0 carries phi and the head's dA term.
  float phi = 0.0f, dA_acc = 0.0f;
  if (tid == 0 && L > 0) phi = p.ws_phi0[bh] + p.ws_u[(b * L + L - 1) * H + h];

  auto reduce_tile = [&](int64_t t0) __attribute__((always_inline)) {
    for (int e = tid; e < kTT * N; e += 256) {
      const int i = e / N, n = e % N;
      const int64_t t = t0 + i;
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) v += sR[i][q][n];
      if (t < L) p.ws_dBh[((b * L + t) * H + h) * N + n] = sDt[i] * v;
    }
    if (tid == 0) {
      for (int i = kTT - 1; i >= 0; --i) {
        const int64_t t = t0 + i;
        if (t >= L) continue;
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) s += sS[i][q];
        const float dl = sDt[i];
        const float gt = phi - dl * s;
        float ddt = fmaf(A, gt, s);
        if (p.dt_softplus) ddt *= 1.0f - __builtin_amdgcn_exp2f(-dl * kLog2e);  // sigmoid(raw + bias) = 1 - e^{-dt}
        stf(gddt, (b * L + t) * H + h, ddt);
        dA_acc = fmaf(dl, gt, dA_acc);
        if (t > 0) phi = gt + p.ws_u[(b * L + t - 1) * H + h];
      }
    }
  };

  const int64_t last = L > 0 ? ((L - 1) / kTT) * kTT : 0;
  for (int64_t t0 = last; t0 >= 0 && L > 0; t0 -= kTT) {
    stage_tile<Tdy, N, HAS_Z>(st, p, b, h, g, t0, bias);
    if (t0 < last) reduce_tile(t0 + kTT);
    __syncthreads();
    if (tid < kTT) sDt[tid] = st.dt[tid];
#pragma unroll
    for (int i = kTT - 1; i >= 0; --i) {
      const float dl = st.dt[i];
      const float al = __builtin_amdgcn_exp2f(dl * Ah);
      float xv[kPB], bv[NB], cv[NB], dyh[kPB];
#pragma unroll
      for (int a = 0; a < kPB; ++a) {
        xv[a] = st.x[i][kPB * pg + a];
        const float dyv = st.dy[i][kPB * pg + a];
        if constexpr (HAS_Z) {
          const float zv = st.z[i][kPB * pg + a];
          dyh[a] = dyv * zv * sigm(zv);
        } else {
          dyh[a] = dyv;
        }
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        bv[k] = st.B[i][NB * ng + k];
        cv[k] = st.C[i][NB * ng + k];
      }
      float sp = 0.0f;
#pragma unroll
      for (int a = 0; a < kPB; ++a) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
          lam[a][k] = fmaf(dyh[a], cv[k], lam[a][k]);
          acc = fmaf(lam[a][k], bv[k], acc);
        }
        const float v = row_sum(acc);   // (Lam_t B_t)[p]
        if (ng == a && t0 + i < L)
          stf(gdx, ((b * L + t0 + i) * H + h) * kP + kPB * pg + a, fmaf(dl, v, Dh * dyh[a]));
        sp = fmaf(xv[a], v, sp);
      }
      if (ng == 0) sS[i][pg] = sp;
      float rp[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        float v = 0.0f;
#pragma unroll
        for (int a = 0; a < kPB; ++a) v = fmaf(lam[a][k], xv[a], v);
        rp[k] = v;
      }
#pragma unroll
      for (int k = 0; k < NB; k += 4)
        *reinterpret_cast<float4 *>(&sR[i][pg][NB * ng + k]) = make_float4(rp[k], rp[k + 1], rp[k + 2], rp[k + 3]);
#pragma unroll
      for (int a = 0; a < kPB; ++a)
#pragma unroll
        for (int k = 0; k < NB; ++k) lam[a][k] *= al;
    }
    __syncthreads();
  }
  if (L > 0) reduce_tile(0);

  // lam now holds alpha_0 Lam_0 = dh0.
  if (p.dh0) {
#pragma unroll
    for (int a = 0; a < kPB; ++a)
#pragma unroll
      for (int k = 0; k < NB; ++k) p.dh0[sbase + a * N + k] = lam[a][k];
  }
  if (tid == 0) p.ws_dApart[bh] = dA_acc;
}

// ---- sums over heads and batch rows -----------------------------------------------
__global__ void __launch_bounds__(256) ssd_bwd_reduce_kernel(const SsdBwdParams p) {
  const int64_t H = p.nheads, G = p.ngroups, N = p.dstate, hpg = H / G;
  const int64_t total = p.batch * p.seqlen * G * N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < total) {
    const int64_t n = i % N, bt_g = i / N, g = bt_g % G, bt = bt_g / G;
    const float *sb = p.ws_dBh + (bt * H + g * hpg) * N + n;
    const float *sc = p.ws_dCh + (bt * H + g * hpg) * N + n;
    float vb = 0.0f, vc = 0.0f;
    for (int64_t k = 0; k < hpg; ++k) {
      vb += sb[k * N];
      vc += sc[k * N];
    }
    p.dB[i] = vb;
    p.dC[i] = vc;
  }
  if (i < H) {
    float va = 0.0f, vd = 0.0f;
    for (int64_t bb = 0; bb < p.batch; ++bb) {
      va += p.ws_dApart[bb * H + i];
      vd += p.ws_dDpart[bb * H + i];
    }
    p.dA[i] = va;
    if (p.dD) p.dD[i] = vd;
  }
}

template <typename Tdy, int N>
hipError_t launch_walks(const SsdBwdParams &p, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(p.batch * p.nheads));
  if (p.z != nullptr) {
    hipLaunchKernelGGL((ssd_bwd_fwd_kernel<Tdy, N, true>), grid, dim3(256), 0, stream, p);
    hipLaunchKernelGGL((ssd_bwd_rev_kernel<Tdy, N, true>), grid, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((ssd_bwd_fwd_kernel<Tdy, N, false>), grid, dim3(256), 0, stream, p);
    hipLaunchKernelGGL((ssd_bwd_rev_kernel<Tdy, N, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_bwd(const SsdBwdParams &p, int dy_bf16, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (p.batch * p.nheads > 0) {
    if (p.dstate == 128)
      e = dy_bf16 ? launch_walks<uint16_t, 128>(p, stream) : launch_walks<float, 128>(p, stream);
    else
      e = dy_bf16 ? launch_walks<uint16_t, 64>(p, stream) : launch_walks<float, 64>(p, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t total = p.batch * p.seqlen * p.ngroups * p.dstate;
  const int64_t work = total > p.nheads ? total : p.nheads;
  if (work > 0) {
    hipLaunchKernelGGL(ssd_bwd_reduce_kernel, dim3(static_cast<uint32_t>((work + 255) / 256)), dim3(256), 0, stream, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace ssm
