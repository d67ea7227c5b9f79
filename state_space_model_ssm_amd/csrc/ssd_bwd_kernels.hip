// Backward of the scalar-decay SSD for gfx950: gradients of x, dt, A, B, C,
// D, z and h0 for upstream gradients dy and dh_last, in the chunked form of
// the forward ("Mamba-3 NKI Kernels for AWS Neuron", section "Kernel
// details": the Mamba-2 chunked SSD with chunk 64; section "Correctness"
// reports backward parity of the SSD but prints no formulas, so the
// gradients are the chain rule on the chunked forward).
//
// One chunk of Q = 64 steps of one (batch, head), a_t = A sum_{r <= t} dt_r
// inside the chunk, S_in the state entering it and dS the gradient of the
// state leaving it (dh_last for the last chunk):
//   forward   Y   = W Xd + diag(e^a) C S_in^T,   W[t][s] = (C_t . B_s) e^{a_t - a_s} [s <= t]
//             S_out = e^{a_last} S_in + Xd^T diag(e^{a_last - a}) B,   Xd = diag(dt) X
//   backward  dXd = W^T dY + diag(e^{a_last - a}) B dS^T          dx = dt dXd + D dY
//             dG  = (dY X^T) e^{a_t - a_s} dt_s [s <= t]
//             dC  = dG B + diag(e^a) dY S_in                      (summed over a group's heads)
//             dB  = dG^T C + diag(dt e^{a_last - a}) X dS         (summed over a group's heads)
//             dS_in = e^{a_last} dS + dY^T diag(e^a) C            (the gradient entering the chunk before)
//   log-decay gradient (R = W o dW, dW = dY Xd^T):
//             da_t = sum_s R[t][s] - sum_u R[u][t] + e^{a_t} (dY S_in)_t . C_t - q_t,
//             q_s  = dt_s e^{a_last - a_s} (X dS)_s . B_s;  da_last += sum_s q_s + e^{a_last} <dS, S_in>
//             ddt_s = x_s . dXd_s + A sum_{t >= s} da_t,      dA = sum_s dt_s sum_{t >= s} da_t
// (dY here is dyhat = dy silu(z); dz = dy yhat silu'(z) with yhat = Y + D x.)
//
// Kernels:
//   * state pass, forward: per (batch, head), the chunk states S_in from h0
//     (the forward's state update, MFMA over the chunk's steps), stored bf16;
//   * state pass, reverse: per (batch, head), dS of every chunk from dh_last,
//     stored bf16, with <dS, S_in> per chunk and dh0;
//   * chunk kernel: every (batch, chunk, block of heads) at once: the products
//     above on matrix cores (v_mfma_f32_16x16x32_bf16), dx, ddt, dz directly,
//     dB and dC summed over the block's heads in registers, dA and dD terms;
//   * a reduction over head blocks (dB, dC) and over batch rows and chunks
//     (dA, dD) in a fixed order: no atomics, equal results on every call.
// Operands are staged in LDS in their natural layouts only ([t][n], [t][p],
// [p][n]); fragments that contract over the other index come from the
// transposing LDS read ds_read_b64_tr_b16 (in each 16-lane group, lane i
// receives element i mod 4 of the 8-byte segments addressed by lanes
// 4j + i / 4, j = 0..3).  Steps past the end of the sequence are zero steps
// (dt = 0, zero rows), so they change nothing.
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int Q = 64;        // chunk length
constexpr int P = 64;        // headdim
constexpr int PP = P + 8;    // padded LDS row of [.][p] arrays (bf16)
constexpr int QPp = Q + 8;   // padded LDS row of [t][s] arrays (bf16)
constexpr int RP = Q + 1;    // padded row of the float32 R matrix

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ __forceinline__ uint16_t f2bf(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
__device__ __forceinline__ float sigm(float z) { return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e)); }

__device__ __forceinline__ floatx4 mfma(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte read (LDS or global) as an MFMA fragment.
__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

// Transposing LDS read of four bf16.
typedef __attribute__((address_space(3))) short4v lds_short4v;
__device__ __forceinline__ bf16x4 ldtr(const uint16_t *p) {
  // The C-style cast is an address-space cast: p points into LDS.
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(p)));
}

// MFMA fragment (row or column i0 + i, k = k0 + 8q .. k0 + 8q + 7) from an
// LDS array stored k-major, T[k][i] with row pitch RPT: lane (q, m) addresses
// T[k0 + 8q + m / 4 (+ 4)][i0 + 4 (m % 4)].
template <int RPT>
__device__ __forceinline__ bf16x8 frag_t(const uint16_t *T, int k0, int i0, int q, int m) {
  const uint16_t *a = T + (k0 + 8 * q + m / 4) * RPT + i0 + 4 * (m % 4);
  const bf16x4 lo = ldtr(a), hi = ldtr(a + 4 * RPT);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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

// Value of lane (l - N) of this lane's 16-lane row, 0 outside the row.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}
template <int J>
__device__ __forceinline__ float lane_value(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), J));
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_prefix(float a, int lane) {
  a += row_shr<1>(a);
  a += row_shr<2>(a);
  a += row_shr<4>(a);
  a += row_shr<8>(a);
  const float r0 = lane_value<15>(a), r1 = lane_value<31>(a), r2 = lane_value<47>(a);
  return a + (lane >= 16 ? r0 : 0.0f) + (lane >= 32 ? r1 : 0.0f) + (lane >= 48 ? r2 : 0.0f);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Eight consecutive elements of dy (float32 or bf16) as float32.
__device__ __forceinline__ void load8(const float *g, int64_t o, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(g + o), b = *reinterpret_cast<const float4 *>(g + o + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t *g, int64_t o, float (&v)[8]) {
  const uint4 r = *reinterpret_cast<const uint4 *>(g + o);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ float ld1(const float *g, int64_t o) { return g[o]; }
__device__ __forceinline__ float ld1(const uint16_t *g, int64_t o) { return bf2f(g[o]); }

__device__ __forceinline__ uint4 pack8(const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = static_cast<uint32_t>(f2bf(v[2 * j])) | (static_cast<uint32_t>(f2bf(v[2 * j + 1])) << 16);
  return uint4{w[0], w[1], w[2], w[3]};
}

// dyhat = dy silu(z) of eight consecutive elements at offset o (0 past the end).
template <typename Tdy, bool HAS_Z>
__device__ __forceinline__ void load_dyhat(const SsdBwdParams &p, int64_t o, bool in, float (&v)[8]) {
  if (!in) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    return;
  }
  load8(static_cast<const Tdy *>(p.dy), o, v);
  if constexpr (HAS_Z) {
    float z[8];
    load8(static_cast<const uint16_t *>(p.z), o, z);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= z[j] * sigm(z[j]);
  }
}

// The chunk's per-step scalars, one lane per step (wavefront 0): the step
// dt (0 past the end) and the inclusive cumulative a_t = A sum dt.
__device__ __forceinline__ void chunk_steps(const SsdBwdParams &p, int64_t b, int64_t h, int64_t c0, int Lc,
                                            float Ah, float bias, int lane, float &dtv, float &a) {
  dtv = 0.0f;
  if (lane < Lc) {
    dtv = bf2f(static_cast<const uint16_t *>(p.dt)[(b * p.seqlen + c0 + lane) * p.nheads + h]);
    if (p.dt_softplus) dtv = dt_softplus(dtv + bias);
  }
  a = wave_prefix(dtv * Ah, lane);
}

// ---- state passes -------------------------------------------------------------
// REV = false: S_in of every chunk from h0 (U = B, V = x, weight dt_t e^{a_last - a_t}),
//   stored as S_in[n][p] (and S_in[p][n] with a gate, for the chunk kernel's Y).
// REV = true: dS of every chunk from dh_last, walking the chunks backwards
//   (U = C, V = dyhat, weight e^{a_t}), stored as dS[p][n], with
//   phi_c = <dS, S_in> per chunk, and dh0 at the end.
// State tiles as in the forward: rows n = 16 ni + 4q + r, column p = 16 w + i.
template <int N, bool REV, typename Tdy, bool HAS_Z>
__global__ void __launch_bounds__(256) ssd_bwd_state_kernel(const SsdBwdParams p) {
  constexpr int NT = N / 16, NPC = N + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sU[Q * NPC];
  __shared__ __attribute__((aligned(16))) uint16_t sV[Q * PP];
  __shared__ __attribute__((aligned(16))) float sOm[Q];
  __shared__ float sDec;
  __shared__ float sRed[4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, q = lane / 16, m = lane % 16;
  const int pcol = 16 * wave + m;
  const int64_t H = p.nheads, L = p.seqlen, G = p.ngroups;
  const int64_t bh = blockIdx.x, b = bh / H, h = bh % H, g = h / (H / G);
  const int64_t nC = p.nchunks;
  const float Ah = p.A[h];
  const float bias = (p.dt_softplus && p.dt_bias) ? p.dt_bias[h] : 0.0f;
  const uint16_t *gU = static_cast<const uint16_t *>(REV ? p.C : p.B);
  const uint16_t *gx = static_cast<const uint16_t *>(p.x);

  floatx4 S[NT];
  const float *init = REV ? p.dh_last : p.h0;
#pragma unroll
  for (int ni = 0; ni < NT; ++ni)
    S[ni] = init ? *reinterpret_cast<const floatx4 *>(init + (bh * P + pcol) * N + 16 * ni + 4 * q)
                 : floatx4{0.f, 0.f, 0.f, 0.f};

  for (int64_t ci = 0; ci < nC; ++ci) {
    const int64_t c = REV ? nC - 1 - ci : ci;
    const int64_t c0 = c * Q;
    const int Lc = static_cast<int>(min(static_cast<int64_t>(Q), L - c0));
    for (int e = tid; e < Q * (N / 8); e += 256) {
      const int t = e / (N / 8), nv = (e % (N / 8)) * 8;
      uint4 v = {0u, 0u, 0u, 0u};
      if (t < Lc) v = *reinterpret_cast<const uint4 *>(gU + ((b * L + c0 + t) * G + g) * N + nv);
      *reinterpret_cast<uint4 *>(&sU[t * NPC + nv]) = v;
    }
    for (int e = tid; e < Q * (P / 8); e += 256) {
      const int t = e / (P / 8), pv = (e % (P / 8)) * 8;
      const int64_t o = ((b * L + c0 + t) * H + h) * P + pv;
      uint4 v = {0u, 0u, 0u, 0u};
      if constexpr (!REV) {
        if (t < Lc) v = *reinterpret_cast<const uint4 *>(gx + o);
      } else {
        float dv[8];
        load_dyhat<Tdy, HAS_Z>(p, o, t < Lc, dv);
        v = pack8(dv);
      }
      *reinterpret_cast<uint4 *>(&sV[t * PP + pv]) = v;
    }
    if (wave == 0) {
      float dtv, a;
      chunk_steps(p, b, h, c0, Lc, Ah, bias, lane, dtv, a);
      const float alast = lane_value<63>(a);
      sOm[lane] = REV ? fast_exp(a) : dtv * fast_exp(alast - a);
      if (lane == 0) sDec = fast_exp(alast);
    }
    __syncthreads();

    // The state of this chunk before its update: S_in (forward) or dS (reverse).
    const int64_t wb = (bh * nC + c) * static_cast<int64_t>(N * P);
    if constexpr (!REV) {
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
#pragma unroll
        for (int r = 0; r < 4; ++r) p.ws_Sn[wb + (16 * ni + 4 * q + r) * P + pcol] = f2bf(S[ni][r]);
        if constexpr (HAS_Z) {
          const uint32_t lo = static_cast<uint32_t>(f2bf(S[ni][0])) | (static_cast<uint32_t>(f2bf(S[ni][1])) << 16);
          const uint32_t hi = static_cast<uint32_t>(f2bf(S[ni][2])) | (static_cast<uint32_t>(f2bf(S[ni][3])) << 16);
          *reinterpret_cast<uint2 *>(p.ws_Sp + wb + pcol * N + 16 * ni + 4 * q) = uint2{lo, hi};
        }
      }
    } else {
      float ph = 0.0f;
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        const uint32_t lo = static_cast<uint32_t>(f2bf(S[ni][0])) | (static_cast<uint32_t>(f2bf(S[ni][1])) << 16);
        const uint32_t hi = static_cast<uint32_t>(f2bf(S[ni][2])) | (static_cast<uint32_t>(f2bf(S[ni][3])) << 16);
        *reinterpret_cast<uint2 *>(p.ws_dSp + wb + pcol * N + 16 * ni + 4 * q) = uint2{lo, hi};
#pragma unroll
        for (int r = 0; r < 4; ++r) ph = fmaf(S[ni][r], bf2f(p.ws_Sn[wb + (16 * ni + 4 * q + r) * P + pcol]), ph);
      }
      ph = wave_sum(ph);
      if (lane == 0) sRed[wave] = ph;
    }

    // S <- e^{a_last} S + U^T diag(omega) V  (K = the chunk's steps).
    const float dec = sDec;
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) S[ni] *= dec;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 vf = frag_t<PP>(sV, 32 * kk, 16 * wave, q, m);
      const floatx4 o0 = *reinterpret_cast<const floatx4 *>(&sOm[32 * kk + 8 * q]);
      const floatx4 o1 = *reinterpret_cast<const floatx4 *>(&sOm[32 * kk + 8 * q + 4]);
      floatx8 wv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wv[j] = static_cast<float>(vf[j]) * o0[j];
        wv[j + 4] = static_cast<float>(vf[j + 4]) * o1[j];
      }
      const bf16x8 bfrag = __builtin_convertvector(wv, bf16x8);
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) S[ni] = mfma(frag_t<NPC>(sU, 32 * kk, 16 * ni, q, m), bfrag, S[ni]);
    }
    __syncthreads();
    if (REV && tid == 0) p.ws_phi[bh * nC + c] = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
  }
  if constexpr (REV) {
    if (p.dh0) {
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) *reinterpret_cast<floatx4 *>(p.dh0 + (bh * P + pcol) * N + 16 * ni + 4 * q) = S[ni];
    }
  }
}

// ---- chunk kernel ---------------------------------------------------------------
// Workgroup: one (batch, chunk) and HPW heads of one group, 4 wavefronts.
// Q x Q tiles (s-tile si, t-tile ti): the 10 with si <= ti plus the zero
// tiles (1, 0) and (3, 2) that the K = 32 steps of the causal products read;
// wavefront w takes tiles w, w + 4, w + 8.  Wavefront w owns headdim columns
// [16 w, 16 w + 16) of dX (and Y) and dstate columns [N/4 w, N/4 (w + 1)) of
// dB and dC.
template <int N, typename Tdy, bool HAS_Z>
__global__ void __launch_bounds__(256) ssd_bwd_chunk_kernel(const SsdBwdParams p) {
  constexpr int NPC = N + 8, NK = N / 32, NTW = N / 64;  // n-tiles per wavefront
  __shared__ __attribute__((aligned(16))) uint16_t sC[Q * NPC];
  __shared__ __attribute__((aligned(16))) uint16_t sB[Q * NPC];
  __shared__ __attribute__((aligned(16))) uint16_t sX[Q * PP];
  __shared__ __attribute__((aligned(16))) uint16_t sDY[Q * PP];
  __shared__ __attribute__((aligned(16))) uint16_t sW[Q * QPp];
  __shared__ __attribute__((aligned(16))) uint16_t sDG[Q * QPp];
  __shared__ __attribute__((aligned(16))) uint16_t sM[HAS_Z ? Q * QPp : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sDS[P * NPC];
  __shared__ float sR[Q * RP];
  __shared__ __attribute__((aligned(16))) float sA[Q];
  __shared__ __attribute__((aligned(16))) float sEa[Q];
  __shared__ __attribute__((aligned(16))) float sWl[Q];
  __shared__ __attribute__((aligned(16))) float sDt[Q];
  __shared__ float sDdt[4][Q], sDaC[4][Q], sDaB[4][Q], sDaR[4][Q];
  __shared__ float sRed[4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, q = lane / 16, m = lane % 16;
  const int64_t H = p.nheads, L = p.seqlen, G = p.ngroups, nC = p.nchunks;
  const int HPW = p.hpw;
  const int64_t HB = H / HPW;
  int64_t id = blockIdx.x;
  const int64_t hb = id % HB;
  id /= HB;
  const int64_t c = id % nC, b = id / nC;
  const int64_t g = (hb * HPW) / (H / G);
  const int64_t c0 = c * Q;
  const int Lc = static_cast<int>(min(static_cast<int64_t>(Q), L - c0));
  const uint16_t *gx = static_cast<const uint16_t *>(p.x);
  const uint16_t *gB = static_cast<const uint16_t *>(p.B);
  const uint16_t *gC = static_cast<const uint16_t *>(p.C);
  uint16_t *gdx = static_cast<uint16_t *>(p.dx);
  uint16_t *gddt = static_cast<uint16_t *>(p.ddt);

  // C and B of the chunk (shared by the heads).
  for (int e = tid; e < 2 * Q * (N / 8); e += 256) {
    const int ee = e % (Q * (N / 8));
    const int t = ee / (N / 8), nv = (ee % (N / 8)) * 8;
    const bool isb = e >= Q * (N / 8);
    uint4 v = {0u, 0u, 0u, 0u};
    if (t < Lc) v = *reinterpret_cast<const uint4 *>((isb ? gB : gC) + ((b * L + c0 + t) * G + g) * N + nv);
    *reinterpret_cast<uint4 *>(&(isb ? sB : sC)[t * NPC + nv]) = v;
  }
  __syncthreads();

  // (si, ti) of the 12 tiles, four bits each: si | ti << 2.
  constexpr uint64_t kTiles = 0x0 | 0x4ull << 4 | 0x5ull << 8 | 0x8ull << 12 | 0x9ull << 16 | 0xAull << 20 |
                              0xCull << 24 | 0xDull << 28 | 0xEull << 32 | 0xFull << 36 | 0x1ull << 40 |
                              0xBull << 44;
  // G^T tiles, G^T[s][t] = B_s . C_t: lane holds s = 16 si + 4q + r, t = 16 ti + m.
  floatx4 Gt[3];
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int code = static_cast<int>((kTiles >> (4 * (wave + 4 * u))) & 0xF);
    const int si = code & 3, ti = code >> 2;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (si <= ti) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        acc = mfma(ld8(&sB[(16 * si + m) * NPC + 32 * kk + 8 * q]), ld8(&sC[(16 * ti + m) * NPC + 32 * kk + 8 * q]), acc);
    }
    Gt[u] = acc;
  }

  floatx4 aB[4][NTW], aC[4][NTW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      aB[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
      aC[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  for (int k = 0; k < HPW; ++k) {
    const int64_t h = hb * HPW + k;
    const int64_t bh = b * H + h, bhc = bh * nC + c;
    const float Ah = p.A[h], Dh = p.D ? p.D[h] : 0.0f;
    const float bias = (p.dt_softplus && p.dt_bias) ? p.dt_bias[h] : 0.0f;

    if (wave == 0) {
      float dtv, a;
      chunk_steps(p, b, h, c0, Lc, Ah, bias, lane, dtv, a);
      const float alast = lane_value<63>(a);
      sA[lane] = a;
      sEa[lane] = fast_exp(a);
      sWl[lane] = fast_exp(alast - a);
      sDt[lane] = dtv;
    }
    // x and dyhat of the head's chunk, and its dD term.
    float dDp = 0.0f;
    for (int e = tid; e < Q * (P / 8); e += 256) {
      const int t = e / (P / 8), pv = (e % (P / 8)) * 8;
      const int64_t o = ((b * L + c0 + t) * H + h) * P + pv;
      uint4 xv = {0u, 0u, 0u, 0u};
      if (t < Lc) xv = *reinterpret_cast<const uint4 *>(gx + o);
      float dv[8], xf[8];
      load_dyhat<Tdy, HAS_Z>(p, o, t < Lc, dv);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xf[2 * j] = __uint_as_float(xw[j] << 16);
        xf[2 * j + 1] = __uint_as_float(xw[j] & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) dDp = fmaf(dv[j], xf[j], dDp);
      *reinterpret_cast<uint4 *>(&sX[t * PP + pv]) = xv;
      *reinterpret_cast<uint4 *>(&sDY[t * PP + pv]) = pack8(dv);
    }
    dDp = wave_sum(dDp);
    if (lane == 0) sRed[wave] = dDp;
    // dS of the chunk, [p][n].
    const uint16_t *gds = p.ws_dSp + bhc * static_cast<int64_t>(P * N);
    for (int e = tid; e < P * (N / 8); e += 256) {
      const int pr = e / (N / 8), nv = (e % (N / 8)) * 8;
      *reinterpret_cast<uint4 *>(&sDS[pr * NPC + nv]) = *reinterpret_cast<const uint4 *>(gds + pr * N + nv);
    }
    __syncthreads();

    // D2^T tiles (D2^T[s][t] = x_s . dyhat_t) and the masked matrices:
    // W[t][s], dG[t][s], M[t][s] = W dt_s (bf16) and R[t][s] (float32).
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int code = static_cast<int>((kTiles >> (4 * (wave + 4 * u))) & 0xF);
      const int si = code & 3, ti = code >> 2;
      floatx4 d2 = {0.f, 0.f, 0.f, 0.f};
      if (si <= ti) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          d2 = mfma(ld8(&sX[(16 * si + m) * PP + 32 * kk + 8 * q]), ld8(&sDY[(16 * ti + m) * PP + 32 * kk + 8 * q]), d2);
      }
      const int t = 16 * ti + m, sb = 16 * si + 4 * q;
      const float at = sA[t];
      const floatx4 as4 = *reinterpret_cast<const floatx4 *>(&sA[sb]);
      const floatx4 dt4 = *reinterpret_cast<const floatx4 *>(&sDt[sb]);
      uint16_t wv[4], gv[4], mv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = sb + r;
        const float e = s <= t ? fast_exp(fminf(at - as4[r], 0.0f)) : 0.0f;
        const float w = Gt[u][r] * e;
        const float dg = dt4[r] * d2[r] * e;
        wv[r] = f2bf(w);
        gv[r] = f2bf(dg);
        mv[r] = f2bf(w * dt4[r]);
        sR[t * RP + s] = dg * Gt[u][r];
      }
      *reinterpret_cast<uint2 *>(&sW[t * QPp + sb]) = *reinterpret_cast<const uint2 *>(wv);
      *reinterpret_cast<uint2 *>(&sDG[t * QPp + sb]) = *reinterpret_cast<const uint2 *>(gv);
      if constexpr (HAS_Z) *reinterpret_cast<uint2 *>(&sM[t * QPp + sb]) = *reinterpret_cast<const uint2 *>(mv);
    }
    __syncthreads();

    // Row and column sums of R (s <= t only): thread (u, part) takes a
    // quarter of the row u and of the column u.
    {
      const int u = tid % 64, part = tid / 64;
      float v = 0.0f;
      for (int s = 16 * part; s < 16 * part + 16 && s <= u; ++s) v += sR[u * RP + s];
      for (int t = max(16 * part, u); t < 16 * part + 16; ++t) v -= sR[t * RP + u];
      sDaR[part][u] = v;
    }

    // dXd = W^T dyhat + diag(e^{a_last - a}) B dS^T; dx, and x . dXd per step.
    {
      const int pc = 16 * wave + m;
#pragma unroll
      for (int si = 0; si < 4; ++si) {
        floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = (si >= 2 ? 1 : 0); kk < 2; ++kk)
          a1 = mfma(frag_t<QPp>(sW, 32 * kk, 16 * si, q, m), frag_t<PP>(sDY, 32 * kk, 16 * wave, q, m), a1);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          a2 = mfma(ld8(&sB[(16 * si + m) * NPC + 32 * kk + 8 * q]), ld8(&sDS[pc * NPC + 32 * kk + 8 * q]), a2);
        const int sb = 16 * si + 4 * q;
        const floatx4 wl4 = *reinterpret_cast<const floatx4 *>(&sWl[sb]);
        const floatx4 dt4 = *reinterpret_cast<const floatx4 *>(&sDt[sb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = sb + r;
          const float dxd = fmaf(wl4[r], a2[r], a1[r]);
          const float xs = bf2f(sX[s * PP + pc]);
          const float dys = bf2f(sDY[s * PP + pc]);
          if (s < Lc) gdx[((b * L + c0 + s) * H + h) * P + pc] = f2bf(fmaf(dt4[r], dxd, Dh * dys));
          const float part = row_sum(xs * dxd);
          if (m == r) sDdt[wave][s] = part;
        }
      }
    }

    // dz = dy yhat silu'(z), yhat = M x + diag(e^a) C S_in^T + D x.
    if constexpr (HAS_Z) {
      const int pc = 16 * wave + m;
      const uint16_t *gsp = p.ws_Sp + bhc * static_cast<int64_t>(P * N) + pc * N;
      const Tdy *gdy = static_cast<const Tdy *>(p.dy);
      const uint16_t *gz = static_cast<const uint16_t *>(p.z);
      uint16_t *gdz = static_cast<uint16_t *>(p.dz);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        floatx4 y1 = {0.f, 0.f, 0.f, 0.f}, y2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          if (32 * kk < 16 * (ti + 1))
            y1 = mfma(ld8(&sM[(16 * ti + m) * QPp + 32 * kk + 8 * q]), frag_t<PP>(sX, 32 * kk, 16 * wave, q, m), y1);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          y2 = mfma(ld8(&sC[(16 * ti + m) * NPC + 32 * kk + 8 * q]), ld8(gsp + 32 * kk + 8 * q), y2);
        const floatx4 ea4 = *reinterpret_cast<const floatx4 *>(&sEa[16 * ti + 4 * q]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * ti + 4 * q + r;
          if (t < Lc) {
            const int64_t o = ((b * L + c0 + t) * H + h) * P + pc;
            const float yh = fmaf(ea4[r], y2[r], y1[r]) + Dh * bf2f(sX[t * PP + pc]);
            const float zv = bf2f(gz[o]);
            const float sg = sigm(zv);
            gdz[o] = f2bf(ld1(gdy, o) * yh * sg * (1.0f + zv * (1.0f - sg)));
          }
        }
      }
    }

    // dC += dG B + diag(e^a) dyhat S_in; and e^{a_t} (dyhat S_in)_t . C_t per step.
    {
      const uint16_t *gsn = p.ws_Sn + bhc * static_cast<int64_t>(N * P);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        float rd[4] = {0.f, 0.f, 0.f, 0.f};
        const floatx4 ea4 = *reinterpret_cast<const floatx4 *>(&sEa[16 * ti + 4 * q]);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const int nt = NTW * wave + j;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            if (32 * kk < 16 * (ti + 1))
              aC[ti][j] = mfma(ld8(&sDG[(16 * ti + m) * QPp + 32 * kk + 8 * q]), frag_t<NPC>(sB, 32 * kk, 16 * nt, q, m), aC[ti][j]);
          floatx4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            tmp = mfma(ld8(&sDY[(16 * ti + m) * PP + 32 * kk + 8 * q]), ld8(gsn + (16 * nt + m) * P + 32 * kk + 8 * q), tmp);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * ti + 4 * q + r;
            rd[r] = fmaf(tmp[r], bf2f(sC[t * NPC + 16 * nt + m]), rd[r]);
            aC[ti][j][r] = fmaf(ea4[r], tmp[r], aC[ti][j][r]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = row_sum(rd[r]);
          if (m == r) sDaC[wave][16 * ti + 4 * q + r] = v * ea4[r];
        }
      }
    }

    // dB += dG^T C + diag(dt e^{a_last - a}) X dS; and (X dS)_s . B_s per step.
#pragma unroll
    for (int si = 0; si < 4; ++si) {
      float rq[4] = {0.f, 0.f, 0.f, 0.f};
      const floatx4 wl4 = *reinterpret_cast<const floatx4 *>(&sWl[16 * si + 4 * q]);
      const floatx4 dt4 = *reinterpret_cast<const floatx4 *>(&sDt[16 * si + 4 * q]);
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int nt = NTW * wave + j;
#pragma unroll
        for (int kk = (si >= 2 ? 1 : 0); kk < 2; ++kk)
          aB[si][j] = mfma(frag_t<QPp>(sDG, 32 * kk, 16 * si, q, m), frag_t<NPC>(sC, 32 * kk, 16 * nt, q, m), aB[si][j]);
        floatx4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          tmp = mfma(ld8(&sX[(16 * si + m) * PP + 32 * kk + 8 * q]), frag_t<NPC>(sDS, 32 * kk, 16 * nt, q, m), tmp);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * si + 4 * q + r;
          const float ws = dt4[r] * wl4[r];
          rq[r] = fmaf(tmp[r], bf2f(sB[s * NPC + 16 * nt + m]), rq[r]);
          aB[si][j][r] = fmaf(ws, tmp[r], aB[si][j][r]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = row_sum(rq[r]);
        if (m == r) sDaB[wave][16 * si + 4 * q + r] = v * dt4[r] * wl4[r];
      }
    }
    __syncthreads();

    // da per step, its suffix sums, ddt and the dA and dD terms (wavefront 0).
    if (wave == 0) {
      const int u = lane;
      float da = (sDaR[0][u] + sDaR[1][u]) + (sDaR[2][u] + sDaR[3][u]);
      da += (sDaC[0][u] + sDaC[1][u]) + (sDaC[2][u] + sDaC[3][u]);
      const float qu = (sDaB[0][u] + sDaB[1][u]) + (sDaB[2][u] + sDaB[3][u]);
      da -= qu;
      const float qtot = wave_sum(qu);
      if (u == Q - 1) da += qtot + sEa[Q - 1] * p.ws_phi[bhc];
      // Suffix sums: rc_u = sum_{t >= u} da_t.
      float rc = da;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_down(rc, off, 64);
        if (u + off < 64) rc += o;
      }
      const float dtv = sDt[u];
      float ddt = (sDdt[0][u] + sDdt[1][u]) + (sDdt[2][u] + sDdt[3][u]);
      ddt = fmaf(Ah, rc, ddt);
      if (p.dt_softplus) ddt *= 1.0f - __builtin_amdgcn_exp2f(-dtv * kLog2e);  // sigmoid(raw + bias) = 1 - e^{-dt}
      if (u < Lc) gddt[(b * L + c0 + u) * H + h] = f2bf(ddt);
      const float dap = wave_sum(dtv * rc);
      if (u == 0) {
        p.ws_dApart[bhc] = dap;
        p.ws_dDpart[bhc] = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
      }
    }
    __syncthreads();
  }

  // The head block's dB and dC terms.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int n = 16 * (NTW * wave + j) + m;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * i + 4 * q + r;
        if (t < Lc) {
          const int64_t o = ((b * L + c0 + t) * HB + hb) * N + n;
          p.ws_dBp[o] = aB[i][j][r];
          p.ws_dCp[o] = aC[i][j][r];
        }
      }
    }
  }
}

// ---- sums over head blocks, batch rows and chunks ------------------------------------
__global__ void __launch_bounds__(256) ssd_bwd_reduce_kernel(const SsdBwdParams p) {
  const int64_t H = p.nheads, G = p.ngroups, N = p.dstate, HB = H / p.hpw, bpg = HB / G;
  const int64_t total = p.batch * p.seqlen * G * N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < total) {
    const int64_t n = i % N, bt_g = i / N, g = bt_g % G, bt = bt_g / G;
    const float *sb = p.ws_dBp + (bt * HB + g * bpg) * N + n;
    const float *sc = p.ws_dCp + (bt * HB + g * bpg) * N + n;
    float vb = 0.0f, vc = 0.0f;
    for (int64_t k = 0; k < bpg; ++k) {
      vb += sb[k * N];
      vc += sc[k * N];
    }
    p.dB[i] = vb;
    p.dC[i] = vc;
  }
  if (i < H) {
    float va = 0.0f, vd = 0.0f;
    for (int64_t bb = 0; bb < p.batch; ++bb)
      for (int64_t c = 0; c < p.nchunks; ++c) {
        va += p.ws_dApart[(bb * H + i) * p.nchunks + c];
        vd += p.ws_dDpart[(bb * H + i) * p.nchunks + c];
      }
    p.dA[i] = va;
    if (p.dD) p.dD[i] = vd;
  }
}

template <int N, typename Tdy, bool HAS_Z>
hipError_t launch_all(const SsdBwdParams &p, hipStream_t stream) {
  const dim3 grid_bh(static_cast<uint32_t>(p.batch * p.nheads));
  if (p.nchunks > 0)
    hipLaunchKernelGGL((ssd_bwd_state_kernel<N, false, Tdy, HAS_Z>), grid_bh, dim3(256), 0, stream, p);
  hipLaunchKernelGGL((ssd_bwd_state_kernel<N, true, Tdy, HAS_Z>), grid_bh, dim3(256), 0, stream, p);
  if (p.nchunks > 0) {
    const dim3 grid(static_cast<uint32_t>(p.batch * p.nchunks * (p.nheads / p.hpw)));
    hipLaunchKernelGGL((ssd_bwd_chunk_kernel<N, Tdy, HAS_Z>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

template <int N, typename Tdy>
hipError_t launch_z(const SsdBwdParams &p, hipStream_t stream) {
  return p.z != nullptr ? launch_all<N, Tdy, true>(p, stream) : launch_all<N, Tdy, false>(p, stream);
}

}  // namespace

int ssd_bwd_heads_per_block(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups) {
  // The most heads (up to 8) that divide a group's heads while the chunk
  // kernel's grid keeps at least kSsdBwdMinBlocks workgroups.
  const int64_t hpg = nheads / ngroups, nc = (seqlen + Q - 1) / Q;
  for (int hpw = 8; hpw >= 2; hpw /= 2)
    if (hpg % hpw == 0 && batch * nc * (nheads / hpw) >= kSsdBwdMinBlocks) return hpw;
  return 1;
}

hipError_t launch_ssd_bwd(const SsdBwdParams &p, int dy_bf16, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (p.batch * p.nheads > 0) {
    if (p.dstate == 128)
      e = dy_bf16 ? launch_z<128, uint16_t>(p, stream) : launch_z<128, float>(p, stream);
    else
      e = dy_bf16 ? launch_z<64, uint16_t>(p, stream) : launch_z<64, float>(p, stream);
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
