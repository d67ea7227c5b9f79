// Selective-scan forward kernels for gfx950 (CDNA4, wave64).
//
// Math ("We brought Mamba to Trainium", section "Mamba: bringing an unsupported
// model to the chip"; discretisation and gate from "Mamba-3 NKI Kernels for
// AWS Neuron", section "How it works", Phases 0 and 5):
//   h_t[n] = exp(dt_t A[d,n]) h_{t-1}[n] + dt_t B_t[n] u_t
//   y_t    = (sum_n C_t[n] h_t[n] + D[d] u_t) * silu(z_t)
//
// Work decomposition
//   * One thread owns one (channel d, state n) pair and keeps h[n] in a float32
//     register for its whole time range.  A 256-thread workgroup covers
//     256 / N channels of one (batch, group), so the B_t/C_t tile it stages in
//     LDS is shared by every channel of the block.
//   * Time is walked in tiles of T steps.  Per tile the block stages, in LDS,
//     delta and w = delta * u for its channels and B, C for its group (the
//     global loads of tile i+1 are issued into registers before tile i is
//     computed).  Each thread then runs T steps of the recurrence and writes its
//     readout partial C_t[n] h_t[n] to LDS; after a barrier the same 256
//     threads, now one per (channel, step) element, sum the N partials, add the
//     D skip, apply the gate and store y with coalesced writes.
//   * The sequence may be split into chunks that run in parallel (grid.y).
//     A first pass (SUMMARY) reduces every chunk but the last to the pair
//     (prod_t exp(dt_t A), local end state); the sweep pass for chunk c folds
//     the pairs of chunks 0..c-1 with the associative combine
//     (P1, h1) o (P2, h2) = (P1 P2, P2 h1 + h2)  ("We brought Mamba to
//     Trainium", section "We built the parallel scan") to get its start state.
//
// Padding rule: time steps past the end of a chunk are staged with delta = 0
// and w = 0, so exp(0) = 1 and the state passes through them unchanged.
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct alignas(16) F4 {
  float v[4];
};

__device__ __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t *p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

__device__ __forceinline__ void st(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t *p, int64_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // round to nearest even
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * kLog2e));
}

template <int N>
struct TileCfg {
  static constexpr int CH = 256 / N;                             // channels per block
  static constexpr int T = N >= 4 ? 32 : (N == 2 ? 16 : 8);      // time steps per tile
  static constexpr int TP = T + 4;                               // padded LDS row
  static constexpr int EPT = (CH * T + 255) / 256;               // channel-tile elements / thread
  static constexpr int BPT = (N * T + 255) / 256;                // B/C-tile elements / thread
};

template <typename Tin, typename Tout, int N, bool SUMMARY>
__global__ void __launch_bounds__(256) scan_chunk_kernel(const ScanParams p) {
  using Cfg = TileCfg<N>;
  constexpr int CH = Cfg::CH, T = Cfg::T, TP = Cfg::TP, EPT = Cfg::EPT, BPT = Cfg::BPT;
  static_assert(T % 4 == 0 && TP % 4 == 0, "tiles are read four steps at a time");

  __shared__ F4 sDl4[CH * TP / 4];
  __shared__ F4 sW4[CH * TP / 4];
  __shared__ F4 sB4[N * TP / 4];
  __shared__ F4 sC4[SUMMARY ? 1 : N * TP / 4];
  __shared__ F4 sP4[SUMMARY ? 1 : 256 * TP / 4];
  float *sDl = sDl4[0].v, *sW = sW4[0].v, *sB = sB4[0].v, *sC = sC4[0].v, *sP = sP4[0].v;

  const Tin *__restrict__ gu = static_cast<const Tin *>(p.u);
  const Tin *__restrict__ gdl = static_cast<const Tin *>(p.delta);
  const Tin *__restrict__ gB = static_cast<const Tin *>(p.B);
  const Tin *__restrict__ gC = static_cast<const Tin *>(p.C);
  const Tin *__restrict__ gz = static_cast<const Tin *>(p.z);
  Tout *__restrict__ gy = static_cast<Tout *>(p.y);
  const bool has_z = !SUMMARY && gz != nullptr;

  const int tid = threadIdx.x;
  const int n = tid % N;
  const int chl = tid / N;

  int64_t blk = blockIdx.x;
  const int64_t tile = blk % p.tiles_per_group;
  blk /= p.tiles_per_group;
  const int64_t g = blk % p.ngroups;
  const int64_t b = blk / p.ngroups;
  const int c = static_cast<int>(blockIdx.y);
  const int64_t L = p.seqlen;
  const int64_t ch0 = tile * CH;
  const int nvalid = static_cast<int>(min(static_cast<int64_t>(CH), p.dim_per_group - ch0));
  const int64_t d0 = g * p.dim_per_group + ch0;
  const int64_t t_begin = static_cast<int64_t>(c) * p.chunk_len;
  const int64_t t_end = min(L, t_begin + p.chunk_len);

  // ---- this thread's state ------------------------------------------------
  const bool mine = chl < nvalid;
  const int64_t d = d0 + chl;
  const float a2 = mine ? p.A[d * N + n] * kLog2e : 0.0f;
  float h = 0.0f;
  float prod = 1.0f;
  if (!SUMMARY && c > 0 && mine) {
    const float *cr = p.carry + (b * p.dim + d) * static_cast<int64_t>(p.n_chunks - 1) * (2 * N);
    for (int j = 0; j < c; ++j) h = fmaf(cr[j * 2 * N + n], h, cr[j * 2 * N + N + n]);
  }

  // ---- staging / epilogue element map: element k of this thread ------------
  int col[EPT], loff[EPT];
  bool act[EPT], inrange[EPT];
  int64_t gbase[EPT];
  float dsk[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int idx = tid + 256 * k;
    const int row = idx / T;
    col[k] = idx % T;
    inrange[k] = idx < CH * T;
    act[k] = inrange[k] && row < nvalid;
    loff[k] = row * TP + col[k];
    gbase[k] = act[k] ? (b * p.dim + d0 + row) * L + col[k] : 0;
    dsk[k] = (act[k] && p.D != nullptr) ? p.D[d0 + row] : 0.0f;
  }
  int bcol[BPT], boff[BPT];
  bool bin[BPT];
  int64_t bbase[BPT];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int idx = tid + 256 * k;
    const int nn = idx / T;
    bcol[k] = idx % T;
    bin[k] = idx < N * T;
    boff[k] = nn * TP + bcol[k];
    bbase[k] = bin[k] ? ((b * p.ngroups + g) * N + nn) * L + bcol[k] : 0;
  }

  float rdl[EPT], ru[EPT], rz[EPT], rb[BPT], rc[BPT];
  auto prefetch = [&](int64_t t0) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      rdl[k] = 0.0f;
      ru[k] = 0.0f;
      rz[k] = 0.0f;
      if (act[k] && t0 + col[k] < t_end) {
        rdl[k] = ld(gdl, gbase[k] + t0);
        ru[k] = ld(gu, gbase[k] + t0);
        if (has_z) rz[k] = ld(gz, gbase[k] + t0);
      }
    }
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      rb[k] = 0.0f;
      rc[k] = 0.0f;
      if (bin[k] && t0 + bcol[k] < t_end) {
        rb[k] = ld(gB, bbase[k] + t0);
        if (!SUMMARY) rc[k] = ld(gC, bbase[k] + t0);
      }
    }
  };

  prefetch(t_begin);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += T) {
    // ---- stage tile t0 from registers into LDS ----------------------------
    float du[EPT], zz[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      if (inrange[k]) {
        sDl[loff[k]] = rdl[k];
        sW[loff[k]] = rdl[k] * ru[k];
      }
      du[k] = dsk[k] * ru[k];
      zz[k] = rz[k];
    }
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      if (bin[k]) {
        sB[boff[k]] = rb[k];
        if (!SUMMARY) sC[boff[k]] = rc[k];
      }
    }
    __syncthreads();
    if (t0 + T < t_end) prefetch(t0 + T);

    // ---- recurrence over the tile ------------------------------------------
#pragma unroll
    for (int tt = 0; tt < T; tt += 4) {
      const F4 dl4 = sDl4[(chl * TP + tt) / 4];
      const F4 w4 = sW4[(chl * TP + tt) / 4];
      const F4 b4 = sB4[(n * TP + tt) / 4];
      if constexpr (SUMMARY) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = fast_exp2(dl4.v[j] * a2);
          h = fmaf(a, h, w4.v[j] * b4.v[j]);
          prod *= a;
        }
      } else {
        const F4 c4 = sC4[(n * TP + tt) / 4];
        F4 pr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = fast_exp2(dl4.v[j] * a2);
          h = fmaf(a, h, w4.v[j] * b4.v[j]);
          pr.v[j] = c4.v[j] * h;
        }
        sP4[((chl * N + n) * TP + tt) / 4] = pr;
      }
    }
    __syncthreads();

    // ---- epilogue: sum the N partials, D skip, gate, store y ----------------
    if constexpr (!SUMMARY) {
#pragma unroll
      for (int k = 0; k < EPT; ++k) {
        if (act[k] && t0 + col[k] < t_end) {
          const int row = (tid + 256 * k) / T;
          const float *pp = sP + row * N * TP + col[k];
          float s = 0.0f;
#pragma unroll
          for (int nn = 0; nn < N; ++nn) s += pp[nn * TP];
          float yv = s + du[k];
          if (has_z) yv *= silu(zz[k]);
          st(gy, gbase[k] + t0, yv);
        }
      }
    }
  }

  if constexpr (SUMMARY) {
    if (mine) {
      float *cr = p.carry + ((b * p.dim + d) * static_cast<int64_t>(p.n_chunks - 1) + c) * (2 * N);
      cr[n] = prod;
      cr[N + n] = h;
    }
  } else {
    if (c == p.n_chunks - 1 && p.h_last != nullptr && mine) p.h_last[(b * p.dim + d) * N + n] = h;
  }
}

template <typename Tin, typename Tout, int N>
hipError_t launch_typed(const ScanParams &p, hipStream_t stream) {
  const int64_t blocks = p.batch * p.ngroups * p.tiles_per_group;
  if (blocks == 0) return hipSuccess;
  if (p.n_chunks > 1) {
    hipLaunchKernelGGL((scan_chunk_kernel<Tin, Tout, N, true>),
                       dim3(static_cast<uint32_t>(blocks), static_cast<uint32_t>(p.n_chunks - 1)),
                       dim3(256), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((scan_chunk_kernel<Tin, Tout, N, false>),
                     dim3(static_cast<uint32_t>(blocks), static_cast<uint32_t>(p.n_chunks)),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_n(const ScanParams &p, hipStream_t stream) {
  switch (p.dstate) {
    case 1: return launch_typed<Tin, Tout, 1>(p, stream);
    case 2: return launch_typed<Tin, Tout, 2>(p, stream);
    case 4: return launch_typed<Tin, Tout, 4>(p, stream);
    case 8: return launch_typed<Tin, Tout, 8>(p, stream);
    case 16: return launch_typed<Tin, Tout, 16>(p, stream);
    case 32: return launch_typed<Tin, Tout, 32>(p, stream);
    case 64: return launch_typed<Tin, Tout, 64>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int scan_channels_per_block(int dstate) { return dstate > 0 ? 256 / dstate : 0; }

hipError_t launch_scan(const ScanParams &p, int in_bf16, int out_bf16, hipStream_t stream) {
  if (!in_bf16 && !out_bf16) return launch_n<float, float>(p, stream);
  if (!in_bf16 && out_bf16) return launch_n<float, uint16_t>(p, stream);
  if (in_bf16 && !out_bf16) return launch_n<uint16_t, float>(p, stream);
  return launch_n<uint16_t, uint16_t>(p, stream);
}

}  // namespace ssm
