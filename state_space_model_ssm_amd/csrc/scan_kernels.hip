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
//     LDS is shared by every channel of the block.  Time is walked in tiles of
//     T steps whose global loads are issued DEPTH tiles ahead into a static
//     register ring; each thread runs T steps of the recurrence and writes its
//     readout partial C_t[n] h_t[n] to LDS, and lanes of the same wavefront,
//     one per (channel, step) element, then sum the N partials, add the D
//     skip, apply the gate and store y.
//   * N >= 16 (scan_row_kernel): a channel's states fill whole 16-lane DPP
//     rows.  Lane j of a row loads its channel's dt, u and z at step j of each
//     16-step block directly from global memory, so dt and w = dt * u reach
//     the row by a broadcast fused into the multiplies (v_mul_f32_dpp
//     row_newbcast) and the lane reading out (channel, step j) holds u and z;
//     only B and C are staged in LDS.
//   * N < 16 (scan_chunk_kernel): several channels share a 16-lane row, so
//     the block also stages dt, w = dt * u and D * u in LDS.
//   * The sequence may be split into chunks that run in parallel (grid.y).
//     A first pass (SUMMARY) reduces every chunk but the last to the pair
//     (prod_t exp(dt_t A), local end state); the sweep pass for chunk c folds
//     the pairs of chunks 0..c-1 with the associative combine
//     (P1, h1) o (P2, h2) = (P1 P2, P2 h1 + h2)  ("We brought Mamba to
//     Trainium", section "We built the parallel scan") to get its start state.
//
// Padding rule: time steps past the end of a chunk take dt = 0 and w = 0, so
// exp(0) = 1 and the state passes through them unchanged.
#include <utility>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct alignas(16) F4 {
  float v[4];
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t raw(const float *p, int64_t i) { return __float_as_uint(p[i]); }
__device__ __forceinline__ uint32_t raw(const uint16_t *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float from_raw(uint32_t r, const float *) { return __uint_as_float(r); }
__device__ __forceinline__ float from_raw(uint32_t r, const uint16_t *) { return __uint_as_float(r << 16); }

__device__ __forceinline__ void st(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t *p, int64_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // round to nearest even
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * kLog2e));
}

// Value of lane J of this lane's 16-lane DPP row.  Folded by the compiler
// into the consuming VOP2 instruction (v_mul_f32_dpp ... row_newbcast:J).
template <int J>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + J, 0xF, 0xF, true));
}

// Decays and input terms of a whole 16-step block, computed ahead of the
// serial state updates so the transcendental latency overlaps.
template <int... J>
__device__ __forceinline__ void dpp_coeffs(float dl16, float w16, float a2, const F4 *b4, float *av,
                                           float *bx, std::integer_sequence<int, J...>) {
  ((av[J] = fast_exp2(row_bcast<J>(dl16) * a2)), ...);
  ((bx[J] = row_bcast<J>(w16) * b4[J / 4].v[J % 4]), ...);
}

// W 32-bit words of one row segment, loaded as a single vector.
template <int W>
struct alignas(4 * W) Words {
  uint32_t v[W];
};

// Unpack the storage elements held in W words into floats.
__device__ __forceinline__ void unpack(const uint32_t *w, int nw, float *o, const float *) {
  for (int i = 0; i < nw; ++i) o[i] = __uint_as_float(w[i]);
}
__device__ __forceinline__ void unpack(const uint32_t *w, int nw, float *o, const uint16_t *) {
  for (int i = 0; i < nw; ++i) {
    o[2 * i] = bf_lo(w[i]);
    o[2 * i + 1] = bf_hi(w[i]);
  }
}

// A row segment that is misaligned or crosses the end of the chunk: element
// loads, zero past t_end, packed into the same words as a vector load.
__device__ __forceinline__ uint32_t elem_bits(const float *row, int64_t t, int64_t t_end) {
  return t < t_end ? __float_as_uint(row[t]) : 0u;
}
__device__ __forceinline__ uint32_t elem_bits(const uint16_t *row, int64_t t, int64_t t_end) {
  return t < t_end ? static_cast<uint32_t>(row[t]) : 0u;
}
template <int W>
__device__ __forceinline__ Words<W> load_seg_tail(const float *row, int64_t t, int64_t t_end) {
  Words<W> r;
#pragma unroll
  for (int i = 0; i < W; ++i) r.v[i] = elem_bits(row, t + i, t_end);
  return r;
}
template <int W>
__device__ __forceinline__ Words<W> load_seg_tail(const uint16_t *row, int64_t t, int64_t t_end) {
  Words<W> r;
#pragma unroll
  for (int i = 0; i < W; ++i)
    r.v[i] = elem_bits(row, t + 2 * i, t_end) | (elem_bits(row, t + 2 * i + 1, t_end) << 16);
  return r;
}

// Row kernel (N >= 16): 32-step time tiles.  Measured against 16- and
// 64-step tiles.
constexpr int kDppTile = 32;

// Small-state kernel (N < 16): tile shapes.
template <int N>
struct TileCfg {
  static_assert(N < 16, "N >= 16 runs on the row kernel");
  static constexpr int CH = 256 / N;                             // channels per block
  static constexpr int CPW = 64 / N;                             // channels per wavefront
  // Time steps per tile.
  static constexpr int T = N >= 4 ? 32 : (N == 2 ? 16 : 8);
  static constexpr int TP = T + 4;                               // padded LDS row (floats)
  static constexpr int BS = T < 16 ? T : 16;                     // steps per readout block
  static constexpr int NB = T / BS;                              // readout blocks per tile
  static constexpr int OPL = (CPW * BS + 63) / 64;               // readout outputs per lane per block
  // Readout partials of a block live as [channel][step][state]: JS floats per
  // step (rows padded by 4 floats), RS per channel.  A recurrence store (one
  // step, lanes over states) hits consecutive banks, and RS = N (mod 64)
  // keeps the channel rows a wavefront stores at once on disjoint banks.
  static constexpr int JS = N >= 4 ? N + 4 : N;
  static constexpr int RS_ALIGN = N >= 4 ? N : 4;
  static constexpr int RS = BS * JS + ((RS_ALIGN - (BS * JS) % 64) % 64 + 64) % 64;
};

// One block's view of the tensors and its fixed index math.
template <typename Tin, int N, bool SUMMARY>
struct Block {
  using Cfg = TileCfg<N>;
  static constexpr int CH = Cfg::CH, T = Cfg::T;
  // Storage elements per staging load: one 16-byte vector.
  static constexpr int VEC = 16 / static_cast<int>(sizeof(Tin));
  static constexpr int WORDS = VEC * static_cast<int>(sizeof(Tin)) / 4;  // 32-bit words per load
  static constexpr int SEG = (T + VEC - 1) / VEC;   // loads per tile row
  static constexpr int PAIR_JOBS = CH * SEG;        // (dt, u) row segments
  static constexpr int BC_JOBS = N * SEG;           // (B, C) row segments
  static constexpr int JOBS = PAIR_JOBS + BC_JOBS;
  static constexpr int JPT = (JOBS + 255) / 256;    // staging jobs per thread
};

// Registers holding one tile's global data between its load and its staging.
template <typename Tin, int N, bool SUMMARY>
struct TileRegs {
  using Cfg = TileCfg<N>;
  using Bk = Block<Tin, N, SUMMARY>;
  Words<Bk::WORDS> a[Bk::JPT];       // dt segment, or B segment
  Words<Bk::WORDS> b[Bk::JPT];       // u segment, or C segment
  uint32_t z[Cfg::NB * Cfg::OPL];    // raw storage bits of z; converted in the readout
};


// Orders this wavefront's LDS accesses across lanes.  LDS instructions of one
// wavefront execute in issue order, so a later load sees an earlier store of
// any lane of the same wavefront; the fences keep the compiler from moving
// LDS accesses across.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Store M consecutive floats to LDS (M a multiple of 4 at a 16-byte aligned
// address, or M == 2 at an 8-byte aligned one).
struct alignas(8) F2 {
  float v[2];
};
template <int M>
__device__ __forceinline__ void store_row(float *dst, const float *v) {
  if constexpr (M % 4 == 0) {
#pragma unroll
    for (int i = 0; i < M; i += 4) *reinterpret_cast<F4 *>(dst + i) = F4{{v[i], v[i + 1], v[i + 2], v[i + 3]}};
  } else {
    *reinterpret_cast<F2 *>(dst) = F2{{v[0], v[1]}};
  }
}

// SUMMARY: no readout; reduce the chunk to (decay product, end state).
// CKPT (with SUMMARY, one chunk): instead store the state at every
// kScanCkptStep-step boundary, from h0, for the backward pass.
template <typename Tin, typename Tout, int N, bool SUMMARY, int DEPTH, bool HAS_Z, bool CKPT = false>
__global__ void __launch_bounds__(256) scan_chunk_kernel(const ScanParams p) {
  using Cfg = TileCfg<N>;
  using Bk = Block<Tin, N, SUMMARY>;
  using Regs = TileRegs<Tin, N, SUMMARY>;
  constexpr int CH = Cfg::CH, CPW = Cfg::CPW, T = Cfg::T, TP = Cfg::TP, BS = Cfg::BS, NB = Cfg::NB;
  constexpr int OPL = Cfg::OPL, JS = Cfg::JS, RS = Cfg::RS;
  constexpr int VEC = Bk::VEC, SEG = Bk::SEG, JPT = Bk::JPT, WORDS = Bk::WORDS;
  static_assert(T % BS == 0 && BS % 4 == 0 && TP % 4 == 0 && RS % 4 == 0, "tile shape");

  // Staged inputs of a tile, double-buffered by tile parity: there is one
  // barrier per tile, so a wavefront may stage tile i+1 while others still
  // read tile i (never tile i-1, which the barrier of tile i has retired).
  __shared__ F4 sDl4[2 * CH * TP / 4];
  __shared__ F4 sW4[2 * CH * TP / 4];
  __shared__ F4 sDu4[SUMMARY ? 1 : 2 * CH * TP / 4];
  __shared__ F4 sB4[2 * N * TP / 4];
  __shared__ F4 sC4[SUMMARY ? 1 : 2 * N * TP / 4];
  // Readout partials C_t[n] h_t[n] of one BS-step block.  A channel's rows are
  // written and read only by the wavefront that owns the channel.
  __shared__ F4 sP4[SUMMARY ? 1 : CH * RS / 4];
  float *sDl = sDl4[0].v, *sW = sW4[0].v, *sDu = sDu4[0].v;
  float *sP = sP4[0].v;

  const Tin *__restrict__ gu = static_cast<const Tin *>(p.u);
  const Tin *__restrict__ gdl = static_cast<const Tin *>(p.delta);
  const Tin *__restrict__ gB = static_cast<const Tin *>(p.B);
  const Tin *__restrict__ gC = static_cast<const Tin *>(p.C);
  const Tin *__restrict__ gz = static_cast<const Tin *>(p.z);
  Tout *__restrict__ gy = static_cast<Tout *>(p.y);
  constexpr bool has_z = !SUMMARY && HAS_Z;
  const bool vec_ok = p.vec_ok != 0;

  const int tid = threadIdx.x;
  const int n = tid % N;
  const int chl = tid / N;
  const int lane = tid % 64;
  const int wave = tid / 64;

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
  const int ntiles = static_cast<int>((t_end - t_begin + T - 1) / T);

  // ---- this thread's state ------------------------------------------------
  const bool mine = chl < nvalid;
  const int64_t d = d0 + chl;
  const float a2 = mine ? p.A[d * N + n] * kLog2e : 0.0f;
  float h = ((!SUMMARY || CKPT) && p.h0 != nullptr && mine) ? p.h0[(b * p.dim + d) * N + n] : 0.0f;
  float prod = 1.0f;
  if (!SUMMARY && c > 0 && mine) {
    const float *cr = p.carry + (b * p.dim + d) * static_cast<int64_t>(p.n_chunks - 1) * (2 * N);
    for (int j = 0; j < c; ++j) h = fmaf(cr[j * 2 * N + n], h, cr[j * 2 * N + N + n]);
  }

  // ---- staging jobs: job k of this thread loads one row segment of VEC steps
  // from two tensors: (dt, u) of a channel row, or (B, C) of a state row.
  // Whether a thread has job k is uniform over its wavefront when the job
  // count is a multiple of 64, which keeps the loads free of divergence.
  const Tin *jsrc1[JPT], *jsrc2[JPT];
  int jkind[JPT], jrow[JPT], jcol[JPT];
  bool jon[JPT];
  int64_t jbase[JPT];
  float jdsk[JPT], jbias[JPT];
#pragma unroll
  for (int k = 0; k < JPT; ++k) {
    int job = tid + 256 * k;
    jon[k] = job < Bk::JOBS;
    if constexpr (Bk::JOBS % 64 == 0)
      jon[k] = __builtin_amdgcn_readfirstlane(static_cast<int>(jon[k])) != 0;
    if (!jon[k]) job = 0;
    const int kind = job < Bk::PAIR_JOBS ? 0 : 1;
    if (kind == 1) job -= Bk::PAIR_JOBS;
    jkind[k] = kind;
    jrow[k] = job / SEG;
    jcol[k] = (job % SEG) * VEC;
    if (kind == 0) {
      // Rows past the group's last channel load a valid row's data; their
      // states are never written out.
      const int r = min(jrow[k], nvalid - 1);
      jbase[k] = (b * p.dim + d0 + r) * L;
      jdsk[k] = (jrow[k] < nvalid && p.D != nullptr) ? p.D[d0 + jrow[k]] : 0.0f;
      jbias[k] = p.dt_bias != nullptr ? p.dt_bias[d0 + r] : 0.0f;
      jsrc1[k] = gdl;
      jsrc2[k] = gu;
    } else {
      jbase[k] = ((b * p.ngroups + g) * N + jrow[k]) * L;
      jdsk[k] = 0.0f;
      jbias[k] = 0.0f;
      jsrc1[k] = gB;
      jsrc2[k] = gC;
    }
  }

  // ---- readout map: output k of this lane in a BS-step block is step ej[k]
  // of channel row erow[k], one of this wavefront's CPW rows.
  int erow[OPL], ej[OPL];
  bool eact[OPL];
  int64_t ebase[OPL];
#pragma unroll
  for (int k = 0; k < OPL; ++k) {
    const int o = lane + 64 * k;
    const bool live = o < CPW * BS;
    erow[k] = wave * CPW + (live ? o / BS : 0);  // an LDS row of this wave for every lane
    ej[k] = o % BS;
    eact[k] = live && erow[k] < nvalid;
    ebase[k] = (b * p.dim + d0 + (eact[k] ? erow[k] : 0)) * L;
  }

  // Tiles wholly inside [t_begin, t_end) with 16-byte aligned rows load
  // with branch-free vector loads; the last partial tile (or every tile when
  // rows are misaligned) loads element by element, zero past t_end.
  const int nfast = vec_ok ? static_cast<int>((t_end - t_begin) / T) : 0;

  auto prefetch_fast = [&](Regs &R, int ti) __attribute__((always_inline)) {
    const int64_t t0 = t_begin + static_cast<int64_t>(ti) * T;
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
      if (jon[k]) {
        const int64_t o = jbase[k] + t0 + jcol[k];
        R.a[k] = *reinterpret_cast<const Words<WORDS> *>(jsrc1[k] + o);
        R.b[k] = *reinterpret_cast<const Words<WORDS> *>(jsrc2[k] + o);
      }
    }
    if constexpr (has_z) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
        for (int k = 0; k < OPL; ++k) R.z[bb * OPL + k] = raw(gz, ebase[k] + t0 + bb * BS + ej[k]);
      }
    }
  };

  auto prefetch_slow = [&](Regs &R, int ti) __attribute__((always_inline)) {
    const int64_t t0 = t_begin + static_cast<int64_t>(ti) * T;
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
      if (jon[k]) {
        const int64_t t = t0 + jcol[k];
        R.a[k] = load_seg_tail<WORDS>(jsrc1[k] + jbase[k], t, t_end);
        R.b[k] = load_seg_tail<WORDS>(jsrc2[k] + jbase[k], t, t_end);
      }
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
      for (int k = 0; k < OPL; ++k) {
        R.z[bb * OPL + k] = 0u;
        if constexpr (has_z) {
          const int64_t t = t0 + bb * BS + ej[k];
          if (t < t_end) R.z[bb * OPL + k] = raw(gz, ebase[k] + t);
        }
      }
    }
  };

  auto stage = [&](const Regs &R, int par, int64_t t0) __attribute__((always_inline)) {
    static_assert(VEC % 4 == 0 || VEC == 2, "staging store width");
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
      if (!jon[k]) continue;
      float va[VEC], vb[VEC];
      unpack(R.a[k].v, WORDS, va, gu);
      unpack(R.b[k].v, WORDS, vb, gu);
      const int o = jrow[k] * TP + jcol[k];
      if (jkind[k] == 0) {
        if (p.dt_softplus) {
          // The raw step: softplus(delta + bias) inside the sequence; padded
          // steps past its end stay zero steps.
#pragma unroll
          for (int i = 0; i < VEC; ++i)
            va[i] = t0 + jcol[k] + i < t_end ? dt_softplus(va[i] + jbias[k]) : 0.0f;
        }
        const int ob = par * CH * TP + o;
        float vw[VEC], vd[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          vw[i] = va[i] * vb[i];
          vd[i] = jdsk[k] * vb[i];
        }
        store_row<VEC>(sDl + ob, va);
        store_row<VEC>(sW + ob, vw);
        if (!SUMMARY) store_row<VEC>(sDu + ob, vd);
      } else {
        const int ob = par * N * TP + o;
        store_row<VEC>(sB4[0].v + ob, va);
        if (!SUMMARY) store_row<VEC>(sC4[0].v + ob, vb);
      }
    }
  };

  // Steps blk*BS .. blk*BS+BS-1 of the tile staged in buffer `par` for this
  // thread's (channel, state); the readout partials go to LDS.
  auto recur_block = [&](int par, int blk, int64_t t0) __attribute__((always_inline)) {
    if constexpr (CKPT) {
      static_assert(kScanCkptStep % BS == 0 || BS % kScanCkptStep == 0, "checkpoint grid");
      const int64_t ts = t0 + blk * BS;
      if (mine && ts < t_end && (ts - t_begin) % kScanCkptStep == 0)
        p.carry[((b * p.dim + d) * ((L + kScanCkptStep - 1) / kScanCkptStep) + ts / kScanCkptStep) * N + n] = h;
    }
    {
      const int tb = blk * BS;
      const int dbase = par * CH * TP + chl * TP + tb;
      const int bbase = par * N * TP + n * TP + tb;
#pragma unroll
      for (int tt = 0; tt < BS; tt += 4) {
        const F4 dl4 = sDl4[(dbase + tt) / 4];
        const F4 w4 = sW4[(dbase + tt) / 4];
        const F4 b4 = sB4[(bbase + tt) / 4];
        const F4 c4 = SUMMARY ? F4{} : sC4[(bbase + tt) / 4];
        F4 pr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = fast_exp2(dl4.v[i] * a2);
          h = fmaf(a, h, w4.v[i] * b4.v[i]);
          if constexpr (SUMMARY) prod *= a;
          else pr.v[i] = c4.v[i] * h;
        }
        if constexpr (!SUMMARY) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sP[chl * RS + (tt + i) * JS + n] = pr.v[i];
        }
      }
    }
  };

  // Readout of block blk: sum the N partials of each of this lane's outputs
  // (pairwise), add the D skip, gate, store.  LDS reads are
  // unconditional (rows of this wave for every lane); only stores depend on
  // the output being live.  readout_load issues the LDS reads, readout_finish
  // consumes them.
  struct Partials {
    float v[OPL][N];
    float du[OPL];
  };
  auto readout_load = [&](int par, int blk, Partials &P) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < OPL; ++k) {
      const float *row = sP + erow[k] * RS + ej[k] * JS;
      if constexpr (N % 4 == 0) {
#pragma unroll
        for (int q = 0; q < N / 4; ++q) {
          const F4 v4 = *reinterpret_cast<const F4 *>(row + 4 * q);
          P.v[k][4 * q] = v4.v[0];
          P.v[k][4 * q + 1] = v4.v[1];
          P.v[k][4 * q + 2] = v4.v[2];
          P.v[k][4 * q + 3] = v4.v[3];
        }
      } else {
#pragma unroll
        for (int i = 0; i < N; ++i) P.v[k][i] = row[i];
      }
      P.du[k] = sDu[par * CH * TP + erow[k] * TP + blk * BS + ej[k]];
    }
  };
  auto readout_finish = [&](int blk, int64_t t0, const uint32_t *zz, Partials &P) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < OPL; ++k) {
      float *v = P.v[k];
#pragma unroll
      for (int w = N / 2; w >= 1; w /= 2) {
#pragma unroll
        for (int i = 0; i < w; ++i) v[i] += v[i + w];
      }
      float y = v[0] + P.du[k];
      if constexpr (has_z) y *= silu(from_raw(zz[blk * OPL + k], gz));
      const int64_t t = t0 + blk * BS + ej[k];
      if (eact[k] && t < t_end) st(gy, ebase[k] + t, y);
    }
  };

  // One tile: stage from registers, one barrier, then per readout block the
  // recurrence and this wavefront's readout.  `pf` refills R with the tile
  // DEPTH ahead on the fast path.
  auto do_tile = [&](Regs &R, int ti, bool pf) __attribute__((always_inline)) {
    const int64_t t0 = t_begin + static_cast<int64_t>(ti) * T;
    uint32_t zz[NB * OPL];
#pragma unroll
    for (int e = 0; e < NB * OPL; ++e) zz[e] = R.z[e];
    const int par = ti & 1;
    stage(R, par, t0);
    __syncthreads();
    if (pf && ti + DEPTH < nfast) prefetch_fast(R, ti + DEPTH);
    if constexpr (SUMMARY) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) recur_block(par, bb, t0);
    } else {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        recur_block(par, bb, t0);
        wave_lds_sync();
        Partials P;
        readout_load(par, bb, P);
        readout_finish(bb, t0, zz, P);
        compiler_fence();
      }
    }
  };

  // Fast tiles: tile ti lives in ring slot ti % DEPTH; the loop is unrolled
  // DEPTH times so every slot index is a compile-time constant.
  static_assert(DEPTH >= 1 && DEPTH <= 3, "ring depth");
  Regs ring[DEPTH];
#pragma unroll
  for (int k = 0; k < DEPTH; ++k)
    if (k < nfast) prefetch_fast(ring[k], k);
  for (int ti0 = 0; ti0 < nfast; ti0 += DEPTH) {
    do_tile(ring[0], ti0, true);
    if constexpr (DEPTH > 1) {
      if (ti0 + 1 < nfast) do_tile(ring[1], ti0 + 1, true);
    }
    if constexpr (DEPTH > 2) {
      if (ti0 + 2 < nfast) do_tile(ring[2], ti0 + 2, true);
    }
  }
  // Remaining tiles: element loads, one tile at a time.
  for (int ti = nfast; ti < ntiles; ++ti) {
    prefetch_slow(ring[0], ti);
    do_tile(ring[0], ti, false);
  }

  if constexpr (SUMMARY && !CKPT) {
    if (mine) {
      float *cr = p.carry + ((b * p.dim + d) * static_cast<int64_t>(p.n_chunks - 1) + c) * (2 * N);
      cr[n] = prod;
      cr[N + n] = h;
    }
  } else {
    if (c == p.n_chunks - 1 && p.h_last != nullptr && mine) p.h_last[(b * p.dim + d) * N + n] = h;
  }
}

// ---------------------------------------------------------------------------
// Row kernel (N >= 16): one (channel, state) per thread, a channel's states
// filling whole 16-lane DPP rows.
//
// Lane j of a row loads its own channel's dt, u (and z) at step j of every
// 16-step block straight from global memory: a row reads 16 consecutive steps
// of one channel row (32 or 64 contiguous bytes), so the loads coalesce by
// rows.  dt and w = dt u then reach the row's lanes by DPP row broadcasts from
// registers, and the lane that reads out (channel, step j) already holds u
// and z.  Only B and C (shared by every channel of the block) are staged in
// LDS, double-buffered by tile parity with one barrier per tile, and the
// readout partials C_t[n] h_t[n] pass through LDS within each wavefront.  The
// sweep is bound by LDS throughput, so dt, w and D u no longer occupy it.
// ---------------------------------------------------------------------------
// B/C staging loads of the row kernel: 2 steps per load, so that the 16 x 32
// B/C tile of N = 16 is one job per thread.
constexpr int kRowVec = 2;
// Row kernel for N = 16: registers held to this many wavefronts per SIMD,
// and tiles in flight per block by input dtype.
constexpr int kRowWaves16 = 4;
template <typename Tin>
constexpr int kRowDepth = sizeof(Tin) == 2 ? 3 : 2;

template <typename Tin, typename Tout, int N, bool SUMMARY, int DEPTH, bool HAS_Z, bool CKPT = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(N == 16 ? kRowWaves16 : 1)))
scan_row_kernel(const ScanParams p) {
  static_assert(N >= 16 && N <= 64 && N % 16 == 0, "row kernel state counts");
  constexpr int CH = 256 / N;                 // channels per block
  constexpr int RPC = N / 16;                 // DPP rows per channel
  constexpr int T = kDppTile, BS = 16, NB = T / BS;
  constexpr int TP = T + 4;                   // padded LDS row of B and C (floats)
  constexpr int VEC = kRowVec;                // B/C staging: elements per load
  constexpr int WORDS = VEC * static_cast<int>(sizeof(Tin)) / 4;
  constexpr int SEG = T / VEC;                // loads per B/C row per tile
  constexpr int BC_JOBS = N * SEG;
  constexpr int JPT = (BC_JOBS + 255) / 256;  // B/C staging jobs per thread
  constexpr int G4 = N / 4;                   // 16-byte groups per partial row
  // Partials of one block: [channel][step][state], RS floats per channel with
  // RS = N (mod 64) so the rows of one store instruction fall on disjoint banks.
  constexpr int RS = BS * N + (((N < 64 ? N : 0) - (BS * N) % 64) % 64 + 64) % 64;
  static_assert(T % BS == 0 && TP % 4 == 0 && RS % 4 == 0 && BC_JOBS % 64 == 0, "tile shape");
  constexpr bool has_z = !SUMMARY && HAS_Z;

  __shared__ F4 sB4[2 * N * TP / 4];
  __shared__ F4 sC4[SUMMARY ? 1 : 2 * N * TP / 4];
  __shared__ F4 sP4[SUMMARY ? 1 : CH * RS / 4];
  float *sP = sP4[0].v;

  const Tin *__restrict__ gu = static_cast<const Tin *>(p.u);
  const Tin *__restrict__ gdl = static_cast<const Tin *>(p.delta);
  const Tin *__restrict__ gB = static_cast<const Tin *>(p.B);
  const Tin *__restrict__ gC = static_cast<const Tin *>(p.C);
  const Tin *__restrict__ gz = static_cast<const Tin *>(p.z);
  Tout *__restrict__ gy = static_cast<Tout *>(p.y);

  const int tid = threadIdx.x;
  const int n = tid % N;
  const int chl = tid / N;
  const int j = tid % 16;                            // step of a block this lane loads and reads out
  const bool reader = ((tid / 16) % RPC) == 0;       // the channel's first row reads out

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
  const int ntiles = static_cast<int>((t_end - t_begin + T - 1) / T);

  // ---- this thread's state and its channel row ------------------------------
  const bool mine = chl < nvalid;
  const int64_t d = d0 + chl;
  const int64_t crow = d0 + min(chl, nvalid - 1);    // rows past the group load a valid row
  const int64_t ebase = (b * p.dim + crow) * L;
  const float a2 = mine ? p.A[d * N + n] * kLog2e : 0.0f;
  const float dskip = (!SUMMARY && p.D != nullptr) ? p.D[crow] : 0.0f;
  const float bias = p.dt_bias != nullptr ? p.dt_bias[crow] : 0.0f;
  float h = ((!SUMMARY || CKPT) && p.h0 != nullptr && mine) ? p.h0[(b * p.dim + d) * N + n] : 0.0f;
  float prod = 1.0f;
  if (!SUMMARY && c > 0 && mine) {
    const float *cr = p.carry + (b * p.dim + d) * static_cast<int64_t>(p.n_chunks - 1) * (2 * N);
    for (int k = 0; k < c; ++k) h = fmaf(cr[k * 2 * N + n], h, cr[k * 2 * N + N + n]);
  }

  // ---- B/C staging jobs: job k loads VEC steps of one B row and one C row ----
  int jrow[JPT], jcol[JPT];
  bool jon[JPT];
  int64_t jbase[JPT];
#pragma unroll
  for (int k = 0; k < JPT; ++k) {
    int job = tid + 256 * k;
    jon[k] = __builtin_amdgcn_readfirstlane(static_cast<int>(job < BC_JOBS)) != 0;  // uniform: BC_JOBS % 64 == 0
    if (!jon[k]) job = 0;
    jrow[k] = job / SEG;
    jcol[k] = (job % SEG) * VEC;
    jbase[k] = ((b * p.ngroups + g) * N + jrow[k]) * L;
  }

  struct Regs {
    uint32_t dl[NB], u[NB], z[NB];   // raw storage bits of this lane's step in each block
    Words<WORDS> bw[JPT], cw[JPT];   // B and C row segments
  };

  // Tiles wholly inside [t_begin, t_end) with aligned B/C rows take vector
  // loads; the last partial tile (or every tile when rows are misaligned)
  // loads B/C element by element and zeroes steps past t_end.
  const int nfast = p.vec_ok ? static_cast<int>((t_end - t_begin) / T) : 0;

  auto prefetch = [&](Regs &R, int ti, bool fast) __attribute__((always_inline)) {
    const int64_t t0 = t_begin + static_cast<int64_t>(ti) * T;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int64_t t = t0 + bb * BS + j;
      const bool in = fast || t < t_end;
      const int64_t ti_ = in ? t : t_begin;  // a valid step for every lane
      R.dl[bb] = in ? raw(gdl, ebase + ti_) : 0u;
      R.u[bb] = in ? raw(gu, ebase + ti_) : 0u;
      if constexpr (has_z) R.z[bb] = in ? raw(gz, ebase + ti_) : 0u;
    }
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
      if (!jon[k]) continue;
      if (fast) {
        const int64_t o = jbase[k] + t0 + jcol[k];
        R.bw[k] = *reinterpret_cast<const Words<WORDS> *>(gB + o);
        if constexpr (!SUMMARY) R.cw[k] = *reinterpret_cast<const Words<WORDS> *>(gC + o);
      } else {
        R.bw[k] = load_seg_tail<WORDS>(gB + jbase[k], t0 + jcol[k], t_end);
        if constexpr (!SUMMARY) R.cw[k] = load_seg_tail<WORDS>(gC + jbase[k], t0 + jcol[k], t_end);
      }
    }
  };

  auto stage = [&](const Regs &R, int par) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < JPT; ++k) {
      if (!jon[k]) continue;
      float vb[VEC], vc[VEC];
      unpack(R.bw[k].v, WORDS, vb, gu);
      const int o = par * N * TP + jrow[k] * TP + jcol[k];
      store_row<VEC>(sB4[0].v + o, vb);
      if constexpr (!SUMMARY) {
        unpack(R.cw[k].v, WORDS, vc, gu);
        store_row<VEC>(sC4[0].v + o, vc);
      }
    }
  };

  // B and C of this thread's state for the 16 steps of block bb.
  struct Ops {
    F4 b4[4], c4[4];
  };
  auto load_ops = [&](int par, int bb, Ops &o) __attribute__((always_inline)) {
    const int q0 = (par * N * TP + n * TP + bb * BS) / 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o.b4[q] = sB4[q0 + q];
      o.c4[q] = SUMMARY ? F4{} : sC4[q0 + q];
    }
  };

  // The step (softplus(dt + bias) when asked; zero past the end) and w = dt u
  // of this lane's step in block bb.
  auto step_vals = [&](uint32_t rdl, uint32_t ru, int64_t t, float &dl, float &w, float &uv)
                       __attribute__((always_inline)) {
    dl = from_raw(rdl, gu);
    uv = from_raw(ru, gu);
    if (p.dt_softplus) dl = t < t_end ? dt_softplus(dl + bias) : 0.0f;
    w = dl * uv;
  };

  // 16 recurrence steps of block bb; on the sweep the partials C_t[n] h_t[n]
  // go to this wavefront's LDS rows.
  auto recur = [&](float dl, float w, const Ops &o, int64_t ts) __attribute__((always_inline)) {
    if constexpr (CKPT) {
      static_assert(kScanCkptStep == BS, "checkpoint grid");
      if (mine && ts < t_end)
        p.carry[((b * p.dim + d) * ((L + kScanCkptStep - 1) / kScanCkptStep) + ts / kScanCkptStep) * N + n] = h;
    }
    float av[16], bx[16];
    dpp_coeffs(dl, w, a2, o.b4, av, bx, std::make_integer_sequence<int, 16>{});
    F4 pr[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      h = fmaf(av[i], h, bx[i]);
      if constexpr (SUMMARY) prod *= av[i];
      else pr[i / 4].v[i % 4] = o.c4[i / 4].v[i % 4] * h;
    }
    if constexpr (!SUMMARY) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sP[chl * RS + i * N + n] = pr[i / 4].v[i % 4];
    }
  };

  // Readout of (channel, step j) of a block: sum the N partials pairwise
  // (16-byte groups visited in the order q ^ swz so the 16 lanes of a row hit
  // distinct banks), add the D skip, gate, store.
  auto readout_load = [&](float (&v)[N]) __attribute__((always_inline)) {
    const float *row = sP + chl * RS + j * N;
    const int f = (j / (16 / G4)) % G4;
#pragma unroll
    for (int q = 0; q < G4; ++q) {
      const F4 v4 = *reinterpret_cast<const F4 *>(row + 4 * (q ^ f));
      v[4 * q] = v4.v[0];
      v[4 * q + 1] = v4.v[1];
      v[4 * q + 2] = v4.v[2];
      v[4 * q + 3] = v4.v[3];
    }
  };
  auto readout_finish = [&](float (&v)[N], float uv, uint32_t zr, int64_t t) __attribute__((always_inline)) {
#pragma unroll
    for (int wd = N / 2; wd >= 1; wd /= 2) {
#pragma unroll
      for (int i = 0; i < wd; ++i) v[i] += v[i + wd];
    }
    float y = fmaf(dskip, uv, v[0]);
    if constexpr (has_z) y *= silu(from_raw(zr, gz));
    if (reader && mine && t < t_end) st(gy, ebase + t, y);
  };

  auto do_tile = [&](Regs &R, int ti, bool pf) __attribute__((always_inline)) {
    const int64_t t0 = t_begin + static_cast<int64_t>(ti) * T;
    uint32_t rdl[NB], ru[NB], zr[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      rdl[bb] = R.dl[bb];
      ru[bb] = R.u[bb];
      zr[bb] = has_z ? R.z[bb] : 0u;
    }
    const int par = ti & 1;
    stage(R, par);
    __syncthreads();
    if (pf && ti + DEPTH < nfast) prefetch(R, ti + DEPTH, true);
    Ops o;
    load_ops(par, 0, o);
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      float dl, w, uv;
      step_vals(rdl[bb], ru[bb], t0 + bb * BS + j, dl, w, uv);
      recur(dl, w, o, t0 + bb * BS);
      if constexpr (SUMMARY) {
        if (bb + 1 < NB) load_ops(par, bb + 1, o);
      } else {
        wave_lds_sync();
        float v[N];
        readout_load(v);
        if (bb + 1 < NB) load_ops(par, bb + 1, o);  // the next block's operands load before the sums
        readout_finish(v, uv, zr[bb], t0 + bb * BS + j);
        compiler_fence();
      }
    }
  };

  // Fast tiles: tile ti lives in ring slot ti % DEPTH; the slot loop is
  // unrolled so every slot index is a compile-time constant.
  static_assert(DEPTH >= 1 && DEPTH <= 6, "ring depth");
  Regs ring[DEPTH];
#pragma unroll
  for (int k = 0; k < DEPTH; ++k)
    if (k < nfast) prefetch(ring[k], k, true);
  for (int ti0 = 0; ti0 < nfast; ti0 += DEPTH) {
#pragma unroll
    for (int k = 0; k < DEPTH; ++k)
      if (ti0 + k < nfast) do_tile(ring[k], ti0 + k, true);
  }
  for (int ti = nfast; ti < ntiles; ++ti) {
    prefetch(ring[0], ti, false);
    do_tile(ring[0], ti, false);
  }

  if constexpr (SUMMARY && !CKPT) {
    if (mine) {
      float *cr = p.carry + ((b * p.dim + d) * static_cast<int64_t>(p.n_chunks - 1) + c) * (2 * N);
      cr[n] = prod;
      cr[N + n] = h;
    }
  } else {
    if (c == p.n_chunks - 1 && p.h_last != nullptr && mine) p.h_last[(b * p.dim + d) * N + n] = h;
  }
}

// Prefetch depth (tiles in flight per block) by input dtype: bf16 tiles are
// half the bytes, so they keep one more tile in flight.
template <typename Tin>
constexpr int kDepth = sizeof(Tin) == 2 ? 3 : 2;

template <typename Tin, typename Tout, int N>
hipError_t launch_typed(const ScanParams &p, hipStream_t stream) {
  const int64_t blocks = p.batch * p.ngroups * p.tiles_per_group;
  if (blocks == 0) return hipSuccess;
  constexpr bool kRow = N >= 16;
  constexpr int kD = kRow ? kRowDepth<Tin> : kDepth<Tin>;
  if (p.n_chunks > 1) {
    const dim3 sgrid(static_cast<uint32_t>(blocks), static_cast<uint32_t>(p.n_chunks - 1));
    if constexpr (kRow)
      hipLaunchKernelGGL((scan_row_kernel<Tin, Tout, N, true, kD, false>), sgrid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((scan_chunk_kernel<Tin, Tout, N, true, kD, false>), sgrid, dim3(256), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(static_cast<uint32_t>(blocks), static_cast<uint32_t>(p.n_chunks));
  if constexpr (kRow) {
    if (p.z != nullptr)
      hipLaunchKernelGGL((scan_row_kernel<Tin, Tout, N, false, kD, true>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((scan_row_kernel<Tin, Tout, N, false, kD, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (p.z != nullptr)
      hipLaunchKernelGGL((scan_chunk_kernel<Tin, Tout, N, false, kD, true>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((scan_chunk_kernel<Tin, Tout, N, false, kD, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename Tin, int N>
hipError_t launch_ckpt_n(const ScanParams &p, hipStream_t stream) {
  const int64_t blocks = p.batch * p.ngroups * p.tiles_per_group;
  if (blocks == 0) return hipSuccess;
  if constexpr (N >= 16)
    hipLaunchKernelGGL((scan_row_kernel<Tin, Tin, N, true, kRowDepth<Tin>, false, true>),
                       dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((scan_chunk_kernel<Tin, Tin, N, true, kDepth<Tin>, false, true>),
                       dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, p);
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

int scan_vector_elems(int in_bf16) { return in_bf16 ? 8 : 4; }

hipError_t launch_scan_ckpt(const ScanParams &p, int in_bf16, hipStream_t stream) {
  switch (p.dstate) {
#define SSM_CKPT_CASE(NN) \
    case NN: return in_bf16 ? launch_ckpt_n<uint16_t, NN>(p, stream) : launch_ckpt_n<float, NN>(p, stream);
    SSM_CKPT_CASE(1) SSM_CKPT_CASE(2) SSM_CKPT_CASE(4) SSM_CKPT_CASE(8) SSM_CKPT_CASE(16)
    SSM_CKPT_CASE(32) SSM_CKPT_CASE(64)
#undef SSM_CKPT_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan(const ScanParams &p, int in_bf16, int out_bf16, hipStream_t stream) {
  if (!in_bf16 && !out_bf16) return launch_n<float, float>(p, stream);
  if (!in_bf16 && out_bf16) return launch_n<float, uint16_t>(p, stream);
  if (in_bf16 && !out_bf16) return launch_n<uint16_t, float>(p, stream);
  return launch_n<uint16_t, uint16_t>(p, stream);
}

}  // namespace ssm
