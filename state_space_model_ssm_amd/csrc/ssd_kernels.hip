// Scalar-decay chunked SSD forward for gfx950: bf16 matrix cores (MFMA
// 16x16x32, float32 accumulation) for the intra-chunk contractions.
//
// Structure ("Mamba-3 NKI Kernels for AWS Neuron", section "Kernel details",
// mamba3_siso_ssd_kernel: the Mamba-2 chunked SSD with chunk 64; section
// "Repository layout": segsum and causal masks).  For one (batch b, head h)
// and one chunk of Q = 64 steps, with a_t the inclusive cumulative sum of
// dt_s * A_h inside the chunk:
//   G^T[s][t] = B_s . C_t                                  (MFMA, K = N)
//   M[t][s]   = G^T[s][t] exp(a_t - a_s) dt_s  if s <= t, else 0   (segsum mask)
//   Y         = diag(exp(a_t)) C S_prev^T  +  M X          (MFMA, K = N and K = Q)
//   S_new     = exp(a_last) S_prev + sum_s exp(a_last - a_s) dt_s x_s B_s^T  (MFMA, K = Q)
//   y         = (Y + D_h x) * silu(z)
// S is the (headdim x dstate) state; passing it from chunk to chunk is the
// associative (decay, state) combine of "We brought Mamba to Trainium",
// section "We built the parallel scan", with a scalar decay per head.
//
// Four wavefronts per (b, h) walk the chunks in order and keep S^T in float32
// MFMA accumulators: wavefront w of a head owns the 16 headdim columns p in
// [16w, 16w+16) for all dstate rows.  A workgroup takes one, two or four heads
// of one group (which share B and C).  Chunk operands are staged in LDS as
// bf16 (x transposed to [p][s], B also transposed to [n][s]) so that every
// MFMA operand fragment is one 16-byte (or two 8-byte) LDS read.
//
// MFMA 16x16x32 bf16 lane layout (lane l, q = l / 16, i = l % 16):
//   A fragment: row i, k = 8q .. 8q+7;  B fragment: column i, k = 8q .. 8q+7;
//   D: column i, rows 4q .. 4q+3.
// A contraction may permute k as long as both fragments use one permutation:
// the C S^T product uses k-slot 8q + j -> n = 32kk + 4q + j (j < 4) and
// n = 32kk + 16 + 4q + j - 4 (j >= 4), which is exactly what two S^T
// accumulator tiles hold per lane, so S feeds the MFMA without a transpose.
#include <type_traits>

#include "ssm_internal.h"


namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int Q = 64;   // chunk length
constexpr int P = 64;   // headdim
// Padded LDS rows (bf16 elements) of the [.][s] arrays; with the [.][n] rows
// N + 24, measured ~4% faster than 8-element pads (fewer bank conflicts in
// the fragment reads and the transposed stores).
constexpr int QP = Q + 16;

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ __forceinline__ uint16_t f2bf(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }

__device__ __forceinline__ floatx4 mfma(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t *p) {  // 16-byte LDS read
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ void st(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t *p, int64_t i, float v) { p[i] = f2bf(v); }

// Value of lane (l - N) of this lane's 16-lane row, or 0 when that lane is
// outside the row (DPP row_shr with bound_ctrl).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}

// Value of lane J (wave-uniform).
template <int J>
__device__ __forceinline__ float lane_value(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), J));
}

__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Transposed chunk copies ([col][t] for COLS columns, rows of QP bf16): the
// XOR applied to the index of the 32-bit step pair (t / 2) in row `col`.  A
// staging store instruction covers 64 / (COLS / 8) consecutive pairs of each
// of COLS / 8 rows; rows 16 apart get distinct multiples of that span.
template <int COLS>
__device__ __forceinline__ int tswz(int col) {
  constexpr int span = 64 / (COLS / 8);
  return span * ((col >> 4) & (COLS / 16 - 1));
}

// Element index of (col, t) in a transposed copy.
template <int COLS>
__device__ __forceinline__ int tidx(int col, int t) {
  return col * QP + 2 * ((t >> 1) ^ tswz<COLS>(col)) + (t & 1);
}

// TRAP: the trapezoidal (Mamba-3 SISO) three-term form.  Its chunked form is
// this SSD with the input of step s weighted by scale_s = gamma_s +
// dt_{s+1} (1 - lam_{s+1}) wherever it reaches a later step, and by
// gamma_s = lam_s dt_s at its own step (the diagonal of M).
//
// HPB heads per workgroup (4 HPB wavefronts): the heads of one group share B
// and C, so the workgroup stages B and C once per chunk and computes each
// G^T tile once, masking it with every head's decays; each head keeps its own
// four wavefronts, x, M and state.  Four heads per workgroup put four
// wavefronts on every SIMD, which hides the latency of each head's chain of
// dependent LDS reads, MFMAs and barriers.
template <typename Tout, int N, bool HAS_Z, bool TRAP, int HPB>
__global__ void __launch_bounds__(256 * HPB)
__attribute__((amdgpu_waves_per_eu(HPB == 4 ? 4 : 2, HPB == 4 ? 4 : 2)))
ssd_chunk_kernel(const SsdParams p) {
  constexpr int NTH = 256 * HPB;  // threads per workgroup
  constexpr int NP = N + 24;      // padded LDS row of [.][n] arrays
  constexpr int NT = N / 16;      // dstate tiles of S^T
  constexpr int NK = N / 32;      // K steps over dstate
  // bf16 y leaves through LDS as 16-byte row vectors (in each head's M
  // buffer; 2-byte stores from the MFMA layout measured 6% slower); float32 y
  // is stored from the MFMA layout directly.
  constexpr bool kStageY = sizeof(Tout) == 2;
  constexpr int YV = 8;                        // bf16 y elements per 16-byte vector
  constexpr int YP = P + YV;                   // padded y row
  constexpr int YJ = Q * (P / YV) / 256;       // y vectors per thread of a head per chunk
  constexpr int SM = (kStageY && Q * YP > Q * QP) ? Q * YP : Q * QP;  // one head's M (or y) buffer
  // One LDS block, laid out by hand: the small per-head arrays first, at
  // addresses that fit the immediate offset of an LDS instruction (so their
  // per-lane addresses need no registers of their own), then the tiles.
  // Per head: a_t, exp(a_t), exp(a_last - a_s) w_s, w_s (dt_s, or scale_s
  // when TRAP), gamma_s (TRAP) and exp(a_last).
  constexpr int kHeadF = HPB * Q * 4;                       // bytes of one per-head float array
  constexpr int kOffA = 0, kOffEa = kOffA + kHeadF, kOffW = kOffEa + kHeadF, kOffDt = kOffW + kHeadF;
  constexpr int kOffGam = kOffDt + kHeadF;
  constexpr int kOffDecay = kOffGam + (TRAP ? kHeadF : 16);
  constexpr int kOffC = kOffDecay + 16 * ((HPB * 4 + 15) / 16);
  constexpr int kOffB = kOffC + Q * NP * 2;                 // C[t][n], then B[s][n] (n reordered)
  constexpr int kOffBt = kOffB + Q * NP * 2;                // B[n][s]
  constexpr int kOffXt = kOffBt + N * QP * 2;               // per head: x[p][s]
  constexpr int kOffM = kOffXt + HPB * P * QP * 2;          // per head: M[t][s], then y[t][p]
  constexpr int kLds = kOffM + HPB * SM * 2;
  static_assert(kOffC % 16 == 0 && kOffBt % 16 == 0 && kOffXt % 16 == 0 && kOffM % 16 == 0, "LDS layout");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  float *const sAH = reinterpret_cast<float *>(smem + kOffA);
  float *const sEaH = reinterpret_cast<float *>(smem + kOffEa);
  float *const sWH = reinterpret_cast<float *>(smem + kOffW);
  float *const sDtH = reinterpret_cast<float *>(smem + kOffDt);
  float *const sGamH = reinterpret_cast<float *>(smem + kOffGam);
  float *const sDecayH = reinterpret_cast<float *>(smem + kOffDecay);
  uint16_t *const sC = reinterpret_cast<uint16_t *>(smem + kOffC);
  uint16_t *const sB = reinterpret_cast<uint16_t *>(smem + kOffB);
  uint16_t *const sBt = reinterpret_cast<uint16_t *>(smem + kOffBt);
  uint16_t *const sXtH = reinterpret_cast<uint16_t *>(smem + kOffXt);
  uint16_t *const sMH = reinterpret_cast<uint16_t *>(smem + kOffM);

  const uint16_t *__restrict__ gx = static_cast<const uint16_t *>(p.x);
  const uint16_t *__restrict__ gdt = static_cast<const uint16_t *>(p.dt);
  const uint16_t *__restrict__ gB = static_cast<const uint16_t *>(p.B);
  const uint16_t *__restrict__ gC = static_cast<const uint16_t *>(p.C);
  const uint16_t *__restrict__ gz = static_cast<const uint16_t *>(p.z);
  const uint16_t *__restrict__ glam = static_cast<const uint16_t *>(p.lam);
  Tout *__restrict__ gy = static_cast<Tout *>(p.y);

  const int64_t L = p.seqlen, H = p.nheads, G = p.ngroups;
  const int64_t hblocks = H / HPB;  // workgroups per batch row
  // Workgroups of one batch row share B and C.  Consecutive workgroup ids are
  // dealt round-robin to the 8 XCDs, so remap ids to give each XCD a
  // contiguous run of (b, head block) pairs and keep a batch row's B/C in one L2.
  const int64_t nblk = p.batch * hblocks;
  int64_t id = blockIdx.x;
  if (nblk % 8 == 0) id = (id % 8) * (nblk / 8) + id / 8;
  const int64_t b = id / hblocks;
  const int64_t h0i = (id % hblocks) * HPB;  // first head of the workgroup
  const int64_t g = h0i / (H / G);

  int tid = threadIdx.x;
  // The wavefront index is uniform over a wavefront; taking it from the first
  // lane lets everything derived from it (head, LDS bases, per-head scalars)
  // live in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  int lane = tid % 64;
  int q = lane / 16;
  int r16 = lane % 16;
  const int hs = wave / 4;                  // this wavefront's head slot
  int htid = tid % 256;               // thread index within the head's wavefronts
  int pcol = (wave % 4) * 16 + r16;   // this lane's headdim column in S^T and Y
  const int64_t h = h0i + hs;
  uint16_t *const sXt = sXtH + hs * (P * QP);
  uint16_t *const sM = sMH + hs * SM;
  const float *const sA = sAH + hs * Q;
  const float *const sEa = sEaH + hs * Q;
  const float *const sW = sWH + hs * Q;

  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.0f;
  // Phase-0 maps of the raw inputs when asked for: the step softplus(dt +
  // dt_bias[h]) and the trapezoid weight sigmoid(lam).
  const float dt_bias = (p.dt_softplus && p.dt_bias != nullptr) ? p.dt_bias[h] : 0.0f;
  auto step_of = [&](float raw) __attribute__((always_inline)) {
    return p.dt_softplus ? dt_softplus(raw + dt_bias) : raw;
  };
  auto lam_of = [&](float raw) __attribute__((always_inline)) {
    return p.lam_sigmoid ? 1.0f / (1.0f + expf(-raw)) : raw;
  };

  floatx4 S[NT];  // S^T tiles: rows n = 16 ni + 4q + r, column p = pcol
#pragma unroll
  for (int i = 0; i < NT; ++i) S[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (p.h0) {
    const float *h0 = p.h0 + ((b * H + h) * P + pcol) * N;
#pragma unroll
    for (int i = 0; i < NT; ++i) S[i] = *reinterpret_cast<const floatx4 *>(h0 + i * 16 + 4 * q);
  }
  if constexpr (TRAP) {
    // The token before the sequence: the first token's previous-token term
    // beta_0 x_prev B_prev^T, with beta_0 = dt_0 (1 - lam_0) alpha_0, enters
    // through the initial state, alpha_0 (S + dt_0 (1 - lam_0) x_prev B_prev^T).
    if (p.x_prev != nullptr && L > 0) {
      const int64_t i0 = b * L * H + h;  // dt and lam of this head's step 0
      const float w0 = step_of(bf2f(gdt[i0])) * (1.0f - lam_of(bf2f(glam[i0])));
      const float xw = w0 * bf2f(static_cast<const uint16_t *>(p.x_prev)[(b * H + h) * P + pcol]);
      const uint16_t *bp = static_cast<const uint16_t *>(p.B_prev) + (b * G + g) * N + 4 * q;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const uint2 v = *reinterpret_cast<const uint2 *>(bp + 16 * i);
        S[i][0] = fmaf(xw, bf2f(static_cast<uint16_t>(v.x)), S[i][0]);
        S[i][1] = fmaf(xw, bf2f(static_cast<uint16_t>(v.x >> 16)), S[i][1]);
        S[i][2] = fmaf(xw, bf2f(static_cast<uint16_t>(v.y)), S[i][2]);
        S[i][3] = fmaf(xw, bf2f(static_cast<uint16_t>(v.y >> 16)), S[i][3]);
      }
    }
  }
  // Retire the initial-state loads here (s_waitcnt vmcnt(0)).  Otherwise they
  // may count as outstanding at the top of the chunk loop, and the first use
  // of S in every chunk would wait for all loads in flight, prefetches included.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // Staging jobs: a job covers steps (2 tp, 2 tp + 1) of one 8-column group;
  // the 8-column groups of a row go to consecutive lanes, so a wavefront's
  // global loads read whole rows.  The transposed copies ([col][t], 32-bit
  // step pairs) XOR the pair index with a multiple of the wavefront's tp span
  // chosen by the row, which spreads one store instruction over all 64 banks;
  // fragment reads apply the same XOR, and keep 16-byte groups contiguous.
  // B and C jobs (one tensor each: jobs below BC_JOBS / 2 are B's) are spread
  // over the whole workgroup, so whole wavefronts take one or none; x jobs
  // over each head's 256 threads.
  constexpr int BC_JOBS = 2 * (Q / 2) * (N / 8);
  constexpr int BJ = (BC_JOBS + NTH - 1) / NTH;  // B/C jobs per thread per chunk
  static_assert(BC_JOBS % 128 == 0 && (Q / 2) * (P / 8) == 256 && QP % 2 == 0, "staging map");
  uint32_t *sBt32 = reinterpret_cast<uint32_t *>(sBt);
  uint32_t *sXt32 = reinterpret_cast<uint32_t *>(sXt);
  auto pair_lo = [](uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); };
  auto pair_hi = [](uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); };
  auto put_t = [&](uint32_t *dst, int col0, int tp, const uint4 &r0, const uint4 &r1, auto cols)
                   __attribute__((always_inline)) {
    constexpr int COLS = decltype(cols)::value;
    const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
    const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = col0 + 2 * i;
      dst[c * (QP / 2) + (tp ^ tswz<COLS>(c))] = pair_lo(w0[i], w1[i]);
      dst[(c + 1) * (QP / 2) + (tp ^ tswz<COLS>(c + 1))] = pair_hi(w0[i], w1[i]);
    }
  };

  // One chunk's global inputs in registers: loaded a chunk ahead (while the
  // previous chunk computes), then written to LDS.  Steps past the end of the
  // sequence load copies of the last step: their dt is taken as 0, so they
  // reach no output row that is stored and add nothing to the state (their
  // weights in M and in the state update are 0).  The loads are branch-free.
  struct ChunkRegs {
    uint4 bc[BJ][2];  // steps 2 tp and 2 tp + 1 of a B or C job
    uint4 xv[2];
    uint32_t dt;  // raw bf16 bits of this head's dt at step `lane` (its first wavefront uses it)
    uint32_t lam, dtn, lamn;  // TRAP: lam at step `lane`, dt and lam at step `lane` + 1
  };
  // Global addresses: a uniform base at the chunk's first step plus a 32-bit
  // lane offset (the host keeps 64 rows of x and of B/C below 2^31 elements).
  const int rx = static_cast<int>(H * P), rbc = static_cast<int>(G * N), rdt = static_cast<int>(H);
  auto load_chunk = [&](int64_t c0, ChunkRegs &R) __attribute__((always_inline)) {
    const int last = static_cast<int>(min(static_cast<int64_t>(Q), L - c0) - 1);  // last valid step offset
#pragma unroll
    for (int k = 0; k < BJ; ++k) {
      const int v = tid + NTH * k;
      if (BC_JOBS % NTH == 0 || v < BC_JOBS) {
        const int vv = v % (BC_JOBS / 2);
        const int tp = vv / (N / 8);
        const int nv = (vv % (N / 8)) * 8;
        const uint16_t *src = (v < BC_JOBS / 2 ? gB : gC) + ((b * L + c0) * G + g) * N;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          R.bc[k][e] = *reinterpret_cast<const uint4 *>(src + min(2 * tp + e, last) * rbc + nv);
      }
    }
    {
      const int tp = htid / (P / 8);
      const int pv = (htid % (P / 8)) * 8;
      const uint16_t *src = gx + ((b * L + c0) * H + h) * P;
#pragma unroll
      for (int e = 0; e < 2; ++e) R.xv[e] = *reinterpret_cast<const uint4 *>(src + min(2 * tp + e, last) * rx + pv);
    }
    // Loads from clamped steps, so no lane branches.  Only each head's first
    // wavefront stages dt (a wave-uniform branch): the other wavefronts skip
    // the per-step gathers (trapezoidal form 2% faster).
    const int64_t dbase = (b * L + c0) * H + h;
    const int lastn = static_cast<int>(min(static_cast<int64_t>(Q) + 1, L - c0) - 1);  // the next chunk's first step too
    if (wave % 4 == 0) {
      R.dt = gdt[dbase + min(lane, last) * rdt];
      if constexpr (TRAP) {
        R.lam = glam[dbase + min(lane, last) * rdt];
        R.dtn = gdt[dbase + min(lane + 1, lastn) * rdt];
        R.lamn = glam[dbase + min(lane + 1, lastn) * rdt];
      }
    }
  };
  auto stage_chunk = [&](const ChunkRegs &R, int64_t c0) __attribute__((always_inline)) {
    // B and C: [t][n] rows (n reordered, below), B also transposed to [n][t].
#pragma unroll
    for (int k = 0; k < BJ; ++k) {
      const int v = tid + NTH * k;
      if (BC_JOBS % NTH == 0 || v < BC_JOBS) {
        const int vv = v % (BC_JOBS / 2);
        const int tp = vv / (N / 8);
        const int nv = (vv % (N / 8)) * 8;
        const bool is_b = v < BC_JOBS / 2;  // uniform over a wavefront
        uint16_t *dst = is_b ? sB : sC;
        // Within each block of 32 dstate columns, slot 8i + j (i < 4, j < 8)
        // holds n = 4i + j for j < 4 and n = 16 + 4i + (j - 4) for j >= 4:
        // the order in which the state tiles pair n in the K slots of Y_off,
        // so that a lane's C fragment there is one 16-byte read.  The mask
        // tiles contract B and C over n, which any common order leaves alone.
        const int o = nv % 32;  // 0, 8, 16 or 24: this vector's n = nv .. nv + 7
        const int slot = (nv - o) + 8 * ((o % 16) / 4) + 4 * (o / 16);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          uint16_t *row = &dst[(2 * tp + e) * NP + slot];
          *reinterpret_cast<uint2 *>(row) = uint2{R.bc[k][e].x, R.bc[k][e].y};
          *reinterpret_cast<uint2 *>(row + 8) = uint2{R.bc[k][e].z, R.bc[k][e].w};
        }
        if (is_b) put_t(sBt32, nv, tp, R.bc[k][0], R.bc[k][1], std::integral_constant<int, N>{});
      }
    }
    // x transposed to [p][t].
    put_t(sXt32, (htid % (P / 8)) * 8, htid / (P / 8), R.xv[0], R.xv[1], std::integral_constant<int, P>{});
    // dt and the in-chunk cumulative decay (the head's first wavefront: one
    // lane per step).
    if (wave % 4 == 0) {
      const float dtv = (c0 + lane < L) ? step_of(bf2f(static_cast<uint16_t>(R.dt))) : 0.0f;
      // Inclusive prefix sum over the 64 lanes: within each 16-lane row by
      // DPP row shifts (lanes shifted in from outside the row read 0), then
      // the totals of the rows below, read from lanes 15, 31 and 47.
      float a = dtv * Ah;
      a += row_shr<1>(a);
      a += row_shr<2>(a);
      a += row_shr<4>(a);
      a += row_shr<8>(a);
      const float r0 = lane_value<15>(a), r1 = lane_value<31>(a), r2 = lane_value<47>(a);
      a += (lane >= 16 ? r0 : 0.0f) + (lane >= 32 ? r1 : 0.0f) + (lane >= 48 ? r2 : 0.0f);
      const float alast = lane_value<63>(a);
      float w = dtv;
      if constexpr (TRAP) {
        // Weight of this step's input wherever it reaches a later step; the
        // step after the sequence has dt = 0, so the last step keeps gamma.
        const float gam = (c0 + lane < L) ? lam_of(bf2f(static_cast<uint16_t>(R.lam))) * dtv : 0.0f;
        const bool nx = c0 + lane + 1 < L;
        const float dtn = nx ? step_of(bf2f(static_cast<uint16_t>(R.dtn))) : 0.0f;
        const float lamn = nx ? lam_of(bf2f(static_cast<uint16_t>(R.lamn))) : 0.0f;
        w = gam + dtn * (1.0f - lamn);
        sGamH[hs * Q + lane] = gam;
      }
      sAH[hs * Q + lane] = a;
      sEaH[hs * Q + lane] = fast_exp(a);
      sWH[hs * Q + lane] = fast_exp(alast - a) * w;
      sDtH[hs * Q + lane] = w;
      if (lane == 0) sDecayH[hs] = fast_exp(alast);
    }
  };

  ChunkRegs R;
  if (L > 0) load_chunk(0, R);  // an empty sequence reads nothing (its step indexes would be -1)
  for (int64_t c0 = 0; c0 < L; c0 += Q) {
    if constexpr (HPB == 4) {
      // At four wavefronts per SIMD (128 registers) the lane indices pass
      // through an empty asm each chunk, so the LDS and global addresses
      // derived from them are recomputed (a few VALU operations) instead of
      // being held, or spilled, across the loop.
      asm volatile("" : "+v"(tid), "+v"(lane), "+v"(q), "+v"(r16), "+v"(htid), "+v"(pcol));
    }
    stage_chunk(R, c0);
    __syncthreads();
    if (c0 + Q < L) load_chunk(c0 + Q, R);

    // Y_off and the state update need only what the staging wrote (not M),
    // so they come before the mask tiles: the wavefronts without a tile work
    // while the others build M (4-6% faster than after the M barrier).
    // ---- Y_off = diag(exp(a_t)) C S_prev^T ---------------------------------
    floatx4 Y[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) Y[ti] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const floatx8 sf = {S[2 * kk][0], S[2 * kk][1], S[2 * kk][2], S[2 * kk][3],
                          S[2 * kk + 1][0], S[2 * kk + 1][1], S[2 * kk + 1][2], S[2 * kk + 1][3]};
      const bf16x8 bfrag = __builtin_convertvector(sf, bf16x8);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const bf16x8 afrag = lds8(&sC[(ti * 16 + r16) * NP + 32 * kk + 8 * q]);
        Y[ti] = mfma(afrag, bfrag, Y[ti]);
      }
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const floatx4 ea = *reinterpret_cast<const floatx4 *>(&sEa[ti * 16 + 4 * q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) Y[ti][r] *= ea[r];
    }

    // ---- S_new = exp(a_last) S_prev + B^T (w x) ----------------------------
    {
      const float decay = sDecayH[hs];
#pragma unroll
      for (int i = 0; i < NT; ++i) S[i] *= decay;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int s0 = 32 * kk + 8 * q;
        const bf16x8 xs = lds8(&sXt[tidx<P>(pcol, s0)]);
        const floatx4 w0 = *reinterpret_cast<const floatx4 *>(&sW[s0]);
        const floatx4 w1 = *reinterpret_cast<const floatx4 *>(&sW[s0 + 4]);
        floatx8 wx;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wx[j] = static_cast<float>(xs[j]) * w0[j];
          wx[j + 4] = static_cast<float>(xs[j + 4]) * w1[j];
        }
        const bf16x8 bfrag = __builtin_convertvector(wx, bf16x8);
#pragma unroll
        for (int ni = 0; ni < NT; ++ni) {
          const bf16x8 afrag = lds8(&sBt[tidx<N>(ni * 16 + r16, s0)]);
          S[ni] = mfma(afrag, bfrag, S[ni]);
        }
      }
    }
    // After the last chunk's update S is the final state: h_last leaves here,
    // so that its stores overlap the chunk's remaining products and epilogue.
    if (p.h_last != nullptr && c0 + Q >= L) {
      float *hl = p.h_last + ((b * H + h) * P + pcol) * N;
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
        *reinterpret_cast<floatx4 *>(hl + ni * 16 + 4 * q) = S[ni];
    }

    // ---- M = mask(G^T) into LDS, for every head of the workgroup -----------
    // 12 tiles (si, ti): the lower-triangular tiles plus the two upper tiles
    // (1,0) and (3,2) that the K = 32 steps of Y_diag read; those are written
    // as zeros.  Tile k goes to wavefront k mod (4 HPB).
    {
      // (si, ti) pairs, four bits each: si | ti << 2, in the order listed above.
      constexpr uint64_t kTiles = 0x0 | 0x4ull << 4 | 0x5ull << 8 | 0x8ull << 12 | 0x9ull << 16 |
                                  0xAull << 20 | 0xCull << 24 | 0xDull << 28 | 0xEull << 32 |
                                  0xFull << 36 | 0x1ull << 40 | 0xBull << 44;
      constexpr int kRounds = (12 + 4 * HPB - 1) / (4 * HPB);
#pragma unroll
      for (int u = 0; u < kRounds; ++u) {
        const int k = wave + 4 * HPB * u;
        if (12 % (4 * HPB) == 0 || k < 12) {
          const int code = static_cast<int>((kTiles >> (4 * k)) & 0xF);
          const int si = code & 3;
          const int ti = code >> 2;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
          if (si <= ti) {
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
              const bf16x8 afrag = lds8(&sB[(si * 16 + r16) * NP + 32 * kk + 8 * q]);
              const bf16x8 bfrag = lds8(&sC[(ti * 16 + r16) * NP + 32 * kk + 8 * q]);
              acc = mfma(afrag, bfrag, acc);
            }
          }
          const int t = ti * 16 + r16;
          const int sb = si * 16 + 4 * q;
#pragma unroll
          for (int j = 0; j < HPB; ++j) {
            const float at = sAH[j * Q + t];
            const floatx4 as4 = *reinterpret_cast<const floatx4 *>(&sAH[j * Q + sb]);
            const floatx4 dt4 = *reinterpret_cast<const floatx4 *>(&sDtH[j * Q + sb]);
            floatx4 gm4 = dt4;
            if constexpr (TRAP) gm4 = *reinterpret_cast<const floatx4 *>(&sGamH[j * Q + sb]);
            uint16_t m[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              // Branch-free: above the diagonal the exponent is clamped to 0
              // (a_t - a_s > 0 there) and the product is multiplied by 0.
              const int s = sb + r;
              const float ws = s < t ? dt4[r] : gm4[r];
              const float keep = s <= t ? 1.0f : 0.0f;
              m[r] = f2bf(acc[r] * fast_exp(fminf(at - as4[r], 0.0f)) * ws * keep);
            }
            *reinterpret_cast<uint2 *>(&sMH[j * SM + t * QP + si * 16 + 4 * q]) =
                *reinterpret_cast<const uint2 *>(m);
          }
        }
      }
    }
    __syncthreads();

    // ---- Y += M X (causal: K steps at or below the diagonal) ---------------
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (32 * kk < 16 * (ti + 1)) {
          const bf16x8 afrag = lds8(&sM[(ti * 16 + r16) * QP + 32 * kk + 8 * q]);
          const bf16x8 bfrag = lds8(&sXt[tidx<P>(pcol, 32 * kk + 8 * q)]);
          Y[ti] = mfma(afrag, bfrag, Y[ti]);
        }
      }
    }

    // ---- epilogue: D skip and gate in the MFMA layout ------------------------
    // The gate's z values are loaded first, all together, from clamped steps,
    // so the loads are waited for once.
    uint32_t zr[16];
    const int64_t ybase = ((b * L + c0) * H + h) * P;  // (c0, h, 0) of x, z and y
    if constexpr (HAS_Z) {
      const int last = static_cast<int>(min(static_cast<int64_t>(Q), L - c0) - 1);
#pragma unroll
      for (int e = 0; e < 16; ++e) zr[e] = gz[ybase + min((e / 4) * 16 + 4 * q + (e % 4), last) * rx + pcol];
    }
    float yv[16];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = ti * 16 + 4 * q + r;
        float v = Y[ti][r] + Dh * bf2f(sXt[tidx<P>(pcol, t)]);
        if constexpr (HAS_Z) v *= silu(bf2f(static_cast<uint16_t>(zr[ti * 4 + r])));
        yv[ti * 4 + r] = v;
      }
    }
    // Every wavefront is done reading M and x: the M buffers take y, and the
    // next chunk may be staged.
    __syncthreads();
    if constexpr (kStageY) {
      Tout *sY = reinterpret_cast<Tout *>(sM);
#pragma unroll
      for (int e = 0; e < 16; ++e) st(sY, ((e / 4) * 16 + 4 * q + (e % 4)) * YP + pcol, yv[e]);
      __syncthreads();
      // y rows of the chunk as 16-byte vectors: P / YV vectors per step.
#pragma unroll
      for (int k = 0; k < YJ; ++k) {
        const int v = htid + 256 * k;
        const int t = v / (P / YV);
        const int pv = (v % (P / YV)) * YV;
        if (c0 + t < L)
          *reinterpret_cast<uint4 *>(gy + ybase + t * rx + pv) =
              *reinterpret_cast<const uint4 *>(&sY[t * YP + pv]);
      }
      // No barrier here: the next chunk's staging writes none of the y
      // buffers, and they are rewritten (as M) only after the next barrier.
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = (e / 4) * 16 + 4 * q + (e % 4);
        if (c0 + t < L) st(gy + ybase, t * rx + pcol, yv[e]);
      }
    }
  }

  if (p.h_last != nullptr && L == 0) {  // an empty sequence: h_last is the initial state
    float *hl = p.h_last + ((b * H + h) * P + pcol) * N;
#pragma unroll
    for (int ni = 0; ni < NT; ++ni)
      *reinterpret_cast<floatx4 *>(hl + ni * 16 + 4 * q) = S[ni];
  }
}

template <typename Tout, int N, bool TRAP, int HPB>
hipError_t launch_hpb(const SsdParams &p, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(p.batch * (p.nheads / HPB)));
  if (p.z != nullptr)
    hipLaunchKernelGGL((ssd_chunk_kernel<Tout, N, true, TRAP, HPB>), grid, dim3(256 * HPB), 0, stream, p);
  else
    hipLaunchKernelGGL((ssd_chunk_kernel<Tout, N, false, TRAP, HPB>), grid, dim3(256 * HPB), 0, stream, p);
  return hipGetLastError();
}

template <typename Tout, int N, bool TRAP>
hipError_t launch_n(const SsdParams &p, hipStream_t stream) {
  switch (ssd_heads_per_block(p.batch, p.nheads, p.ngroups, 4)) {
    case 4: return launch_hpb<Tout, N, TRAP, 4>(p, stream);
    case 2: return launch_hpb<Tout, N, TRAP, 2>(p, stream);
    default: return launch_hpb<Tout, N, TRAP, 1>(p, stream);
  }
}

template <typename Tout>
hipError_t launch_typed(const SsdParams &p, hipStream_t stream) {
  if (p.lam != nullptr) {
    if (p.dstate == 128) return launch_n<Tout, 128, true>(p, stream);
    if (p.dstate == 64) return launch_n<Tout, 64, true>(p, stream);
  } else {
    if (p.dstate == 128) return launch_n<Tout, 128, false>(p, stream);
    if (p.dstate == 64) return launch_n<Tout, 64, false>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int ssd_heads_per_block(int64_t batch, int64_t nheads, int64_t ngroups, int max_hpb) {
  // The most heads (up to max_hpb) that divide a group's heads while the grid
  // still gives every CU a workgroup.
  const int64_t hpg = nheads / ngroups;
  for (int hpb = max_hpb; hpb >= 2; hpb /= 2)
    if (hpg % hpb == 0 && batch * nheads / hpb >= kSsdMinBlocks) return hpb;
  return 1;
}

hipError_t launch_ssd(const SsdParams &p, int out_bf16, hipStream_t stream) {
  if (p.headdim != P || p.chunk != Q) return hipErrorInvalidValue;
  return out_bf16 ? launch_typed<uint16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ssm
