// Chunked SSD with the rotary step on B and C fused in (Mamba-3's
// complex-valued state), for gfx950.
//
// Math: the rotary step of "Mamba-3 NKI Kernels for AWS Neuron", section "How
// it works", Phase 1 (angles phi_t = angle0 - sum_{s <= t} dt_s theta_s, B and
// C rotated pairwise by them, per head), followed by the chunked SSD of Phase 2
// (the scalar-decay form, or the trapezoidal three-term form) on the rotated,
// per-head B and C.  For state pair k < N/2 (states k and k + N/2):
//   B_rot[k]       = B[k] cos phi[k] - B[k + N/2] sin phi[k]
//   B_rot[k + N/2] = B[k] sin phi[k] + B[k + N/2] cos phi[k],   C alike.
// The SSD part follows the chunk kernel of ssd_kernels.hip (see there for
// the chunk products), at one head per workgroup.
//
// The rotated B and C never reach HBM.  Each workgroup (batch row b, head h,
// eight wavefronts) reads the group's shared B and C rows and theta, and per
// chunk:
//   - an angle pass (for the next chunk, during this one) fills a table of
//     phi_t[k] for the chunk's 64 steps: the increments dt_t theta_t[k] are
//     written lane-per-step as loaded, read back lane-per-(pair, 8-step
//     segment), summed in registers and combined over the segments with a DPP
//     scan, in float32 revolutions on top of the angle at the chunk's start,
//     which is carried from chunk to chunk in float64 and reduced to
//     [-1/2, 1/2] revolutions after every chunk;
//   - the staging rotates one 16-byte piece of B and of C per thread (8 pairs
//     of one step, both halves, loaded coalesced) with the hardware sine and
//     cosine (which take revolutions) and writes the rotated rows to LDS.
// The state update's B operand comes from the natural [s][n] rows through
// the transposing LDS read (ds_read_b64_tr_b16), so no transposed copy is
// kept: ~77 KB of LDS, two workgroups per CU.
#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInvTwoPiF = 0.15915494309189533577f;
constexpr double kTwoPi = 6.28318530717958647692529;
constexpr double kInvTwoPi = 0.15915494309189533576888;
constexpr int Q = 64;        // chunk length
constexpr int P = 64;        // headdim
constexpr int QP = Q + 16;   // padded [.][s] LDS rows (bf16)

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float bf2f(uint32_t v16) { return __uint_as_float(v16 << 16); }
__device__ __forceinline__ uint16_t f2bf(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ floatx4 mfma(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t *p) {  // 16-byte LDS read
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}

// Transposing LDS read of four bf16.
typedef __attribute__((address_space(3))) short4v lds_short4v;
__device__ __forceinline__ bf16x4 ldtr(const uint16_t *p) {
  // The C-style cast is an address-space cast: p points into LDS.
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(p)));
}

// MFMA fragment (row or column i0 + i, k = k0 + 8q .. k0 + 8q + 7) from an
// LDS array stored k-major, T[k][i] with row pitch RPT: lane (q, i) addresses
// T[k0 + 8q + i / 4 (+ 4)][i0 + 4 (i % 4)].
template <int RPT>
__device__ __forceinline__ bf16x8 frag_t(const uint16_t *T, int k0, int i0, int q, int i) {
  const uint16_t *a = T + (k0 + 8 * q + i / 4) * RPT + i0 + 4 * (i % 4);
  const bf16x4 lo = ldtr(a), hi = ldtr(a + 4 * RPT);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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

// Inclusive prefix sum over the 64 lanes: within each 16-lane row by DPP row
// shifts (lanes shifted in from outside the row read 0), then the totals of
// the rows below, read from lanes 15, 31 and 47.
__device__ __forceinline__ float wave_prefix(float a, int lane) {
  a += row_shr<1>(a);
  a += row_shr<2>(a);
  a += row_shr<4>(a);
  a += row_shr<8>(a);
  const float r0 = lane_value<15>(a), r1 = lane_value<31>(a), r2 = lane_value<47>(a);
  return a + (lane >= 16 ? r0 : 0.0f) + (lane >= 32 ? r1 : 0.0f) + (lane >= 48 ? r2 : 0.0f);
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two float32 rounded to bf16 (nearest even) in one 32-bit word, lo first.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v{lo, hi}), bf16x2));
}

__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Transposed copy of x ([p][t], rows of QP bf16): the XOR applied to the index
// of the 32-bit step pair (t / 2) in row p, so that a staging store
// instruction (64 / 8 consecutive pairs of each of 8 rows) spreads over all
// banks; fragment reads apply the same XOR.
__device__ __forceinline__ int tswz(int col) { return 8 * ((col >> 4) & 3); }
__device__ __forceinline__ int tidx(int col, int t) { return col * QP + 2 * ((t >> 1) ^ tswz(col)) + (t & 1); }

// One workgroup per (batch row, head) of eight wavefronts (two workgroups,
// four wavefronts per SIMD, per CU).  Wavefront w owns the headdim columns
// [16 (w % 4), 16 (w % 4) + 16) and the dstate rows [(w / 4) N/2, (w / 4) N/2
// + N/2) of the state, and the output rows [32 (w / 4), 32 (w / 4) + 32) of
// each chunk: the two wavefronts of a column block each take Y_off over their
// half of dstate for all rows, and swap the partial sums of each other's rows
// through LDS.
template <typename Tout, int N, bool HAS_Z, bool TRAP>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4)))
ssd_rope_kernel(const SsdRopeParams rp) {
  const SsdParams &p = rp.ssd;
  constexpr int NTH = 512;        // threads
  constexpr int KP = N / 2;       // state pairs
  constexpr int PG = KP / 8;      // groups of 8 pairs (one 16-byte vector of each half row)
  constexpr int NJOB = Q * PG;    // rotation jobs (step, pair group) per chunk
  constexpr int PPW = KP / 8;     // pairs per wavefront in the angle pass
  constexpr int SEGS = 64 / PPW;  // angle pass: step segments (lanes per pair)
  constexpr int SLEN = Q / SEGS;  // angle pass: steps per segment
  constexpr int KA = KP + 1;      // row of the angle table (floats): conflict-free by rows and by columns
  constexpr int NP = N + 24;      // padded LDS row of [.][n] arrays
  constexpr int NT = N / 16;      // dstate tiles of S^T
  constexpr int NT2 = NT / 2;     // dstate tiles of this wavefront's half
  constexpr int NK2 = N / 64;     // K steps over this wavefront's half of dstate
  constexpr int NK = N / 32;      // K steps over dstate
  static_assert(NJOB <= NTH && NTH % NJOB == 0 && PPW % 4 == 0, "rotation map");
  constexpr bool kStageY = sizeof(Tout) == 2;
  constexpr int YV = 8;                        // bf16 y elements per 16-byte vector
  constexpr int YP = P + YV;                   // padded y row
  static_assert(Q * (P / YV) == NTH, "one y vector per thread per chunk");
  constexpr int SM = (kStageY && Q * YP > Q * QP) ? Q * YP : Q * QP;  // M (or y) buffer
  // One LDS block: the small per-step arrays first (a_t, exp(a_t),
  // exp(a_last - a_s) w_s, w_s, gamma_s when TRAP, exp(a_last)), then the
  // tiles and the angle table.
  constexpr int kF = Q * 4;
  constexpr int kOffA = 0, kOffEa = kOffA + kF, kOffW = kOffEa + kF, kOffDt = kOffW + kF;
  constexpr int kOffGam = kOffDt + kF;
  constexpr int kOffDecay = kOffGam + (TRAP ? kF : 0);
  constexpr int kOffC = kOffDecay + 16;
  constexpr int kOffB = kOffC + Q * NP * 2;                 // C_rot[t][n], then B_rot[s][n]
  constexpr int kOffXt = kOffB + Q * NP * 2;                // x[p][s]
  constexpr int kOffM = kOffXt + P * QP * 2;                // M[t][s], then y[t][p]
  constexpr int kOffAng = kOffM + SM * 2;                   // angle[t][k] (revolutions, in [0, 1))
  // The angle table's space also carries the Y_off halves (8 wavefronts x 2
  // tiles x 64 lanes x 4 floats) between the angle passes.
  constexpr int kAngF = Q * KA > 8 * 2 * 64 * 4 ? Q * KA : 8 * 2 * 64 * 4;
  constexpr int kLds = kOffAng + kAngF * 4;
  static_assert(kOffC % 16 == 0 && kOffB % 16 == 0 && kOffXt % 16 == 0 && kOffM % 16 == 0 && kOffAng % 16 == 0,
                "LDS layout");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  float *const sA = reinterpret_cast<float *>(smem + kOffA);
  float *const sEa = reinterpret_cast<float *>(smem + kOffEa);
  float *const sW = reinterpret_cast<float *>(smem + kOffW);
  float *const sDt = reinterpret_cast<float *>(smem + kOffDt);
  float *const sGam = reinterpret_cast<float *>(smem + kOffGam);
  float *const sDecay = reinterpret_cast<float *>(smem + kOffDecay);
  uint16_t *const sC = reinterpret_cast<uint16_t *>(smem + kOffC);
  uint16_t *const sB = reinterpret_cast<uint16_t *>(smem + kOffB);
  uint16_t *const sXt = reinterpret_cast<uint16_t *>(smem + kOffXt);
  uint16_t *const sM = reinterpret_cast<uint16_t *>(smem + kOffM);
  float *const sAng = reinterpret_cast<float *>(smem + kOffAng);

  const uint16_t *__restrict__ gx = static_cast<const uint16_t *>(p.x);
  const uint16_t *__restrict__ gdt = static_cast<const uint16_t *>(p.dt);
  const uint16_t *__restrict__ gB = static_cast<const uint16_t *>(p.B);
  const uint16_t *__restrict__ gC = static_cast<const uint16_t *>(p.C);
  const uint16_t *__restrict__ gz = static_cast<const uint16_t *>(p.z);
  const uint16_t *__restrict__ glam = static_cast<const uint16_t *>(p.lam);
  const uint16_t *__restrict__ gth = static_cast<const uint16_t *>(rp.theta);
  Tout *__restrict__ gy = static_cast<Tout *>(p.y);

  const int64_t L = p.seqlen, H = p.nheads, G = p.ngroups, TH = rp.theta_heads;
  // The heads of a batch row read the same B, C (and theta when shared).
  // Consecutive workgroup ids are dealt round-robin to the 8 XCDs, so remap
  // ids to give each XCD a contiguous run of (b, h) and keep a batch row's
  // shared rows in one L2.
  const int64_t nblk = p.batch * H;
  int64_t id = blockIdx.x;
  if (nblk % 8 == 0) id = (id % 8) * (nblk / 8) + id / 8;
  const int64_t b = id / H;
  const int64_t h = id % H;
  const int64_t g = h / (H / G);
  const int64_t th = TH == 1 ? 0 : h;

  int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  int lane = tid % 64;
  int q = lane / 16;
  int r16 = lane % 16;
  int pcol = (wave % 4) * 16 + r16;  // this lane's headdim column in S^T and Y
  const int tr = wave / 4;   // this wavefront's output rows (tiles 2 tr, 2 tr + 1) and dstate half
  const int nb = tr * (N / 2);  // first dstate row of the half
  // Rotation job (the last NJOB threads) and x staging job (the first 256).
  const int jv = tid - (NTH - NJOB);
  const bool has_job = jv >= 0;
  int jt = max(jv, 0) / PG, jk0 = 8 * (max(jv, 0) % PG);
  const int kw = wave * PPW;  // the angle pass's first pair for this wavefront
  // Angle pass, second half: this lane's pair kw + aj and step segment ag.
  const int aj = lane / SEGS, ag = lane % SEGS;

  const float Ah = p.A[h];
  const float Dh = p.D ? p.D[h] : 0.0f;
  const float dt_bias = (p.dt_softplus && p.dt_bias != nullptr) ? p.dt_bias[h] : 0.0f;
  auto step_of = [&](float raw) __attribute__((always_inline)) {
    return p.dt_softplus ? dt_softplus(raw + dt_bias) : raw;
  };
  auto lam_of = [&](float raw) __attribute__((always_inline)) {
    return p.lam_sigmoid ? 1.0f / (1.0f + expf(-raw)) : raw;
  };

  // The angle of pair kw + aj at the start of the next chunk whose angles
  // are to be computed, in revolutions reduced to [-1/2, 1/2], float64 (the
  // SEGS lanes of a pair hold the same value).  angle0 is read here, before
  // anything is written, so angle_last may be angle0 itself.
  double base = rp.angle0 != nullptr ? static_cast<double>(rp.angle0[(b * H + h) * KP + kw + aj]) * kInvTwoPi : 0.0;
  base -= rint(base);

  floatx4 S[NT2];  // S^T tiles: rows n = nb + 16 i + 4q + r, column p = pcol
#pragma unroll
  for (int i = 0; i < NT2; ++i) S[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (p.h0) {
    const float *h0 = p.h0 + ((b * H + h) * P + pcol) * N + nb;
#pragma unroll
    for (int i = 0; i < NT2; ++i) S[i] = *reinterpret_cast<const floatx4 *>(h0 + i * 16 + 4 * q);
  }
  if constexpr (TRAP) {
    // The token before the sequence (its B already rotated, per head) enters
    // through the initial state, as in the trapezoidal SSD.
    if (p.x_prev != nullptr && L > 0) {
      const int64_t i0 = b * L * H + h;
      const float w0 = step_of(bf2f(gdt[i0])) * (1.0f - lam_of(bf2f(glam[i0])));
      const float xw = w0 * bf2f(static_cast<const uint16_t *>(p.x_prev)[(b * H + h) * P + pcol]);
      const uint16_t *bp = static_cast<const uint16_t *>(p.B_prev) + (b * H + h) * N + nb + 4 * q;
#pragma unroll
      for (int i = 0; i < NT2; ++i) {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(bp + 16 * i);
        S[i][0] = fmaf(xw, lo_bf(v.x), S[i][0]);
        S[i][1] = fmaf(xw, hi_bf(v.x), S[i][1]);
        S[i][2] = fmaf(xw, lo_bf(v.y), S[i][2]);
        S[i][3] = fmaf(xw, hi_bf(v.y), S[i][3]);
      }
    }
  }
  // Retire the initial loads here (s_waitcnt vmcnt(0)), so that the first use
  // of S in a chunk does not also wait for that chunk's prefetches.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  uint32_t *const sXt32 = reinterpret_cast<uint32_t *>(sXt);
  auto pair_lo = [](uint32_t a, uint32_t c) { return (a & 0xffffu) | (c << 16); };
  auto pair_hi = [](uint32_t a, uint32_t c) { return (a >> 16) | (c & 0xffff0000u); };

  // One chunk's global inputs in registers, loaded a chunk ahead.  Steps past
  // the end of the sequence load copies of the last step; their dt is taken
  // as 0, so they turn no angle, reach no stored output and add nothing to
  // the state.  The loads are branch-free.
  //   Rotation job (t, pg) = step t, pairs [8 pg, 8 pg + 8): B and C of both
  //   halves of those pairs, 16 bytes each.  Consecutive lanes take
  //   consecutive pair groups of one step, so a load instruction reads whole
  //   128-byte half rows.
  //   theta for the angle pass: this wavefront's PPW pairs at step `lane`.
  struct ChunkRegs {
    u32x4 bc[4];       // B[k], B[k + N/2], C[k], C[k + N/2] of the job's pairs
    u32x4 xv[2];       // x: steps 2 tp and 2 tp + 1 of one 8-column group
    uint32_t th[PPW / 2];  // raw bf16 bits of theta, two pairs per word
    uint32_t dt;       // raw bf16 bits of dt at step `lane`
    uint32_t lam, dtn, lamn;  // TRAP: lam at step `lane`, dt and lam at step `lane` + 1
  };
  // Global addresses: a uniform base at the chunk's first step plus a 32-bit
  // lane offset (the host keeps 64 rows of x and of B/C below 2^31 elements).
  const int rx = static_cast<int>(H * P), rbc = static_cast<int>(G * N), rdt = static_cast<int>(H);
  const int rth = static_cast<int>(TH * KP);
  auto load_chunk = [&](int64_t c0, ChunkRegs &R) __attribute__((always_inline)) {
    const int last = static_cast<int>(min(static_cast<int64_t>(Q), L - c0) - 1);  // last valid step offset
    // dt and theta first: the angle pass waits for them (loads complete in order).
    const int64_t dbase = (b * L + c0) * H + h;
    const int lastn = static_cast<int>(min(static_cast<int64_t>(Q) + 1, L - c0) - 1);  // the next chunk's first step too
    R.dt = gdt[dbase + min(lane, last) * rdt];
    if (TRAP && wave == 4) {  // the weights are built by the decay wavefront only
      R.lam = glam[dbase + min(lane, last) * rdt];
      R.dtn = gdt[dbase + min(lane + 1, lastn) * rdt];
      R.lamn = glam[dbase + min(lane + 1, lastn) * rdt];
    }
    {
      const uint16_t *tb = gth + ((b * L + c0) * TH + th) * KP + kw + min(lane, last) * rth;
      if constexpr (PPW == 8) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(tb);
        R.th[0] = v.x, R.th[1] = v.y, R.th[2] = v.z, R.th[3] = v.w;
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(tb);
        R.th[0] = v.x, R.th[1] = v.y;
      }
    }
    const uint16_t *bbase = gB + ((b * L + c0) * G + g) * N;
    const uint16_t *cbase = gC + ((b * L + c0) * G + g) * N;
    if (has_job) {
      const int off = min(jt, last) * rbc + jk0;
      R.bc[0] = *reinterpret_cast<const u32x4 *>(bbase + off);
      R.bc[1] = *reinterpret_cast<const u32x4 *>(bbase + off + KP);
      R.bc[2] = *reinterpret_cast<const u32x4 *>(cbase + off);
      R.bc[3] = *reinterpret_cast<const u32x4 *>(cbase + off + KP);
    }
    if (wave < 4) {
      const int tp = tid / (P / 8);
      const int pv = (tid % (P / 8)) * 8;
      const uint16_t *src = gx + ((b * L + c0) * H + h) * P;
#pragma unroll
      for (int e = 0; e < 2; ++e) R.xv[e] = *reinterpret_cast<const u32x4 *>(src + min(2 * tp + e, last) * rx + pv);
    }
  };

  // ---- angle pass (this wavefront's PPW pairs, every step of a chunk) -----
  // phi_t = base - sum_{s <= t} dt_s theta_s as a fraction of a revolution,
  // into the table; then the base moves to the next chunk's start.  The
  // table first takes the increments dt_t theta_t (lane = step, as loaded);
  // the wavefront then reads back its own columns with lane = (pair aj,
  // segment ag of SLEN steps), sums each segment in registers, combines the
  // segments with a scan over the SEGS lanes of the pair and writes the
  // angles over the increments.  Only this wavefront touches these columns.
  auto angle_pass = [&](const ChunkRegs &R, int64_t c0) __attribute__((always_inline)) {
    const float sr = (c0 + lane < L) ? step_of(bf2f(R.dt)) * kInvTwoPiF : 0.0f;  // revolutions per unit theta
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const uint32_t tw = R.th[j / 2];
      sAng[lane * KA + kw + j] = sr * ((j & 1) ? hi_bf(tw) : lo_bf(tw));
    }
    __builtin_amdgcn_wave_barrier();
    float part[SLEN];
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < SLEN; ++i) {
      acc += sAng[(ag * SLEN + i) * KA + kw + aj];
      part[i] = acc;
    }
    // Inclusive scan of the segment sums over the pair's SEGS consecutive
    // lanes (within a 16-lane row; with SEGS = 8 a row holds two pairs, and
    // the lanes of the other pair are masked off).
    float incl = acc;
#pragma unroll
    for (int sh = 1; sh < SEGS; sh *= 2) {
      float v;
      if (sh == 1) v = row_shr<1>(incl);
      else if (sh == 2) v = row_shr<2>(incl);
      else if (sh == 4) v = row_shr<4>(incl);
      else v = row_shr<8>(incl);
      if constexpr (SEGS < 16) v = ag >= sh ? v : 0.0f;
      incl += v;
    }
    const float excl = incl - acc;
    // The chunk's turn of the pair: the inclusive sum of its last segment
    // (lane 15, or lanes 7 and 15 of the row), broadcast within the row.
    float tot;
    if constexpr (SEGS == 16) {
      tot = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, incl), 0x15F, 0xF, 0xF, true));
    } else {
      const float t7 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, incl), 0x157, 0xF, 0xF, true));
      const float t15 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, incl), 0x15F, 0xF, 0xF, true));
      tot = (lane & 8) ? t15 : t7;
    }
    const float bf = static_cast<float>(base);
#pragma unroll
    for (int i = 0; i < SLEN; ++i)
      sAng[(ag * SLEN + i) * KA + kw + aj] = __builtin_amdgcn_fractf(bf - (excl + part[i]));
    base -= static_cast<double>(tot);
    base -= rint(base);
    if (c0 + Q >= L && rp.angle_last != nullptr && ag == 0)  // after the last chunk
      rp.angle_last[(b * H + h) * KP + kw + aj] = static_cast<float>(base * kTwoPi);
  };

  auto stage_chunk = [&](const ChunkRegs &R, int64_t c0) __attribute__((always_inline)) {
    // ---- rotary step: the job's 8 pairs at its step ------------------------
    if (has_job) {
      const int t = jt, k0 = jk0;
      float ang[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ang[i] = sAng[t * KA + k0 + i];
      u32x4 ob[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float o[2][4];  // [pair 2e + hw][B_rot lo, B_rot hi, C_rot lo, C_rot hi]
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          const int i = 2 * e + hw;
          const float rev = ang[i];
          const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
#pragma unroll
          for (int m = 0; m < 2; ++m) {  // B, then C
            const uint32_t w1 = R.bc[2 * m][e], w2 = R.bc[2 * m + 1][e];
            const float x1 = hw ? hi_bf(w1) : lo_bf(w1), x2 = hw ? hi_bf(w2) : lo_bf(w2);
            o[hw][2 * m] = x1 * cs - x2 * sn;
            o[hw][2 * m + 1] = x1 * sn + x2 * cs;
          }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) ob[m][e] = pack2(o[0][m], o[1][m]);
      }
      *reinterpret_cast<u32x4 *>(&sB[t * NP + k0]) = ob[0];
      *reinterpret_cast<u32x4 *>(&sB[t * NP + KP + k0]) = ob[1];
      *reinterpret_cast<u32x4 *>(&sC[t * NP + k0]) = ob[2];
      *reinterpret_cast<u32x4 *>(&sC[t * NP + KP + k0]) = ob[3];
      // The rotated B of the sequence's last step, for a later call's
      // previous-token term.
      if (rp.B_last != nullptr && c0 + t == L - 1) {
        uint16_t *bl = static_cast<uint16_t *>(rp.B_last) + (b * H + h) * N + k0;
        *reinterpret_cast<u32x4 *>(bl) = ob[0];
        *reinterpret_cast<u32x4 *>(bl + KP) = ob[1];
      }
    }
    // x transposed to [p][t].
    if (wave < 4) {
      const int col0 = (tid % (P / 8)) * 8, tp = tid / (P / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = col0 + 2 * i;
        sXt32[c * (QP / 2) + (tp ^ tswz(c))] = pair_lo(R.xv[0][i], R.xv[1][i]);
        sXt32[(c + 1) * (QP / 2) + (tp ^ tswz(c + 1))] = pair_hi(R.xv[0][i], R.xv[1][i]);
      }
    }
    // dt and the in-chunk cumulative decay (one lane per step; on a
    // wavefront that stages no x).
    if (wave == 4) {
      const float dtv = (c0 + lane < L) ? step_of(bf2f(R.dt)) : 0.0f;
      const float a = wave_prefix(dtv * Ah, lane);
      const float alast = lane_value<63>(a);
      float w = dtv;
      if constexpr (TRAP) {
        const float gam = (c0 + lane < L) ? lam_of(bf2f(R.lam)) * dtv : 0.0f;
        const bool nx = c0 + lane + 1 < L;
        const float dtn = nx ? step_of(bf2f(R.dtn)) : 0.0f;
        const float lamn = nx ? lam_of(bf2f(R.lamn)) : 0.0f;
        w = gam + dtn * (1.0f - lamn);
        sGam[lane] = gam;
      }
      sA[lane] = a;
      sEa[lane] = fast_exp(a);
      sW[lane] = fast_exp(alast - a) * w;
      sDt[lane] = w;
      if (lane == 0) sDecay[0] = fast_exp(alast);
    }
  };

  ChunkRegs R;
  if (L > 0) {  // an empty sequence reads nothing (its step indexes would be -1)
    load_chunk(0, R);
    angle_pass(R, 0);
    __syncthreads();
  }
  for (int64_t c0 = 0; c0 < L; c0 += Q) {
    // The lane indices pass through an empty asm each chunk, so the LDS and
    // global addresses derived from them are recomputed (a few VALU
    // operations) instead of being held, or spilled, across the loop.
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(q), "+v"(r16), "+v"(pcol), "+v"(jt), "+v"(jk0));
    const bool more = c0 + Q < L;
    stage_chunk(R, c0);
    __syncthreads();

    // ---- M = mask(G^T) into LDS: 12 tiles (si, ti) over the 8 wavefronts ----
    // (the two all-zero tiles listed last go to the second round)
    {
      constexpr uint64_t kTiles = 0x0 | 0x4ull << 4 | 0x5ull << 8 | 0x8ull << 12 | 0x9ull << 16 |
                                  0xAull << 20 | 0xCull << 24 | 0xDull << 28 | 0xEull << 32 |
                                  0xFull << 36 | 0x1ull << 40 | 0xBull << 44;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int k = wave + 8 * u;
        if (k >= 12) break;
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
        const float at = sA[t];
        const floatx4 as4 = *reinterpret_cast<const floatx4 *>(&sA[sb]);
        const floatx4 dt4 = *reinterpret_cast<const floatx4 *>(&sDt[sb]);
        floatx4 gm4 = dt4;
        if constexpr (TRAP) gm4 = *reinterpret_cast<const floatx4 *>(&sGam[sb]);
        uint16_t m[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = sb + r;
          const float ws = s < t ? dt4[r] : gm4[r];
          const float keep = s <= t ? 1.0f : 0.0f;
          m[r] = f2bf(acc[r] * fast_exp(fminf(at - as4[r], 0.0f)) * ws * keep);
        }
        *reinterpret_cast<u32x2 *>(&sM[t * QP + si * 16 + 4 * q]) = *reinterpret_cast<const u32x2 *>(m);
      }
    }
    // ---- Y_off = diag(exp(a_t)) C S_prev^T over this half of dstate --------
    // (all four row tiles; the partner wavefront's two go to it through LDS,
    // in the angle table's space, which is free until the next angle pass)
    float *const sX = sAng;
    floatx4 Y[2];
    {
      floatx4 Yp[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) Yp[ti] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK2; ++kk) {
        const floatx8 sf = {S[2 * kk][0], S[2 * kk][1], S[2 * kk][2], S[2 * kk][3],
                            S[2 * kk + 1][0], S[2 * kk + 1][1], S[2 * kk + 1][2], S[2 * kk + 1][3]};
        const bf16x8 bfrag = __builtin_convertvector(sf, bf16x8);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          const uint16_t *crow = &sC[(ti * 16 + r16) * NP + nb + 32 * kk + 4 * q];
          const bf16x4 lo = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2 *>(crow));
          const bf16x4 hi = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2 *>(crow + 16));
          const bf16x8 afrag = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          Yp[ti] = mfma(afrag, bfrag, Yp[ti]);
        }
      }
      // Selected with a wave-uniform condition, not a run-time register
      // index (which would compile to indexed register moves).
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        *reinterpret_cast<floatx4 *>(&sX[((wave * 2 + i) * 64 + lane) * 4]) = tr ? Yp[i] : Yp[2 + i];
        Y[i] = tr ? Yp[2 + i] : Yp[i];
      }
    }

    // ---- S_new = exp(a_last) S_prev + B^T (w x) over this half of dstate ---
    {
      const float decay = sDecay[0];
#pragma unroll
      for (int i = 0; i < NT2; ++i) S[i] *= decay;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int s0 = 32 * kk + 8 * q;
        const bf16x8 xs = lds8(&sXt[tidx(pcol, s0)]);
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
        for (int i = 0; i < NT2; ++i) S[i] = mfma(frag_t<NP>(sB, 32 * kk, nb + 16 * i, q, r16), bfrag, S[i]);
      }
    }
    if (p.h_last != nullptr && !more) {
      float *hl = p.h_last + ((b * H + h) * P + pcol) * N + nb;
#pragma unroll
      for (int i = 0; i < NT2; ++i) *reinterpret_cast<floatx4 *>(hl + i * 16 + 4 * q) = S[i];
    }
    // The next chunk's inputs.
    if (more) load_chunk(c0 + Q, R);
    __syncthreads();

    // The partner's half of Y_off for this wavefront's rows, then exp(a_t).
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      Y[i] += *reinterpret_cast<const floatx4 *>(&sX[(((wave ^ 4) * 2 + i) * 64 + lane) * 4]);
      const floatx4 ea = *reinterpret_cast<const floatx4 *>(&sEa[(2 * tr + i) * 16 + 4 * q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) Y[i][r] *= ea[r];
    }

    // ---- Y += M X (causal: K steps at or below the diagonal) ---------------
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ti = 2 * tr + i;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk <= tr) {  // 32 kk < 16 (ti + 1)
          const bf16x8 afrag = lds8(&sM[(ti * 16 + r16) * QP + 32 * kk + 8 * q]);
          const bf16x8 bfrag = lds8(&sXt[tidx(pcol, 32 * kk + 8 * q)]);
          Y[i] = mfma(afrag, bfrag, Y[i]);
        }
      }
    }

    // ---- epilogue: D skip and gate in the MFMA layout ------------------------
    // Element e of this lane: step t = (2 tr + e / 4) 16 + 4q + e % 4.
    uint32_t zr[8];
    const int64_t ybase = ((b * L + c0) * H + h) * P;  // (c0, h, 0) of x, z and y
    if constexpr (HAS_Z) {
      const int last = static_cast<int>(min(static_cast<int64_t>(Q), L - c0) - 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) zr[e] = gz[ybase + min((2 * tr + e / 4) * 16 + 4 * q + (e % 4), last) * rx + pcol];
    }
    float yv[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = (2 * tr + i) * 16 + 4 * q + r;
        float v = Y[i][r] + Dh * bf2f(sXt[tidx(pcol, t)]);
        if constexpr (HAS_Z) v *= silu(bf2f(zr[i * 4 + r]));
        yv[i * 4 + r] = v;
      }
    }
    // Every wavefront is done reading M, x and the Y_off halves: the M buffer
    // takes y, and the angle table the next chunk's angles (its theta and dt
    // were loaded during this chunk's products; this chunk's table was read
    // before the first barrier).
    __syncthreads();
    if (more) angle_pass(R, c0 + Q);
    if constexpr (kStageY) {
      Tout *sY = reinterpret_cast<Tout *>(sM);
#pragma unroll
      for (int e = 0; e < 8; ++e) st(sY, ((2 * tr + e / 4) * 16 + 4 * q + (e % 4)) * YP + pcol, yv[e]);
      __syncthreads();
      {
        const int t = tid / (P / YV);
        const int pv = (tid % (P / YV)) * YV;
        if (c0 + t < L)
          *reinterpret_cast<u32x4 *>(gy + ybase + t * rx + pv) = *reinterpret_cast<const u32x4 *>(&sY[t * YP + pv]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = (2 * tr + e / 4) * 16 + 4 * q + (e % 4);
        if (c0 + t < L) st(gy + ybase, t * rx + pcol, yv[e]);
      }
      if (more) __syncthreads();  // the angle table is complete before the next staging
    }
  }

  if (L == 0) {  // an empty sequence: h_last is the initial state, angle_last the initial angle
    if (p.h_last != nullptr) {
      float *hl = p.h_last + ((b * H + h) * P + pcol) * N + nb;
#pragma unroll
      for (int i = 0; i < NT2; ++i) *reinterpret_cast<floatx4 *>(hl + i * 16 + 4 * q) = S[i];
    }
    if (rp.angle_last != nullptr && ag == 0)
      rp.angle_last[(b * H + h) * KP + kw + aj] = static_cast<float>(base * kTwoPi);
  }
}

template <typename Tout, int N, bool TRAP>
hipError_t launch_n(const SsdRopeParams &p, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>(p.ssd.batch * p.ssd.nheads));
  if (p.ssd.z != nullptr)
    hipLaunchKernelGGL((ssd_rope_kernel<Tout, N, true, TRAP>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((ssd_rope_kernel<Tout, N, false, TRAP>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <typename Tout>
hipError_t launch_typed(const SsdRopeParams &p, hipStream_t stream) {
  if (p.ssd.lam != nullptr) {
    if (p.ssd.dstate == 128) return launch_n<Tout, 128, true>(p, stream);
    if (p.ssd.dstate == 64) return launch_n<Tout, 64, true>(p, stream);
  } else {
    if (p.ssd.dstate == 128) return launch_n<Tout, 128, false>(p, stream);
    if (p.ssd.dstate == 64) return launch_n<Tout, 64, false>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ssd_rope(const SsdRopeParams &p, int out_bf16, hipStream_t stream) {
  if (p.ssd.headdim != P || p.ssd.chunk != Q) return hipErrorInvalidValue;
  return out_bf16 ? launch_typed<uint16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ssm
