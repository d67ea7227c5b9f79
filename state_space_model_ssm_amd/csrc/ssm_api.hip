// C ABI of libssm (declared in include/ssm.h): argument checks, chunk-count
// resolution, workspace sizing and dispatch to the HIP launchers.
//
// Every check runs on the host before any HIP call, so a rejected request
// launches nothing and writes nothing.
#include "ssm.h"

#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "ssm_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SSM_OK;
}

bool valid_dtype(int32_t t) { return t == SSM_F32 || t == SSM_BF16; }
size_t dtype_size(int32_t t) { return t == SSM_F32 ? 4 : 2; }
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int32_t kMaxChunks = 4096;
constexpr int64_t kMaxGridX = 2147483647;

// Byte range [p, p + bytes) of one tensor, for the overlap check.
struct Span {
  const void *p;
  size_t bytes;
};
bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// ---------------------------------------------------------------------------
// Selective scan
// ---------------------------------------------------------------------------

// dims.flags may hold only `allowed` bits; dt_bias needs SSM_DT_SOFTPLUS.
int check_dt_flags(int32_t flags, int32_t allowed, const float *dt_bias) {
  if ((flags & ~allowed) != 0) return fail(SSM_ERR_SHAPE, "flags 0x%x: unknown or unsupported bits", flags);
  if (dt_bias != nullptr && !(flags & SSM_DT_SOFTPLUS))
    return fail(SSM_ERR_SHAPE, "dt_bias is read only with SSM_DT_SOFTPLUS");
  if (!aligned(dt_bias, 4)) return fail(SSM_ERR_ALIGN, "dt_bias must be 4-byte aligned");
  return SSM_OK;
}

int check_scan_dims(const ssm_scan_dims_t *d) {
  if (!d) return fail(SSM_ERR_NULL, "dims is NULL");
  int rc0 = SSM_OK;
  if (d->batch < 0 || d->dim < 0 || d->seqlen < 0)
    return fail(SSM_ERR_SHAPE, "negative size (batch=%lld dim=%lld seqlen=%lld)",
                (long long)d->batch, (long long)d->dim, (long long)d->seqlen);
  if (d->dstate < 1) return fail(SSM_ERR_SHAPE, "dstate must be >= 1 (got %lld)", (long long)d->dstate);
  if (d->ngroups < 1) return fail(SSM_ERR_SHAPE, "ngroups must be >= 1 (got %lld)", (long long)d->ngroups);
  if (d->dim % d->ngroups != 0)
    return fail(SSM_ERR_SHAPE, "ngroups (%lld) must divide dim (%lld)", (long long)d->ngroups,
                (long long)d->dim);
  if (!valid_dtype(d->in_dtype)) return fail(SSM_ERR_DTYPE, "in_dtype %d is not an ssm_dtype_t", d->in_dtype);
  if (!valid_dtype(d->out_dtype)) return fail(SSM_ERR_DTYPE, "out_dtype %d is not an ssm_dtype_t", d->out_dtype);
  rc0 = check_dt_flags(d->flags, SSM_DT_SOFTPLUS, d->dt_bias);
  if (rc0 != SSM_OK) return rc0;
  if (d->n_chunks < 0 || d->n_chunks > kMaxChunks)
    return fail(SSM_ERR_SHAPE, "n_chunks must be in [0, %d] (got %d)", kMaxChunks, d->n_chunks);
  const int64_t N = d->dstate;
  if (N != 1 && N != 2 && N != 4 && N != 8 && N != 16 && N != 32 && N != 64)
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not supported (1, 2, 4, 8, 16, 32 or 64)", (long long)N);
  const int64_t cpb = ssm::scan_channels_per_block(static_cast<int>(N));
  const int64_t tiles = d->ngroups ? ceil_div(d->dim / d->ngroups, cpb) : 0;
  if (d->batch > 0 && d->ngroups * tiles > kMaxGridX / d->batch)
    return fail(SSM_ERR_UNSUPPORTED, "batch * ngroups * channel tiles exceeds the grid limit");
  return SSM_OK;
}

// Chunk count the call uses.  0 asks the library: split the sequence only when
// the channels alone give fewer than 1024 wavefronts (one per SIMD of the
// 256-CU part) and the sequence has at least 384 steps; then aim at ~4096
// wavefronts with chunks of at least 128 steps (at most 64 chunks).  Measured
// on 1536 channels: 384 steps and fewer run fastest in one pass (the summary
// pass and a second launch cost more than they save), 4096 steps take 65 us
// in 8-16 chunks against 149 us in one.
int32_t resolve_chunks(const ssm_scan_dims_t *d, int64_t *chunk_len) {
  const int64_t L = d->seqlen;
  if (L <= 1 || d->batch == 0 || d->dim == 0) {
    *chunk_len = L > 0 ? L : 1;
    return 1;
  }
  int64_t want = d->n_chunks;
  if (want == 0) {
    const int64_t waves = d->batch * d->dim * d->dstate / 64;
    if (waves >= 1024 || L < 384) {
      want = 1;
    } else {
      want = ceil_div(4096, waves > 0 ? waves : 1);
      const int64_t cap = L / 128;
      if (want > cap) want = cap;
      if (want > 64) want = 64;
    }
  }
  if (want > L) want = L;
  int64_t len = ceil_div(L, want);
  if (want > 1) len = ceil_div(len, ssm::kScanChunkAlign) * ssm::kScanChunkAlign;
  *chunk_len = len;
  return static_cast<int32_t>(ceil_div(L, len));
}

size_t scan_workspace(const ssm_scan_dims_t *d, int32_t chunks) {
  if (chunks <= 1) return 0;
  return static_cast<size_t>(8) * d->batch * d->dim * (chunks - 1) * d->dstate;
}

}  // namespace

extern "C" {

int ssm_scan_workspace_size(const ssm_scan_dims_t *dims, size_t *bytes) {
  if (!bytes) return fail(SSM_ERR_NULL, "bytes is NULL");
  const int rc = check_scan_dims(dims);
  if (rc != SSM_OK) return rc;
  int64_t len;
  *bytes = scan_workspace(dims, resolve_chunks(dims, &len));
  return ok();
}

size_t ssm_scan_workspace_bytes(const ssm_scan_dims_t *dims) {
  size_t bytes = 0;
  return ssm_scan_workspace_size(dims, &bytes) == SSM_OK ? bytes : SIZE_MAX;
}

int ssm_scan_resolved_chunks(const ssm_scan_dims_t *dims, int32_t *n_chunks) {
  if (!n_chunks) return fail(SSM_ERR_NULL, "n_chunks is NULL");
  const int rc = check_scan_dims(dims);
  if (rc != SSM_OK) return rc;
  int64_t len;
  *n_chunks = resolve_chunks(dims, &len);
  return ok();
}

}  // extern "C"

namespace {

// Scratch of ssm_scan_fwd_noalloc: the chunked carry of every call on a
// device lives in this file-scope array (one copy per device, held until the
// process ends).  Host code never uses the array's name as an address: the
// device address is looked up once per device with hipGetSymbolAddress and
// kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t{16} << 20;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the
// first call there).
int scratch_on_current_device(float **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SSM_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch covers", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(SSM_ERR_HIP, "hipGetSymbolAddress of the static scratch failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float *>(g_scratch_ptr[dev]);
  return SSM_OK;
}

// ssm_scan_fwd and ssm_scan_fwd_noalloc: the same checks and kernels; the
// chunked carry lives in the caller's workspace, or (noalloc) in `scratch`.
int scan_fwd_run(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *h0, void *y, float *h_last,
                 const ssm_scan_dims_t *dims, void *stream, bool noalloc) {
  int rc = check_scan_dims(dims);
  if (rc != SSM_OK) return rc;
  const ssm_scan_dims_t &d = *dims;
  const int64_t n_bdl = d.batch * d.dim * d.seqlen;
  const int64_t n_bc = d.batch * d.ngroups * d.dstate * d.seqlen;
  const int64_t n_a = d.dim * d.dstate;
  const int64_t n_h = d.batch * d.dim * d.dstate;
  if (n_bdl > 0 && (!u || !delta || !y)) return fail(SSM_ERR_NULL, "u, delta and y are required");
  if (n_bc > 0 && (!B || !C)) return fail(SSM_ERR_NULL, "B and C are required");
  if (n_a > 0 && !A) return fail(SSM_ERR_NULL, "A is required");
  const size_t ei = dtype_size(d.in_dtype), eo = dtype_size(d.out_dtype);
  if (!aligned(u, ei) || !aligned(delta, ei) || !aligned(B, ei) || !aligned(C, ei) || !aligned(z, ei))
    return fail(SSM_ERR_ALIGN, "input pointers must be aligned to %zu bytes", ei);
  if (!aligned(y, eo)) return fail(SSM_ERR_ALIGN, "y must be aligned to %zu bytes", eo);
  if (!aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 4) || !aligned(h_last, 4))
    return fail(SSM_ERR_ALIGN, "A, D, h0 and h_last must be 4-byte aligned");
  int64_t chunk_len = 1;
  const int32_t chunks = resolve_chunks(&d, &chunk_len);
  const Span ins[] = {{u, n_bdl * ei}, {delta, n_bdl * ei}, {z, n_bdl * ei}, {B, n_bc * ei},
                      {C, n_bc * ei},  {A, n_a * 4ull},    {D, d.dim * 4ull}, {d.dt_bias, d.dim * 4ull}};
  const Span sy{y, n_bdl * eo}, sh{h_last, n_h * 4ull}, s0{h0, n_h * 4ull};
  for (const Span &s : ins)
    if (overlap(s, sy) || overlap(s, sh) || overlap(s, s0))
      return fail(SSM_ERR_SHAPE, "an output or h0 overlaps an input");
  if (overlap(sy, sh) || overlap(sy, s0)) return fail(SSM_ERR_SHAPE, "y overlaps h_last or h0");
  // h_last may replace h0 in place when one pass reads each state once and
  // writes it after; chunked passes read h0 from every chunk.
  if (overlap(s0, sh) && !(h0 == h_last && chunks == 1))
    return fail(SSM_ERR_SHAPE, "h_last overlaps h0 (only h_last == h0 with one pass is allowed)");
  const size_t need = scan_workspace(&d, chunks);
  if (noalloc) {
    if (need > kScratchBytes)
      return fail(SSM_ERR_WORKSPACE,
                  "the chunked carry of %d chunks needs %zu bytes, more than the %zu-byte static scratch of "
                  "ssm_scan_fwd_noalloc (ask for fewer chunks)",
                  chunks, need, kScratchBytes);
  } else if (need > 0) {
    if (!d.workspace || d.workspace_bytes < need)
      return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required for %d chunks (got %zu)", need,
                  chunks, d.workspace ? d.workspace_bytes : (size_t)0);
    if (!aligned(d.workspace, 4)) return fail(SSM_ERR_ALIGN, "workspace must be 4-byte aligned");
    const Span sw{d.workspace, need};
    for (const Span &s : ins)
      if (overlap(s, sw)) return fail(SSM_ERR_SHAPE, "workspace overlaps an input");
    if (overlap(sw, s0)) return fail(SSM_ERR_SHAPE, "workspace overlaps h0");
    if (overlap(sw, sy) || overlap(sw, sh)) return fail(SSM_ERR_SHAPE, "workspace overlaps an output");
  }
  if (d.batch == 0 || d.dim == 0) return ok();
  float *carry = nullptr;
  if (need > 0) {
    if (noalloc) {
      rc = scratch_on_current_device(&carry);
      if (rc != SSM_OK) return rc;
    } else {
      carry = static_cast<float *>(d.workspace);
    }
  }

  ssm::ScanParams p{};
  p.u = u;
  p.delta = delta;
  p.B = B;
  p.C = C;
  p.z = z;
  p.A = A;
  p.D = D;
  p.h0 = h0;
  p.y = y;
  p.h_last = h_last;
  p.dt_bias = d.dt_bias;
  p.dt_softplus = (d.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
  p.carry = carry;
  p.batch = d.batch;
  p.dim = d.dim;
  p.seqlen = d.seqlen;
  p.ngroups = d.ngroups;
  p.dim_per_group = d.dim / d.ngroups;
  p.chunk_len = chunk_len;
  p.tiles_per_group = ceil_div(p.dim_per_group, ssm::scan_channels_per_block(static_cast<int>(d.dstate)));
  p.n_chunks = chunks;
  p.dstate = static_cast<int32_t>(d.dstate);
  const int vec = ssm::scan_vector_elems(d.in_dtype == SSM_BF16);
  p.vec_ok = (d.seqlen % vec == 0) && aligned(u, 16) && aligned(delta, 16) && aligned(B, 16) &&
             aligned(C, 16);
  const hipError_t e = ssm::launch_scan(p, d.in_dtype == SSM_BF16, d.out_dtype == SSM_BF16,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "scan launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int ssm_scan_fwd(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *h0, void *y, float *h_last,
                 const ssm_scan_dims_t *dims, void *stream) {
  return scan_fwd_run(u, delta, A, B, C, D, z, h0, y, h_last, dims, stream, false);
}

int ssm_scan_fwd_noalloc(const void *u, const void *delta, const float *A, const void *B, const void *C,
                         const float *D, const void *z, const float *h0, void *y, float *h_last,
                         const ssm_scan_dims_t *dims, void *stream) {
  return scan_fwd_run(u, delta, A, B, C, D, z, h0, y, h_last, dims, stream, true);
}

// ---------------------------------------------------------------------------
// Selective-scan backward
// ---------------------------------------------------------------------------

// Backward workspace, in floats: the state checkpoints, then the dB and dC
// terms of every channel tile, then the per-batch dA and dD terms.
struct BwdWorkspace {
  size_t ckpt, part_bc, part_a, part_d;
  size_t bytes() const { return 4 * (ckpt + 2 * part_bc + part_a + part_d); }
};

static BwdWorkspace scan_bwd_layout(const ssm_scan_dims_t *d) {
  const int64_t tiles =
      d->ngroups > 0 ? ceil_div(d->dim / d->ngroups, ssm::scan_channels_per_block(static_cast<int>(d->dstate))) : 0;
  BwdWorkspace w;
  w.ckpt = static_cast<size_t>(d->batch * d->dim * d->dstate * ceil_div(d->seqlen, ssm::kScanCkptStep));
  w.part_bc = static_cast<size_t>(d->batch * d->ngroups * tiles * d->dstate * d->seqlen);
  w.part_a = static_cast<size_t>(d->batch * d->dim * d->dstate);
  w.part_d = static_cast<size_t>(d->batch * d->dim);
  return w;
}

static size_t scan_bwd_workspace(const ssm_scan_dims_t *d) { return scan_bwd_layout(d).bytes(); }

int ssm_scan_bwd_workspace_size(const ssm_scan_dims_t *dims, size_t *bytes) {
  if (!bytes) return fail(SSM_ERR_NULL, "bytes is NULL");
  const int rc = check_scan_dims(dims);
  if (rc != SSM_OK) return rc;
  *bytes = scan_bwd_workspace(dims);
  return ok();
}

int ssm_scan_bwd(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *h0, const void *dy, const float *dh_last,
                 void *du, void *ddelta, float *dA, float *dB, float *dC, float *dD, void *dz, float *dh0,
                 const ssm_scan_dims_t *dims, void *stream) {
  int rc = check_scan_dims(dims);
  if (rc != SSM_OK) return rc;
  const ssm_scan_dims_t &d = *dims;
  const int64_t n_bdl = d.batch * d.dim * d.seqlen;
  const int64_t n_bc = d.batch * d.ngroups * d.dstate * d.seqlen;
  const int64_t n_a = d.dim * d.dstate;
  const int64_t n_h = d.batch * d.dim * d.dstate;
  if (n_bdl > 0 && (!u || !delta || !dy || !du || !ddelta))
    return fail(SSM_ERR_NULL, "u, delta, dy, du and ddelta are required");
  if (n_bc > 0 && (!B || !C || !dB || !dC)) return fail(SSM_ERR_NULL, "B, C, dB and dC are required");
  if (n_a > 0 && (!A || !dA)) return fail(SSM_ERR_NULL, "A and dA are required");
  if (n_bdl > 0 && z && !dz) return fail(SSM_ERR_NULL, "dz is required when z is given");
  if (d.dim > 0 && D && !dD) return fail(SSM_ERR_NULL, "dD is required when D is given");
  if (!z) dz = nullptr;
  if (!D) dD = nullptr;
  const size_t ei = dtype_size(d.in_dtype), eo = dtype_size(d.out_dtype);
  if (!aligned(u, ei) || !aligned(delta, ei) || !aligned(B, ei) || !aligned(C, ei) || !aligned(z, ei) ||
      !aligned(du, ei) || !aligned(ddelta, ei) || !aligned(dz, ei))
    return fail(SSM_ERR_ALIGN, "input-dtype pointers must be aligned to %zu bytes", ei);
  if (!aligned(dy, eo)) return fail(SSM_ERR_ALIGN, "dy must be aligned to %zu bytes", eo);
  if (!aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 4) || !aligned(dh_last, 4) || !aligned(dA, 4) ||
      !aligned(dB, 4) || !aligned(dC, 4) || !aligned(dD, 4) || !aligned(dh0, 4))
    return fail(SSM_ERR_ALIGN, "float32 pointers must be 4-byte aligned");
  const Span ins[] = {{u, n_bdl * ei},  {delta, n_bdl * ei}, {z, n_bdl * ei},   {B, n_bc * ei},
                      {C, n_bc * ei},   {A, n_a * 4ull},     {D, d.dim * 4ull}, {h0, n_h * 4ull},
                      {dy, n_bdl * eo}, {dh_last, n_h * 4ull}, {d.dt_bias, d.dim * 4ull}};
  const Span outs[] = {{du, n_bdl * ei}, {ddelta, n_bdl * ei}, {dz, n_bdl * ei},  {dA, n_a * 4ull},
                       {dB, n_bc * 4ull}, {dC, n_bc * 4ull},    {dD, d.dim * 4ull}, {dh0, n_h * 4ull}};
  for (const Span &o : outs) {
    for (const Span &i : ins)
      if (overlap(o, i)) return fail(SSM_ERR_SHAPE, "a gradient output overlaps an input");
    for (const Span &o2 : outs)
      if (&o != &o2 && overlap(o, o2)) return fail(SSM_ERR_SHAPE, "two gradient outputs overlap");
  }
  const size_t need = scan_bwd_workspace(&d);
  if (need > 0) {
    if (!d.workspace || d.workspace_bytes < need)
      return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required for checkpoints and partial sums (got %zu)",
                  need, d.workspace ? d.workspace_bytes : (size_t)0);
    if (!aligned(d.workspace, 4)) return fail(SSM_ERR_ALIGN, "workspace must be 4-byte aligned");
    const Span sw{d.workspace, need};
    for (const Span &s : ins)
      if (overlap(s, sw)) return fail(SSM_ERR_SHAPE, "workspace overlaps an input");
    for (const Span &s : outs)
      if (overlap(s, sw)) return fail(SSM_ERR_SHAPE, "workspace overlaps an output");
  }
  // An empty batch or channel set still writes zeros to dA and dD (sums over
  // nothing); the backward kernel then launches no workgroup.
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t tiles = ceil_div(d.dim / d.ngroups, ssm::scan_channels_per_block(static_cast<int>(d.dstate)));
  ssm::ScanParams f{};
  f.u = u;
  f.delta = delta;
  f.B = B;
  f.C = C;
  f.A = A;
  f.h0 = h0;
  f.dt_bias = d.dt_bias;
  f.dt_softplus = (d.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
  f.carry = static_cast<float *>(d.workspace);
  f.batch = d.batch;
  f.dim = d.dim;
  f.seqlen = d.seqlen;
  f.ngroups = d.ngroups;
  f.dim_per_group = d.dim / d.ngroups;
  f.chunk_len = d.seqlen > 0 ? d.seqlen : 1;
  f.tiles_per_group = tiles;
  f.n_chunks = 1;
  f.dstate = static_cast<int32_t>(d.dstate);
  const int vec = ssm::scan_vector_elems(d.in_dtype == SSM_BF16);
  f.vec_ok = (d.seqlen % vec == 0) && aligned(u, 16) && aligned(delta, 16) && aligned(B, 16) && aligned(C, 16);
  hipError_t e = hipSuccess;
  if (need > 0) e = ssm::launch_scan_ckpt(f, d.in_dtype == SSM_BF16, st);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "checkpoint launch failed: %s", hipGetErrorString(e));
  ssm::ScanBwdParams p{};
  p.u = u;
  p.delta = delta;
  p.B = B;
  p.C = C;
  p.z = z;
  p.A = A;
  p.D = D;
  p.dy = dy;
  p.dh_last = dh_last;
  p.du = du;
  p.ddelta = ddelta;
  p.dz = dz;
  p.dA = dA;
  p.dB = dB;
  p.dC = dC;
  p.dD = dD;
  p.dh0 = dh0;
  p.dt_bias = d.dt_bias;
  p.dt_softplus = f.dt_softplus;
  p.ckpt = static_cast<const float *>(d.workspace);
  const BwdWorkspace wl = scan_bwd_layout(&d);
  float *ws = static_cast<float *>(d.workspace);
  p.part_dB = ws + wl.ckpt;
  p.part_dC = p.part_dB + wl.part_bc;
  p.part_dA = p.part_dC + wl.part_bc;
  p.part_dD = p.part_dA + wl.part_a;
  p.batch = d.batch;
  p.dim = d.dim;
  p.seqlen = d.seqlen;
  p.ngroups = d.ngroups;
  p.dim_per_group = d.dim / d.ngroups;
  p.tiles_per_group = tiles;
  p.dstate = static_cast<int32_t>(d.dstate);
  e = ssm::launch_scan_bwd(p, d.in_dtype == SSM_BF16, d.out_dtype == SSM_BF16, st);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
// Scalar-decay chunked SSD
// ---------------------------------------------------------------------------

static int check_ssd_dims(const ssd_dims_t *d) {
  if (!d) return fail(SSM_ERR_NULL, "dims is NULL");
  if (d->batch < 0 || d->seqlen < 0 || d->nheads < 0)
    return fail(SSM_ERR_SHAPE, "negative size (batch=%lld seqlen=%lld nheads=%lld)", (long long)d->batch,
                (long long)d->seqlen, (long long)d->nheads);
  if (d->headdim < 1 || d->dstate < 1 || d->chunk < 1)
    return fail(SSM_ERR_SHAPE, "headdim, dstate and chunk must be >= 1");
  if (d->ngroups < 1) return fail(SSM_ERR_SHAPE, "ngroups must be >= 1 (got %lld)", (long long)d->ngroups);
  if (d->nheads % d->ngroups != 0)
    return fail(SSM_ERR_SHAPE, "ngroups (%lld) must divide nheads (%lld)", (long long)d->ngroups,
                (long long)d->nheads);
  if (!valid_dtype(d->in_dtype)) return fail(SSM_ERR_DTYPE, "in_dtype %d is not an ssm_dtype_t", d->in_dtype);
  if (!valid_dtype(d->out_dtype)) return fail(SSM_ERR_DTYPE, "out_dtype %d is not an ssm_dtype_t", d->out_dtype);
  if (d->reserved != 0) return fail(SSM_ERR_SHAPE, "reserved must be 0");
  const int rc0 = check_dt_flags(d->flags, SSM_DT_SOFTPLUS | SSM_LAM_SIGMOID, d->dt_bias);
  if (rc0 != SSM_OK) return rc0;
  if (d->in_dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "ssd_chunked_fwd takes bf16 inputs only (matrix-core operands)");
  if (d->headdim != 64) return fail(SSM_ERR_UNSUPPORTED, "headdim %lld not supported (64)", (long long)d->headdim);
  if (d->dstate != 64 && d->dstate != 128)
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not supported (64 or 128)", (long long)d->dstate);
  if (d->chunk != 64) return fail(SSM_ERR_UNSUPPORTED, "chunk %lld not supported (64)", (long long)d->chunk);
  if (d->batch > 0 && d->nheads > kMaxGridX / d->batch)
    return fail(SSM_ERR_UNSUPPORTED, "batch * nheads exceeds the grid limit");
  // A chunk's rows of x, z, y and of B, C are addressed with 32-bit offsets.
  if (d->nheads * d->headdim >= (1ll << 25) || d->ngroups * d->dstate >= (1ll << 25))
    return fail(SSM_ERR_UNSUPPORTED, "nheads * headdim and ngroups * dstate must be below 2^25");
  return SSM_OK;
}

int ssd_workspace_size(const ssd_dims_t *dims, size_t *bytes) {
  if (!bytes) return fail(SSM_ERR_NULL, "bytes is NULL");
  const int rc = check_ssd_dims(dims);
  if (rc != SSM_OK) return rc;
  *bytes = 0;
  return ok();
}

size_t ssd_workspace_bytes(const ssd_dims_t *dims) {
  size_t bytes = 0;
  return ssd_workspace_size(dims, &bytes) == SSM_OK ? bytes : SIZE_MAX;
}

// The rotary step's arguments of the fused forms (ssd_rope_chunked_fwd,
// ssd_rope_trap_chunked_fwd).
struct SsdRopeArgs {
  const void *theta;
  int64_t theta_heads;
  const float *angle0;
  float *angle_last;
  void *B_last;
};

static int ssd_run(const void *x, const void *dt, const void *lam, bool trap, const float *A, const void *B,
                   const void *C, const float *D, const void *z, const float *h0, const void *x_prev,
                   const void *B_prev, void *y, float *h_last, const ssd_dims_t *dims, void *stream,
                   const SsdRopeArgs *rope = nullptr) {
  const int rc = check_ssd_dims(dims);
  if (rc != SSM_OK) return rc;
  const ssd_dims_t &d = *dims;
  const int64_t n_x = d.batch * d.seqlen * d.nheads * d.headdim;
  const int64_t n_dt = d.batch * d.seqlen * d.nheads;
  const int64_t n_bc = d.batch * d.seqlen * d.ngroups * d.dstate;
  const int64_t n_h = d.batch * d.nheads * d.headdim * d.dstate;
  if (n_x > 0 && (!x || !dt || !y)) return fail(SSM_ERR_NULL, "x, dt and y are required");
  if (n_bc > 0 && (!B || !C)) return fail(SSM_ERR_NULL, "B and C are required");
  if (d.nheads > 0 && !A) return fail(SSM_ERR_NULL, "A is required");
  const size_t eo = dtype_size(d.out_dtype);
  if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(z, 16))
    return fail(SSM_ERR_ALIGN, "x, z, B and C must be 16-byte aligned");
  if (trap && n_dt > 0 && !lam) return fail(SSM_ERR_NULL, "lam is required");
  if (!trap && (d.flags & SSM_LAM_SIGMOID))
    return fail(SSM_ERR_SHAPE, "SSM_LAM_SIGMOID applies to ssd_trap_chunked_fwd only");
  if (!aligned(dt, 2) || !aligned(lam, 2)) return fail(SSM_ERR_ALIGN, "dt and lam must be 2-byte aligned");
  if (!aligned(y, eo)) return fail(SSM_ERR_ALIGN, "y must be aligned to %zu bytes", eo);
  if (!aligned(A, 4) || !aligned(D, 4)) return fail(SSM_ERR_ALIGN, "A and D must be 4-byte aligned");
  if (!aligned(h0, 16) || !aligned(h_last, 16))
    return fail(SSM_ERR_ALIGN, "h0 and h_last must be 16-byte aligned");
  if ((x_prev == nullptr) != (B_prev == nullptr))
    return fail(SSM_ERR_NULL, "x_prev and B_prev are given together or not at all");
  if (!aligned(x_prev, 16) || !aligned(B_prev, 16))
    return fail(SSM_ERR_ALIGN, "x_prev and B_prev must be 16-byte aligned");
  // With the rotary step B_prev is per head (rotated by that head's angle).
  const int64_t n_xp = d.batch * d.nheads * d.headdim;
  const int64_t n_bp = d.batch * (rope ? d.nheads : d.ngroups) * d.dstate;
  const int64_t n_ang = d.batch * d.nheads * (d.dstate / 2);
  const int64_t th_heads = rope ? rope->theta_heads : 0;
  const void *theta = rope ? rope->theta : nullptr;
  const float *angle0 = rope ? rope->angle0 : nullptr;
  float *angle_last = rope ? rope->angle_last : nullptr;
  void *B_last = rope ? rope->B_last : nullptr;
  if (rope) {
    if (th_heads != 1 && th_heads != d.nheads)
      return fail(SSM_ERR_SHAPE, "theta_heads must be 1 or nheads (got %lld)", (long long)th_heads);
    if (d.batch * d.seqlen > 0 && !theta) return fail(SSM_ERR_NULL, "theta is required");
    if (!aligned(theta, 16) || !aligned(B_last, 16)) return fail(SSM_ERR_ALIGN, "theta and B_last must be 16-byte aligned");
    if (!aligned(angle0, 4) || !aligned(angle_last, 4)) return fail(SSM_ERR_ALIGN, "angles must be 4-byte aligned");
  }
  const Span ins[] = {{x, n_x * 2ull},  {dt, n_dt * 2ull},     {z, n_x * 2ull},
                      {B, n_bc * 2ull}, {C, n_bc * 2ull},     {A, d.nheads * 4ull},
                      {D, d.nheads * 4ull}, {lam, n_dt * 2ull}, {d.dt_bias, d.nheads * 4ull},
                      {x_prev, n_xp * 2ull}, {B_prev, n_bp * 2ull},
                      {theta, d.batch * d.seqlen * th_heads * (d.dstate / 2) * 2ull}, {angle0, n_ang * 4ull}};
  const Span sy{y, n_x * eo}, sh{h_last, n_h * 4ull}, s0{h0, n_h * 4ull};
  const Span sa{angle_last, n_ang * 4ull}, sbl{B_last, d.batch * d.nheads * d.dstate * 2ull};
  for (const Span &s : ins) {
    if (overlap(s, sy) || overlap(s, sh) || overlap(s, s0) || overlap(s, sbl))
      return fail(SSM_ERR_SHAPE, "an output or h0 overlaps an input");
    // angle_last may be exactly angle0 (each is read before it is written).
    if (overlap(s, sa) && !(s.p == angle0 && angle_last == angle0))
      return fail(SSM_ERR_SHAPE, "angle_last overlaps an input (only angle_last == angle0 is allowed)");
  }
  if (overlap(sy, sh) || overlap(sy, s0)) return fail(SSM_ERR_SHAPE, "y overlaps h_last or h0");
  if (overlap(sa, sy) || overlap(sa, sh) || overlap(sa, s0) || overlap(sa, sbl) || overlap(sbl, sy) ||
      overlap(sbl, sh) || overlap(sbl, s0))
    return fail(SSM_ERR_SHAPE, "outputs overlap each other");
  // One workgroup per (batch, head) reads its state first and writes it last.
  if (overlap(s0, sh) && h0 != h_last)
    return fail(SSM_ERR_SHAPE, "h_last overlaps h0 (only h_last == h0 is allowed)");
  if (d.batch == 0 || d.nheads == 0) return ok();

  ssm::SsdParams p{};
  p.x = x;
  p.dt = dt;
  p.lam = trap ? lam : nullptr;
  p.x_prev = trap ? x_prev : nullptr;
  p.B_prev = trap ? B_prev : nullptr;
  p.B = B;
  p.C = C;
  p.z = z;
  p.A = A;
  p.D = D;
  p.h0 = h0;
  p.y = y;
  p.h_last = h_last;
  p.dt_bias = d.dt_bias;
  p.dt_softplus = (d.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
  p.lam_sigmoid = (d.flags & SSM_LAM_SIGMOID) ? 1 : 0;
  p.batch = d.batch;
  p.seqlen = d.seqlen;
  p.nheads = d.nheads;
  p.headdim = d.headdim;
  p.dstate = d.dstate;
  p.ngroups = d.ngroups;
  p.chunk = d.chunk;
  hipError_t e;
  if (rope) {
    ssm::SsdRopeParams rp{};
    rp.ssd = p;
    rp.theta = theta;
    rp.angle0 = angle0;
    rp.angle_last = angle_last;
    rp.B_last = B_last;
    rp.theta_heads = th_heads;
    e = ssm::launch_ssd_rope(rp, d.out_dtype == SSM_BF16, static_cast<hipStream_t>(stream));
  } else {
    e = ssm::launch_ssd(p, d.out_dtype == SSM_BF16, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "ssd launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ssd_chunked_fwd(const void *x, const void *dt, const float *A, const void *B, const void *C,
                    const float *D, const void *z, const float *h0, void *y, float *h_last,
                    const ssd_dims_t *dims, void *stream) {
  return ssd_run(x, dt, nullptr, false, A, B, C, D, z, h0, nullptr, nullptr, y, h_last, dims, stream);
}

int ssd_trap_chunked_fwd(const void *x, const void *dt, const void *lam, const float *A, const void *B,
                         const void *C, const float *D, const void *z, const float *h0, const void *x_prev,
                         const void *B_prev, void *y, float *h_last, const ssd_dims_t *dims, void *stream) {
  return ssd_run(x, dt, lam, true, A, B, C, D, z, h0, x_prev, B_prev, y, h_last, dims, stream);
}

int ssd_rope_chunked_fwd(const void *x, const void *dt, const float *A, const void *B, const void *C,
                         const void *theta, int64_t theta_heads, const float *angle0, const float *D,
                         const void *z, const float *h0, void *y, float *h_last, float *angle_last,
                         void *B_last, const ssd_dims_t *dims, void *stream) {
  const SsdRopeArgs r{theta, theta_heads, angle0, angle_last, B_last};
  return ssd_run(x, dt, nullptr, false, A, B, C, D, z, h0, nullptr, nullptr, y, h_last, dims, stream, &r);
}

int ssd_rope_trap_chunked_fwd(const void *x, const void *dt, const void *lam, const float *A, const void *B,
                              const void *C, const void *theta, int64_t theta_heads, const float *angle0,
                              const float *D, const void *z, const float *h0, const void *x_prev,
                              const void *B_prev, void *y, float *h_last, float *angle_last, void *B_last,
                              const ssd_dims_t *dims, void *stream) {
  const SsdRopeArgs r{theta, theta_heads, angle0, angle_last, B_last};
  return ssd_run(x, dt, lam, true, A, B, C, D, z, h0, x_prev, B_prev, y, h_last, dims, stream, &r);
}

// ---------------------------------------------------------------------------
// Scalar-decay SSD backward
// ---------------------------------------------------------------------------

// Backward workspace: per (batch, head, chunk) two bf16 state matrices
// (S_in and dS) and two floats; per (batch, step, head block) the float32 dB
// and dC terms; for the trapezoidal form three floats per (batch, step, head),
// one per (batch, head) and dstate per (batch, head).  Each region starts on a
// 256-byte boundary.  One size serves both forms.
struct SsdBwdWorkspace {
  int64_t nchunks;
  int32_t hpw;
  size_t state, per_bhc, bp, steps, bh;  // elements of one region
  static size_t up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
  size_t bytes() const {
    return 2 * up(2 * state) + 2 * up(4 * per_bhc) + 2 * up(4 * bp) + 3 * up(4 * steps) + up(4 * bh) + up(4 * bp_prev);
  }
  size_t bp_prev;
};

static SsdBwdWorkspace ssd_bwd_layout(const ssd_dims_t *d) {
  SsdBwdWorkspace w;
  w.nchunks = (d->seqlen + 63) / 64;
  w.hpw = d->nheads > 0 ? ssm::ssd_bwd_heads_per_block(d->batch, d->seqlen, d->nheads, d->ngroups) : 1;
  w.per_bhc = static_cast<size_t>(d->batch * d->nheads * w.nchunks);
  w.state = w.per_bhc * static_cast<size_t>(d->headdim * d->dstate);
  w.bp = static_cast<size_t>(d->batch * d->seqlen * (d->nheads / w.hpw) * d->dstate);
  w.steps = static_cast<size_t>(d->batch * d->seqlen * d->nheads);
  w.bh = static_cast<size_t>(d->batch * d->nheads);
  w.bp_prev = w.bh * static_cast<size_t>(d->dstate);
  return w;
}

int ssd_bwd_workspace_size(const ssd_dims_t *dims, size_t *bytes) {
  if (!bytes) return fail(SSM_ERR_NULL, "bytes is NULL");
  const int rc = check_ssd_dims(dims);
  if (rc != SSM_OK) return rc;
  *bytes = ssd_bwd_layout(dims).bytes();
  return ok();
}

// Checks and launch shared by ssd_bwd and ssd_trap_bwd (trap: lam non-null).
static int ssd_bwd_run(const void *x, const void *dt, const void *lam, const float *A, const void *B, const void *C,
                       const float *D, const void *z, const float *h0, const void *x_prev, const void *B_prev,
                       const void *dy, const float *dh_last, void *dx, void *ddt, void *dlam, float *dA, float *dB,
                       float *dC, float *dD, void *dz, float *dh0, void *dx_prev, float *dB_prev,
                       const ssd_dims_t *dims, void *stream, bool trap) {
  int rc = check_ssd_dims(dims);
  if (rc != SSM_OK) return rc;
  const ssd_dims_t &d = *dims;
  if (!trap && (d.flags & SSM_LAM_SIGMOID))
    return fail(SSM_ERR_SHAPE, "SSM_LAM_SIGMOID applies to the trapezoidal form only");
  const int64_t n_x = d.batch * d.seqlen * d.nheads * d.headdim;
  const int64_t n_dt = d.batch * d.seqlen * d.nheads;
  const int64_t n_bc = d.batch * d.seqlen * d.ngroups * d.dstate;
  const int64_t n_h = d.batch * d.nheads * d.headdim * d.dstate;
  const int64_t n_xp = d.batch * d.nheads * d.headdim, n_bp = d.batch * d.ngroups * d.dstate;
  if (n_x > 0 && (!x || !dt || !dy || !dx || !ddt)) return fail(SSM_ERR_NULL, "x, dt, dy, dx and ddt are required");
  if (n_bc > 0 && (!B || !C || !dB || !dC)) return fail(SSM_ERR_NULL, "B, C, dB and dC are required");
  if (d.nheads > 0 && (!A || !dA)) return fail(SSM_ERR_NULL, "A and dA are required");
  if (n_x > 0 && z && !dz) return fail(SSM_ERR_NULL, "dz is required when z is given");
  if (d.nheads > 0 && D && !dD) return fail(SSM_ERR_NULL, "dD is required when D is given");
  if (trap && n_dt > 0 && (!lam || !dlam)) return fail(SSM_ERR_NULL, "lam and dlam are required");
  if ((x_prev == nullptr) != (B_prev == nullptr))
    return fail(SSM_ERR_NULL, "x_prev and B_prev are given together or not at all");
  if (x_prev && n_xp > 0 && (!dx_prev || !dB_prev))
    return fail(SSM_ERR_NULL, "dx_prev and dB_prev are required with x_prev and B_prev");
  if (!z) dz = nullptr;
  if (!D) dD = nullptr;
  if (!x_prev) {
    dx_prev = nullptr;
    dB_prev = nullptr;
  }
  const size_t eo = dtype_size(d.out_dtype);
  if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(z, 16) || !aligned(dy, 16))
    return fail(SSM_ERR_ALIGN, "x, z, B, C and dy must be 16-byte aligned");
  if (!aligned(dt, 2) || !aligned(lam, 2) || !aligned(x_prev, 2) || !aligned(B_prev, 2) || !aligned(dx, 2) ||
      !aligned(ddt, 2) || !aligned(dlam, 2) || !aligned(dz, 2) || !aligned(dx_prev, 2))
    return fail(SSM_ERR_ALIGN, "bf16 pointers must be 2-byte aligned");
  if (!aligned(A, 4) || !aligned(D, 4) || !aligned(dA, 4) || !aligned(dB, 4) || !aligned(dC, 4) || !aligned(dD, 4) ||
      !aligned(dB_prev, 4))
    return fail(SSM_ERR_ALIGN, "A, D, dA, dB, dC, dD and dB_prev must be 4-byte aligned");
  if (!aligned(h0, 16) || !aligned(dh_last, 16) || !aligned(dh0, 16))
    return fail(SSM_ERR_ALIGN, "h0, dh_last and dh0 must be 16-byte aligned");
  const Span ins[] = {{x, n_x * 2ull},       {dt, n_dt * 2ull},    {z, n_x * 2ull},        {B, n_bc * 2ull},
                      {C, n_bc * 2ull},      {A, d.nheads * 4ull}, {D, d.nheads * 4ull},  {h0, n_h * 4ull},
                      {dy, n_x * eo},        {dh_last, n_h * 4ull}, {d.dt_bias, d.nheads * 4ull},
                      {lam, n_dt * 2ull},    {x_prev, n_xp * 2ull}, {B_prev, n_bp * 2ull}};
  const Span outs[] = {{dx, n_x * 2ull},     {ddt, n_dt * 2ull},   {dz, n_x * 2ull},       {dA, d.nheads * 4ull},
                       {dB, n_bc * 4ull},    {dC, n_bc * 4ull},    {dD, d.nheads * 4ull},  {dh0, n_h * 4ull},
                       {dlam, n_dt * 2ull},  {dx_prev, n_xp * 2ull}, {dB_prev, n_bp * 4ull}};
  for (const Span &o : outs) {
    for (const Span &i : ins)
      if (overlap(o, i)) return fail(SSM_ERR_SHAPE, "a gradient output overlaps an input");
    for (const Span &o2 : outs)
      if (&o != &o2 && overlap(o, o2)) return fail(SSM_ERR_SHAPE, "two gradient outputs overlap");
  }
  if (n_bc / 256 >= kMaxGridX || n_dt / 256 >= kMaxGridX)
    return fail(SSM_ERR_UNSUPPORTED, "batch * seqlen * (ngroups * dstate or nheads) exceeds the grid limit");
  const SsdBwdWorkspace wl = ssd_bwd_layout(&d);
  if (d.batch * d.nheads > kMaxGridX / 2 ||
      (d.batch > 0 && wl.nchunks > 0 && d.nheads / wl.hpw > kMaxGridX / d.batch / wl.nchunks))
    return fail(SSM_ERR_UNSUPPORTED, "batch * nheads * chunks exceeds the grid limit");
  const size_t need = wl.bytes();
  if (need > 0) {
    if (!d.workspace || d.workspace_bytes < need)
      return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need,
                  d.workspace ? d.workspace_bytes : (size_t)0);
    if (!aligned(d.workspace, 16)) return fail(SSM_ERR_ALIGN, "workspace must be 16-byte aligned");
    const Span sw{d.workspace, need};
    for (const Span &s : ins)
      if (overlap(s, sw)) return fail(SSM_ERR_SHAPE, "workspace overlaps an input");
    for (const Span &s : outs)
      if (overlap(s, sw)) return fail(SSM_ERR_SHAPE, "workspace overlaps an output");
  }
  if (d.nheads == 0) return ok();
  ssm::SsdBwdParams p{};
  p.x = x;
  p.dt = dt;
  p.B = B;
  p.C = C;
  p.z = z;
  p.dy = dy;
  p.A = A;
  p.D = D;
  p.h0 = h0;
  p.dh_last = dh_last;
  p.dt_bias = d.dt_bias;
  p.dt_softplus = (d.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
  p.lam_sigmoid = (d.flags & SSM_LAM_SIGMOID) ? 1 : 0;
  p.dx = dx;
  p.ddt = ddt;
  p.dz = dz;
  p.dA = dA;
  p.dB = dB;
  p.dC = dC;
  p.dD = dD;
  p.dh0 = dh0;
  p.lam = trap ? lam : nullptr;
  p.x_prev = trap ? x_prev : nullptr;
  p.B_prev = trap ? B_prev : nullptr;
  p.dlam = dlam;
  p.dx_prev = dx_prev;
  p.dB_prev = dB_prev;
  uint8_t *ws = static_cast<uint8_t *>(d.workspace);
  const size_t st = SsdBwdWorkspace::up(2 * wl.state), sc = SsdBwdWorkspace::up(4 * wl.per_bhc);
  const size_t sb = SsdBwdWorkspace::up(4 * wl.bp), ss = SsdBwdWorkspace::up(4 * wl.steps);
  const size_t sh = SsdBwdWorkspace::up(4 * wl.bh);
  p.ws_Sp = reinterpret_cast<uint16_t *>(ws);
  p.ws_dSp = reinterpret_cast<uint16_t *>(ws + st);
  p.ws_dApart = reinterpret_cast<float *>(ws + 2 * st);
  p.ws_dDpart = reinterpret_cast<float *>(ws + 2 * st + sc);
  p.ws_dBp = reinterpret_cast<float *>(ws + 2 * st + 2 * sc);
  p.ws_dCp = reinterpret_cast<float *>(ws + 2 * st + 2 * sc + sb);
  p.ws_dsc = reinterpret_cast<float *>(ws + 2 * st + 2 * sc + 2 * sb);
  p.ws_dga = reinterpret_cast<float *>(ws + 2 * st + 2 * sc + 2 * sb + ss);
  p.ws_rc = reinterpret_cast<float *>(ws + 2 * st + 2 * sc + 2 * sb + 2 * ss);
  p.ws_dw0 = reinterpret_cast<float *>(ws + 2 * st + 2 * sc + 2 * sb + 3 * ss);
  p.ws_dBpp = reinterpret_cast<float *>(ws + 2 * st + 2 * sc + 2 * sb + 3 * ss + sh);
  p.nchunks = wl.nchunks;
  p.hpw = wl.hpw;
  p.batch = d.batch;
  p.seqlen = d.seqlen;
  p.nheads = d.nheads;
  p.ngroups = d.ngroups;
  p.dstate = d.dstate;
  const hipError_t e = ssm::launch_ssd_bwd(p, d.out_dtype == SSM_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "ssd backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ssd_bwd(const void *x, const void *dt, const float *A, const void *B, const void *C, const float *D,
            const void *z, const float *h0, const void *dy, const float *dh_last, void *dx, void *ddt, float *dA,
            float *dB, float *dC, float *dD, void *dz, float *dh0, const ssd_dims_t *dims, void *stream) {
  return ssd_bwd_run(x, dt, nullptr, A, B, C, D, z, h0, nullptr, nullptr, dy, dh_last, dx, ddt, nullptr, dA, dB, dC,
                     dD, dz, dh0, nullptr, nullptr, dims, stream, false);
}

int ssd_trap_bwd(const void *x, const void *dt, const void *lam, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *h0, const void *x_prev, const void *B_prev,
                 const void *dy, const float *dh_last, void *dx, void *ddt, void *dlam, float *dA, float *dB,
                 float *dC, float *dD, void *dz, float *dh0, void *dx_prev, float *dB_prev, const ssd_dims_t *dims,
                 void *stream) {
  return ssd_bwd_run(x, dt, lam, A, B, C, D, z, h0, x_prev, B_prev, dy, dh_last, dx, ddt, dlam, dA, dB, dC, dD, dz,
                     dh0, dx_prev, dB_prev, dims, stream, true);
}

// ---------------------------------------------------------------------------
// Decode steps
// ---------------------------------------------------------------------------

static bool step_dstate_ok(int64_t n) {
  return n == 1 || n == 2 || n == 4 || n == 8 || n == 16 || n == 32 || n == 64 || n == 128 || n == 256;
}

// Shared checks and launch of both decode steps: `chan` channels per batch
// row, A of `n_a` floats, dt of `n_dt` elements, D of `n_d` floats.
static int step_common(const void *u, const void *delta, const float *A, const void *B, const void *C,
                       const float *D, const void *z, float *state, void *y, int64_t batch, int64_t chan,
                       int64_t dstate, int64_t ngroups, int64_t headdim, int64_t n_a, int64_t n_dt,
                       int64_t n_d, int32_t in_dtype, int32_t out_dtype, int per_head, int32_t flags,
                       const float *dt_bias, void *stream, const void *lam = nullptr,
                       const void *x_prev = nullptr, const void *B_prev = nullptr) {
  const int64_t n_x = batch * chan;
  const int64_t n_bc = batch * ngroups * dstate;
  const int64_t n_h = n_x * dstate;
  if (n_x > 0 && (!u || !delta || !y || !state)) return fail(SSM_ERR_NULL, "input, dt, state and y are required");
  if (n_bc > 0 && (!B || !C)) return fail(SSM_ERR_NULL, "B and C are required");
  if (n_a > 0 && !A) return fail(SSM_ERR_NULL, "A is required");
  if ((x_prev == nullptr) != (B_prev == nullptr))
    return fail(SSM_ERR_NULL, "x_prev and B_prev are given together or not at all");
  const size_t ei = dtype_size(in_dtype), eo = dtype_size(out_dtype);
  if (!aligned(u, ei) || !aligned(delta, ei) || !aligned(B, ei) || !aligned(C, ei) || !aligned(z, ei) ||
      !aligned(lam, ei) || !aligned(x_prev, ei) || !aligned(B_prev, ei))
    return fail(SSM_ERR_ALIGN, "input pointers must be aligned to %zu bytes", ei);
  if (!aligned(y, eo)) return fail(SSM_ERR_ALIGN, "y must be aligned to %zu bytes", eo);
  if (!aligned(A, 4) || !aligned(D, 4)) return fail(SSM_ERR_ALIGN, "A and D must be 4-byte aligned");
  if (!aligned(state, dstate >= 4 ? 16 : 4))
    return fail(SSM_ERR_ALIGN, "state must be %d-byte aligned", dstate >= 4 ? 16 : 4);
  const Span ins[] = {{u, n_x * ei},      {delta, n_dt * ei},    {z, n_x * ei},          {B, n_bc * ei},
                      {C, n_bc * ei},      {A, n_a * 4ull},       {D, n_d * 4ull},        {dt_bias, n_d * 4ull},
                      {lam, n_dt * ei},    {x_prev, n_x * ei},    {B_prev, n_bc * ei}};
  const Span sy{y, n_x * eo}, ss{state, n_h * 4ull};
  for (const Span &s : ins)
    if (overlap(s, sy) || overlap(s, ss)) return fail(SSM_ERR_SHAPE, "y or the state overlaps an input");
  if (overlap(sy, ss)) return fail(SSM_ERR_SHAPE, "y overlaps the state");
  const int64_t tpc = dstate < 4 ? 1 : dstate / 4;
  if (n_x > 0 && ceil_div(n_x, 256) > kMaxGridX / tpc)
    return fail(SSM_ERR_UNSUPPORTED, "batch * channels exceeds the grid limit");
  if (n_x == 0) return ok();

  ssm::StepParams p{};
  p.u = u;
  p.delta = delta;
  p.B = B;
  p.C = C;
  p.z = z;
  p.A = A;
  p.D = D;
  p.state = state;
  p.y = y;
  p.dt_bias = dt_bias;
  p.dt_softplus = (flags & SSM_DT_SOFTPLUS) ? 1 : 0;
  p.lam = lam;
  p.x_prev = x_prev;
  p.B_prev = B_prev;
  p.lam_sigmoid = (flags & SSM_LAM_SIGMOID) ? 1 : 0;
  p.batch = batch;
  p.dim = chan;
  p.ngroups = ngroups;
  p.headdim = headdim;
  p.dstate = static_cast<int32_t>(dstate);
  const hipError_t e = ssm::launch_step(p, per_head, in_dtype == SSM_BF16, out_dtype == SSM_BF16,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "step launch failed: %s", hipGetErrorString(e));
  return ok();
}

int ssm_scan_step(const void *u, const void *delta, const float *A, const void *B, const void *C,
                  const float *D, const void *z, float *state, void *y, const ssm_step_dims_t *dims,
                  void *stream) {
  if (!dims) return fail(SSM_ERR_NULL, "dims is NULL");
  const ssm_step_dims_t &d = *dims;
  if (d.batch < 0 || d.dim < 0) return fail(SSM_ERR_SHAPE, "negative size");
  if (d.dstate < 1 || d.ngroups < 1) return fail(SSM_ERR_SHAPE, "dstate and ngroups must be >= 1");
  if (d.dim % d.ngroups != 0) return fail(SSM_ERR_SHAPE, "ngroups must divide dim");
  if (!valid_dtype(d.in_dtype) || !valid_dtype(d.out_dtype)) return fail(SSM_ERR_DTYPE, "bad dtype code");
  if (d.reserved != 0) return fail(SSM_ERR_SHAPE, "reserved must be 0");
  const int rc = check_dt_flags(d.flags, SSM_DT_SOFTPLUS, d.dt_bias);
  if (rc != SSM_OK) return rc;
  if (!step_dstate_ok(d.dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not supported (a power of two up to 256)", (long long)d.dstate);
  return step_common(u, delta, A, B, C, D, z, state, y, d.batch, d.dim, d.dstate, d.ngroups, 1,
                     d.dim * d.dstate, d.batch * d.dim, d.dim, d.in_dtype, d.out_dtype, 0, d.flags, d.dt_bias,
                     stream);
}

// Checks shared by the SSD decode steps; `allowed` are the flag bits the
// step takes.
static int check_ssd_step_dims(const ssd_step_dims_t *dims, int32_t allowed) {
  if (!dims) return fail(SSM_ERR_NULL, "dims is NULL");
  const ssd_step_dims_t &d = *dims;
  if (d.batch < 0 || d.nheads < 0) return fail(SSM_ERR_SHAPE, "negative size");
  if (d.headdim < 1 || d.dstate < 1 || d.ngroups < 1)
    return fail(SSM_ERR_SHAPE, "headdim, dstate and ngroups must be >= 1");
  if (d.nheads % d.ngroups != 0) return fail(SSM_ERR_SHAPE, "ngroups must divide nheads");
  if (!valid_dtype(d.in_dtype) || !valid_dtype(d.out_dtype)) return fail(SSM_ERR_DTYPE, "bad dtype code");
  if (d.reserved != 0) return fail(SSM_ERR_SHAPE, "reserved must be 0");
  const int rc = check_dt_flags(d.flags, allowed, d.dt_bias);
  if (rc != SSM_OK) return rc;
  if (!step_dstate_ok(d.dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not supported (a power of two up to 256)", (long long)d.dstate);
  if (d.nheads > 0 && d.headdim > kMaxGridX / d.nheads) return fail(SSM_ERR_UNSUPPORTED, "too many channels");
  return SSM_OK;
}

int ssd_trap_step(const void *x, const void *dt, const void *lam, const float *A, const void *B, const void *C,
                  const float *D, const void *z, const void *x_prev, const void *B_prev, float *state, void *y,
                  const ssd_step_dims_t *dims, void *stream) {
  const int rc = check_ssd_step_dims(dims, SSM_DT_SOFTPLUS | SSM_LAM_SIGMOID);
  if (rc != SSM_OK) return rc;
  const ssd_step_dims_t &d = *dims;
  if (d.batch * d.nheads > 0 && !lam) return fail(SSM_ERR_NULL, "lam is required");
  return step_common(x, dt, A, B, C, D, z, state, y, d.batch, d.nheads * d.headdim, d.dstate, d.ngroups,
                     d.headdim, d.nheads, d.batch * d.nheads, d.nheads, d.in_dtype, d.out_dtype, 1, d.flags,
                     d.dt_bias, stream, lam, x_prev, B_prev);
}

int ssd_step(const void *x, const void *dt, const float *A, const void *B, const void *C, const float *D,
             const void *z, float *state, void *y, const ssd_step_dims_t *dims, void *stream) {
  if (!dims) return fail(SSM_ERR_NULL, "dims is NULL");
  const ssd_step_dims_t &d = *dims;
  if (d.batch < 0 || d.nheads < 0) return fail(SSM_ERR_SHAPE, "negative size");
  if (d.headdim < 1 || d.dstate < 1 || d.ngroups < 1)
    return fail(SSM_ERR_SHAPE, "headdim, dstate and ngroups must be >= 1");
  if (d.nheads % d.ngroups != 0) return fail(SSM_ERR_SHAPE, "ngroups must divide nheads");
  if (!valid_dtype(d.in_dtype) || !valid_dtype(d.out_dtype)) return fail(SSM_ERR_DTYPE, "bad dtype code");
  if (d.reserved != 0) return fail(SSM_ERR_SHAPE, "reserved must be 0");
  const int rc = check_dt_flags(d.flags, SSM_DT_SOFTPLUS, d.dt_bias);
  if (rc != SSM_OK) return rc;
  if (!step_dstate_ok(d.dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not supported (a power of two up to 256)", (long long)d.dstate);
  if (d.nheads > 0 && d.headdim > kMaxGridX / d.nheads) return fail(SSM_ERR_UNSUPPORTED, "too many channels");
  return step_common(x, dt, A, B, C, D, z, state, y, d.batch, d.nheads * d.headdim, d.dstate, d.ngroups,
                     d.headdim, d.nheads, d.batch * d.nheads, d.nheads, d.in_dtype, d.out_dtype, 1, d.flags,
                     d.dt_bias, stream);
}

// ---------------------------------------------------------------------------
// Rotary step on B and C
// ---------------------------------------------------------------------------

// Checks shared by the rotary step and its backward.
static int check_rope_dims(const ssm_rope_dims_t *dims) {
  if (!dims) return fail(SSM_ERR_NULL, "dims is NULL");
  const ssm_rope_dims_t &d = *dims;
  if (d.batch < 0 || d.seqlen < 0) return fail(SSM_ERR_SHAPE, "negative size");
  if (d.nheads < 1 || d.ngroups < 1) return fail(SSM_ERR_SHAPE, "nheads and ngroups must be >= 1");
  if (d.nheads % d.ngroups != 0) return fail(SSM_ERR_SHAPE, "ngroups must divide nheads");
  if (d.theta_heads != 1 && d.theta_heads != d.nheads) return fail(SSM_ERR_SHAPE, "theta_heads must be 1 or nheads");
  if (!valid_dtype(d.in_dtype) || !valid_dtype(d.out_dtype)) return fail(SSM_ERR_DTYPE, "bad dtype code");
  if (d.reserved != 0) return fail(SSM_ERR_SHAPE, "reserved must be 0");
  const int rc = check_dt_flags(d.flags, SSM_DT_SOFTPLUS, d.dt_bias);
  if (rc != SSM_OK) return rc;
  if (d.dstate < 2 || !step_dstate_ok(d.dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not supported (a power of two from 2 to 256)", (long long)d.dstate);
  if (d.batch > 0 && d.nheads > kMaxGridX / d.batch) return fail(SSM_ERR_UNSUPPORTED, "batch * nheads exceeds the grid limit");
  return SSM_OK;
}

int ssm_rope_bc(const void *dt, const void *theta, const void *B, const void *C, const float *angle0,
                void *B_rot, void *C_rot, float *angle_last, const ssm_rope_dims_t *dims, void *stream) {
  const int rc = check_rope_dims(dims);
  if (rc != SSM_OK) return rc;
  const ssm_rope_dims_t &d = *dims;
  const int64_t rows = d.batch * d.seqlen;
  const int64_t half = d.dstate / 2;
  if (rows > 0 && (!dt || !theta || !B || !C || !B_rot || !C_rot))
    return fail(SSM_ERR_NULL, "dt, theta, B, C, B_rot and C_rot are required");
  const size_t ei = dtype_size(d.in_dtype), eo = dtype_size(d.out_dtype);
  if (!aligned(dt, ei)) return fail(SSM_ERR_ALIGN, "dt must be aligned to %zu bytes", ei);
  if (!aligned(theta, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(B_rot, 16) || !aligned(C_rot, 16))
    return fail(SSM_ERR_ALIGN, "theta, B, C, B_rot and C_rot must be 16-byte aligned");
  if (!aligned(angle0, 4) || !aligned(angle_last, 4)) return fail(SSM_ERR_ALIGN, "angles must be 4-byte aligned");
  const int64_t n_ang = d.batch * d.nheads * half;
  const Span ins[] = {{dt, rows * d.nheads * ei},
                      {theta, rows * d.theta_heads * half * ei},
                      {B, rows * d.ngroups * d.dstate * ei},
                      {C, rows * d.ngroups * d.dstate * ei},
                      {d.dt_bias, d.nheads * 4ull},
                      {angle0, n_ang * 4ull}};
  const Span sb{B_rot, rows * d.nheads * d.dstate * eo}, sc{C_rot, rows * d.nheads * d.dstate * eo};
  const Span sa{angle_last, n_ang * 4ull};
  for (const Span &s : ins) {
    if (overlap(s, sb) || overlap(s, sc)) return fail(SSM_ERR_SHAPE, "B_rot or C_rot overlaps an input");
    if (s.p != angle0 && overlap(s, sa)) return fail(SSM_ERR_SHAPE, "angle_last overlaps an input");
  }
  if (angle_last != nullptr && angle0 != nullptr && angle_last != angle0 && overlap(sa, Span{angle0, n_ang * 4ull}))
    return fail(SSM_ERR_SHAPE, "angle_last overlaps angle0 without being it");
  if (overlap(sb, sc) || overlap(sb, sa) || overlap(sc, sa)) return fail(SSM_ERR_SHAPE, "outputs overlap each other");
  if (d.batch * d.nheads == 0 || (rows == 0 && angle_last == nullptr)) return ok();

  ssm::RopeParams p{};
  p.dt = dt;
  p.theta = theta;
  p.B = B;
  p.C = C;
  p.angle0 = angle0;
  p.dt_bias = d.dt_bias;
  p.B_rot = B_rot;
  p.C_rot = C_rot;
  p.angle_last = angle_last;
  p.dt_softplus = (d.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
  p.dstate = static_cast<int32_t>(d.dstate);
  p.batch = d.batch;
  p.seqlen = d.seqlen;
  p.nheads = d.nheads;
  p.ngroups = d.ngroups;
  p.theta_heads = d.theta_heads;
  const hipError_t e = ssm::launch_rope(p, d.in_dtype == SSM_BF16, d.out_dtype == SSM_BF16,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "rope launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Workspace of the rotary backward: the angle before every tile and the
// tiles' sums of the angle gradient, (batch, nheads, ntile, dstate / 2)
// float32 each, and the parts of ddt when a step's pairs span several
// wavefronts; each rounded up to 256 bytes.
struct RopeBwdTiling {
  ssm::RopeBwdTilingCfg c;
  int64_t ntile;
  size_t one, ddt;  // bytes of one angle array, of the ddt parts
};
static RopeBwdTiling rope_bwd_tiling(const ssm_rope_dims_t &d) {
  RopeBwdTiling t{};
  t.c = ssm::rope_bwd_tiling(d.dstate, d.nheads, d.ngroups);
  t.ntile = (d.seqlen + t.c.tile_len - 1) / t.c.tile_len;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  t.one = up(static_cast<size_t>(d.batch) * d.nheads * t.ntile * (d.dstate / 2) * 4);
  t.ddt = t.c.parts > 1 ? up(static_cast<size_t>(d.batch) * d.seqlen * d.nheads * t.c.parts * 4) : 0;
  return t;
}
static size_t rope_bwd_workspace(const ssm_rope_dims_t &d) {
  const RopeBwdTiling t = rope_bwd_tiling(d);
  return 2 * t.one + t.ddt;
}

int ssm_rope_bc_bwd_workspace_size(const ssm_rope_dims_t *dims, size_t *bytes) {
  if (!bytes) return fail(SSM_ERR_NULL, "bytes is NULL");
  const int rc = check_rope_dims(dims);
  if (rc != SSM_OK) return rc;
  *bytes = rope_bwd_workspace(*dims);
  return ok();
}

int ssm_rope_bc_bwd(const void *dt, const void *theta, const void *B, const void *C, const float *angle0,
                    const void *dB_rot, const void *dC_rot, const float *dangle_last, float *ddt, float *dtheta,
                    float *dB, float *dC, float *dangle0, void *workspace, size_t workspace_bytes,
                    const ssm_rope_dims_t *dims, void *stream) {
  int rc = check_rope_dims(dims);
  if (rc != SSM_OK) return rc;
  const ssm_rope_dims_t &d = *dims;
  const int64_t rows = d.batch * d.seqlen;
  const int64_t half = d.dstate / 2;
  if (rows > 0 && (!dt || !theta || !B || !C || !dB_rot || !dC_rot))
    return fail(SSM_ERR_NULL, "dt, theta, B, C, dB_rot and dC_rot are required");
  if (rows > 0 && (!ddt || !dtheta || !dB || !dC)) return fail(SSM_ERR_NULL, "ddt, dtheta, dB and dC are required");
  const size_t ei = dtype_size(d.in_dtype), eg = dtype_size(d.out_dtype);
  if (!aligned(dt, ei)) return fail(SSM_ERR_ALIGN, "dt must be aligned to %zu bytes", ei);
  if (!aligned(theta, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(dB_rot, 16) || !aligned(dC_rot, 16) ||
      !aligned(dtheta, 16) || !aligned(dB, 16) || !aligned(dC, 16))
    return fail(SSM_ERR_ALIGN, "theta, B, C, dB_rot, dC_rot, dtheta, dB and dC must be 16-byte aligned");
  if (!aligned(ddt, 4) || !aligned(angle0, 4) || !aligned(dangle_last, 4) || !aligned(dangle0, 4))
    return fail(SSM_ERR_ALIGN, "ddt and the angle arrays must be 4-byte aligned");
  const int64_t n_ang = d.batch * d.nheads * half;
  const Span ins[] = {{dt, rows * d.nheads * ei},
                      {theta, rows * d.theta_heads * half * ei},
                      {B, rows * d.ngroups * d.dstate * ei},
                      {C, rows * d.ngroups * d.dstate * ei},
                      {dB_rot, rows * d.nheads * d.dstate * eg},
                      {dC_rot, rows * d.nheads * d.dstate * eg},
                      {d.dt_bias, d.nheads * 4ull},
                      {angle0, n_ang * 4ull},
                      {dangle_last, n_ang * 4ull}};
  const Span outs[] = {{ddt, rows * d.nheads * 4ull},
                       {dtheta, rows * d.theta_heads * half * 4ull},
                       {dB, rows * d.ngroups * d.dstate * 4ull},
                       {dC, rows * d.ngroups * d.dstate * 4ull},
                       {dangle0, n_ang * 4ull}};
  for (const Span &o : outs) {
    for (const Span &i : ins)
      if (overlap(o, i)) return fail(SSM_ERR_SHAPE, "a gradient output overlaps an input");
    for (const Span &o2 : outs)
      if (&o != &o2 && overlap(o, o2)) return fail(SSM_ERR_SHAPE, "two gradient outputs overlap");
  }
  const size_t need = rope_bwd_workspace(d);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(SSM_ERR_ALIGN, "workspace must be 16-byte aligned");
    const Span sw{workspace, need};
    for (const Span &s : ins)
      if (overlap(s, sw)) return fail(SSM_ERR_SHAPE, "workspace overlaps an input");
    for (const Span &s : outs)
      if (overlap(s, sw)) return fail(SSM_ERR_SHAPE, "workspace overlaps an output");
  }
  const RopeBwdTiling tl = rope_bwd_tiling(d);
  if (d.batch * tl.ntile >= kMaxGridX || rows / 4 >= kMaxGridX)
    return fail(SSM_ERR_UNSUPPORTED, "batch * seqlen exceeds the grid limit");
  if (d.batch * d.nheads == 0 || (rows == 0 && dangle0 == nullptr)) return ok();

  ssm::RopeBwdParams p{};
  p.dt = dt;
  p.theta = theta;
  p.B = B;
  p.C = C;
  p.dB_rot = dB_rot;
  p.dC_rot = dC_rot;
  p.angle0 = angle0;
  p.dangle_last = dangle_last;
  p.dt_bias = d.dt_bias;
  p.ddt = ddt;
  p.dtheta = dtheta;
  p.dB = dB;
  p.dC = dC;
  p.dangle0 = dangle0;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  p.ws_ang = reinterpret_cast<float *>(ws);
  p.ws_tot = reinterpret_cast<float *>(ws + tl.one);
  p.ws_ddt = tl.ddt > 0 ? reinterpret_cast<float *>(ws + 2 * tl.one) : nullptr;
  p.tile_len = tl.c.tile_len;
  p.slots = tl.c.slots;
  p.ws_parts = tl.c.parts;
  p.ntile = tl.ntile;
  p.dt_softplus = (d.flags & SSM_DT_SOFTPLUS) ? 1 : 0;
  p.dstate = static_cast<int32_t>(d.dstate);
  p.batch = d.batch;
  p.seqlen = d.seqlen;
  p.nheads = d.nheads;
  p.ngroups = d.ngroups;
  p.theta_heads = d.theta_heads;
  const hipError_t e = ssm::launch_rope_bwd(p, d.in_dtype == SSM_BF16, d.out_dtype == SSM_BF16,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "rope backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
// Diagnostics
// ---------------------------------------------------------------------------

const char *ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_NULL: return "SSM_ERR_NULL";
    case SSM_ERR_SHAPE: return "SSM_ERR_SHAPE";
    case SSM_ERR_DTYPE: return "SSM_ERR_DTYPE";
    case SSM_ERR_ALIGN: return "SSM_ERR_ALIGN";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED";
    case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE";
    case SSM_ERR_HIP: return "SSM_ERR_HIP";
    default: return "SSM_ERR_UNKNOWN";
  }
}

const char *ssm_last_error(void) { return g_last_error.c_str(); }

const char *ssm_last_error_message(void) { return g_last_error.c_str(); }

int ssm_version(void) { return 500; }

}  // extern "C"
