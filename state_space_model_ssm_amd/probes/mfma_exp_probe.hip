// In-bounds probe of the gfx950 16x16x32 bf16 MFMA lane layout: one wave,
// each lane reads its own 8+8 operand values and writes its 4 results.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <math.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
__global__ void probe(const float *a, const float *b, float *out) {
  int l = threadIdx.x;
  floatx8 fa, fb;
  for (int j = 0; j < 8; ++j) { fa[j] = a[l * 8 + j]; fb[j] = b[l * 8 + j]; }
  bf16x8 A = __builtin_convertvector(fa, bf16x8), B = __builtin_convertvector(fb, bf16x8);
  floatx4 c = {0, 0, 0, 0};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c, 0, 0, 0);
  for (int r = 0; r < 4; ++r) out[l * 4 + r] = c[r];
}
// exp2 accuracy/throughput probe: v_exp_f32 on a grid of arguments.
__global__ void exp_acc(const float *x, float *y, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = __builtin_amdgcn_exp2f(x[i]);
}
__global__ void exp_rate(float *out, int iters, float seed) {
  float v0 = seed + threadIdx.x * 1e-7f, v1 = v0 * 0.5f, v2 = v0 * 0.25f, v3 = v0 * 0.125f;
  float v4 = v0 * 0.3f, v5 = v0 * 0.6f, v6 = v0 * 0.7f, v7 = v0 * 0.9f;
  for (int i = 0; i < iters; ++i) {
    v0 = __builtin_amdgcn_exp2f(v0) - 1.5f; v1 = __builtin_amdgcn_exp2f(v1) - 1.5f;
    v2 = __builtin_amdgcn_exp2f(v2) - 1.5f; v3 = __builtin_amdgcn_exp2f(v3) - 1.5f;
    v4 = __builtin_amdgcn_exp2f(v4) - 1.5f; v5 = __builtin_amdgcn_exp2f(v5) - 1.5f;
    v6 = __builtin_amdgcn_exp2f(v6) - 1.5f; v7 = __builtin_amdgcn_exp2f(v7) - 1.5f;
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = v0 + v1 + v2 + v3 + v4 + v5 + v6 + v7;
}
__global__ void fma_rate(float *out, int iters, float seed) {
  float v0 = seed + threadIdx.x * 1e-7f, v1 = v0 * 0.5f, v2 = v0 * 0.25f, v3 = v0 * 0.125f;
  float v4 = v0 * 0.3f, v5 = v0 * 0.6f, v6 = v0 * 0.7f, v7 = v0 * 0.9f;
  for (int i = 0; i < iters; ++i) {
    v0 = fmaf(v0, 0.999f, 0.001f); v1 = fmaf(v1, 0.999f, 0.001f); v2 = fmaf(v2, 0.999f, 0.001f);
    v3 = fmaf(v3, 0.999f, 0.001f); v4 = fmaf(v4, 0.999f, 0.001f); v5 = fmaf(v5, 0.999f, 0.001f);
    v6 = fmaf(v6, 0.999f, 0.001f); v7 = fmaf(v7, 0.999f, 0.001f);
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = v0 + v1 + v2 + v3 + v4 + v5 + v6 + v7;
}
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)
int main() {
  // ---- MFMA layout ----
  float ha[512], hb[512], ho[256];
  srand(7);
  for (int i = 0; i < 512; ++i) { ha[i] = (float)(rand() % 5 - 2); hb[i] = (float)(rand() % 5 - 2); }
  float *da, *db, *dout;
  CK(hipMalloc(&da, 512 * 4)); CK(hipMalloc(&db, 512 * 4)); CK(hipMalloc(&dout, 256 * 4));
  CK(hipMemcpy(da, ha, 2048, hipMemcpyHostToDevice)); CK(hipMemcpy(db, hb, 2048, hipMemcpyHostToDevice));
  hipLaunchKernelGGL(probe, dim3(1), dim3(64), 0, 0, da, db, dout);
  CK(hipDeviceSynchronize());
  CK(hipMemcpy(ho, dout, 1024, hipMemcpyDeviceToHost));
  // hypothesis: A[i][k]: i=l%16, k=8*(l/16)+j ; B[k][n]: n=l%16, k=8*(l/16)+j ; D[i][n]: i=4*(l/16)+r, n=l%16
  float A[16][32], B[32][16];
  for (int l = 0; l < 64; ++l) for (int j = 0; j < 8; ++j) { A[l % 16][8 * (l / 16) + j] = ha[l * 8 + j]; B[8 * (l / 16) + j][l % 16] = hb[l * 8 + j]; }
  int bad = 0;
  for (int l = 0; l < 64; ++l) for (int r = 0; r < 4; ++r) {
    int i = 4 * (l / 16) + r, n = l % 16; float s = 0;
    for (int k = 0; k < 32; ++k) s += A[i][k] * B[k][n];
    if (s != ho[l * 4 + r]) ++bad;
  }
  printf("MFMA_16x16x32_bf16 layout hypothesis mismatches: %d of 256\n", bad);
  // ---- exp2 accuracy over [-24, 0] ----
  const int n = 1 << 20;
  float *hx = (float *)malloc(n * 4), *hy = (float *)malloc(n * 4);
  for (int i = 0; i < n; ++i) hx[i] = -24.0f * (float)i / n;
  float *dx, *dy; CK(hipMalloc(&dx, n * 4)); CK(hipMalloc(&dy, n * 4));
  CK(hipMemcpy(dx, hx, n * 4, hipMemcpyHostToDevice));
  hipLaunchKernelGGL(exp_acc, dim3(n / 256), dim3(256), 0, 0, dx, dy, n);
  CK(hipDeviceSynchronize());
  CK(hipMemcpy(hy, dy, n * 4, hipMemcpyDeviceToHost));
  double sum_rel = 0, max_rel = 0, sum_ulp = 0, max_ulp = 0;
  for (int i = 0; i < n; ++i) {
    double ref = exp2((double)hx[i]);
    double rel = ((double)hy[i] - ref) / ref;
    double ulp = ((double)hy[i] - ref) / (ldexp(1.0, ilogb((float)ref) - 23));
    sum_rel += rel; if (fabs(rel) > max_rel) max_rel = fabs(rel);
    sum_ulp += ulp; if (fabs(ulp) > max_ulp) max_ulp = fabs(ulp);
  }
  printf("v_exp_f32 over [-24,0]: mean rel err %.3e, max |rel| %.3e, mean ulp %.4f, max |ulp| %.3f\n",
         sum_rel / n, max_rel, sum_ulp / n, max_ulp);
  // ---- rates ----
  float *dr; CK(hipMalloc(&dr, 1024 * 256 * 4 * 8));
  hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  const int iters = 4096, blocks = 1024 * 8;
  for (int rep = 0; rep < 2; ++rep) {
    CK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(exp_rate, dim3(blocks), dim3(256), 0, 0, dr, iters, 0.5f);
    CK(hipEventRecord(e1, 0)); CK(hipEventSynchronize(e1));
    float ms; CK(hipEventElapsedTime(&ms, e0, e1));
    double ops = (double)blocks * 256 * iters * 8;
    if (rep) printf("exp2+add: %.2f ms, %.3f T exp/s (%.3f T lane-instr/s incl. the add)\n", ms, ops / ms / 1e9, 2 * ops / ms / 1e9);
    CK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(fma_rate, dim3(blocks), dim3(256), 0, 0, dr, iters, 0.5f);
    CK(hipEventRecord(e1, 0)); CK(hipEventSynchronize(e1));
    CK(hipEventElapsedTime(&ms, e0, e1));
    if (rep) printf("fma: %.2f ms, %.3f T fma/s\n", ms, ops / ms / 1e9);
  }
  int dev; hipDeviceProp_t prop; CK(hipGetDevice(&dev)); CK(hipGetDeviceProperties(&prop, dev));
  printf("device %s CUs %d clock %d kHz L2 %d\n", prop.gcnArchName, prop.multiProcessorCount, prop.clockRate, prop.l2CacheSize);
  return bad != 0;
}
