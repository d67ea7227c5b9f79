// VALU issue-rate probes (in-bounds: each thread writes one float of a buffer
// sized blocks*256).
#include <hip/hip_runtime.h>
#include <stdio.h>
template <int K>
__global__ void exp_fma(float *out, int iters, float seed) {
  float v[8], w[8];
  for (int j = 0; j < 8; ++j) { v[j] = seed * (0.1f + 0.1f * j) + threadIdx.x * 1e-7f; w[j] = v[j]; }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = __builtin_amdgcn_exp2f(-v[j]);
#pragma unroll
      for (int k = 0; k < K; ++k) w[j] = fmaf(w[j], 0.999f, v[j]);
    }
  }
  float s = 0; for (int j = 0; j < 8; ++j) s += v[j] + w[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s\n", hipGetErrorString(e)); return 1; } } while (0)
template <int K> int run(float *dr, int blocks, int iters, int threads) {
  hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  float ms = 0;
  for (int rep = 0; rep < 2; ++rep) {
    CK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(exp_fma<K>, dim3(blocks), dim3(threads), 0, 0, dr, iters, 0.5f);
    CK(hipEventRecord(e1, 0)); CK(hipEventSynchronize(e1));
    CK(hipEventElapsedTime(&ms, e0, e1));
  }
  double lanes = (double)blocks * threads * iters * 8;
  printf("exp + %d fma: %.3f ms  exp %.2f T/s  fma %.2f T/s  (slots if exp=4: %.2f T/s)\n", K, ms,
         lanes / ms / 1e9, K * lanes / ms / 1e9, (4 + K) * lanes / ms / 1e9);
  return 0;
}
int main() {
  float *dr; const int blocks = 8192, threads = 256, iters = 2048;
  CK(hipMalloc(&dr, (size_t)blocks * threads * 4));
  run<0>(dr, blocks, iters, threads); run<1>(dr, blocks, iters, threads); run<2>(dr, blocks, iters, threads);
  run<4>(dr, blocks, iters, threads); run<8>(dr, blocks, iters, threads);
  return 0;
}
