// gfx950 issue-rate probes used to set the scan kernel's design and the ALU
// roofline: fp32 FMA and v_exp_f32 rates versus wavefronts per SIMD, and LDS
// ds_read_b128 bandwidth for broadcast and distinct addresses.
//
// Every kernel is in bounds by construction: each thread writes out[gid] of a
// buffer sized to the grid, and LDS indices are masked to the allocation.
#include <hip/hip_runtime.h>
#include <stdio.h>

extern __shared__ float dyn_lds[];

// ILP independent FMA chains; optional exp per iteration.
template <int ILP, bool EXP>
__global__ void valu_kernel(float *out, int iters) {
  if (threadIdx.x == 0) dyn_lds[0] = 0.f;  // touch the LDS that pins one block per CU
  float v[ILP];
#pragma unroll
  for (int j = 0; j < ILP; ++j) v[j] = 0.001f * (threadIdx.x + j);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < ILP; ++j) {
      if (EXP) v[j] = __builtin_amdgcn_exp2f(-v[j]);
      v[j] = fmaf(v[j], 0.999f, 0.0001f);
      v[j] = fmaf(v[j], 0.999f, 0.0001f);
      v[j] = fmaf(v[j], 0.999f, 0.0001f);
      v[j] = fmaf(v[j], 0.999f, 0.0001f);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < ILP; ++j) s += v[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// LDS read bandwidth: each thread reads 16 B per ds_read_b128 from an index
// that is either the same for the whole wavefront (broadcast) or distinct.
// One integer xor per read keeps the VALU out of the way.
template <bool BROADCAST>
__global__ void lds_kernel(float *out, int iters) {
  __shared__ uint4 buf[4096];  // 64 KiB
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  uint32_t acc = 0;
  const int idx = BROADCAST ? (threadIdx.x / 64) * 8 : threadIdx.x;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 t = buf[(idx + j * 256 + i) & 4095];
      acc += t.x + t.y + t.z + t.w;
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)acc;
}


// Throughput of DPP-modified VALU ops: v_mul_f32 with a row_newbcast (or
// row_ror:8) source, against the same loop without DPP.
template <int CTRL, bool USE_DPP>
__global__ void dpp_kernel(float *out, int iters) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = 1.0f + 0.001f * (threadIdx.x + j);
  const float s = 0.9999f + 1e-7f * threadIdx.x;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float src = v[(j + 1) & 7];
      if (USE_DPP)
        src = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, src), CTRL, 0xF, 0xF, false));
      v[j] = src * s;
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc += v[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <int CTRL, bool USE_DPP>
int run_dpp(float *dout, int blocks, int iters, const char *name) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  float ms = 0.f;
  for (int rep = 0; rep < 2; ++rep) {
    (void)hipEventRecord(e0, 0);
    hipLaunchKernelGGL((dpp_kernel<CTRL, USE_DPP>), dim3(blocks), dim3(256), 0, 0, dout, iters);
    if (hipGetLastError() != hipSuccess) return 1;
    (void)hipEventRecord(e1, 0);
    (void)hipEventSynchronize(e1);
    (void)hipEventElapsedTime(&ms, e0, e1);
  }
  const double ops = (double)blocks * 256 * iters * 8;
  printf("%-28s %.3f ms, %.2f T ops/s (%.0f%% of 78.6)\n", name, ms, ops / ms / 1e9, 100.0 * ops / ms / 1e9 / 78.64);
  return 0;
}

#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)

template <int ILP, bool EXP>
int run_valu(float *dout, int threads, int iters, int ncu) {
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  const size_t lds = 96 * 1024;  // > half the CU's LDS: one block per CU
  CK(hipFuncSetAttribute((const void *)valu_kernel<ILP, EXP>, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
  float ms = 0.f;
  for (int rep = 0; rep < 2; ++rep) {
    CK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL((valu_kernel<ILP, EXP>), dim3(ncu), dim3(threads), lds, 0, dout, iters);
    CK(hipGetLastError());
    CK(hipEventRecord(e1, 0)); CK(hipEventSynchronize(e1));
    CK(hipEventElapsedTime(&ms, e0, e1));
  }
  const double lanes = (double)ncu * threads * iters * ILP;
  const double slots = lanes * (4 + (EXP ? 4 : 0));
  printf("valu ILP=%d exp=%d waves/SIMD=%d: %.3f ms, %.2f T slots/s (%.0f%% of 78.6)\n", ILP, EXP, threads / 256,
         ms, slots / ms / 1e9, 100.0 * slots / ms / 1e9 / 78.64);
  return 0;
}

template <bool BC>
int run_lds(float *dout, int blocks, int threads, int iters) {
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  float ms = 0.f;
  for (int rep = 0; rep < 2; ++rep) {
    CK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL((lds_kernel<BC>), dim3(blocks), dim3(threads), 0, 0, dout, iters);
    CK(hipGetLastError());
    CK(hipEventRecord(e1, 0)); CK(hipEventSynchronize(e1));
    CK(hipEventElapsedTime(&ms, e0, e1));
  }
  const double bytes = (double)blocks * threads * iters * 16 * 16;
  printf("lds b128 %s: %.3f ms, %.1f TB/s delivered to lanes (%.0f B/clk/CU)\n", BC ? "broadcast" : "distinct ", ms,
         bytes / ms / 1e9, bytes / (ms * 1e-3) / 256 / 2.4e9);
  return 0;
}

int main() {
  int dev;
  hipDeviceProp_t prop;
  CK(hipGetDevice(&dev));
  CK(hipGetDeviceProperties(&prop, dev));
  const int ncu = prop.multiProcessorCount;
  float *dout;
  CK(hipMalloc(&dout, (size_t)ncu * 1024 * 64 * sizeof(float)));
  const int it = 4096;
  run_valu<8, false>(dout, 256, it, ncu);
  run_valu<8, false>(dout, 512, it, ncu);
  run_valu<8, false>(dout, 1024, it, ncu);
  run_valu<4, false>(dout, 256, it, ncu);
  run_valu<2, false>(dout, 256, it, ncu);
  run_valu<4, true>(dout, 256, it / 2, ncu);
  run_valu<4, true>(dout, 512, it / 2, ncu);
  run_valu<8, true>(dout, 256, it / 2, ncu);
  run_dpp<0x150, false>(dout, ncu * 16, 4096, "v_mul_f32 (no dpp)");
  run_dpp<0x155, true>(dout, ncu * 16, 4096, "v_mul_f32_dpp row_newbcast");
  run_dpp<0x128, true>(dout, ncu * 16, 4096, "v_mul_f32_dpp row_ror:8");
  run_lds<true>(dout, ncu * 8, 256, 1024);
  run_lds<false>(dout, ncu * 8, 256, 1024);
  return 0;
}
