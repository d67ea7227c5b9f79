// gfx950 LDS bank-conflict probe: time per wavefront-wide LDS instruction
// (ds_read / ds_write of 4, 8 or 16 bytes per lane) when lane L of every
// wavefront addresses word L * S of the allocation, for a range of strides S.
// A stride whose accesses fall on distinct banks for every group of lanes the
// LDS serves at once runs at the conflict-free time; a k-way conflict takes
// about k times as long.
//
// In bounds by construction: LDS word indices are masked to the 16384-word
// allocation (64 KiB) after rounding down to the access width, and each thread
// writes out[gid] of a buffer sized to the grid.
#include <hip/hip_runtime.h>
#include <stdio.h>

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWords = 16384;
constexpr int kThreads = 1024;
constexpr int kInner = 16;

template <int W>
struct Vec;
template <>
struct Vec<1> { typedef unsigned T; };
template <>
struct Vec<2> { typedef u32x2 T; };
template <>
struct Vec<4> { typedef u32x4 T; };

__device__ __forceinline__ unsigned sum(unsigned v) { return v; }
__device__ __forceinline__ unsigned sum(u32x2 v) { return v.x + v.y; }
__device__ __forceinline__ unsigned sum(u32x4 v) { return v.x + v.y + v.z + v.w; }

// Each (iteration, wavefront, j) adds a word offset that is a multiple of 256
// words to every lane alike, so the lane-to-bank pattern is that of stride S
// (and the reads cannot be hoisted out of the loop).
template <int W, bool WRITE>
__global__ void __launch_bounds__(kThreads) lds_kernel(unsigned *out, int stride, int iters) {
  extern __shared__ unsigned buf[];
  typedef typename Vec<W>::T T;
  for (int i = threadIdx.x; i < kWords; i += blockDim.x) buf[i] = i;
  __syncthreads();
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int base = (lane * stride) & ~(W - 1);
  unsigned acc = 0;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kInner; ++j) {
      const int w = (base + ((i + wave * kInner + j) * 256)) & (kWords - 1) & ~(W - 1);
      T *p = reinterpret_cast<T *>(buf + w);
      if (WRITE) {
        *p = T(acc + j);
      } else {
        acc += sum(*p);
      }
    }
    if (WRITE) acc += i;
  }
  __syncthreads();
  acc += buf[(threadIdx.x * 7) & (kWords - 1)];
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <int W, bool WRITE>
float run(unsigned *out, int stride, int blocks, int iters) {
  hipEvent_t e0, e1;
  hipEventCreate(&e0);
  hipEventCreate(&e1);
  // 96 KiB of dynamic LDS pins one workgroup (16 wavefronts, four per SIMD) per CU.
  const size_t lds = 96 * 1024;
  hipLaunchKernelGGL((lds_kernel<W, WRITE>), dim3(blocks), dim3(kThreads), lds, 0, out, stride, 4);
  hipEventRecord(e0);
  hipLaunchKernelGGL((lds_kernel<W, WRITE>), dim3(blocks), dim3(kThreads), lds, 0, out, stride, iters);
  hipEventRecord(e1);
  hipEventSynchronize(e1);
  if (hipGetLastError() != hipSuccess) return -1.0f;
  float ms = 0.f;
  hipEventElapsedTime(&ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  // nanoseconds per LDS instruction of one CU (16 wavefronts issue them)
  return ms * 1e6f / (float(kThreads / 64) * iters * kInner);
}

int main() {
  const int blocks = 256, iters = 1024;
  unsigned *out;
  hipMalloc(&out, blocks * kThreads * sizeof(unsigned));
  const void *kernels[] = {(const void *)lds_kernel<1, false>, (const void *)lds_kernel<2, false>,
                           (const void *)lds_kernel<4, false>, (const void *)lds_kernel<1, true>,
                           (const void *)lds_kernel<2, true>,  (const void *)lds_kernel<4, true>};
  for (const void *k : kernels)
    if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024) != hipSuccess) {
      printf("cannot raise the dynamic LDS limit\n");
      return 1;
    }
  const int strides[] = {1, 2, 4, 8, 12, 16, 20, 24, 28, 32, 36, 40, 44, 48, 64, 68, 72, 76, 80, 128, 132, 136};
  printf("stride_words  rd_b32  rd_b64  rd_b128  wr_b32  wr_b64  wr_b128   (ns per wavefront instruction per CU)\n");
  for (int s : strides) {
    printf("%12d  %6.2f  %6.2f  %7.2f  %6.2f  %6.2f  %7.2f\n", s, run<1, false>(out, s, blocks, iters),
           run<2, false>(out, s, blocks, iters), run<4, false>(out, s, blocks, iters),
           run<1, true>(out, s, blocks, iters), run<2, true>(out, s, blocks, iters),
           run<4, true>(out, s, blocks, iters));
  }
  hipFree(out);
  return 0;
}
