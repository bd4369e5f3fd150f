// Measurement probe: dense bf16 MFMA throughput of this device at the clock it
// runs under load, for the "% of measured peak" figure next to the spec peak.
#include "../../include/attn_det.h"

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"

namespace attn {

__device__ unsigned long long g_probe_clk[kMaxGrid][2];

// Each wave keeps four independent 32x32 accumulators busy: back-to-back
// v_mfma_f32_32x32x16_bf16 with no dependency between neighbours.
__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float seed, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = to_bf16(seed * (float)(threadIdx.x + e));
    b[e] = to_bf16(seed * (float)(e - (int)threadIdx.x));
  }
  f32x16 c0 = zero16(), c1 = zero16(), c2 = zero16(), c3 = zero16();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += c0[k] + c1[k] + c2[k] + c3[k];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (s == 1234.5f) sink[threadIdx.x] = s;  // keeps the work alive; never true for the seeds used
  if (threadIdx.x == 0 && blockIdx.x < kMaxGrid) {
    g_probe_clk[blockIdx.x][0] = t0;
    g_probe_clk[blockIdx.x][1] = t1;
  }
}

// fp32 atomic-add throughput in the access pattern of the atomic-dQ variant:
// each instruction adds into 64 consecutive floats (256 bytes), sixteen
// instructions cover a 4 KB block, and every wave walks its own sequence of
// blocks (no two waves on one block at a time).
__global__ void __launch_bounds__(256) atomic_probe_kernel(float* buf, long long n_blocks, int iters) {
  const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long n_waves = (long long)gridDim.x * 4;
  const int lane = threadIdx.x & 63;
  for (int it = 0; it < iters; ++it) {
    const long long blk = (wave + (long long)it * n_waves) % n_blocks;
    float* base = buf + blk * 1024 + lane;
#pragma unroll
    for (int e = 0; e < 16; ++e) atomicAdd(base + 64 * e, 1.0f);
  }
}

}  // namespace attn

using namespace attn;

extern "C" int attn_probe_atomic(void* buffer, size_t bytes, int iterations, void* stream, double* gops) {
  if (!buffer || bytes < 4096 || iterations <= 0 || !gops) return ATTN_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(buffer) & 255u) != 0) return ATTN_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0, num_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return ATTN_ERR_HIP;
  const int grid = num_cu * 8;  // eight 4-wave workgroups per CU
  const long long n_blocks = (long long)(bytes / 4096);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return ATTN_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    hipEventDestroy(e0);
    return ATTN_ERR_HIP;
  }
  int st = ATTN_OK;
  float ms = 0.0f;
  for (int rep = 0; rep < 2 && st == ATTN_OK; ++rep) {  // warm-up launch, then the timed one
    if (rep == 1 && hipEventRecord(e0, s) != hipSuccess) st = ATTN_ERR_HIP;
    hipLaunchKernelGGL(atomic_probe_kernel, dim3(grid), dim3(256), 0, s, static_cast<float*>(buffer), n_blocks,
                       iterations);
    if (hipGetLastError() != hipSuccess) st = ATTN_ERR_HIP;
    if (rep == 1 && st == ATTN_OK && hipEventRecord(e1, s) != hipSuccess) st = ATTN_ERR_HIP;
  }
  if (st == ATTN_OK && hipEventSynchronize(e1) != hipSuccess) st = ATTN_ERR_HIP;
  if (st == ATTN_OK && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) st = ATTN_ERR_HIP;
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (st != ATTN_OK) return st;
  *gops = (double)grid * 4.0 * iterations * 16.0 * 64.0 / (ms * 1e-3) / 1e9;
  return ATTN_OK;
}

extern "C" int attn_probe_mfma(int iterations, void* stream, double* tflops, double* ghz) {
  if (iterations <= 0 || !tflops || !ghz) return ATTN_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0, num_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (hipDeviceGetAttribute(&num_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return ATTN_ERR_HIP;
  const int grid = num_cu < kMaxGrid ? num_cu : kMaxGrid;  // one workgroup (one wave per SIMD) per CU
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return ATTN_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    hipEventDestroy(e0);
    return ATTN_ERR_HIP;
  }
  int st = ATTN_OK;
  float ms = 0.0f;
  // warm-up launch, then the timed one
  for (int rep = 0; rep < 2 && st == ATTN_OK; ++rep) {
    if (rep == 1 && hipEventRecord(e0, s) != hipSuccess) st = ATTN_ERR_HIP;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(256), 0, s, iterations, 1.0f / 4096.0f, nullptr);
    if (hipGetLastError() != hipSuccess) st = ATTN_ERR_HIP;
    if (rep == 1 && st == ATTN_OK && hipEventRecord(e1, s) != hipSuccess) st = ATTN_ERR_HIP;
  }
  if (st == ATTN_OK && hipEventSynchronize(e1) != hipSuccess) st = ATTN_ERR_HIP;
  if (st == ATTN_OK && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) st = ATTN_ERR_HIP;
  unsigned long long clk[kMaxGrid][2];
  if (st == ATTN_OK && hipMemcpyFromSymbol(clk, HIP_SYMBOL(g_probe_clk), sizeof(clk)) != hipSuccess) st = ATTN_ERR_HIP;
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (st != ATTN_OK) return st;
  // 4 waves x 4 MFMAs x iterations per workgroup, 2*32*32*16 flops each
  const double flops = (double)grid * 4.0 * 4.0 * iterations * 32768.0;
  *tflops = flops / (ms * 1e-3) / 1e12;
  double cyc = 0.0;
  for (int g = 0; g < grid; ++g) cyc += (double)(clk[g][1] - clk[g][0]);
  *ghz = cyc / grid / (ms * 1e-3) / 1e9;  // shader-clock counter ticks per second, one workgroup's span
  return ATTN_OK;
}
