// Measurement probes: the ceilings the attention and indexer kernels are measured
// against on the running GPU, as opposed to the data-sheet peaks.
//
//  * mfma_burn_kernel: 8 independent chains of 32x32x16 bf16 MFMAs from registers,
//    four waves per workgroup (one per SIMD when the grid is a multiple of the
//    compute-unit count). Each wave records the shader-clock cycles and the
//    constant-rate wall-clock ticks of its loop, which give the sustained matrix
//    rate and the shader clock it runs at under full matrix load.
//  * stream kernels: a 16-byte-per-lane grid-stride copy (HBM read + write) and a
//    read-only pass with non-temporal loads (each thread folds what it read into one
//    word), over buffers much larger than the last-level cache.
#include "common.h"
#include "kernels.h"

namespace dsa {

__global__ __launch_bounds__(256) void mfma_burn_kernel(long long* __restrict__ cycles, long long* __restrict__ wall,
                                                        float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
  const long long w0 = wall_clock64(), t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32x32x16(a, b, c0);
    c1 = mfma32x32x16(a, b, c1);
    c2 = mfma32x32x16(a, b, c2);
    c3 = mfma32x32x16(a, b, c3);
    c4 = mfma32x32x16(a, b, c4);
    c5 = mfma32x32x16(a, b, c5);
    c6 = mfma32x32x16(a, b, c6);
    c7 = mfma32x32x16(a, b, c7);
  }
  const long long t1 = clock64(), w1 = wall_clock64();
  const f32x16 s = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += s[i];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
  if (lane == 0) {
    cycles[(size_t)blockIdx.x * 4 + wave] = t1 - t0;
    wall[(size_t)blockIdx.x * 4 + wave] = w1 - w0;
  }
}

// n16: 16-byte elements (a multiple of 4). Every thread moves 4 elements per round,
// all four loads issued before the stores.
__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256 * 4;
  for (size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; e < n16; e += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[e + u];
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[e + u] = v[u];
  }
}

// Eight 16-byte loads per thread in flight, non-temporal (streamed past the caches:
// measured the fastest way to read HBM on this chip, 6.7-7.0 TB/s against 6.0-6.3 TB/s
// for ordinary loads).
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ sink,
                                                          size_t n16) {
  constexpr int U = 8;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  uint32_t acc = 0;
  for (size_t c = (size_t)blockIdx.x * 256 * U; c < n16; c += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t e = c + 256 * u + threadIdx.x;
      v[u] = e < n16 ? __builtin_nontemporal_load(src + e) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_mfma_burn(int grid, int iters, long long* cycles, long long* wall, float* sink,
                            hipStream_t stream) {
  KernelTrace kt("probe_mfma_burn", stream);
  hipLaunchKernelGGL(mfma_burn_kernel, dim3(grid), dim3(256), 0, stream, cycles, wall, sink, iters);
  return hipGetLastError();
}

hipError_t launch_stream(int mode, const void* src, void* dst, size_t bytes, int grid, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (mode == 0) {
    KernelTrace kt("probe_stream_copy", stream);
    hipLaunchKernelGGL(stream_copy_kernel, dim3(grid), dim3(256), 0, stream, (const u32x4*)src, (u32x4*)dst, n16);
  } else {
    KernelTrace kt("probe_stream_read", stream);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, stream, (const u32x4*)src, (uint32_t*)dst, n16);
  }
  return hipGetLastError();
}

}  // namespace dsa
