// Streaming read of a device buffer: the achievable HBM read bandwidth that
// the sparse FFN's gathers and predictor streams are measured against.
//
// kStrBlocks workgroups walk the buffer in a grid-stride loop of 16-byte
// non-temporal loads, kStrUnroll per thread in flight, and fold every word
// into an XOR that each workgroup writes out (so no load can be dropped and
// the result is checkable bit for bit).
#include "pi_internal.h"

namespace pi {
namespace {

constexpr int kStrThreads = 256;
constexpr int kStrUnroll = 8;

__global__ __launch_bounds__(kStrThreads) void k_stream_read(const u32x4* __restrict__ src, size_t n_units,
                                                             uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kStrThreads;
  size_t u = (size_t)blockIdx.x * kStrThreads + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; u + (kStrUnroll - 1) * stride < n_units; u += kStrUnroll * stride) {
    u32x4 v[kStrUnroll];
#pragma unroll
    for (int k = 0; k < kStrUnroll; ++k) v[k] = __builtin_nontemporal_load(src + u + k * stride);
#pragma unroll
    for (int k = 0; k < kStrUnroll; ++k) acc ^= v[k];
  }
  for (; u < n_units; u += stride) acc ^= src[u];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, kWave);
  __shared__ uint32_t red[kStrThreads / kWave];
  if (lane_id() == 0) red[wave_id()] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kStrThreads / kWave; ++w) r ^= red[w];
    out[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(kStrThreads), 0, s, static_cast<const u32x4*>(src), bytes / 16,
                     out);
  return hipGetLastError();
}

}  // namespace pi
