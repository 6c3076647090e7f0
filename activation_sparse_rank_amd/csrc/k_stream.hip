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

// Gathered read of listed rows: wave w of the grid reads rows[w], rows[w +
// waves], ... whole, 16-byte non-temporal loads, kStrUnroll per lane in
// flight (8 KB per wave), and folds every word into the same XOR as
// k_stream_read.  This is the access pattern of the sparse FFN's weight
// gathers without their arithmetic: the ceiling a gather of these rows can
// reach.
__global__ __launch_bounds__(kStrThreads) void k_gather_read(const uint8_t* __restrict__ src, int n_rows,
                                                             int row_bytes, const int32_t* __restrict__ rows,
                                                             const int32_t* __restrict__ count_ptr, int max_count,
                                                             uint32_t* __restrict__ out) {
  int n = *count_ptr;
  n = n < 0 ? 0 : (n < max_count ? n : max_count);
  const int waves = gridDim.x * (kStrThreads / kWave);
  const int units = row_bytes / 16;
  const int lane = lane_id();
  u32x4 acc = {0, 0, 0, 0};
  for (int k = blockIdx.x * (kStrThreads / kWave) + wave_id(); k < n; k += waves) {
    const int r = __builtin_amdgcn_readfirstlane(rows[k]);
    if ((unsigned)r >= (unsigned)n_rows) continue;          // an entry outside the matrix reads nothing
    const u32x4* p = reinterpret_cast<const u32x4*>(src + (size_t)r * row_bytes);
    for (int u0 = lane; u0 < units; u0 += kWave * kStrUnroll) {
      u32x4 v[kStrUnroll];
#pragma unroll
      for (int k2 = 0; k2 < kStrUnroll; ++k2) {
        const int u = u0 + kWave * k2;
        v[k2] = u < units ? __builtin_nontemporal_load(p + u) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int k2 = 0; k2 < kStrUnroll; ++k2) acc ^= v[k2];
    }
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, kWave);
  __shared__ uint32_t red[kStrThreads / kWave];
  if (lane == 0) red[wave_id()] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
#pragma unroll
    for (int w = 0; w < kStrThreads / kWave; ++w) v ^= red[w];
    out[blockIdx.x] = v;
  }
}

}  // namespace

hipError_t launch_gather_read(const void* src, int n_rows, int row_bytes, const int32_t* rows, const int32_t* count,
                              int max_count, uint32_t* out, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(k_gather_read, dim3(blocks), dim3(kStrThreads), 0, s, static_cast<const uint8_t*>(src), n_rows,
                     row_bytes, rows, count, max_count, out);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(kStrThreads), 0, s, static_cast<const u32x4*>(src), bytes / 16,
                     out);
  return hipGetLastError();
}

}  // namespace pi
