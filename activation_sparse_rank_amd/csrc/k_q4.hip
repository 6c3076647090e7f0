// Q4_0 weights: repacking from canonical blocks into the kernels' layout.
//
// [GN] "Lượng tử hóa và tương thích": INT4 Q4_0 is the supported quantized
// format.  A canonical block is 18 bytes (fp16 scale, then 16 bytes of 4-bit
// codes), which is not 16-byte aligned; the kernels want every row's code
// bytes contiguous and 16-byte aligned.  The repacked layout therefore puts
// all code groups first ([rows][cols/32][16] bytes) and all scales after them
// ([rows][cols/32] fp16); the nibble order inside a code group is unchanged.
#include "pi_internal.h"

namespace pi {
namespace {

__global__ __launch_bounds__(256) void k_q4_0_repack(const uint8_t* __restrict__ src, long long n_blocks,
                                                     uint8_t* __restrict__ dst) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= n_blocks) return;
  const uint8_t* s = src + b * 18;
  uint8_t* codes = dst + b * 16;
  uint8_t* scales = dst + n_blocks * 16 + b * 2;
  scales[0] = s[0];
  scales[1] = s[1];
#pragma unroll
  for (int j = 0; j < 16; ++j) codes[j] = s[2 + j];
}

}  // namespace

hipError_t launch_q4_0_repack(const void* src, int rows, int cols, void* dst, hipStream_t s) {
  const long long n_blocks = (long long)rows * (cols / 32);
  if (n_blocks == 0) return hipSuccess;
  const long long grid = (n_blocks + 255) / 256;
  hipLaunchKernelGGL(k_q4_0_repack, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint8_t*>(src),
                     n_blocks, static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

}  // namespace pi
