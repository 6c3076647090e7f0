// Q4_0 weights: repacking from canonical blocks into the kernels' layout.
//
// [GN] "Lượng tử hóa và tương thích": INT4 Q4_0 is the supported quantized
// format.  A canonical block is 18 bytes: an fp16 scale d, then 16 bytes in
// which byte j holds code j (low nibble) and code j+16 (high nibble); code q
// means the weight d*(q-8).  18-byte blocks are not 16-byte aligned, and their
// nibble order does not line up with pairs of consecutive activations, so the
// kernels read a repacked layout:
//
//   * all code groups first, [rows][cols/32][16] bytes, then all scales,
//     [rows][cols/32] fp16 -- every row's codes are contiguous and 16-byte
//     aligned;
//   * inside a code group, 32-bit word k (k = 0..3) holds the codes of weight
//     pairs p = 4k+u (u = 0..3): code 2p in bits [4u, 4u+4) and code 2p+1 in
//     bits [16+4u, 16+4u+4).  (w >> 4u) & 0x000F000F then holds the two codes
//     of pair p in the two 16-bit halves, ready to become an fp16 pair that
//     multiplies the activation pair (x[2p], x[2p+1]).
#include "pi_internal.h"

namespace pi {
namespace {

__global__ __launch_bounds__(256) void k_q4_0_repack(const uint8_t* __restrict__ src, long long n_blocks,
                                                     uint8_t* __restrict__ dst) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= n_blocks) return;
  const uint8_t* s = src + b * 18;
  unsigned q[32];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const unsigned byte = s[2 + j];
    q[j] = byte & 0xFu;
    q[j + 16] = byte >> 4;
  }
  unsigned* codes = reinterpret_cast<unsigned*>(dst + b * 16);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    unsigned w = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = 4 * k + u;
      w |= q[2 * p] << (4 * u);
      w |= q[2 * p + 1] << (16 + 4 * u);
    }
    codes[k] = w;
  }
  uint8_t* scales = dst + n_blocks * 16 + b * 2;
  scales[0] = s[0];
  scales[1] = s[1];
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
