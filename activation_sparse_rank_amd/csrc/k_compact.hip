// Active-neuron compaction: masks -> ascending int32 list + device count.
//
// [QB] "Гибридный дизайн вывода CPU/GPU": the predictor's output is a set of
// neuron numbers (the worked example names {3, 4, 5}).  This kernel turns the
// per-token masks into that set as an ordered list, taking the union over
// tokens when several share one call.
//
// One 1024-thread workgroup (16 waves) walks the mask in tiles of 16 bytes
// per thread.  Per tile: each thread ORs its 16 bytes over the tokens and
// packs them into a 16-bit flag word; a wave-level inclusive scan of the
// per-thread popcounts (lane shuffles) plus an LDS scan of the 16 wave totals
// gives every thread its output offset, so the list comes out in ascending
// order with no atomics.  The work is latency-bound (32 KB in, ~13 KB out at
// 32768 neurons), so one workgroup is the right size.
#include "pi_internal.h"

namespace pi {
namespace {

constexpr int kCThreads = 1024;
constexpr int kCWaves = kCThreads / kWave;
constexpr int kCBytes = 16;    // mask bytes per thread per tile
constexpr int kCTok = 8;       // token rows in flight per thread

// Bit b (b < 4) of the result is set when byte b of v is nonzero.
__device__ __forceinline__ unsigned nz_bytes4(unsigned v) {
  unsigned t = v | (v >> 4);
  t |= t >> 2;
  t |= t >> 1;
  t &= 0x01010101u;               // bit 0 of every nonzero byte
  // Multiplying by 0x204081 moves bits 0, 8, 16, 24 to bits 21..24 with no
  // carries (the shifted copies never overlap).
  return ((t * 0x00204081u) >> 21) & 0xFu;
}

__global__ __launch_bounds__(kCThreads) void k_compact(const uint8_t* __restrict__ mask, int n_tok, int d_ff,
                                                       int vec_ok, int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ count) {
  __shared__ int wave_tot[kCWaves];
  __shared__ int wave_off[kCWaves + 1];
  const int lane = lane_id();
  const int wave = wave_id();
  int base = 0;
  for (int tile = 0; tile < d_ff; tile += kCThreads * kCBytes) {
    const int p = tile + threadIdx.x * kCBytes;
    unsigned flags = 0;
    if (p < d_ff) {
      if (vec_ok && p + kCBytes <= d_ff) {
        // kCTok token rows per round, all loads in flight together; past the
        // last token the last row is read again (OR is idempotent), so the
        // loads carry no condition.
        u32x4 acc = {0, 0, 0, 0};
        if (n_tok == 1) acc = ld16(mask + p);
        else for (int t0 = 0; t0 < n_tok; t0 += kCTok) {
          u32x4 v[kCTok];
#pragma unroll
          for (int u = 0; u < kCTok; ++u) {
            const int t = t0 + u < n_tok ? t0 + u : n_tok - 1;
            v[u] = ld16(mask + (size_t)t * d_ff + p);
          }
#pragma unroll
          for (int u = 0; u < kCTok; ++u) acc |= v[u];
        }
        flags = nz_bytes4(acc.x) | (nz_bytes4(acc.y) << 4) | (nz_bytes4(acc.z) << 8) | (nz_bytes4(acc.w) << 12);
      } else {
        const int nb = d_ff - p < kCBytes ? d_ff - p : kCBytes;
        for (int b = 0; b < nb; ++b) {
          unsigned any = 0;
          for (int t = 0; t < n_tok; ++t) any |= mask[(size_t)t * d_ff + p + b];
          flags |= (any ? 1u : 0u) << b;
        }
      }
    }
    const int cnt = __builtin_popcount(flags);
    // inclusive scan over the wave
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
      int s = 0;
      for (int w = 0; w < kCWaves; ++w) {
        wave_off[w] = s;
        s += wave_tot[w];
      }
      wave_off[kCWaves] = s;
    }
    __syncthreads();
    int off = base + wave_off[wave] + incl - cnt;
    while (flags) {
      const int b = __builtin_ctz(flags);
      idx[off++] = p + b;
      flags &= flags - 1;
    }
    base += wave_off[kCWaves];
    __syncthreads();
  }
  if (threadIdx.x == 0) *count = base;
}

}  // namespace

hipError_t launch_compact(const uint8_t* mask, int n_tok, int d_ff, int32_t* idx, int32_t* count, hipStream_t s) {
  const int vec_ok = ((reinterpret_cast<uintptr_t>(mask) & 15) == 0) && (d_ff % 16 == 0);
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(kCThreads), 0, s, mask, n_tok, d_ff, vec_ok, idx, count);
  return hipGetLastError();
}

}  // namespace pi
