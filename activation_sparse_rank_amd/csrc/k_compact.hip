// Active-neuron compaction: masks -> ascending int32 list + device count.
//
// [QB] "Гибридный дизайн вывода CPU/GPU": the predictor's output is a set of
// neuron numbers (the worked example names {3, 4, 5}).  This kernel turns the
// per-token masks into that set as an ordered list, taking the union over
// tokens when several share one call.
//
// Two kernels, both without atomics or communication between workgroups:
//   k_compact_tiles -- (16-byte aligned mask rows) one workgroup per tile of
//                      4096 neurons; each counts the marked neurons before its
//                      tile from the masks themselves, so every tile is listed
//                      at once (one round trip to memory);
//   k_compact       -- (any d_ff) one 1024-thread workgroup walks the mask in
//                      tiles of 16 bytes per thread.
// In both, a thread ORs its mask bytes over the tokens and packs them into a
// flag word; a wave-level inclusive scan of the per-thread popcounts (lane
// shuffles) plus an LDS scan of the wave totals gives every thread its output
// offset, so the list comes out in ascending order.  The work is
// latency-bound (32 KB in, ~13 KB out per token at 32768 neurons).
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

// ---------------------------------------------------------------------------
// k_compact_tiles: the same list from one workgroup per tile of kTTile
// neurons, with no communication between workgroups.  Workgroup g counts the
// marked neurons of all tiles before its own by reading their masks itself
// (16-byte loads, OR over the tokens, nonzero bytes counted), all of those
// loads in flight together with its own tile's, so the list takes one
// round trip to memory instead of one per tile.  The redundant reads of the
// earlier tiles (g tiles for workgroup g) hit the cache.  Needs 16-byte
// aligned mask rows (d_ff % 16 == 0); the last workgroup writes the count.
// ---------------------------------------------------------------------------
constexpr int kTThreads = 1024;
constexpr int kTWaves = kTThreads / kWave;
constexpr int kTTile = 4 * kTThreads;          // neurons per workgroup (4 per thread)
constexpr int kTPre = 2;                        // 16-byte prefix groups per thread per round

__device__ __forceinline__ unsigned nz_bytes16(u32x4 v) {
  return nz_bytes4(v.x) | (nz_bytes4(v.y) << 4) | (nz_bytes4(v.z) << 8) | (nz_bytes4(v.w) << 12);
}

template <int kTTok>     // token rows in flight per round
__global__ __launch_bounds__(kTThreads) void k_compact_tiles(const uint8_t* __restrict__ mask, int n_tok, int d_ff,
                                                             int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ int red[kTWaves];
  __shared__ int scan[kTWaves];
  const int lane = lane_id(), wave = wave_id();
  const int g = blockIdx.x;
  const int base = g * kTTile;
  // own tile: neurons base + 4t .. +3 (one 32-bit word per token); earlier
  // tiles: 16-neuron groups e = t, t + kTThreads, ... < base / 16.  kTTok
  // token rows per round, every load of a round in flight together; past the
  // last token the last row is read again (OR is idempotent), and a group or
  // word past the end reads group 0 / the tile's first word and is dropped.
  const int p = base + 4 * (int)threadIdx.x;
  const bool p_ok = p < d_ff;
  const int n_groups = base / 16;
  unsigned own = 0;
  int before = 0;
  for (int e0 = 0; e0 == 0 || e0 < n_groups; e0 += kTThreads * kTPre) {
    u32x4 acc[kTPre];
#pragma unroll
    for (int k = 0; k < kTPre; ++k) acc[k] = u32x4{0, 0, 0, 0};
    for (int t0 = 0; t0 < n_tok; t0 += kTTok) {
      u32x4 v[kTTok][kTPre];
      unsigned w[kTTok];
#pragma unroll
      for (int u = 0; u < kTTok; ++u) {
        const int t = t0 + u < n_tok ? t0 + u : n_tok - 1;
        const uint8_t* row = mask + (size_t)t * d_ff;
#pragma unroll
        for (int k = 0; k < kTPre; ++k) {
          const int e = e0 + k * kTThreads + (int)threadIdx.x;
          v[u][k] = ld16(row + (size_t)(e < n_groups ? e : 0) * 16);
        }
        w[u] = *reinterpret_cast<const unsigned*>(row + (p_ok ? p : base));
      }
#pragma unroll
      for (int u = 0; u < kTTok; ++u) {
#pragma unroll
        for (int k = 0; k < kTPre; ++k) acc[k] |= v[u][k];
        own |= w[u];
      }
    }
#pragma unroll
    for (int k = 0; k < kTPre; ++k)
      if (e0 + k * kTThreads + (int)threadIdx.x < n_groups) before += __builtin_popcount(nz_bytes16(acc[k]));
  }
  if (!p_ok) own = 0;
  const unsigned flags = nz_bytes4(own);
  const int cnt = __builtin_popcount(flags);
  // the marked neurons before this tile: a sum over the workgroup
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) before += __shfl_xor(before, m, kWave);
  // this tile: inclusive scan over the wave, then over the wave totals
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) {
    red[wave] = before;
    scan[wave] = incl;
  }
  __syncthreads();
  int off = 0, tile = 0, pre = 0;
#pragma unroll
  for (int w = 0; w < kTWaves; ++w) {
    pre += red[w];
    off += w < wave ? scan[w] : 0;
    tile += scan[w];
  }
  int o = pre + off + incl - cnt;
  unsigned f = flags;
  while (f) {
    const int b = __builtin_ctz(f);
    idx[o++] = p + b;
    f &= f - 1;
  }
  if (g == (int)gridDim.x - 1 && threadIdx.x == 0) *count = pre + tile;
}

}  // namespace

hipError_t launch_compact(const uint8_t* mask, int n_tok, int d_ff, int32_t* idx, int32_t* count, hipStream_t s) {
  const int vec_ok = ((reinterpret_cast<uintptr_t>(mask) & 15) == 0) && (d_ff % 16 == 0);
  if (vec_ok) {
    const dim3 grid((d_ff + kTTile - 1) / kTTile);
    if (n_tok == 1)
      hipLaunchKernelGGL(k_compact_tiles<1>, grid, dim3(kTThreads), 0, s, mask, n_tok, d_ff, idx, count);
    else
      hipLaunchKernelGGL(k_compact_tiles<8>, grid, dim3(kTThreads), 0, s, mask, n_tok, d_ff, idx, count);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(kCThreads), 0, s, mask, n_tok, d_ff, vec_ok, idx, count);
  return hipGetLastError();
}

}  // namespace pi
