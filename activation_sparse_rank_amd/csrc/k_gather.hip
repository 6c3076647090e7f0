// Neuron-aware sparse FFN over a list of active neurons (fp16 / fp32 weights).
//
// [QB] "Что такое «разреженная активация»?": only the activated neurons are
// computed; the others add nothing.  [QB] "Гибридный дизайн вывода CPU/GPU"
// and "Общая архитектура PowerInfer": the partial results of separately
// computed neuron groups are merged into the layer output.  Here the groups
// are chunks of the active list on one GPU and the merge is a fixed-order sum.
//
// Three kernels per token tile:
//   up    -- one wave per listed neuron: its w_up (and w_gate) row is read
//            with 16-byte loads (1 KB per wave instruction), dotted with x,
//            summed across the wave and passed through the activation;
//            h[k] is written in fp32.
//   down  -- a workgroup per (column slice, chunk of the list): each wave
//            walks rows of the chunk and accumulates h[k] * w_down_t[idx[k]]
//            over its slice (one 16-byte load per lane per row); the 8 waves
//            are summed in LDS in wave order and the chunk's partial sums
//            are written to the workspace.
//   merge -- y = sum over chunks of the partials, in chunk order.
// No atomics anywhere, and every sum has a fixed order, so y is bitwise
// reproducible.  All three are bound by HBM bandwidth on the weight rows.
#include "pi_internal.h"

namespace pi {
namespace {

template <typename W>
__device__ __forceinline__ float dotc(u32x4 w, u32x4 x, float acc);
template <>
__device__ __forceinline__ float dotc<f16>(u32x4 w, u32x4 x, float acc) { return dot8_f16(w, x, acc); }
template <>
__device__ __forceinline__ float dotc<float>(u32x4 w, u32x4 x, float acc) { return dot4_f32(w, x, acc); }

// ---------------------------------------------------------------------------
// up: h[j][k] = act(w_up[idx[k]] . x[j] (+ bias)), one wave per listed row.
// ---------------------------------------------------------------------------
constexpr int kUpThreads = 256;
constexpr int kUpWaves = kUpThreads / kWave;
constexpr int kUpChunks = 16;   // 16-byte chunks per lane per pass (16 KB of row per wave)

template <int ACT>
__device__ __forceinline__ float activate(float up, float gate) {
  if (ACT == ACT_REGLU) return (gate > 0.f ? gate : 0.f) * up;
  const float r = up > 0.f ? up : 0.f;
  return ACT == ACT_RELU2 ? r * r : r;
}

template <typename W, int ACT, int NT>
__global__ __launch_bounds__(kUpThreads) void k_up(const W* __restrict__ w_up, const W* __restrict__ w_gate,
                                                   const float* __restrict__ bias, const W* __restrict__ x,
                                                   int d, int d_ff, int nt, const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ count_ptr, int max_count,
                                                   float* __restrict__ h, int ld_h) {
  constexpr int E = 16 / sizeof(W);
  constexpr bool GATED = ACT == ACT_REGLU;
  const int nch = d / E;
  const int lane = lane_id();
  const char* xb = reinterpret_cast<const char*>(x);
  // x tile in LDS when several tokens share a row; one token reads x from L2.
  extern __shared__ u32x4 x_lds[];   // [NT][nch] when NT > 1
  if (NT > 1) {
    const int tot = nt * nch;
    for (int e = threadIdx.x; e < tot; e += kUpThreads) x_lds[e] = ld16(xb + (size_t)e * 16);
    __syncthreads();
  }
  int cnt = *count_ptr;
  cnt = cnt < max_count ? cnt : max_count;
  const int n_waves = gridDim.x * kUpWaves;
  for (int k = blockIdx.x * kUpWaves + wave_id(); k < cnt; k += n_waves) {
    const int i = idx[k];
    if ((unsigned)i >= (unsigned)d_ff) {
      // Outside the weight matrix: the list is malformed; the row adds nothing.
      if (lane == 0)
        for (int j = 0; j < nt; ++j) h[(size_t)j * ld_h + k] = 0.f;
      continue;
    }
    const char* up = reinterpret_cast<const char*>(w_up + (size_t)i * d);
    const char* gt = GATED ? reinterpret_cast<const char*>(w_gate + (size_t)i * d) : nullptr;
    float au[NT], ag[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) au[j] = ag[j] = 0.f;
    for (int pass = 0; pass < nch; pass += kWave * kUpChunks) {
      u32x4 wu[kUpChunks], wg[GATED ? kUpChunks : 1];
#pragma unroll
      for (int m = 0; m < kUpChunks; ++m) {
        const int ch = pass + lane + kWave * m;
        const bool ok = ch < nch;
        wu[m] = ok ? ld_nt(up + (size_t)ch * 16) : u32x4{0, 0, 0, 0};
        if (GATED) wg[m] = ok ? ld_nt(gt + (size_t)ch * 16) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int m = 0; m < kUpChunks; ++m) {
        const int ch = pass + lane + kWave * m;
        if (ch < nch) {
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            if (j < nt) {
              const u32x4 xv = NT > 1 ? x_lds[j * nch + ch] : ld16(xb + (size_t)ch * 16);
              au[j] = dotc<W>(wu[m], xv, au[j]);
              if (GATED) ag[j] = dotc<W>(wg[m], xv, ag[j]);
            }
          }
        }
      }
    }
    const float b = bias ? bias[i] : 0.f;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j < nt) {
        const float u = wave_sum(au[j]);
        const float g = GATED ? wave_sum(ag[j]) : 0.f;
        if (lane == 0) h[(size_t)j * ld_h + k] = GATED ? activate<ACT>(u, g + b) : activate<ACT>(u + b, 0.f);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down: part[c][j][col] = sum_{k in chunk c} h[j][k] * w_down_t[idx[k]][col]
// ---------------------------------------------------------------------------
constexpr int kDnThreads = 512;
constexpr int kDnWaves = kDnThreads / kWave;
constexpr int kDnUnroll = 8;    // rows in flight per wave

template <typename W>
__device__ __forceinline__ void axpy_chunk(float* acc, float hv, u32x4 w);
template <>
__device__ __forceinline__ void axpy_chunk<f16>(float* acc, float hv, u32x4 w) {
  const unsigned wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f16x2 p = as_h2(wd[q]);
    acc[2 * q] = __builtin_fmaf(hv, (float)p.x, acc[2 * q]);
    acc[2 * q + 1] = __builtin_fmaf(hv, (float)p.y, acc[2 * q + 1]);
  }
}
template <>
__device__ __forceinline__ void axpy_chunk<float>(float* acc, float hv, u32x4 w) {
  acc[0] = __builtin_fmaf(hv, as_f(w.x), acc[0]);
  acc[1] = __builtin_fmaf(hv, as_f(w.y), acc[1]);
  acc[2] = __builtin_fmaf(hv, as_f(w.z), acc[2]);
  acc[3] = __builtin_fmaf(hv, as_f(w.w), acc[3]);
}

template <typename W, int NT>
__global__ __launch_bounds__(kDnThreads) void k_down(const W* __restrict__ w_dt, int d, int d_ff,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ count_ptr, int max_count,
                                                     const float* __restrict__ h, int ld_h, int nt,
                                                     int n_chunks, float* __restrict__ part) {
  constexpr int E = 16 / sizeof(W);
  constexpr int SW = kWave * E;               // columns per slice
  extern __shared__ float red[];              // [kDnWaves][NT][SW]
  const int lane = lane_id();
  const int wave = wave_id();
  const int col = blockIdx.x * SW + lane * E;
  const bool cv = col < d;
  const int c = blockIdx.y;
  int cnt = *count_ptr;
  cnt = cnt < max_count ? cnt : max_count;
  const int k0 = (int)(((long long)c * cnt) / n_chunks);
  const int k1 = (int)(((long long)(c + 1) * cnt) / n_chunks);

  float acc[NT][E];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[j][e] = 0.f;

  const char* base = reinterpret_cast<const char*>(w_dt) + (size_t)col * sizeof(W);
  for (int kb = k0 + wave; kb < k1; kb += kDnWaves * kDnUnroll) {
    u32x4 v[kDnUnroll];
    int rows[kDnUnroll];
#pragma unroll
    for (int u = 0; u < kDnUnroll; ++u) {
      const int k = kb + kDnWaves * u;
      const int i = k < k1 ? idx[k] : -1;
      rows[u] = (unsigned)i < (unsigned)d_ff ? i : -1;   // a malformed entry adds nothing
    }
#pragma unroll
    for (int u = 0; u < kDnUnroll; ++u)
      v[u] = (rows[u] >= 0 && cv) ? ld_nt(base + (size_t)rows[u] * d * sizeof(W)) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kDnUnroll; ++u) {
      const int k = kb + kDnWaves * u;
      if (rows[u] >= 0) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
          if (j < nt) axpy_chunk<W>(acc[j], h[(size_t)j * ld_h + k], v[u]);
      }
    }
  }
  // Sum the waves of this workgroup in wave order.
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) red[(wave * NT + j) * SW + lane * E + e] = acc[j][e];
  __syncthreads();
  for (int o = threadIdx.x; o < nt * SW; o += kDnThreads) {
    const int j = o / SW, cc = o % SW;
    const int gcol = blockIdx.x * SW + cc;
    if (gcol < d) {
      float s = red[j * SW + cc];
#pragma unroll
      for (int w = 1; w < kDnWaves; ++w) s += red[(w * NT + j) * SW + cc];
      part[((size_t)c * nt + j) * d + gcol] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// merge: y[j][col] = sum_{c = 0 .. n_chunks-1} part[c][j][col]
// ---------------------------------------------------------------------------
template <typename Y>
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ part, int n_chunks, int n,
                                               Y* __restrict__ y) {
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + e);
  for (int c = 1; c < n_chunks; ++c) s += *reinterpret_cast<const f32x4*>(part + (size_t)c * n + e);
  if constexpr (sizeof(Y) == 4) {
    *reinterpret_cast<f32x4*>(y + e) = s;
  } else {
    y[e] = (f16)s.x;
    y[e + 1] = (f16)s.y;
    y[e + 2] = (f16)s.z;
    y[e + 3] = (f16)s.w;
  }
}

template <typename W, int NT>
hipError_t run_tile(const SparseArgs& a, int t0, int nt, hipStream_t s) {
  constexpr int E = 16 / sizeof(W);
  const int d = a.d;
  const W* x = static_cast<const W*>(a.x) + (size_t)t0 * d;
  const float* bias = a.act == ACT_REGLU ? a.b_gate : a.b_up;
  const int ld_h = a.d_ff;

  // up: about 12 resident waves per CU on 256 CUs, no more than the list
  const int max_waves = 3072;
  int waves = a.max_count < max_waves ? a.max_count : max_waves;
  if (waves < 1) waves = 1;
  const int grid_up = (waves + kUpWaves - 1) / kUpWaves;
  const size_t lds_up = NT > 1 ? (size_t)NT * (d / E) * 16 : 0;
  const W* wu = static_cast<const W*>(a.w_up);
  const W* wg = static_cast<const W*>(a.w_gate);
  if (a.act == ACT_REGLU)
    hipLaunchKernelGGL((k_up<W, ACT_REGLU, NT>), dim3(grid_up), dim3(kUpThreads), lds_up, s, wu, wg, bias, x, d,
                       a.d_ff, nt, a.idx, a.count, a.max_count, a.h, ld_h);
  else if (a.act == ACT_RELU2)
    hipLaunchKernelGGL((k_up<W, ACT_RELU2, NT>), dim3(grid_up), dim3(kUpThreads), lds_up, s, wu, wg, bias, x, d,
                       a.d_ff, nt, a.idx, a.count, a.max_count, a.h, ld_h);
  else
    hipLaunchKernelGGL((k_up<W, ACT_RELU, NT>), dim3(grid_up), dim3(kUpThreads), lds_up, s, wu, wg, bias, x, d,
                       a.d_ff, nt, a.idx, a.count, a.max_count, a.h, ld_h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  constexpr int SW = kWave * E;
  const int slices = (d + SW - 1) / SW;
  const size_t lds_dn = (size_t)kDnWaves * NT * SW * sizeof(float);
  hipLaunchKernelGGL((k_down<W, NT>), dim3(slices, a.n_chunks), dim3(kDnThreads), lds_dn, s,
                     static_cast<const W*>(a.w_down_t), d, a.d_ff, a.idx, a.count, a.max_count, a.h, ld_h, nt,
                     a.n_chunks, a.part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n = nt * d;
  const int grid_m = (n / 4 + 255) / 256;
  if (a.ytype == 1)
    hipLaunchKernelGGL((k_merge<f16>), dim3(grid_m), dim3(256), 0, s, a.part, a.n_chunks, n,
                       static_cast<f16*>(a.y) + (size_t)t0 * d);
  else
    hipLaunchKernelGGL((k_merge<float>), dim3(grid_m), dim3(256), 0, s, a.part, a.n_chunks, n,
                       static_cast<float*>(a.y) + (size_t)t0 * d);
  return hipGetLastError();
}

template <typename W>
hipError_t run_all(const SparseArgs& a, hipStream_t s) {
  const int tile = sparse_tile(a.wtype, a.d);
  for (int t0 = 0; t0 < a.n_tok; t0 += tile) {
    const int nt = a.n_tok - t0 < tile ? a.n_tok - t0 : tile;
    hipError_t e;
    if (nt == 1)
      e = run_tile<W, 1>(a, t0, nt, s);
    else if (nt == 2)
      e = run_tile<W, 2>(a, t0, nt, s);
    else if (nt <= 4)
      e = run_tile<W, 4>(a, t0, nt, s);
    else
      e = run_tile<W, 8>(a, t0, nt, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

int sparse_tile(int wtype, int d) {
  // Tokens per pass: the x tile of the up kernel (tile * d * elem bytes) and
  // the wave-sum buffer of the down kernel (8 * tile * slice * 4 bytes) must
  // each fit in 64 KB of LDS.
  const int eb = wtype == 1 ? 2 : 4;
  const int E = 16 / eb;
  int tile = 8;
  while (tile > 1 && ((size_t)tile * d * eb > 65536 || (size_t)kDnWaves * tile * kWave * E * 4 > 65536)) tile >>= 1;
  return tile;
}

int sparse_chunks(int wtype, int d, int d_ff, int n_tok) {
  (void)d_ff;
  (void)n_tok;
  const int E = wtype == 1 ? 8 : 4;
  const int slices = (d + kWave * E - 1) / (kWave * E);
  // Aim for about 2048 waves (8 per CU) in the down kernel.
  int c = (2048 / kDnWaves + slices - 1) / slices;
  if (c < 1) c = 1;
  if (c > 64) c = 64;
  return c;
}

hipError_t launch_sparse_ffn(const SparseArgs& a, hipStream_t s) {
  if (a.wtype == 1) return run_all<f16>(a, s);
  return run_all<float>(a, s);
}

}  // namespace pi
