// Activation predictor of one layer: t = p1 x (stage 1), then
// l = p2 t + c and the threshold test l > theta (stage 2).
//
// [QB] "Что такое «разреженная активация»?": a small per-layer model predicts
// which neurons an input activates, before the layer is computed.  The form
// implemented is a low-rank linear pair with a sigmoid threshold; the
// sigmoid is never evaluated: sigmoid(l) > tau holds exactly when
// l > ln(tau / (1 - tau)) = theta, which the host computes once.
//
// Both stages are dense GEMVs at about 1 flop per byte, so they are bound by
// HBM bandwidth: the kernels stream p1 and p2 with 16-byte non-temporal loads
// and keep the small vectors (x, t) in L2 / LDS.  t stays in fp32.
#include "pi_internal.h"

namespace pi {
namespace {

// ---------------------------------------------------------------------------
// Stage 1: t[n][r] = p1[r] . x[n].  One 256-thread workgroup per row of p1;
// the row is split into 16-byte chunks, thread j taking chunks j, j+256, ...
// Sum order: per-thread chunk order, then the wave butterfly, then waves
// 0..3 in order -- fixed, so results are bitwise reproducible.
// ---------------------------------------------------------------------------
template <typename W>
__device__ __forceinline__ float dot_chunk(u32x4 w, u32x4 x, float acc);
template <>
__device__ __forceinline__ float dot_chunk<f16>(u32x4 w, u32x4 x, float acc) { return dot8_f16(w, x, acc); }
template <>
__device__ __forceinline__ float dot_chunk<float>(u32x4 w, u32x4 x, float acc) { return dot4_f32(w, x, acc); }

constexpr int kP1Threads = 256;
constexpr int kP1Chunks = 4;   // chunks per thread per pass
constexpr int kP1Tok = 8;      // tokens per pass over the row

template <typename W>
__global__ __launch_bounds__(kP1Threads) void k_pred1(const W* __restrict__ p1, const W* __restrict__ x,
                                                      int n_tok, int d, int rank, float* __restrict__ t) {
  constexpr int E = 16 / sizeof(W);
  const int row = blockIdx.x;
  const int nch = d / E;
  const char* rowp = reinterpret_cast<const char*>(p1 + (size_t)row * d);
  const char* xb = reinterpret_cast<const char*>(x);
  __shared__ float red[kP1Threads / kWave][kP1Tok];

  for (int t0 = 0; t0 < n_tok; t0 += kP1Tok) {
    const int nt = min(kP1Tok, n_tok - t0);
    float acc[kP1Tok];
#pragma unroll
    for (int j = 0; j < kP1Tok; ++j) acc[j] = 0.f;
    for (int pass = 0; pass < nch; pass += kP1Threads * kP1Chunks) {
      u32x4 w[kP1Chunks];
#pragma unroll
      for (int m = 0; m < kP1Chunks; ++m) {
        const int ch = pass + threadIdx.x + kP1Threads * m;
        w[m] = ch < nch ? ld_nt(rowp + (size_t)ch * 16) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < kP1Tok; ++j) {
        if (j < nt) {
          const char* xr = xb + (size_t)(t0 + j) * d * sizeof(W);
#pragma unroll
          for (int m = 0; m < kP1Chunks; ++m) {
            const int ch = pass + threadIdx.x + kP1Threads * m;
            if (ch < nch) acc[j] = dot_chunk<W>(w[m], ld16(xr + (size_t)ch * 16), acc[j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kP1Tok; ++j) {
      if (j < nt) {
        const float v = wave_sum(acc[j]);
        if (lane_id() == 0) red[wave_id()][j] = v;
      }
    }
    __syncthreads();
    if ((int)threadIdx.x < nt) {
      float s = red[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < kP1Threads / kWave; ++w) s += red[w][threadIdx.x];
      t[(size_t)(t0 + threadIdx.x) * rank + row] = s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Stage 2: l[n][i] = p2[i] . t[n] + c[i]; mask = l > theta.
// Rows of p2 are short (rank elements), so 16 lanes share a row: a wave
// covers 4 rows per step and a 256-thread workgroup 16 rows.  Each lane
// takes chunks g, g+16, ... of its row; the token tile of t sits in LDS.
// Sum order: per-lane chunk order, then a 16-lane butterfly -- fixed.
// ---------------------------------------------------------------------------
constexpr int kP2Threads = 256;
constexpr int kP2Group = 16;                          // lanes per row
constexpr int kP2Rows = kP2Threads / kP2Group;        // rows per workgroup step
constexpr int kP2Chunks = 8;                          // chunks per lane per pass

template <typename W>
__device__ __forceinline__ float dot_chunk_t(u32x4 w, const float* tv, float acc);
template <>
__device__ __forceinline__ float dot_chunk_t<f16>(u32x4 w, const float* tv, float acc) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(tv);
  const f32x4 b = *reinterpret_cast<const f32x4*>(tv + 4);
  const f16x2 h0 = as_h2(w.x), h1 = as_h2(w.y), h2 = as_h2(w.z), h3 = as_h2(w.w);
  acc = __builtin_fmaf((float)h0.x, a.x, acc);
  acc = __builtin_fmaf((float)h0.y, a.y, acc);
  acc = __builtin_fmaf((float)h1.x, a.z, acc);
  acc = __builtin_fmaf((float)h1.y, a.w, acc);
  acc = __builtin_fmaf((float)h2.x, b.x, acc);
  acc = __builtin_fmaf((float)h2.y, b.y, acc);
  acc = __builtin_fmaf((float)h3.x, b.z, acc);
  acc = __builtin_fmaf((float)h3.y, b.w, acc);
  return acc;
}
template <>
__device__ __forceinline__ float dot_chunk_t<float>(u32x4 w, const float* tv, float acc) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(tv);
  acc = __builtin_fmaf(as_f(w.x), a.x, acc);
  acc = __builtin_fmaf(as_f(w.y), a.y, acc);
  acc = __builtin_fmaf(as_f(w.z), a.z, acc);
  acc = __builtin_fmaf(as_f(w.w), a.w, acc);
  return acc;
}

template <typename W, int NT>
__global__ __launch_bounds__(kP2Threads) void k_pred2(const W* __restrict__ p2, const float* __restrict__ c,
                                                      const float* __restrict__ t, int nt, int rank, int d_ff,
                                                      float theta, uint8_t* __restrict__ mask,
                                                      float* __restrict__ logits) {
  constexpr int E = 16 / sizeof(W);
  extern __shared__ float t_lds[];   // [NT][rank]
  // Stage the token tile of t (nt rows of rank floats) into LDS.
  const int tot4 = nt * rank / 4;
  for (int e = threadIdx.x; e < tot4; e += kP2Threads)
    reinterpret_cast<f32x4*>(t_lds)[e] = reinterpret_cast<const f32x4*>(t)[e];
  __syncthreads();

  const int lane = lane_id();
  const int g = lane & (kP2Group - 1);
  const int q = lane / kP2Group;
  const int nch = rank / E;
  const int n_steps = (d_ff + kP2Rows - 1) / kP2Rows;
  for (int step = blockIdx.x; step < n_steps; step += gridDim.x) {
    const int row = step * kP2Rows + wave_id() * (kWave / kP2Group) + q;
    const bool rv = row < d_ff;
    const char* rowp = reinterpret_cast<const char*>(p2 + (size_t)(rv ? row : 0) * rank);
    float acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = 0.f;
    for (int pass = 0; pass < nch; pass += kP2Group * kP2Chunks) {
      u32x4 w[kP2Chunks];
#pragma unroll
      for (int m = 0; m < kP2Chunks; ++m) {
        const int ch = pass + g + kP2Group * m;
        w[m] = (rv && ch < nch) ? ld_nt(rowp + (size_t)ch * 16) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int m = 0; m < kP2Chunks; ++m) {
        const int ch = pass + g + kP2Group * m;
        if (ch < nch) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
            if (j < nt) acc[j] = dot_chunk_t<W>(w[m], t_lds + j * rank + ch * E, acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = group_sum<kP2Group>(acc[j]);
    if (g == 0 && rv) {
      const float cb = c[row];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (j < nt) {
          const float l = acc[j] + cb;
          mask[(size_t)j * d_ff + row] = (l > theta) ? 1 : 0;
          if (logits) logits[(size_t)j * d_ff + row] = l;
        }
      }
    }
  }
}

template <typename W, int NT>
hipError_t launch_pred2_tile(const W* p2, const float* c, const float* t, int nt, int rank, int d_ff,
                             float theta, uint8_t* mask, float* logits, hipStream_t s) {
  const int n_steps = (d_ff + kP2Rows - 1) / kP2Rows;
  const int grid = n_steps < 4096 ? n_steps : 4096;
  const size_t lds = (size_t)NT * rank * sizeof(float);
  hipLaunchKernelGGL((k_pred2<W, NT>), dim3(grid), dim3(kP2Threads), lds, s, p2, c, t, nt, rank, d_ff, theta,
                     mask, logits);
  return hipGetLastError();
}

template <typename W>
hipError_t pred2_all(const W* p2, const float* c, const float* t, int n_tok, int rank, int d_ff, float theta,
                     uint8_t* mask, float* logits, hipStream_t s) {
  // Token tiles share one pass over p2; a tile of t must fit 64 KB of LDS.
  int tile = 8;
  while (tile > 1 && tile * rank > 16384) tile >>= 1;
  for (int t0 = 0; t0 < n_tok; t0 += tile) {
    const int nt = n_tok - t0 < tile ? n_tok - t0 : tile;
    const float* tt = t + (size_t)t0 * rank;
    uint8_t* mt = mask + (size_t)t0 * d_ff;
    float* lt = logits ? logits + (size_t)t0 * d_ff : nullptr;
    hipError_t e;
    if (nt == 1)
      e = launch_pred2_tile<W, 1>(p2, c, tt, nt, rank, d_ff, theta, mt, lt, s);
    else if (nt == 2)
      e = launch_pred2_tile<W, 2>(p2, c, tt, nt, rank, d_ff, theta, mt, lt, s);
    else if (nt <= 4)
      e = launch_pred2_tile<W, 4>(p2, c, tt, nt, rank, d_ff, theta, mt, lt, s);
    else
      e = launch_pred2_tile<W, 8>(p2, c, tt, nt, rank, d_ff, theta, mt, lt, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_predict_stage1(int wtype, const void* p1, const void* x, int n_tok, int d, int rank, float* t,
                                 hipStream_t s) {
  if (wtype == 1)
    hipLaunchKernelGGL((k_pred1<f16>), dim3(rank), dim3(kP1Threads), 0, s, static_cast<const f16*>(p1),
                       static_cast<const f16*>(x), n_tok, d, rank, t);
  else
    hipLaunchKernelGGL((k_pred1<float>), dim3(rank), dim3(kP1Threads), 0, s, static_cast<const float*>(p1),
                       static_cast<const float*>(x), n_tok, d, rank, t);
  return hipGetLastError();
}

hipError_t launch_predict_stage2(int wtype, const void* p2, const float* c, const float* t, int n_tok, int rank,
                                 int d_ff, float theta, uint8_t* mask, float* logits, hipStream_t s) {
  if (wtype == 1)
    return pred2_all<f16>(static_cast<const f16*>(p2), c, t, n_tok, rank, d_ff, theta, mask, logits, s);
  return pred2_all<float>(static_cast<const float*>(p2), c, t, n_tok, rank, d_ff, theta, mask, logits, s);
}

}  // namespace pi
