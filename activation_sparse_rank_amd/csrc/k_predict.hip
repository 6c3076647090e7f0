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
#include "predict_device.h"

namespace pi {
namespace {

template <typename W>
__device__ __forceinline__ float dot_chunk(u32x4 w, u32x4 x, float acc);
template <>
__device__ __forceinline__ float dot_chunk<f16>(u32x4 w, u32x4 x, float acc) { return dot8_f16(w, x, acc); }
template <>
__device__ __forceinline__ float dot_chunk<float>(u32x4 w, u32x4 x, float acc) { return dot4_f32(w, x, acc); }

// ---------------------------------------------------------------------------
// Stage 1: t[n][r] = p1[r] . x[n].  One 256-thread workgroup per row of p1;
// the row is split into 16-byte chunks, thread j taking chunks j, j+256, ...
// Sum order: per-thread chunk order, then the wave butterfly, then waves
// 0..3 in order -- fixed, so results are bitwise reproducible.
// Block 0 also clears `zero_n` words at `zero_ptr` (counters a later kernel
// of the same call relies on); NULL skips it.
// ---------------------------------------------------------------------------
constexpr int kP1Threads = 256;
constexpr int kP1Chunks = 4;   // chunks per thread per pass
constexpr int kP1Tok = 8;      // tokens per pass over the row

template <typename W>
__global__ __launch_bounds__(kP1Threads) void k_pred1(const W* __restrict__ p1, const W* __restrict__ x,
                                                      int n_tok, int d, int rank, float* __restrict__ t,
                                                      unsigned* __restrict__ zero_ptr, int zero_n) {
  constexpr int E = 16 / sizeof(W);
  if (zero_ptr != nullptr && blockIdx.x == 0)
    for (int e = threadIdx.x; e < zero_n; e += kP1Threads) zero_ptr[e] = 0u;
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
// 16 lanes share a row: a wave covers 4 rows per step and a 256-thread
// workgroup 16 rows; the token tile of t sits in LDS.
// ---------------------------------------------------------------------------
constexpr int kP2Threads = 256;
constexpr int kP2Rows = kP2Threads / kP2Group;   // rows per workgroup step

template <typename W, int NT>
__global__ __launch_bounds__(kP2Threads) void k_pred2(const W* __restrict__ p2, const float* __restrict__ c,
                                                      const float* __restrict__ t, int nt, int rank, int d_ff,
                                                      float theta, uint8_t* __restrict__ mask,
                                                      float* __restrict__ logits) {
  extern __shared__ float t_lds[];   // [NT][rank]
  const int lane = lane_id();
  const int g = lane & (kP2Group - 1);
  const int q = lane / kP2Group;
  const int n_steps = (d_ff + kP2Rows - 1) / kP2Rows;
  int step = blockIdx.x;
  int rows[1] = {step * kP2Rows + wave_id() * (kWave / kP2Group) + q};
  bool rv[1] = {rows[0] < d_ff};
  // The first step's p2 loads go out before t is staged.
  u32x4 w0[1][kP2Chunks];
  issue_pass<W, 1>(p2, rows, rv, rank, g, 0, w0);
  stage_t<W>(t, t_lds, nt, rank);
  __syncthreads();
  while (step < n_steps) {
    float acc[1][NT];
    finish_logits<W, NT, 1>(p2, rows, rv, rank, t_lds, nt, g, w0, acc);
    if (g == 0 && rv[0]) {
      const float cb = c[rows[0]];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (j < nt) {
          const float l = acc[0][j] + cb;
          mask[(size_t)j * d_ff + rows[0]] = (l > theta) ? 1 : 0;
          if (logits) logits[(size_t)j * d_ff + rows[0]] = l;
        }
      }
    }
    step += gridDim.x;
    rows[0] = step * kP2Rows + wave_id() * (kWave / kP2Group) + q;
    rv[0] = step < n_steps && rows[0] < d_ff;
    if (step < n_steps) issue_pass<W, 1>(p2, rows, rv, rank, g, 0, w0);
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
  const int tile = pred_tile(rank);
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

int pred_tile(int rank) {
  // A token tile of t must fit 64 KB of LDS.
  int tile = 8;
  while (tile > 1 && tile * rank > 16384) tile >>= 1;
  return tile;
}

hipError_t launch_predict_stage1(int wtype, const void* p1, const void* x, int n_tok, int d, int rank, float* t,
                                 unsigned* zero_ptr, int zero_n, hipStream_t s) {
  const int grid = rank;
  if (wtype == 1)
    hipLaunchKernelGGL((k_pred1<f16>), dim3(grid), dim3(kP1Threads), 0, s, static_cast<const f16*>(p1),
                       static_cast<const f16*>(x), n_tok, d, rank, t, zero_ptr, zero_n);
  else
    hipLaunchKernelGGL((k_pred1<float>), dim3(grid), dim3(kP1Threads), 0, s, static_cast<const float*>(p1),
                       static_cast<const float*>(x), n_tok, d, rank, t, zero_ptr, zero_n);
  return hipGetLastError();
}

hipError_t launch_predict_stage2(int wtype, const void* p2, const float* c, const float* t, int n_tok, int rank,
                                 int d_ff, float theta, uint8_t* mask, float* logits, hipStream_t s) {
  if (wtype == 1)
    return pred2_all<f16>(static_cast<const f16*>(p2), c, t, n_tok, rank, d_ff, theta, mask, logits, s);
  return pred2_all<float>(static_cast<const float*>(p2), c, t, n_tok, rank, d_ff, theta, mask, logits, s);
}

}  // namespace pi
