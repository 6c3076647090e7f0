// Device code shared by the predictor kernels: the per-row logits of the
// second predictor product.  The stand-alone predictor and the fused layer
// kernel both use these functions, so their logits -- and therefore their
// masks -- are bitwise identical.
#pragma once

#include "pi_internal.h"

namespace pi {

constexpr int kP2Group = 16;   // lanes that share one row of p2
constexpr int kP2Chunks = 8;   // 16-byte chunks per lane per pass (128 chunks per row pass)
constexpr int kP2Pass = kP2Group * kP2Chunks;

// t in LDS.  For fp16 weights a 16-byte chunk of a p2 row meets 8 values of
// t; storing them as 8 consecutive floats would put the 16 lanes of a group
// 32 bytes apart (a 4-way LDS bank conflict on every read), so each token's
// t is stored as two arrays of 4-float quads: the first 4 values of every
// chunk, then the last 4 (lane reads then cover 256 contiguous bytes).
// fp32 weights: a chunk meets 4 values; t is stored as it is.
template <typename W>
__device__ __forceinline__ float dot_chunk_t(u32x4 w, const float* t_tok, int ch, int rank, float acc);

template <>
__device__ __forceinline__ float dot_chunk_t<f16>(u32x4 w, const float* t_tok, int ch, int rank, float acc) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(t_tok + ch * 4);
  const f32x4 b = *reinterpret_cast<const f32x4*>(t_tok + rank / 2 + ch * 4);
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
__device__ __forceinline__ float dot_chunk_t<float>(u32x4 w, const float* t_tok, int ch, int, float acc) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(t_tok + ch * 4);
  acc = __builtin_fmaf(as_f(w.x), a.x, acc);
  acc = __builtin_fmaf(as_f(w.y), a.y, acc);
  acc = __builtin_fmaf(as_f(w.z), a.z, acc);
  acc = __builtin_fmaf(as_f(w.w), a.w, acc);
  return acc;
}

// Copy the token tile of t ([nt][rank] fp32) into LDS in the layout above.
// rank % 8 == 0.
template <typename W>
__device__ __forceinline__ void stage_t(const float* __restrict__ t, float* t_lds, int nt, int rank) {
  const int q_tok = rank / 4;                     // 16-byte quads per token
  const int tot4 = nt * q_tok;
  for (int e = threadIdx.x; e < tot4; e += blockDim.x) {
    int dst = e;
    if (sizeof(W) == 2) {
      const int j = e / q_tok, q = e - j * q_tok;   // quad q = chunk q/2, half q%2
      dst = j * q_tok + (q & 1) * (q_tok / 2) + (q >> 1);
    }
    reinterpret_cast<f32x4*>(t_lds)[dst] = reinterpret_cast<const f32x4*>(t)[e];
  }
}

// Logits of S rows per 16-lane group: acc[s][j] = p2[rows[s]] . t[j].
// Lane position g of the group takes chunks g, g+16, ... of each row; sum
// order: the lane's chunks in order, then a 16-lane butterfly -- fixed, so
// every caller gets the same bits for the same row.
//
// Split in three so a caller can put the first pass's loads in flight before
// it stages t (issue_pass for pass 0, then stage, then finish_logits).
template <typename W, int S>
__device__ __forceinline__ void issue_pass(const W* __restrict__ p2, const int (&rows)[S], const bool (&rv)[S],
                                           int rank, int g, int pass, u32x4 (&w)[S][kP2Chunks]) {
  constexpr int E = 16 / sizeof(W);
  const int nch = rank / E;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const char* rowp = reinterpret_cast<const char*>(p2 + (size_t)(rv[s] ? rows[s] : 0) * rank);
#pragma unroll
    for (int m = 0; m < kP2Chunks; ++m) {
      const int ch = pass + g + kP2Group * m;
      w[s][m] = (rv[s] && ch < nch) ? ld_nt(rowp + (size_t)ch * 16) : u32x4{0, 0, 0, 0};
    }
  }
}

template <typename W, int NT, int S>
__device__ __forceinline__ void consume_pass(const u32x4 (&w)[S][kP2Chunks], int rank, const float* t_lds, int nt,
                                             int g, int pass, float (&acc)[S][NT]) {
  constexpr int E = 16 / sizeof(W);
  const int nch = rank / E;
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int m = 0; m < kP2Chunks; ++m) {
      const int ch = pass + g + kP2Group * m;
      if (ch < nch) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
          if (j < nt) acc[s][j] = dot_chunk_t<W>(w[s][m], t_lds + j * rank, ch, rank, acc[s][j]);
      }
    }
  }
}

// Consume the already-issued pass 0, run the remaining passes, reduce.
template <typename W, int NT, int S>
__device__ __forceinline__ void finish_logits(const W* __restrict__ p2, const int (&rows)[S], const bool (&rv)[S],
                                              int rank, const float* t_lds, int nt, int g,
                                              const u32x4 (&w0)[S][kP2Chunks], float (&acc)[S][NT]) {
  constexpr int E = 16 / sizeof(W);
  const int nch = rank / E;
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[s][j] = 0.f;
  consume_pass<W, NT, S>(w0, rank, t_lds, nt, g, 0, acc);
  for (int pass = kP2Pass; pass < nch; pass += kP2Pass) {
    u32x4 w[S][kP2Chunks];
    issue_pass<W, S>(p2, rows, rv, rank, g, pass, w);
    consume_pass<W, NT, S>(w, rank, t_lds, nt, g, pass, acc);
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[s][j] = group_sum<kP2Group>(acc[s][j]);
}

}  // namespace pi
