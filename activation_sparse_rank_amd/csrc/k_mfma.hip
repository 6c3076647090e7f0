// Multi-token sparse FFN on the matrix cores (fp16 and Q4_0 weights).
//
// [QB] "Гибридный дизайн вывода CPU/GPU" and [GN] "Cách suy luận lai CPU/GPU":
// the predicted neurons are the only ones computed.  With several tokens the
// list is the union of their predicted sets (pi_compact), and every token
// evaluates every listed neuron with its own activation.  The gathered rows
// then form two dense products over the list U:
//
//   Z[k][t] = W_up[U_k] . x_t   (and W_gate),   H = act(Z)      (up)
//   part[c][t][:] = sum over k in chunk c of H[t][k] * W_down_t[U_k]   (down)
//
// both done with v_mfma_f32_16x16x32_f16 (fp16 operands, fp32 accumulation).
// Lane layout of that instruction on gfx950, for lane l:
//   A (16 x 32):  row l%16, k = 8*(l/16) + 0..7      (one 16-byte operand)
//   B (32 x 16):  k = 8*(l/16) + 0..7, column l%16
//   D (16 x 16):  rows 4*(l/16) + 0..3, column l%16
//
// k_mup   -- a workgroup owns 64 list positions and all tokens of the tile;
//            its 4 waves split d into quarters.  Rows of W_up are contiguous
//            in k, so lane l loads 64 contiguous bytes (32 k values) of its
//            row and the same 32 k values of x for its token; the four MFMAs
//            of a 128-wide k step each take 8 of them (the same k
//            permutation on both operands leaves the dot product unchanged).
//            The 4 waves' accumulators are added in LDS in wave order, the
//            bias and activation applied, and H stored in fp16 by list
//            position (zeros past the count).
// k_mdown -- a workgroup owns a column tile and a chunk of the list; its 4
//            waves split the chunk.  A row of W_down_t is contiguous in the
//            output column, not in k, so each lane loads 8 rows x 8 columns
//            (16 bytes per row) and transposes the 8x8 fp16 block in
//            registers into 8 B operands (one per column).  The 4 waves'
//            sums are added in LDS in a fixed order and the chunk's partial
//            sums written; k_merge adds the chunks in order.
//
// Q4_0 weights are dequantized in registers to fp16: w = fp16(d * (q - 8))
// (one rounding; q - 8 is exact in fp16).  H is rounded to fp16 once.
// Every sum has a fixed order, so y is bitwise reproducible.
#include <type_traits>

#include "pi_internal.h"

namespace pi {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                 0);
}

template <int ACT>
__device__ __forceinline__ float act_fn(float up, float gate) {
  if (ACT == ACT_REGLU) return (gate > 0.f ? gate : 0.f) * up;
  const float r = up > 0.f ? up : 0.f;
  return ACT == ACT_RELU2 ? r * r : r;
}

// Word k of a repacked Q4_0 code group holds the weight pairs (8k+2u,
// 8k+2u+1), u = 0..3, as 4-bit fields at bits 4u and 16+4u.  Returns the 8
// weights 8k .. 8k+7 in order as fp16: (1024 + q) - 1032 = q - 8 exactly,
// then one rounding multiply by the block scale.
__device__ __forceinline__ u32x4 q4_dequant8(unsigned w, f16x2 sc) {
  unsigned r[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const unsigned bits = ((w >> (4 * u)) & 0x000F000Fu) | 0x64006400u;
    const f16x2 v = (as_h2(bits) - f16x2{(f16)1032.0f, (f16)1032.0f}) * sc;
    r[u] = __builtin_bit_cast(unsigned, v);
  }
  return u32x4{r[0], r[1], r[2], r[3]};
}

__device__ __forceinline__ unsigned dw(u32x4 v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// in[r] holds 8 fp16 values of row r; out[j] gets column j (rows 0..7 in order).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    unsigned o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const unsigned lo = dw(in[2 * m], j / 2), hi = dw(in[2 * m + 1], j / 2);
      o[m] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    out[j] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

__device__ __forceinline__ int clamp_count(const int32_t* count_ptr, int max_count) {
  const int c = *count_ptr;
  return c < 0 ? 0 : (c < max_count ? c : max_count);
}

// ---------------------------------------------------------------------------
// k_mup
// ---------------------------------------------------------------------------
constexpr int kMuThreads = 256;
constexpr int kMuWaves = kMuThreads / kWave;
constexpr int kMuMB = 4;                   // 16-row blocks per wave (all waves share the rows)
constexpr int kMuRows = 16 * kMuMB;        // list positions per workgroup
constexpr int kMuK = 128;                  // k per step: 4 lane groups x 32

// The 4 A operands (k = k0 + 8s .. +8, s = 0..3) of one row for this lane.
template <typename WF>
__device__ __forceinline__ void load_row_k32(const void* w, size_t scale_off, int row, bool ok, int d, int k0,
                                             u32x4 (&a)[4]) {
  if constexpr (std::is_same<WF, Q4>::value) {
    const int nbk = d / 32;
    const size_t blk = (size_t)row * nbk + k0 / 32;
    const u32x4 code = ok ? ld_nt(static_cast<const uint8_t*>(w) + blk * 16) : u32x4{0, 0, 0, 0};
    const f16 sc = ok ? reinterpret_cast<const f16*>(static_cast<const uint8_t*>(w) + scale_off)[blk] : (f16)0.0f;
    const f16x2 s2{sc, sc};
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = q4_dequant8(dw(code, s), s2);
  } else {
    const char* p = static_cast<const char*>(w) + ((size_t)row * d + k0) * sizeof(f16);
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = ok ? ld_nt(p + 16 * s) : u32x4{0, 0, 0, 0};
  }
}

template <typename WF, int ACT, int NB>
__global__ __launch_bounds__(kMuThreads) void k_mup(const void* __restrict__ w_up, const void* __restrict__ w_gate,
                                                    size_t scale_off, const float* __restrict__ bias,
                                                    const f16* __restrict__ x, int d, int d_ff, int nt,
                                                    const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ count_ptr, int max_count,
                                                    f16* __restrict__ h, int ldh) {
  constexpr bool GATED = ACT == ACT_REGLU;
  constexpr int NQ = kMuMB * NB;           // accumulator quads per lane
  __shared__ float red[kMuWaves][NQ][4][kWave];
  const int lane = lane_id();
  const int wave = wave_id();
  const int g = lane >> 4, n16 = lane & 15;
  const int cnt = clamp_count(count_ptr, max_count);
  const int r0 = blockIdx.x * kMuRows;
  if (r0 >= cnt) return;                   // the whole workgroup leaves together

  int row[kMuMB];
  bool rv[kMuMB];
#pragma unroll
  for (int mb = 0; mb < kMuMB; ++mb) {
    const int p = r0 + mb * 16 + n16;
    const int i = p < cnt ? idx[p] : -1;
    rv[mb] = (unsigned)i < (unsigned)d_ff;
    row[mb] = rv[mb] ? i : 0;
  }

  f32x4 au[kMuMB][NB], ag[GATED ? kMuMB : 1][NB];
#pragma unroll
  for (int mb = 0; mb < kMuMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      au[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (GATED) ag[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int ns = d / kMuK;
  const int s0 = wave * ns / kMuWaves, s1 = (wave + 1) * ns / kMuWaves;
  for (int st = s0; st < s1; ++st) {
    const int k0 = st * kMuK + g * 32;
    u32x4 a[kMuMB][4], ga[GATED ? kMuMB : 1][4], b[NB][4];
#pragma unroll
    for (int mb = 0; mb < kMuMB; ++mb) {
      load_row_k32<WF>(w_up, scale_off, row[mb], rv[mb], d, k0, a[mb]);
      if (GATED) load_row_k32<WF>(w_gate, scale_off, row[mb], rv[mb], d, k0, ga[mb]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = nb * 16 + n16;
      const char* xp = reinterpret_cast<const char*>(x + (size_t)t * d + k0);
#pragma unroll
      for (int s = 0; s < 4; ++s) b[nb][s] = t < nt ? ld16(xp + 16 * s) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mb = 0; mb < kMuMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          au[mb][nb] = mfma(a[mb][s], b[nb][s], au[mb][nb]);
          if (GATED) ag[mb][nb] = mfma(ga[mb][s], b[nb][s], ag[mb][nb]);
        }
  }

  // Sum the 4 waves in wave order.  Thread T owns lane position T%64 and the
  // quads q = T/64 + 4*e (e < NB): rows 4*((T%64)/16)+i of block q/NB, token
  // (q%NB)*16 + T%16.
  const int ol = threadIdx.x & (kWave - 1);
  const int oq = threadIdx.x >> 6;
  float su[NB][4], sg[NB][4];
  auto reduce = [&](f32x4 (&acc)[kMuMB][NB], float (&out)[NB][4]) {
#pragma unroll
    for (int mb = 0; mb < kMuMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][mb * NB + nb][i][lane] = acc[mb][nb][i];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NB; ++e) {
      const int q = oq + kMuWaves * e;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = red[0][q][i][ol];
#pragma unroll
        for (int w = 1; w < kMuWaves; ++w) v += red[w][q][i][ol];
        out[e][i] = v;
      }
    }
    __syncthreads();
  };
  if constexpr (GATED) reduce(ag, sg);
  reduce(au, su);

#pragma unroll
  for (int e = 0; e < NB; ++e) {
    const int q = oq + kMuWaves * e;
    const int mb = q / NB, nb = q % NB;
    const int t = nb * 16 + (ol & 15);
    const int p = r0 + mb * 16 + 4 * (ol >> 4);
    if (t < nt) {
      f16 hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = 0.f;
        if (p + i < cnt) {
          const int neuron = idx[p + i];
          if ((unsigned)neuron < (unsigned)d_ff) {
            const float b = bias ? bias[neuron] : 0.f;
            v = GATED ? act_fn<ACT>(su[e][i], sg[e][i] + b) : act_fn<ACT>(su[e][i] + b, 0.f);
          }
        }
        hv[i] = (f16)v;
      }
      u32x2 packed;
      packed.x = __builtin_bit_cast(unsigned, f16x2{hv[0], hv[1]});
      packed.y = __builtin_bit_cast(unsigned, f16x2{hv[2], hv[3]});
      *reinterpret_cast<u32x2*>(h + (size_t)t * ldh + p) = packed;
    }
  }
}

// ---------------------------------------------------------------------------
// k_mdown
// ---------------------------------------------------------------------------
constexpr int kMdThreads = 256;
constexpr int kMdWaves = kMdThreads / kWave;

// Rows r = 0..7 of this lane, 8 columns starting at col, as fp16.
template <typename WF, int CPL>
struct DownRows;

template <int CPL>
struct DownRows<f16, CPL> {
  u32x4 v[8][CPL / 8];
  __device__ __forceinline__ void load(const void* w, size_t, int d, const int (&rows)[8], const bool (&ok)[8],
                                       int col) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const char* p = static_cast<const char*>(w) + ((size_t)rows[r] * d + col) * sizeof(f16);
#pragma unroll
      for (int q = 0; q < CPL / 8; ++q) v[r][q] = ok[r] ? ld_nt(p + 16 * q) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void group(int q, u32x4 (&out)[8]) const {
#pragma unroll
    for (int r = 0; r < 8; ++r) out[r] = v[r][q];
  }
};

template <int CPL>
struct DownRows<Q4, CPL> {
  // CPL columns = CPL/2 bytes of codes of one block (CPL <= 32), one scale.
  unsigned c[8][CPL / 8];
  f16 sc[8];
  __device__ __forceinline__ void load(const void* w, size_t scale_off, int d, const int (&rows)[8],
                                       const bool (&ok)[8], int col) {
    const int nbk = d / 32;
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    const f16* scales = reinterpret_cast<const f16*>(wb + scale_off);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const size_t blk = (size_t)rows[r] * nbk + col / 32;
      const uint8_t* p = wb + blk * 16 + (col % 32) / 2;
      if constexpr (CPL == 32) {
        const u32x4 t = ok[r] ? ld_nt(p) : u32x4{0, 0, 0, 0};
        c[r][0] = t.x; c[r][1] = t.y; c[r][2] = t.z; c[r][3] = t.w;
      } else if constexpr (CPL == 16) {
        const u32x2 t = ok[r] ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)) : u32x2{0, 0};
        c[r][0] = t.x; c[r][1] = t.y;
      } else {
        c[r][0] = ok[r] ? __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p)) : 0u;
      }
      sc[r] = ok[r] ? scales[blk] : (f16)0.0f;
    }
  }
  __device__ __forceinline__ void group(int q, u32x4 (&out)[8]) const {
#pragma unroll
    for (int r = 0; r < 8; ++r) out[r] = q4_dequant8(c[r][q], f16x2{sc[r], sc[r]});
  }
};

template <typename WF, int NB, int CPL>
__global__ __launch_bounds__(kMdThreads) void k_mdown(const void* __restrict__ w_dt, size_t scale_off, int d,
                                                      int d_ff, const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ count_ptr, int max_count,
                                                      const f16* __restrict__ h, int ldh, int nt, int n_chunks,
                                                      float* __restrict__ part) {
  constexpr int NE = CPL * NB;             // accumulator quads per lane
  __shared__ float red[NE][4][kWave];
  const int lane = lane_id();
  const int wave = wave_id();
  const int g = lane >> 4, n16 = lane & 15;
  const int cnt = clamp_count(count_ptr, max_count);
  const int ksteps = (cnt + 31) / 32;
  const int c = blockIdx.y;
  const int kc0 = (int)((long long)c * ksteps / n_chunks), kc1 = (int)((long long)(c + 1) * ksteps / n_chunks);
  const int kw0 = kc0 + wave * (kc1 - kc0) / kMdWaves, kw1 = kc0 + (wave + 1) * (kc1 - kc0) / kMdWaves;
  const int col = blockIdx.x * 16 * CPL + n16 * CPL;
  const bool cv = col < d;

  f32x4 acc[CPL][NB];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kk = kw0; kk < kw1; ++kk) {
    const int p0 = kk * 32 + g * 8;
    int rows[8];
    bool ok[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = p0 + r < cnt ? idx[p0 + r] : -1;
      ok[r] = cv && (unsigned)i < (unsigned)d_ff;
      rows[r] = ok[r] ? i : 0;
    }
    DownRows<WF, CPL> wr;
    wr.load(w_dt, scale_off, d, rows, ok, col);
    u32x4 a[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) a[nb] = ld16(h + (size_t)(nb * 16 + n16) * ldh + p0);
#pragma unroll
    for (int q = 0; q < CPL / 8; ++q) {
      u32x4 rw[8], bt[8];
      wr.group(q, rw);
      transpose8x8(rw, bt);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[8 * q + j][nb] = mfma(a[nb], bt[j], acc[8 * q + j][nb]);
    }
  }

  // ((w3 + w2) + w1) + w0 through one LDS buffer, then wave 0 writes.
  for (int w = kMdWaves - 1; w >= 1; --w) {
    if (wave == w) {
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = acc[j][nb][i];
            if (w < kMdWaves - 1) v = red[j * NB + nb][i][lane] + v;
            red[j * NB + nb][i][lane] = v;
          }
    }
    __syncthreads();
  }
  if (wave == 0 && cv) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = nb * 16 + 4 * g + i;
        if (t < nt) {
          float* dst = part + ((size_t)c * nt + t) * d + col;
#pragma unroll
          for (int j = 0; j < CPL; j += 4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = red[(j + e) * NB + nb][i][lane] + acc[j + e][nb][i];
            *reinterpret_cast<f32x4*>(dst + j) = v;
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int kMfmaTile = 64;              // tokens per pass

template <typename WF>
constexpr int down_cpl(int nb) {
  return std::is_same<WF, Q4>::value ? (nb == 1 ? 32 : (nb == 2 ? 16 : 8)) : 8;
}

int mfma_chunks(int wtype) { return wtype == 2 ? 16 : 8; }

int ldh_of(int d_ff) { return (d_ff + kMuRows - 1) / kMuRows * kMuRows; }

template <typename WF, int ACT, int NB>
hipError_t launch_mup(const SparseArgs& a, const f16* x, int nt, f16* h, int ldh, hipStream_t s) {
  const int grid = (a.max_count + kMuRows - 1) / kMuRows;
  if (grid == 0) return hipSuccess;
  const float* bias = ACT == ACT_REGLU ? a.b_gate : a.b_up;
  const size_t so = std::is_same<WF, Q4>::value ? (size_t)a.d_ff * (a.d / 32) * 16 : 0;
  hipLaunchKernelGGL((k_mup<WF, ACT, NB>), dim3(grid), dim3(kMuThreads), 0, s, a.w_up, a.w_gate, so, bias, x, a.d,
                     a.d_ff, nt, a.idx, a.count, a.max_count, h, ldh);
  return hipGetLastError();
}

template <typename WF, int NB>
hipError_t run_mtile(const SparseArgs& a, int t0, int nt, hipStream_t s) {
  const f16* x = static_cast<const f16*>(a.x) + (size_t)t0 * a.d;
  f16* h = reinterpret_cast<f16*>(a.h);
  const int ldh = ldh_of(a.d_ff);
  hipError_t e;
  if (a.act == ACT_REGLU)
    e = launch_mup<WF, ACT_REGLU, NB>(a, x, nt, h, ldh, s);
  else if (a.act == ACT_RELU2)
    e = launch_mup<WF, ACT_RELU2, NB>(a, x, nt, h, ldh, s);
  else
    e = launch_mup<WF, ACT_RELU, NB>(a, x, nt, h, ldh, s);
  if (e != hipSuccess) return e;
  constexpr int CPL = down_cpl<WF>(NB);
  const int chunks = mfma_chunks(a.wtype);
  const size_t so = std::is_same<WF, Q4>::value ? (size_t)a.d_ff * (a.d / 32) * 16 : 0;
  const dim3 grid((a.d + 16 * CPL - 1) / (16 * CPL), chunks);
  hipLaunchKernelGGL((k_mdown<WF, NB, CPL>), grid, dim3(kMdThreads), 0, s, a.w_down_t, so, a.d, a.d_ff, a.idx,
                     a.count, a.max_count, h, ldh, nt, chunks, a.part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t yoff = (size_t)t0 * a.d * (a.ytype == 1 ? 2 : 4);
  return launch_merge(a.part, chunks, nt * a.d, static_cast<char*>(a.y) + yoff, a.ytype, s);
}

template <typename WF>
hipError_t run_mall(const SparseArgs& a, hipStream_t s) {
  for (int t0 = 0; t0 < a.n_tok; t0 += kMfmaTile) {
    const int nt = a.n_tok - t0 < kMfmaTile ? a.n_tok - t0 : kMfmaTile;
    hipError_t e;
    if (nt <= 16)
      e = run_mtile<WF, 1>(a, t0, nt, s);
    else if (nt <= 32)
      e = run_mtile<WF, 2>(a, t0, nt, s);
    else if (nt <= 48)
      e = run_mtile<WF, 3>(a, t0, nt, s);
    else
      e = run_mtile<WF, 4>(a, t0, nt, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool mfma_path(int wtype, int d, int n_tok) {
  if (wtype != 1 && wtype != 2) return false;     // fp16 and Q4_0 weights
  if (d % kMuK != 0) return false;
  return n_tok > sparse_tile(wtype, d);
}

void mfma_workspace(int wtype, int d, int d_ff, int n_tok, size_t* h_bytes, size_t* part_bytes) {
  const int nt = n_tok < kMfmaTile ? n_tok : kMfmaTile;
  const int nb = (nt + 15) / 16;
  *h_bytes = (size_t)16 * nb * ldh_of(d_ff) * sizeof(f16);
  *part_bytes = (size_t)mfma_chunks(wtype) * nt * d * sizeof(float);
}

hipError_t launch_sparse_ffn_mfma(const SparseArgs& a, hipStream_t s) {
  if (a.wtype == 2) return run_mall<Q4>(a, s);
  return run_mall<f16>(a, s);
}

}  // namespace pi
