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

// The 4 waves of a workgroup hold accumulators for the same NQ output quads
// (16x16 blocks, 4 values per lane); sum them in wave order through LDS
// (red: [4][NQ][4][64] floats).  Thread T gets lane position T%64 of quads
// q = T/64 + 4e, e < quads_per_thread(NQ), in out[e][0..3] (with NQ < 4 only
// the threads with T/64 < NQ own one).
template <int NQ>
constexpr int quads_per_thread() { return NQ >= 4 ? NQ / 4 : 1; }

template <int NQ>
__device__ __forceinline__ void sum_waves(float* red, const f32x4 (&acc)[NQ],
                                          float (&out)[quads_per_thread<NQ>()][4]) {
  static_assert(NQ < 4 || NQ % 4 == 0, "quads must split evenly over the 4 waves");
  const int lane = lane_id(), wave = wave_id();
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * NQ + q) * 4 + i) * kWave + lane] = acc[q][i];
  __syncthreads();
  const int ol = threadIdx.x & (kWave - 1), oq = threadIdx.x >> 6;
#pragma unroll
  for (int e = 0; e < quads_per_thread<NQ>(); ++e) {
    const int q = oq + 4 * e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
      if (q < NQ) {
        v = red[((0 * NQ + q) * 4 + i) * kWave + ol];
#pragma unroll
        for (int w = 1; w < 4; ++w) v += red[((w * NQ + q) * 4 + i) * kWave + ol];
      }
      out[e][i] = v;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// k_mup
// ---------------------------------------------------------------------------
constexpr int kMfmaTokens = 64;           // tokens per pass of the matrix-core path
constexpr int kMuThreads = 256;
constexpr int kMuWaves = kMuThreads / kWave;
constexpr int kMuMB = 4;                   // 16-row blocks per wave (all waves share the rows)
constexpr int kMuRows = 16 * kMuMB;        // list positions per workgroup
constexpr int kMuK = 128;                  // k per step: 4 lane groups x 32

// Operands of one 128-wide k step [kb, kb + 128) for this lane (group g =
// lane/16).  MFMA sub-step s (0..3) multiplies the A and B operands
// a[s], b[s]; both must cover the same 32 k values, in any order.
//
// fp16 rows ("natural order"): sub-step s, group g -> k = kb + 32s + 8g + 0..7,
// so one load instruction reads 64 contiguous bytes of each of 16 rows.
__device__ __forceinline__ void ld_k128(const f16* rowkb, bool ok, int g, bool stream, u32x4 (&a)[4]) {
  const char* p = reinterpret_cast<const char*>(rowkb + 8 * g);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    a[s] = ok ? (stream ? ld_nt(p + 64 * s) : ld16(p + 64 * s)) : u32x4{0, 0, 0, 0};
}

// Q4_0 rows ("block order"): group g owns block kb/32 + g (one 16-byte code
// group and one scale); sub-step s takes its word s -> k = kb + 32g + 8s + 0..7.
// The fp16 operand that meets it must be permuted to match (k_xstep).
__device__ __forceinline__ void ld_k128_q4(const uint8_t* w, size_t scale_off, int row, bool ok, int d, int kb,
                                           int g, u32x4 (&a)[4]) {
  const size_t blk = (size_t)row * (d / 32) + kb / 32 + g;
  const u32x4 code = ok ? ld_nt(w + blk * 16) : u32x4{0, 0, 0, 0};
  const f16 sc = ok ? reinterpret_cast<const f16*>(w + scale_off)[blk] : (f16)0.0f;
  const f16x2 s2{sc, sc};
#pragma unroll
  for (int s = 0; s < 4; ++s) a[s] = q4_dequant8(dw(code, s), s2);
}

template <typename WF>
__device__ __forceinline__ void load_row_k128(const void* w, size_t scale_off, int row, bool ok, int d, int kb, int g,
                                              u32x4 (&a)[4]) {
  if constexpr (std::is_same<WF, Q4>::value)
    ld_k128_q4(static_cast<const uint8_t*>(w), scale_off, row, ok, d, kb, g, a);
  else
    ld_k128(static_cast<const f16*>(w) + (size_t)row * d + kb, ok, g, true, a);
}

// One 128-wide k step of MB 16-row blocks of a weight matrix, held as loaded
// (fp16: the operands themselves; Q4_0: the code groups and scales, turned
// into fp16 operands when used), so that the next step's loads can be in
// flight while this one is multiplied.
template <typename WF, int MB>
struct RowStep {
  u32x4 v[MB][4];
  __device__ __forceinline__ void load(const void* w, size_t, const int (&row)[MB], const bool (&rv)[MB], int d,
                                       int kb, int g) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) ld_k128(static_cast<const f16*>(w) + (size_t)row[mb] * d + kb, rv[mb], g, true, v[mb]);
  }
  __device__ __forceinline__ void operands(int mb, u32x4 (&a)[4]) const {
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = v[mb][s];
  }
};

template <int MB>
struct RowStep<Q4, MB> {
  u32x4 code[MB];
  f16 sc[MB];
  __device__ __forceinline__ void load(const void* w, size_t scale_off, const int (&row)[MB], const bool (&rv)[MB],
                                       int d, int kb, int g) {
    const uint8_t* wb = static_cast<const uint8_t*>(w);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const size_t blk = (size_t)row[mb] * (d / 32) + kb / 32 + g;
      code[mb] = rv[mb] ? ld_nt(wb + blk * 16) : u32x4{0, 0, 0, 0};
      sc[mb] = rv[mb] ? reinterpret_cast<const f16*>(wb + scale_off)[blk] : (f16)0.0f;
    }
  }
  __device__ __forceinline__ void operands(int mb, u32x4 (&a)[4]) const {
    const f16x2 s2{sc[mb], sc[mb]};
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = q4_dequant8(dw(code[mb], s), s2);
  }
  // the code groups only (every lane loads; the scales come from elsewhere)
  __device__ __forceinline__ void load_codes(const void* w, const int (&row)[MB], int d, int kb, int g) {
    const uint8_t* wb = static_cast<const uint8_t*>(w);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) code[mb] = ld_nt(wb + ((size_t)row[mb] * (d / 32) + kb / 32 + g) * 16);
  }
  __device__ __forceinline__ void operands(int mb, f16 scale, u32x4 (&a)[4]) const {
    const f16x2 s2{scale, scale};
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = q4_dequant8(dw(code[mb], s), s2);
  }
};

// The same step of MB 16-row blocks of fp16 rows, loaded the way a gather
// streams fastest: 16 lanes per row, 256 contiguous bytes of one row per 16
// lanes, so one load instruction covers 4 rows (measured on gathered 16 KB
// rows: 6.4 TB/s, against 4.8 TB/s for the 16 rows x 64 bytes per
// instruction of the operand layout itself).  The units are then moved into
// the operand layout -- row l%16, sub-step s, k = 32s + 8(l/16), the natural
// order above, so the products are the same bits -- through a wave-private
// LDS buffer of 16 rows x kTStride units (one unit of padding per row keeps
// the 16 rows of an operand read on different banks).
constexpr int kTStride = kMuK / 8 + 1;

template <int MB>
struct RowStepT {
  u32x4 v[MB][4];        // v[mb][i]: row 4i + l/16 of block mb, unit l%16 of the step
  __device__ __forceinline__ void load(const f16* w, const int (&rowt)[MB][4], const bool (&rvt)[MB][4], int d, int kb,
                                       int lane) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* p = reinterpret_cast<const char*>(w + (size_t)rowt[mb][i] * d + kb) + 16 * (lane & 15);
        v[mb][i] = rvt[mb][i] ? ld_nt(p) : u32x4{0, 0, 0, 0};
      }
  }
  // Operands of block mb (a[s] for sub-step s), through buf (this wave's).
  __device__ __forceinline__ void operands(int mb, u32x4* buf, int lane, u32x4 (&a)[4]) const {
    const int q = lane >> 4, u = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[(4 * i + q) * kTStride + u] = v[mb][i];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");     // the writes land before any lane reads
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = buf[u * kTStride + 4 * s + q];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");     // and the reads before the next block's writes
  }
};

// RowStepT with every lane loading (rows past the count read a valid stand-in
// row) and the stand-in rows zeroed when the operands are formed, so the
// loads carry no lane condition and the compiler can count the ones in
// flight exactly (a load under a lane condition, or a load whose issue
// depends on a branch, makes it wait for every load issued so far).
template <int MB>
struct RowStepTU {
  u32x4 v[MB][4];
  __device__ __forceinline__ void load(const f16* w, const int (&rowt)[MB][4], int d, int kb, int lane) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[mb][i] = ld_nt(reinterpret_cast<const char*>(w + (size_t)rowt[mb][i] * d + kb) + 16 * (lane & 15));
  }
  __device__ __forceinline__ void operands(int mb, const bool (&rvt)[MB][4], u32x4* buf, int lane,
                                           u32x4 (&a)[4]) const {
    const int q = lane >> 4, u = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[(4 * i + q) * kTStride + u] = rvt[mb][i] ? v[mb][i] : u32x4{0, 0, 0, 0};
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");     // the writes land before any lane reads
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = buf[u * kTStride + 4 * s + q];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");     // and the reads before the next block's writes
  }
};

// Row indices of the transposed load: position 4i + l/16 of each block, from
// the lane that holds it in the operand layout (position l%16).
template <int MB>
__device__ __forceinline__ void rows_for_load(const int (&row)[MB], const bool (&rv)[MB], int lane, int (&rowt)[MB][4],
                                              bool (&rvt)[MB][4]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src = 4 * i + (lane >> 4);
      rowt[mb][i] = __shfl(row[mb], src, kWave);
      rvt[mb][i] = __shfl(rv[mb] ? 1 : 0, src, kWave) != 0;
    }
}

// NB 16-token blocks of fp16 activations for step st, from a step-major
// copy xs[step][token][128] (see k_xstep): one step's operands of all tokens
// are one contiguous block, so the many workgroups reading them at once
// spread over the L2 channels instead of meeting on the few that a 16 KB row
// stride maps to.
// Q4_0 code groups of 16 rows x 4 k-steps (256 contiguous bytes of each
// row), loaded 16 lanes per row, 4 rows per instruction (lane l: row 4i +
// l/16, 16-byte unit l%16), and moved into the operand layout through the
// wave's LDS buffer: steps() gives lane l, for step s of the window, the
// code group of row l%16 and lane group l/16 (the group that
// RowStep<Q4>::load_codes gives that lane for that step).
struct CodesTU {
  u32x4 v[4];
  __device__ __forceinline__ void load(const uint8_t* codes, const int (&rowt)[4], size_t row_bytes, size_t off,
                                       int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld_nt(codes + (size_t)rowt[i] * row_bytes + off + 16 * (lane & 15));
  }
  __device__ __forceinline__ void steps(u32x4* buf, int lane, u32x4 (&c)[4]) const {
    const int q = lane >> 4, u = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[(4 * i + q) * kTStride + u] = v[i];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");     // the writes land before any lane reads
#pragma unroll
    for (int s = 0; s < 4; ++s) c[s] = buf[u * kTStride + 4 * s + q];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");     // and the reads before the next window's writes
  }
};

template <int NB>
struct TokStep {
  u32x4 v[NB][4];
  __device__ __forceinline__ void load(const f16* xs, int nt, int st, int g, int n16) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = nb * 16 + n16;
      ld_k128(xs + ((size_t)st * nt + t) * kMuK, t < nt, g, false, v[nb]);
    }
  }
};

// The same operands read from the row-major token tile x[t][d] (each lane
// the 16 bytes of its token), with a copy into the step-major layout above
// (store_step), so that a kernel which reads every step of x once can leave
// the copy for the kernels that read it many times.
template <int NB>
struct TokStepRM {
  u32x4 v[NB][4];
  __device__ __forceinline__ void load(const f16* x, int d, int nt, int st, int g, int n16) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = nb * 16 + n16;                 // slots past nt read the last token (never stored)
      ld_k128(x + (size_t)(t < nt ? t : nt - 1) * d + (size_t)st * kMuK, true, g, false, v[nb]);
    }
  }
  // xs[st][t][32s + 8g .. +8] = the lane's operand of sub-step s (natural
  // order), or with block (operands meeting Q4_0 rows, as k_xstep<true>
  // writes them) xs[st][t][32g + 8s .. +8]
  __device__ __forceinline__ void store_step(f16* xs, int nt, int st, int g, int n16, bool block) const {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = nb * 16 + n16;
      if (t < nt) {
        f16* dst = xs + ((size_t)st * nt + t) * kMuK;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          *reinterpret_cast<u32x4*>(dst + (block ? 32 * g + 8 * s : 32 * s + 8 * g)) = v[nb][s];
      }
    }
  }
};

// Run steps [s0, s1) with two register stages: the loads of step st+1 are
// issued before step st is multiplied.  load(stage, st) and mul(stage) are
// the caller's.
// The steady state issues every load unconditionally and the last one or two
// steps are peeled, so no load's issue depends on a branch: with loads that
// also carry no lane condition the compiler can then wait for exactly the
// step it multiplies (a conditional issue makes it wait for every load).
template <typename Stage, typename Load, typename Mul>
__device__ __forceinline__ void pipeline2(int s0, int s1, Stage& A, Stage& B, Load load, Mul mul) {
  if (s0 >= s1) return;
  load(A, s0);
  int st = s0;
  for (; st + 2 < s1; st += 2) {
    load(B, st + 1);
    mul(A);
    load(A, st + 2);
    mul(B);
  }
  if (st + 1 < s1) {
    load(B, st + 1);
    mul(A);
    mul(B);
  } else {
    mul(A);
  }
}

// Three register stages over a number of steps that is a multiple of 3
// (at least 3): the loads of steps st+1 and st+2 are in flight while step st
// is multiplied, and no load's issue depends on a branch.
template <typename Stage, typename Load, typename Mul>
__device__ __forceinline__ void pipeline3x(int s0, int s1, Stage& A, Stage& B, Stage& C, Load load, Mul mul) {
  load(A, s0);
  load(B, s0 + 1);
  int st = s0;
  for (; st + 3 < s1; st += 3) {
    load(C, st + 2);
    mul(A);
    load(A, st + 3);
    mul(B);
    load(B, st + 4);
    mul(C);
  }
  load(C, st + 2);
  mul(A);
  mul(B);
  mul(C);
}

// k_xstep: xs[st][t][128] = x[t][128 st .. 128 st + 128), the step-major copy
// TokStep reads.  With BLOCK (operands meeting Q4_0 rows, which come in block
// order) the 16-byte groups inside a step are also permuted:
// xs[st][t][32s + 8g + j] = x[t][128 st + 32g + 8s + j].  One thread per
// 16-byte group.
template <bool BLOCK>
__global__ __launch_bounds__(256) void k_xstep(const f16* __restrict__ x, int nt, int d, f16* __restrict__ xs) {
  const int e = blockIdx.x * 256 + threadIdx.x;       // destination group: [st][t][s][g]
  const int groups = nt * d / 8;
  if (e >= groups) return;
  const int q = e & 15, rest = e >> 4;
  const int t = rest % nt, st = rest / nt;
  const int src_q = BLOCK ? ((q & 3) << 2) | (q >> 2) : q;
  *reinterpret_cast<u32x4*>(xs + (size_t)e * 8) =
      *reinterpret_cast<const u32x4*>(x + (size_t)t * d + st * kMuK + src_q * 8);
}

// As TokStep, but every lane loads: token slots past nt read the last real
// token (a valid address; their results are never stored), so the load has
// no lane condition and the compiler can keep it in flight.
template <int NB>
struct TokStepClamped {
  u32x4 v[NB][4];
  __device__ __forceinline__ void load(const f16* xs, int nt, int st, int g, int n16) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int t = nb * 16 + n16;
      const int tc = t < nt ? t : nt - 1;
      ld_k128(xs + ((size_t)st * nt + tc) * kMuK, true, g, false, v[nb]);
    }
  }
};

// 16-row blocks per wave in k_mup: enough rows to reuse each activation
// operand 4 times at 64 tokens, and at few tokens few enough rows per
// workgroup that a small union list still spreads over every CU.
template <int NB>
constexpr int mup_mb() { return NB == 1 ? 1 : (NB == 2 ? 2 : 4); }

template <typename WF, int ACT, int NB>
__global__ __launch_bounds__(kMuThreads) void k_mup(const void* __restrict__ w_up, const void* __restrict__ w_gate,
                                                    size_t scale_off, const float* __restrict__ bias,
                                                    const f16* __restrict__ x, int d, int d_ff, int nt,
                                                    const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ count_ptr, int max_count,
                                                    f16* __restrict__ h, int ldh, unsigned* __restrict__ flags) {
  constexpr bool GATED = ACT == ACT_REGLU;
  constexpr int MB = mup_mb<NB>();
  constexpr int NQ = MB * NB;              // accumulator quads per lane
  constexpr int QT = quads_per_thread<NQ>();
  constexpr bool TR = std::is_same<WF, f16>::value && !GATED;   // transposed row loads (RowStepT)
  __shared__ float red[kMuWaves][NQ][4][kWave];
  constexpr bool Q = std::is_same<WF, Q4>::value;
  constexpr bool TQ = Q && MB == 1;   // Q4_0 code groups by transposed loads (CodesTU)
  __shared__ u32x4 w_l[TR || TQ ? kMuWaves : 1][TR || TQ ? 16 * kTStride : 1];
  __shared__ u32x4 sc_l[Q ? kMuWaves : 1][Q && GATED ? 2 : 1][Q ? MB : 1][16][Q ? 4 : 1];   // Q4_0: a chunk's scales
  const int lane = lane_id();
  const int wave = wave_id();
  const int g = lane >> 4, n16 = lane & 15;
  const int cnt = clamp_count(count_ptr, max_count);
  const int r0 = blockIdx.x * 16 * MB;
  if (r0 >= cnt) return;                   // the whole workgroup leaves together

  int row[MB];
  bool rv[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int p = r0 + mb * 16 + n16;
    const int i = p < cnt ? idx[p] : -1;
    rv[mb] = (unsigned)i < (unsigned)d_ff;
    row[mb] = rv[mb] ? i : 0;
  }

  f32x4 au[MB][NB], ag[GATED ? MB : 1][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      au[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (GATED) ag[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int ns = d / kMuK;
  const int s0 = wave * ns / kMuWaves, s1 = (wave + 1) * ns / kMuWaves;
  int rowt[MB][4];
  bool rvt[MB][4];
  if constexpr (TR || TQ) rows_for_load<MB>(row, rv, lane, rowt, rvt);
  u32x4* wbuf = &w_l[TR || TQ ? wave : 0][0];
  // fp16 rows: every lane loads (stand-in rows and token slots; see RowStepTU)
  using Rows = typename std::conditional<TR, RowStepTU<MB>, RowStep<WF, MB>>::type;
  using Toks = typename std::conditional<TR, TokStepClamped<NB>, TokStep<NB>>::type;
  struct Step {
    Rows up;
    RowStep<WF, GATED ? MB : 1> gate;
    Toks x;
  };
  auto load = [&](Step& S, int st) {
    const int kb = st * kMuK;
    if constexpr (TR)
      S.up.load(static_cast<const f16*>(w_up), rowt, d, kb, lane);
    else
      S.up.load(w_up, scale_off, row, rv, d, kb, g);
    if constexpr (GATED) S.gate.load(w_gate, scale_off, row, rv, d, kb, g);
    S.x.load(x, nt, st, g, n16);
  };
  auto mul = [&](const Step& S) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      u32x4 a[4], ga[4];
      if constexpr (TR)
        S.up.operands(mb, rvt, wbuf, lane, a);
      else
        S.up.operands(mb, a);
      if constexpr (GATED) S.gate.operands(mb, ga);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          au[mb][nb] = mfma(a[s], S.x.v[nb][s], au[mb][nb]);
          if constexpr (GATED) ag[mb][nb] = mfma(ga[s], S.x.v[nb][s], ag[mb][nb]);
        }
    }
  };
  // Two stages in flight unless their registers would crowd out the
  // accumulators.  Q4_0 rows (18 bytes per block) are prefetched kQPre steps
  // at a time -- every lane loads (rows past the count read a valid row whose
  // results are never stored), so all of a chunk's loads are in flight
  // together -- and the activation steps alternate between two register
  // sets, the next one loading while the current one is multiplied.
  constexpr bool kPipe = !(GATED && NB > 2) && !std::is_same<WF, Q4>::value;
  if constexpr (std::is_same<WF, Q4>::value) {
    constexpr int kQPre = GATED && MB == 1 ? 4 : 8 / MB;   // k steps per chunk
    bool all[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) all[mb] = true;
    // The rows' scales of a whole chunk (4 per step, 8 bytes per step and
    // row, contiguous) in one 16-byte load per lane and matrix -- lane (g,
    // n16) takes unit g % SU of row n16 -- staged in this wave's LDS: a 2-byte
    // load per lane and step otherwise costs as many memory instructions as
    // the codes.  With one row block the code groups come by transposed loads
    // (CodesTU).  Needs 16-byte aligned scale rows (d % 256 == 0) and whole
    // chunks.
    constexpr int SU = kQPre / 2;                   // 16-byte scale units per row per chunk
    constexpr int NM = GATED ? 2 : 1;               // matrices: up (and gate)
    const int nbk = d / 32;
    const bool sc_chunk = nbk % 8 == 0 && (s1 - s0) % kQPre == 0;
    const uint8_t* wm[2] = {static_cast<const uint8_t*>(w_up),
                            static_cast<const uint8_t*>(GATED ? w_gate : w_up)};
    for (int c0 = s0; c0 < s1; c0 += kQPre) {
      RowStep<WF, MB> up[kQPre];
      RowStep<WF, GATED ? MB : 1> gt[GATED ? kQPre : 1];
      bool chunked = false;
      if (sc_chunk) {
        u32x4 su[NM][MB];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            su[m][mb] = ld_nt(wm[m] + scale_off + ((size_t)row[mb] * nbk + (size_t)c0 * 4) * 2 + 16 * (g % SU));
        constexpr int NWIN = kQPre / 4 > 0 ? kQPre / 4 : 1;
        CodesTU ct[TQ ? NM : 1][NWIN];
        if constexpr (TQ) {
          static_assert(kQPre % 4 == 0, "whole 4-step windows per chunk");
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int h = 0; h < NWIN; ++h)
              ct[m][h].load(wm[m], rowt[0], (size_t)nbk * 16, ((size_t)c0 * 4 + 16 * h) * 16, lane);
        } else {
#pragma unroll
          for (int j = 0; j < kQPre; ++j) up[j].load_codes(w_up, row, d, (c0 + j) * kMuK, g);
          if constexpr (GATED)
#pragma unroll
            for (int j = 0; j < kQPre; ++j) gt[j].load_codes(w_gate, row, d, (c0 + j) * kMuK, g);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            if (g < SU) sc_l[wave][m][mb][n16][g] = su[m][mb];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");     // the scales land before any lane reads
#pragma unroll
        for (int j = 0; j < kQPre; ++j)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            up[j].sc[mb] = reinterpret_cast<const f16*>(&sc_l[wave][0][mb][n16][0])[4 * j + g];
            if constexpr (GATED) gt[j].sc[mb] = reinterpret_cast<const f16*>(&sc_l[wave][NM - 1][mb][n16][0])[4 * j + g];
          }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");     // and are read before the next chunk's writes
        if constexpr (TQ) {
#pragma unroll
          for (int h = 0; h < NWIN; ++h) {
            u32x4 c[4];
            ct[0][h].steps(wbuf, lane, c);
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) up[4 * h + s2].code[0] = c[s2];
            if constexpr (GATED) {
              ct[NM - 1][h].steps(wbuf, lane, c);
#pragma unroll
              for (int s2 = 0; s2 < 4; ++s2) gt[4 * h + s2].code[0] = c[s2];
            }
          }
        }
        chunked = true;
      }
      if (!chunked) {
#pragma unroll
        for (int j = 0; j < kQPre; ++j) {
          const int st = c0 + j < s1 ? c0 + j : s1 - 1;
          up[j].load(w_up, scale_off, row, all, d, st * kMuK, g);
          if constexpr (GATED) gt[j].load(w_gate, scale_off, row, all, d, st * kMuK, g);
        }
      }
      TokStepClamped<NB> xt[2];
      xt[0].load(x, nt, c0, g, n16);
#pragma unroll
      for (int j = 0; j < kQPre; ++j) {
        if (j + 1 < kQPre) xt[(j + 1) & 1].load(x, nt, c0 + j + 1 < s1 ? c0 + j + 1 : s1 - 1, g, n16);
        if (c0 + j < s1) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            u32x4 a[4], ga[4];
            up[j].operands(mb, a);
            if constexpr (GATED) gt[j].operands(mb, ga);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) {
                au[mb][nb] = mfma(a[s], xt[j & 1].v[nb][s], au[mb][nb]);
                if constexpr (GATED) ag[mb][nb] = mfma(ga[s], xt[j & 1].v[nb][s], ag[mb][nb]);
              }
          }
        }
      }
    }
  } else {
    // The workgroups start their k walk at different steps (workgroup b at
    // step b % steps of its quarter, wrapping around), as in k_mup_wide:
    // all of them in step would read the same few hundred bytes of many
    // rows 16 KB apart at once (Falcon batch-8 FFN 80.7 -> 75.5 us).
    const int nst = s1 - s0;
    const int rot = nst > 0 ? (int)(blockIdx.x % (unsigned)nst) : 0;
    auto load_rot = [&](Step& S, int st) { load(S, s0 + (st - s0 + rot) % nst); };
    if constexpr (kPipe) {
      Step S0, S1;
      pipeline2(s0, s1, S0, S1, load_rot, mul);
    } else {
      for (int st = s0; st < s1; ++st) {
        Step S;
        load_rot(S, st);
        mul(S);
      }
    }
  }

  // Sum the 4 waves in wave order.  Thread T owns lane position T%64 and the
  // quads q = T/64 + 4*e (e < QT): rows 4*((T%64)/16)+i of block q/NB, token
  // (q%NB)*16 + T%16.
  const int ol = threadIdx.x & (kWave - 1);
  const int oq = threadIdx.x >> 6;
  float su[QT][4], sg[QT][4];
  {
    f32x4 flat[NQ];
    if constexpr (GATED) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) flat[q] = ag[q / NB][q % NB];
      sum_waves<NQ>(&red[0][0][0][0], flat, sg);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) flat[q] = au[q / NB][q % NB];
    sum_waves<NQ>(&red[0][0][0][0], flat, su);
  }

  bool over = false;                       // an H value not finite in fp16
#pragma unroll
  for (int e = 0; e < QT; ++e) {
    const int q = oq + kMuWaves * e;
    const int mb = q / NB, nb = q % NB;
    const int t = nb * 16 + (ol & 15);
    const int p = r0 + mb * 16 + 4 * (ol >> 4);
    if (q < NQ && t < nt) {
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
        over |= fp16_overflows(v);
        hv[i] = (f16)v;
      }
      u32x2 packed;
      packed.x = __builtin_bit_cast(unsigned, f16x2{hv[0], hv[1]});
      packed.y = __builtin_bit_cast(unsigned, f16x2{hv[2], hv[3]});
      *reinterpret_cast<u32x2*>(h + (size_t)t * ldh + p) = packed;
    }
  }
  raise_flag_if_any(flags, over, PI_FLAG_FP16_RANGE);
}

// ---------------------------------------------------------------------------
// k_mup_wide (33-64 tokens).  k_mup reads the shared activation tile once per
// 64 rows, and at 64 tokens that tile is as many bytes as the rows: here a
// workgroup of 8 waves owns 256 list positions and stages pieces of
// kMxPiece k steps of x in LDS, which all 8 waves multiply.  To keep enough
// workgroups, k is split over kMxSplit workgroups (grid y) that write fp32
// partial sums zp[split][token][position] (and zg for the gate); k_mfin adds
// the splits in order, applies bias and activation and writes H.  (Letting
// the last workgroup of a row block finish it instead needs device-scope
// fences, which write back and invalidate the L2 and cost far more.)
// ---------------------------------------------------------------------------
// One token's 128 k values are 16 units of 16 bytes; LDS copies give each
// token 17 units, so the 16 tokens of an MFMA operand read fall on
// different banks (with 16 units they would all hit the same ones).
constexpr int kTokStride = kMuK / 8 + 1;
constexpr int kMxThreads = 512;
constexpr int kMxWaves = kMxThreads / kWave;
constexpr int kMxMB = 2;                          // 16-row blocks per wave
constexpr int kMxRows = kMxWaves * 16 * kMxMB;    // 256 list positions per workgroup
constexpr int kMxSplit = 2;
// k steps per staged piece of x: transposed fp16 row loads also need 8 waves x
// 4.25 KB of LDS (RowStepT)
template <typename WF>
constexpr int mx_piece() { return std::is_same<WF, Q4>::value ? 8 : 4; }

template <typename WF, int ACT, int NB>
__global__ __launch_bounds__(kMxThreads) void k_mup_wide(const void* __restrict__ w_up, const void* __restrict__ w_gate,
                                                         size_t scale_off, const f16* __restrict__ xs, int d,
                                                         int d_ff, int nt, const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ count_ptr, int max_count,
                                                         float* __restrict__ zp, float* __restrict__ zg, int ldz) {
  constexpr bool GATED = ACT == ACT_REGLU;
  // fp16 rows are loaded transposed (RowStepT); with the gate as well that
  // would exceed the register budget, so ReGLU keeps the operand-layout loads
  constexpr bool F16 = std::is_same<WF, f16>::value && !GATED;
  constexpr int kMxPiece = F16 ? mx_piece<WF>() : 8;
  constexpr int LU = 16 * NB * kMuK / 8;          // 16-byte units of one step of x (all token slots)
  __shared__ u32x4 x_l[kMxPiece][16 * NB * kTokStride];
  __shared__ u32x4 w_l[F16 ? kMxWaves : 1][F16 ? 16 * kTStride : 1];   // transposed loads (fp16 rows)
  const int lane = lane_id();
  const int wave = wave_id();
  const int g = lane >> 4, n16 = lane & 15;
  const int cnt = clamp_count(count_ptr, max_count);
  if (blockIdx.x * kMxRows >= cnt) return;        // the whole workgroup leaves together
  const int r0 = blockIdx.x * kMxRows + wave * 16 * kMxMB;
  int row[kMxMB];
  bool rv[kMxMB];
#pragma unroll
  for (int mb = 0; mb < kMxMB; ++mb) {
    const int p = r0 + mb * 16 + n16;
    const int i = p < cnt ? idx[p] : -1;
    rv[mb] = (unsigned)i < (unsigned)d_ff;
    row[mb] = rv[mb] ? i : 0;
  }
  f32x4 au[kMxMB][NB], ag[GATED ? kMxMB : 1][NB];
#pragma unroll
  for (int mb = 0; mb < kMxMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      au[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (GATED) ag[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const int ns = d / kMuK;
  const int split = blockIdx.y;
  const int s0 = split * ns / kMxSplit, s1 = (split + 1) * ns / kMxSplit;
  int rowt[kMxMB][4];
  bool rvt[kMxMB][4];
  if constexpr (F16) rows_for_load<kMxMB>(row, rv, lane, rowt, rvt);
  u32x4* wbuf = &w_l[F16 ? wave : 0][0];
  using Rows = typename std::conditional<F16, RowStepT<kMxMB>, RowStep<WF, kMxMB>>::type;
  using GRows = typename std::conditional<F16, RowStepT<GATED ? kMxMB : 1>, RowStep<WF, GATED ? kMxMB : 1>>::type;
  struct Step {
    Rows up;
    GRows gate;
  };
  auto load = [&](Step& S, int st) {
    if constexpr (F16) {
      S.up.load(static_cast<const f16*>(w_up), rowt, rvt, d, st * kMuK, lane);
      if constexpr (GATED) S.gate.load(static_cast<const f16*>(w_gate), rowt, rvt, d, st * kMuK, lane);
    } else {
      S.up.load(w_up, scale_off, row, rv, d, st * kMuK, g);
      if constexpr (GATED) S.gate.load(w_gate, scale_off, row, rv, d, st * kMuK, g);
    }
  };
  const bool whole = s1 > s0 && (s1 - s0) % kMxPiece == 0;
  if constexpr (F16) {
    if (whole) {
      // Whole pieces: a branch-free software pipeline.  Each step's rows are
      // requested one step ahead, and the next piece's x units together with
      // its first step's rows during the piece's last step, every load
      // unconditional, so each wait covers exactly the loads it needs.
      constexpr int XU = kMxPiece * LU / kMxThreads;   // x units per thread per piece
      const int su = nt * (kMuK / 8);
      u32x4 xr[XU];
      auto x_load = [&](int p0) {
#pragma unroll
        for (int k = 0; k < XU; ++k) {
          const int e = threadIdx.x + kMxThreads * k;
          const int q = e / LU, r = e - q * LU;
          const int rr = r < su ? r : su - 1;          // slots past nt: a valid stand-in, zeroed on store
          xr[k] = ld16(xs + ((size_t)(p0 + q) * nt) * kMuK + (size_t)rr * 8);
        }
      };
      auto x_store = [&]() {
#pragma unroll
        for (int k = 0; k < XU; ++k) {
          const int e = threadIdx.x + kMxThreads * k;
          const int q = e / LU, r = e - q * LU;
          x_l[q][(r >> 4) * kTokStride + (r & 15)] = r < su ? xr[k] : u32x4{0, 0, 0, 0};
        }
      };
      RowStepTU<kMxMB> S0, S1;
      auto rows = [&](RowStepTU<kMxMB>& S, int st) { S.load(static_cast<const f16*>(w_up), rowt, d, st * kMuK, lane); };
      auto step = [&](const RowStepTU<kMxMB>& S, int q) {
        u32x4 a[kMxMB][4];
#pragma unroll
        for (int mb = 0; mb < kMxMB; ++mb) S.operands(mb, rvt, wbuf, lane, a[mb]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          u32x4 b[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) b[nb] = x_l[q][(nb * 16 + n16) * kTokStride + 4 * s + g];
#pragma unroll
          for (int mb = 0; mb < kMxMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) au[mb][nb] = mfma(a[mb][s], b[nb], au[mb][nb]);
        }
      };
      // piece p0 (its x in x_l, the rows of its first step in S0); pn: the next piece
      auto piece = [&](int p0, int pn, auto has_next) {
        static_assert(kMxPiece == 4, "the unrolled piece is 4 steps");
        rows(S1, p0 + 1);
        step(S0, 0);
        rows(S0, p0 + 2);
        step(S1, 1);
        rows(S1, p0 + 3);
        step(S0, 2);
        if constexpr (decltype(has_next)::value) {
          x_load(pn);
          rows(S0, pn);
        }
        step(S1, 3);
        if constexpr (decltype(has_next)::value) {
          __syncthreads();                             // every wave is done with this piece's x
          x_store();
          __syncthreads();
        }
      };
      // The workgroups start at different pieces (row block r at piece
      // r % pieces, wrapping around): all of them walking k in step would
      // read the same few hundred bytes of thousands of rows 16 KB apart at
      // once, which the memory channels serve far below their rate
      // (Falcon 64-token FFN 217.5 -> 192.5 us).  Each row's sum over k then
      // runs in that rotated, fixed order.
      const int npc = (s1 - s0) / kMxPiece;
      const int rot = (int)(blockIdx.x % (unsigned)npc);
      auto pstart = [&](int i) { return s0 + ((i + rot) % npc) * kMxPiece; };
      x_load(pstart(0));
      rows(S0, pstart(0));
      x_store();
      __syncthreads();
      int i = 0;
      for (; i + 1 < npc; ++i) piece(pstart(i), pstart(i + 1), std::true_type{});
      piece(pstart(i), 0, std::false_type{});
    }
  }
  for (int p0 = s0; p0 < s1; p0 += kMxPiece) {
    if constexpr (F16) {
      if (whole) break;                                // done above
    }
    const int np = s1 - p0 < kMxPiece ? s1 - p0 : kMxPiece;
    Step cur;
    load(cur, p0);                                  // the first step's rows go out before the staging
    __syncthreads();                                // the previous piece is no longer read
    const int su = nt * (kMuK / 8);                 // units of one step of the nt real tokens
    for (int e = threadIdx.x; e < np * LU; e += kMxThreads) {
      const int q = e / LU, r = e - q * LU;         // token slots past nt hold zeros
      x_l[q][(r >> 4) * kTokStride + (r & 15)] =
          r < su ? ld16(xs + ((size_t)(p0 + q) * nt) * kMuK + (size_t)r * 8) : u32x4{0, 0, 0, 0};
    }
    __syncthreads();
    for (int q = 0; q < np; ++q) {
      Step nxt;
      if (q + 1 < np) load(nxt, p0 + q + 1);
      u32x4 a[kMxMB][4], ga[GATED ? kMxMB : 1][4];
#pragma unroll
      for (int mb = 0; mb < kMxMB; ++mb) {
        if constexpr (F16) {
          cur.up.operands(mb, wbuf, lane, a[mb]);
          if constexpr (GATED) cur.gate.operands(mb, wbuf, lane, ga[mb]);
        } else {
          cur.up.operands(mb, a[mb]);
          if constexpr (GATED) cur.gate.operands(mb, ga[mb]);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 b[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) b[nb] = x_l[q][(nb * 16 + n16) * kTokStride + 4 * s + g];
#pragma unroll
        for (int mb = 0; mb < kMxMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            au[mb][nb] = mfma(a[mb][s], b[nb], au[mb][nb]);
            if constexpr (GATED) ag[mb][nb] = mfma(ga[mb][s], b[nb], ag[mb][nb]);
          }
      }
      if (q + 1 < np) cur = nxt;
    }
  }
  // partial sums: lane holds rows 4g..4g+3 of each 16-row block, token n16 of each token block
#pragma unroll
  for (int mb = 0; mb < kMxMB; ++mb) {
    const int p = r0 + mb * 16 + 4 * g;
    if (p < cnt) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int t = nb * 16 + n16;
        if (t < nt) {
          *reinterpret_cast<f32x4*>(zp + ((size_t)split * kMfmaTokens + t) * ldz + p) = au[mb][nb];
          if constexpr (GATED)
            *reinterpret_cast<f32x4*>(zg + ((size_t)split * kMfmaTokens + t) * ldz + p) = ag[mb][nb];
        }
      }
    }
  }
}

// k_mfin: H[t][p] = act(sum of the splits in split order + bias) for
// p < count, 0 from the count up to the next multiple of 64, fp16.  Each
// thread does 4 consecutive positions of one token.
template <int ACT>
__global__ __launch_bounds__(256) void k_mfin(const float* __restrict__ zp, const float* __restrict__ zg,
                                              const float* __restrict__ bias, const int32_t* __restrict__ idx,
                                              const int32_t* __restrict__ count_ptr, int max_count, int d_ff, int nt,
                                              int ldz, f16* __restrict__ h, int ldh, unsigned* __restrict__ flags) {
  constexpr bool GATED = ACT == ACT_REGLU;
  const int cnt = clamp_count(count_ptr, max_count);
  const int quads = (cnt + 63) / 64 * 16;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const bool live = e < nt * quads;
  if (__ballot(live) == 0ull) return;          // whole waves leave together (the flag check below is per wave)
  const int t = live ? e / quads : 0, p = live ? (e - t * quads) * 4 : cnt;
  f32x4 u{0.f, 0.f, 0.f, 0.f}, gs{0.f, 0.f, 0.f, 0.f};
  if (p < cnt) {
#pragma unroll
    for (int sp = 0; sp < kMxSplit; ++sp) {
      const size_t o = ((size_t)sp * kMfmaTokens + t) * ldz + p;
      u += *reinterpret_cast<const f32x4*>(zp + o);
      if constexpr (GATED) gs += *reinterpret_cast<const f32x4*>(zg + o);
    }
  }
  f16 hv[4];
  bool over = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = p + i < cnt ? idx[p + i] : -1;
    float v = 0.f;
    if ((unsigned)n < (unsigned)d_ff) {
      const float b = bias ? bias[n] : 0.f;
      v = GATED ? act_fn<ACT>(u[i], gs[i] + b) : act_fn<ACT>(u[i] + b, 0.f);
    }
    over |= fp16_overflows(v);
    hv[i] = (f16)v;
  }
  raise_flag_if_any(flags, over, PI_FLAG_FP16_RANGE);
  if (!live) return;
  u32x2 packed;
  packed.x = __builtin_bit_cast(unsigned, f16x2{hv[0], hv[1]});
  packed.y = __builtin_bit_cast(unsigned, f16x2{hv[2], hv[3]});
  *reinterpret_cast<u32x2*>(h + (size_t)t * ldh + p) = packed;
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
  // Every lane loads (the caller passes a valid stand-in row and column for
  // entries it does not use); group_ok then zeroes the rows with ok false.
  __device__ __forceinline__ void load_all(const void* w, size_t, int d, const int (&rows)[8], int col) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const char* p = static_cast<const char*>(w) + ((size_t)rows[r] * d + col) * sizeof(f16);
#pragma unroll
      for (int q = 0; q < CPL / 8; ++q) v[r][q] = ld_nt(p + 16 * q);
    }
  }
  __device__ __forceinline__ void group_ok(int q, const bool (&ok)[8], u32x4 (&out)[8]) const {
#pragma unroll
    for (int r = 0; r < 8; ++r) out[r] = ok[r] ? v[r][q] : u32x4{0, 0, 0, 0};
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
  // Every lane loads (stand-in rows and columns from the caller); group_ok
  // dequantizes the rows with ok false with a zero scale.
  __device__ __forceinline__ void load_all(const void* w, size_t scale_off, int d, const int (&rows)[8], int col) {
    const int nbk = d / 32;
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    const f16* scales = reinterpret_cast<const f16*>(wb + scale_off);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const size_t blk = (size_t)rows[r] * nbk + col / 32;
      const uint8_t* p = wb + blk * 16 + (col % 32) / 2;
      if constexpr (CPL == 32) {
        const u32x4 t = ld_nt(p);
        c[r][0] = t.x; c[r][1] = t.y; c[r][2] = t.z; c[r][3] = t.w;
      } else if constexpr (CPL == 16) {
        const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        c[r][0] = t.x; c[r][1] = t.y;
      } else {
        c[r][0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p));
      }
      sc[r] = scales[blk];
    }
  }
  __device__ __forceinline__ void group_ok(int q, const bool (&ok)[8], u32x4 (&out)[8]) const {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const f16 s = ok[r] ? sc[r] : (f16)0.0f;
      out[r] = q4_dequant8(c[r][q], f16x2{s, s});
    }
  }
};

// The GPU deals the workgroups of a launch to its 8 XCDs round-robin by
// linear index (x fastest), and each XCD has its own L2.  This renumbers a
// 2-D grid so that consecutive logical workgroups (x fastest) share an XCD:
// logical number L = (id % 8) * (total / 8) + id / 8, a bijection when the
// grid size is a multiple of 8 (otherwise the numbering is left as it is).
__device__ __forceinline__ void xcd_grouped(int& x, int& y) {
  const int gx = gridDim.x, total = gx * (int)gridDim.y;
  const int id = (int)blockIdx.x + gx * (int)blockIdx.y;
  const int L = total % 8 == 0 ? (id % 8) * (total / 8) + id / 8 : id;
  x = L % gx;
  y = L / gx;
}

template <typename WF, int NB, int CPL>
__global__ __launch_bounds__(kMdThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_mdown(const void* __restrict__ w_dt, size_t scale_off, int d,
                                                      int d_ff, const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ count_ptr, int max_count,
                                                      const f16* __restrict__ h, int ldh, int nt, int n_chunks,
                                                      float* __restrict__ part,
                                                      unsigned long long* __restrict__ rows_read,
                                                      unsigned long long* __restrict__ up_rows_read) {
  constexpr int NE = CPL * NB;             // accumulator quads per lane
  __shared__ float red[NE][4][kWave];
  const int lane = lane_id();
  const int wave = wave_id();
  const int g = lane >> 4, n16 = lane & 15;
  const int cnt = clamp_count(count_ptr, max_count);
  const int ksteps = (cnt + 31) / 32;
  // Q4_0: the 8 column tiles that share a 128-byte line of scales (2048
  // columns) run on one XCD, so the line is fetched once per XCD, not once
  // per tile
  int tile = blockIdx.x, c = blockIdx.y;
  if constexpr (std::is_same<WF, Q4>::value) xcd_grouped(tile, c);
  const int kc0 = (int)((long long)c * ksteps / n_chunks), kc1 = (int)((long long)(c + 1) * ksteps / n_chunks);
  if ((rows_read || up_rows_read) && tile == 0 && threadIdx.x == 0) {     // the chunk's rows, counted once
    const int r0 = kc0 * 32 < cnt ? kc0 * 32 : cnt, r1 = kc1 * 32 < cnt ? kc1 * 32 : cnt;
    if (r1 > r0 && rows_read) atomicAdd(rows_read, (unsigned long long)(r1 - r0));
    if (r1 > r0 && up_rows_read) atomicAdd(up_rows_read, (unsigned long long)(r1 - r0));   // k_mup read them too
  }
  const int kw0 = kc0 + wave * (kc1 - kc0) / kMdWaves, kw1 = kc0 + (wave + 1) * (kc1 - kc0) / kMdWaves;
  const int col = tile * 16 * CPL + n16 * CPL;
  const bool cv = col < d;

  f32x4 acc[CPL][NB];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The list entries of step kk+1 are loaded while step kk's rows are in
  // flight (clamped to the last valid entry, so the loads carry no lane
  // condition); a step then waits for one round trip, not two.
  // Two register stages (pipeline2): the rows and H of step kk+1 are in
  // flight while step kk is multiplied, and the list entries of step kk+2
  // while those are loaded.  Every lane loads (entries past the count or
  // malformed read row 0, columns past d read column 0, H past the count
  // reads position 0), and the unused values are zeroed when the operands
  // are formed, so no load's issue depends on a branch.
  int nidx[8];
  auto load_idx = [&](int kk) {
    const int q0 = kk * 32 + g * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) nidx[r] = idx[q0 + r < cnt ? q0 + r : cnt - 1];
  };
  const int colc = cv ? col : 0;
  struct Stage {
    DownRows<WF, CPL> wr;
    bool ok[8];
    bool hv;
    u32x4 a[NB];
  };
  auto load = [&](Stage& S, int kk) {
    const int p0 = kk * 32 + g * 8;
    int rows[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = nidx[r];
      S.ok[r] = cv && p0 + r < cnt && (unsigned)i < (unsigned)d_ff;
      rows[r] = S.ok[r] ? i : 0;
    }
    load_idx(kk + 1 < kw1 ? kk + 1 : kk);
    S.wr.load_all(w_dt, scale_off, d, rows, colc);
    S.hv = p0 < cnt;
    const int pc = S.hv ? p0 : 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) S.a[nb] = ld16(h + (size_t)(nb * 16 + n16) * ldh + pc);
  };
  auto mul = [&](const Stage& S) {
    u32x4 a[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) a[nb] = S.hv ? S.a[nb] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < CPL / 8; ++q) {
      u32x4 rw[8], bt[8];
      S.wr.group_ok(q, S.ok, rw);
      transpose8x8(rw, bt);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[8 * q + j][nb] = mfma(a[nb], bt[j], acc[8 * q + j][nb]);
    }
  };
  if (kw0 < kw1) load_idx(kw0);
  Stage S0, S1;
  pipeline2(kw0, kw1, S0, S1, load, mul);

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
// Predictor for many tokens ([QB] "Гибридный дизайн вывода CPU/GPU": the
// predictor maps the input to the neurons expected to fire; two low-rank
// products and a threshold).  Same tiling as k_mup, over all rows:
//   k_mp1    -- part[s][j][r] = sum over k in split s of p1[r][k] * x[j][k]
//               (the k range is split over the grid's y dimension, then over
//               the 4 waves), x read row-major; it also leaves the step-major
//               copy of x for the fp16 FFN;
//   k_tsplit -- t = the splits added in order (fp32), and t_hi = fp16(t),
//               t_lo = fp16(t - t_hi);
//   k_mp2    -- l[j][i] = p2[i] . t[j] + c[i]; mask = l > theta (per token,
//               and optionally the union over the tokens).  t is fp32,
//               so both t_hi and t_lo are multiplied (products exact in fp32;
//               t_hi + t_lo carries 22 significant bits).  Needs |t| < 65504.
// ---------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(kMuThreads) void k_mp1(const f16* __restrict__ p1, const f16* __restrict__ x, int d,
                                                    int rank, int nt, float* __restrict__ part,
                                                    f16* __restrict__ xs, int xs_block) {
  // x: the row-major token tile; the workgroups of row block 0 also write
  // the step-major copy xs (nullable) of the steps they read, in block order
  // when xs_block (for a Q4_0 FFN)
  constexpr int NQ = kMuMB * NB;
  __shared__ float red[kMuWaves][NQ][4][kWave];
  const int lane = lane_id(), wave = wave_id();
  const int g = lane >> 4, n16 = lane & 15;
  const int r0 = blockIdx.x * kMuRows;
  const int split = blockIdx.y, n_split = gridDim.y;
  int row[kMuMB];
  bool rv[kMuMB];
#pragma unroll
  for (int mb = 0; mb < kMuMB; ++mb) {
    row[mb] = r0 + mb * 16 + n16;
    rv[mb] = row[mb] < rank;
  }
  f32x4 acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ns = d / kMuK;
  const int c0 = split * ns / n_split, c1 = (split + 1) * ns / n_split;
  const int s0 = c0 + wave * (c1 - c0) / kMuWaves, s1 = c0 + (wave + 1) * (c1 - c0) / kMuWaves;
#pragma unroll
  for (int mb = 0; mb < kMuMB; ++mb) row[mb] = rv[mb] ? row[mb] : 0;
  const bool copy = xs != nullptr && blockIdx.x == 0;
  // every lane loads (rows past rank read row 0; their sums are never stored).
  // With 1-2 token blocks the p1 rows are loaded in the transposed pattern
  // (RowStepTU: 256 contiguous bytes of a row per 16 lanes) and moved into
  // the operand layout through this wave's LDS buffer; more blocks leave no
  // registers for it and load the operand pattern (64 bytes of 16 rows).
  constexpr bool TU = NB <= 2;
  __shared__ u32x4 w_l[TU ? kMuWaves : 1][TU ? 16 * kTStride : 1];
  int rowt[kMuMB][4];
  bool rvt[kMuMB][4];
  bool all[kMuMB];
#pragma unroll
  for (int mb = 0; mb < kMuMB; ++mb) all[mb] = true;
  if constexpr (TU) rows_for_load<kMuMB>(row, all, lane, rowt, rvt);
  using Rows = typename std::conditional<TU, RowStepTU<kMuMB>, RowStep<f16, kMuMB>>::type;
  struct Step {
    Rows w;
    TokStepRM<NB> x;
    int st;
  };
  auto load = [&](Step& S, int st) {
    if constexpr (TU)
      S.w.load(p1, rowt, d, st * kMuK, lane);
    else
      S.w.load(p1, 0, row, all, d, st * kMuK, g);
    S.x.load(x, d, nt, st, g, n16);
    S.st = st;
  };
  auto mul = [&](const Step& S) {
#pragma unroll
    for (int mb = 0; mb < kMuMB; ++mb) {
      u32x4 a[4];
      if constexpr (TU)
        S.w.operands(mb, rvt, &w_l[TU ? wave : 0][0], lane, a);
      else
        S.w.operands(mb, a);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb * NB + nb] = mfma(a[s], S.x.v[nb][s], acc[mb * NB + nb]);
    }
    if (copy) S.x.store_step(xs, nt, S.st, g, n16, xs_block != 0);
  };
  Step S0, S1;
  pipeline2(s0, s1, S0, S1, load, mul);
  float sum[NB][4];
  sum_waves<NQ>(&red[0][0][0][0], acc, sum);
  const int ol = threadIdx.x & (kWave - 1), oq = threadIdx.x >> 6;
#pragma unroll
  for (int e = 0; e < NB; ++e) {
    const int q = oq + 4 * e;
    const int mb = q / NB, nb = q % NB;
    const int j = nb * 16 + (ol & 15);
    const int r = r0 + mb * 16 + 4 * (ol >> 4);     // rank % 8 == 0: r < rank means r + 3 < rank
    if (j < nt && r < rank)
      *reinterpret_cast<f32x4*>(part + ((size_t)split * nt + j) * rank + r) =
          f32x4{sum[e][0], sum[e][1], sum[e][2], sum[e][3]};
  }
}

// In-kernel compaction of the union mask (layer path, last token tile of
// the predictor): the workgroup's R rows are marked 0/1 in uni[] (LDS).  It
// publishes its marked count as one atomic word that carries its own ready
// flag, adds the counts of the workgroups before it (dispatched before it, so
// the grid needs no co-residency), and writes the marked rows' numbers at
// their list positions in ascending order; the last workgroup writes the
// count.  The list equals k_compact's over the same union row.  status[] and
// *fault are zero at launch (k_tsplit clears them); every wait is bounded
// (hdr[PI_WS_WAIT_POLLS] polls, or kDefaultWaitPolls), so the grid always
// drains; a wait that runs out sets *fault (the merge then writes NaN) and
// PI_FLAG_WAIT_EXPIRED in hdr[0].
// ---------------------------------------------------------------------------
constexpr unsigned kListReady = 0x80000000u;

template <int THREADS, int R>
__device__ void list_marked(const int* __restrict__ uni, int base, int d_ff, unsigned* __restrict__ status,
                            int32_t* __restrict__ idx, int32_t* __restrict__ count, int* wl /* [THREADS/64] */,
                            unsigned* __restrict__ hdr, unsigned* __restrict__ fault) {
  static_assert(R <= THREADS && R % kWave == 0, "one thread per row");
  constexpr int W = THREADS / kWave;
  const int lane = lane_id(), wave = wave_id();
  const int i = threadIdx.x;
  const bool mine = i < R && base + i < d_ff && uni[i] != 0;
  const unsigned long long bm = __ballot(mine);
  if (lane == 0) wl[wave] = __builtin_popcountll(bm);
  __syncthreads();
  int n_g = 0, before = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int cw = wl[w];
    before += w < wave ? cw : 0;
    n_g += cw;
  }
  const int wg = blockIdx.x;
  const unsigned polls_hook = hdr[PI_WS_WAIT_POLLS], skip_hook = hdr[PI_WS_SKIP_PUBLISH];
  const int max_polls = polls_hook ? (int)polls_hook : kDefaultWaitPolls;
  if (threadIdx.x == 0 && skip_hook != (unsigned)wg + 1u)
    __hip_atomic_store(&status[wg], kListReady | (unsigned)n_g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int part = 0;
  bool expired = false;
  for (int p = threadIdx.x; p < wg; p += THREADS) {
    unsigned v = __hip_atomic_load(&status[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int spin = 0; !(v & kListReady) && spin < max_polls; ++spin) {
      __builtin_amdgcn_s_sleep(2);
      v = __hip_atomic_load(&status[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    expired |= !(v & kListReady);
    part += (int)(v & ~kListReady);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m, kWave);
  if (__ballot(expired) != 0ull && lane == 0) {
    raise_flag(fault, 1u);
    raise_flag(hdr + PI_WS_FLAGS, PI_FLAG_WAIT_EXPIRED);
  }
  __syncthreads();                                  // every wave has read wl[] above
  if (lane == 0) wl[wave] = part;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) off += wl[w];
  if (mine) idx[off + before + __builtin_popcountll(bm & ((1ull << lane) - 1ull))] = base + i;
  if (wg == (int)gridDim.x - 1 && threadIdx.x == 0) *count = off + n_g;
}

// ---------------------------------------------------------------------------
// k_tsplit: t = sum of the k splits of the first product in split order
// (fp32), and its fp16 split t_hi = fp16(t), t_lo = fp16(t - t_hi), stored
// step-major ([rank/128][nt][128]) for k_mp2.
// It also clears zero_n words at zero_ptr and the word at fault (the list
// counters of k_mp2 in the same call); NULL skips them.  A t_hi
// that is not finite in fp16 raises PI_FLAG_FP16_RANGE in *flags.
__global__ __launch_bounds__(256) void k_tsplit(const float* __restrict__ part, int n_split, int nt, int rank,
                                                float* __restrict__ t, f16* __restrict__ th, f16* __restrict__ tl,
                                                unsigned* __restrict__ zero_ptr, int zero_n,
                                                unsigned* __restrict__ fault, unsigned* __restrict__ flags) {
  const int n = nt * rank;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (zero_ptr != nullptr && e < zero_n) zero_ptr[e] = 0u;
  if (fault != nullptr && e == 0) *fault = 0u;
  if (__ballot(e < n) == 0ull) return;          // whole waves leave together (the flag check below is per wave)
  const bool live = e < n;
  const int ee = live ? e : 0;
  float v[16];
#pragma unroll
  for (int sp = 0; sp < 16; ++sp) v[sp] = sp < n_split ? part[(size_t)sp * n + ee] : 0.f;
  float sum = v[0];
#pragma unroll
  for (int sp = 1; sp < 16; ++sp)
    if (sp < n_split) sum += v[sp];
  raise_flag_if_any(flags, live && fp16_overflows(sum), PI_FLAG_FP16_RANGE);
  if (!live) return;
  t[e] = sum;
  const f16 hi = (f16)sum;
  const int j = e / rank, r = e - j * rank;
  const size_t o = ((size_t)(r / kMuK) * nt + j) * kMuK + r % kMuK;     // step-major, as TokStep reads
  th[o] = hi;
  tl[o] = (f16)(sum - (float)hi);
}

// ---------------------------------------------------------------------------
// k_mdown_wide: the down projection for 33-64 tokens.  k_mdown's 4 waves
// share one column tile and split the chunk, so every 128 columns re-read H
// from the cache hierarchy (at 64 tokens H is half as many bytes as the
// weight rows).  Here the 4 waves own 4 column tiles and walk the same list
// positions: pieces of kMwPiece k-steps of H (and of the list) are staged in
// LDS once per workgroup, and the next step's weight rows are in flight while
// the current step is multiplied.  Each wave writes its own partial sums.
// ---------------------------------------------------------------------------
constexpr int kMwPiece = 16;                 // k-steps (32 list positions each) per staged piece

template <typename WF, int NB, int CPL>
__global__ __launch_bounds__(kMdThreads) void k_mdown_wide(const void* __restrict__ w_dt, size_t scale_off, int d,
                                                           int d_ff, const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ count_ptr, int max_count,
                                                           const f16* __restrict__ h, int ldh, int nt, int n_chunks,
                                                           float* __restrict__ part,
                                                           unsigned long long* __restrict__ rows_read,
                                                           unsigned long long* __restrict__ up_rows_read) {
  constexpr int HU = kMwPiece * 32 / 8;       // 16-byte units of one token's H in a piece
  constexpr int HS = HU + 1;                  // per-token stride in LDS: tokens on different banks
  __shared__ u32x4 h_l[16 * NB * HS];
  __shared__ int rows_l[kMwPiece * 32];
  const int lane = lane_id();
  const int wave = wave_id();
  const int g = lane >> 4, n16 = lane & 15;
  const int cnt = clamp_count(count_ptr, max_count);
  const int ksteps = (cnt + 31) / 32;
  const int c = blockIdx.y;
  const int kc0 = (int)((long long)c * ksteps / n_chunks), kc1 = (int)((long long)(c + 1) * ksteps / n_chunks);
  if ((rows_read || up_rows_read) && blockIdx.x == 0 && threadIdx.x == 0) {     // the chunk's rows, counted once
    const int r0 = kc0 * 32 < cnt ? kc0 * 32 : cnt, r1 = kc1 * 32 < cnt ? kc1 * 32 : cnt;
    if (r1 > r0 && rows_read) atomicAdd(rows_read, (unsigned long long)(r1 - r0));
    if (r1 > r0 && up_rows_read) atomicAdd(up_rows_read, (unsigned long long)(r1 - r0));   // k_mup read them too
  }
  const int col = (blockIdx.x * kMdWaves + wave) * 16 * CPL + n16 * CPL;
  const bool cv = col < d;

  f32x4 acc[CPL][NB];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_rows = [&](int q, DownRows<WF, CPL>& wr) {
    int rows[8];
    bool ok[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = rows_l[q * 32 + g * 8 + r];
      ok[r] = cv && i >= 0;
      rows[r] = ok[r] ? i : 0;
    }
    wr.load(w_dt, scale_off, d, rows, ok, col);
  };

  for (int pb = kc0; pb < kc1; pb += kMwPiece) {
    const int np = kc1 - pb < kMwPiece ? kc1 - pb : kMwPiece;
    __syncthreads();                           // the previous piece is no longer read
    for (int e = threadIdx.x; e < np * 32; e += kMdThreads) {
      const int p = pb * 32 + e;
      const int i = p < cnt ? idx[p] : -1;
      rows_l[e] = (unsigned)i < (unsigned)d_ff ? i : -1;   // past the count or malformed: adds nothing
    }
    for (int e = threadIdx.x; e < 16 * NB * np * 4; e += kMdThreads) {
      const int t = e / (np * 4), u = e - t * (np * 4);
      const int p = pb * 32 + u * 8;
      h_l[t * HS + u] = p < cnt ? ld16(h + (size_t)t * ldh + p) : u32x4{0, 0, 0, 0};
    }
    __syncthreads();
    DownRows<WF, CPL> cur, nxt;
    load_rows(0, cur);
    for (int q = 0; q < np; ++q) {
      if (q + 1 < np) load_rows(q + 1, nxt);
      u32x4 a[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) a[nb] = h_l[(nb * 16 + n16) * HS + q * 4 + g];
#pragma unroll
      for (int qq = 0; qq < CPL / 8; ++qq) {
        u32x4 rw[8], bt[8];
        cur.group(qq, rw);
        transpose8x8(rw, bt);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[8 * qq + j][nb] = mfma(a[nb], bt[j], acc[8 * qq + j][nb]);
      }
      if (q + 1 < np) cur = nxt;
    }
  }

  if (cv) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = nb * 16 + 4 * g + i;
        if (t < nt) {
          float* dst = part + ((size_t)c * nt + t) * d + col;
#pragma unroll
          for (int j = 0; j < CPL; j += 4)
            *reinterpret_cast<f32x4*>(dst + j) =
                f32x4{acc[j][nb][i], acc[j + 1][nb][i], acc[j + 2][nb][i], acc[j + 3][nb][i]};
        }
      }
  }
}

// 8 rows x 4 fp16 columns (each row's 4 columns in one u32x2) -> 4 B
// operands of 8 rows each, as transpose8x8 does for 8 columns.
__device__ __forceinline__ void transpose8x4(const u32x2 (&in)[8], u32x4 (&out)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    unsigned o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const unsigned lo = j < 2 ? in[2 * m].x : in[2 * m].y, hi = j < 2 ? in[2 * m + 1].x : in[2 * m + 1].y;
      o[m] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    out[j] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

// k_mdown_w4 (fp16 rows, 33-64 tokens): k_mdown_wide with 4 columns per lane
// instead of 8.  Half the accumulators leave room for more rows in flight:
// three register stages over whole pieces of kW4Piece k-steps (pipeline3x;
// a chunk's last, partial piece takes pipeline2), every lane loading
// (entries past the count or malformed read row 0, columns past d read
// column 0, both zeroed when the operands are formed), held to 2 waves per
// SIMD.  With 256 columns per workgroup 16 list chunks still give 512
// workgroups at the Falcon width, so the partial sums that the merge reads
// back are half as many bytes as with 32 chunks.
constexpr int kW4Piece = 18;                 // k-steps per staged piece: a multiple of the 3 row stages

template <int NB>
__global__ __launch_bounds__(kMdThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_mdown_w4(const f16* __restrict__ w_dt, int d, int d_ff,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ count_ptr, int max_count,
                                                         const f16* __restrict__ h, int ldh, int nt, int n_chunks,
                                                         float* __restrict__ part,
                                                         unsigned long long* __restrict__ rows_read,
                                                         unsigned long long* __restrict__ up_rows_read) {
  constexpr int CPL = 4;
  constexpr int HU = kW4Piece * 32 / 8;       // 16-byte units of one token's H in a piece
  constexpr int HS = HU + 1;                  // per-token stride in LDS: tokens on different banks
  __shared__ u32x4 h_l[16 * NB * HS];
  __shared__ int rows_l[kW4Piece * 32];
  const int lane = lane_id();
  const int wave = wave_id();
  const int g = lane >> 4, n16 = lane & 15;
  const int cnt = clamp_count(count_ptr, max_count);
  const int ksteps = (cnt + 31) / 32;
  // the column tiles of a chunk, which all read its H, run on one XCD
  int tile, c;
  xcd_grouped(tile, c);
  const int kc0 = (int)((long long)c * ksteps / n_chunks), kc1 = (int)((long long)(c + 1) * ksteps / n_chunks);
  if ((rows_read || up_rows_read) && tile == 0 && threadIdx.x == 0) {     // the chunk's rows, counted once
    const int r0 = kc0 * 32 < cnt ? kc0 * 32 : cnt, r1 = kc1 * 32 < cnt ? kc1 * 32 : cnt;
    if (r1 > r0 && rows_read) atomicAdd(rows_read, (unsigned long long)(r1 - r0));
    if (r1 > r0 && up_rows_read) atomicAdd(up_rows_read, (unsigned long long)(r1 - r0));   // k_mup read them too
  }
  const int col = (tile * kMdWaves + wave) * 16 * CPL + n16 * CPL;
  const bool cv = col < d;
  const int colc = cv ? col : 0;

  f32x4 acc[CPL][NB];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    u32x2 v[8];
    bool ok[8];
    int q;
  };
  auto load_rows = [&](Stage& S, int q) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = rows_l[q * 32 + g * 8 + r];
      S.ok[r] = cv && i >= 0;
      S.v[r] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2*>(w_dt + (size_t)(S.ok[r] ? i : 0) * d + colc));
    }
    S.q = q;
  };
  auto mul_rows = [&](const Stage& S) {
    u32x4 a[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) a[nb] = h_l[(nb * 16 + n16) * HS + S.q * 4 + g];
    u32x2 rw[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) rw[r] = S.ok[r] ? S.v[r] : u32x2{0, 0};
    u32x4 bt[CPL];
    transpose8x4(rw, bt);
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[j][nb] = mfma(a[nb], bt[j], acc[j][nb]);
  };

  for (int pb = kc0; pb < kc1; pb += kW4Piece) {
    const int np = kc1 - pb < kW4Piece ? kc1 - pb : kW4Piece;
    __syncthreads();                           // the previous piece is no longer read
    for (int e = threadIdx.x; e < np * 32; e += kMdThreads) {
      const int p = pb * 32 + e;
      const int i = p < cnt ? idx[p] : -1;
      rows_l[e] = (unsigned)i < (unsigned)d_ff ? i : -1;   // past the count or malformed: adds nothing
    }
    for (int e = threadIdx.x; e < 16 * NB * np * 4; e += kMdThreads) {
      const int t = e / (np * 4), u = e - t * (np * 4);
      const int p = pb * 32 + u * 8;
      h_l[t * HS + u] = p < cnt ? ld16(h + (size_t)t * ldh + p) : u32x4{0, 0, 0, 0};
    }
    __syncthreads();
    Stage S0, S1, S2;
    if (np == kW4Piece)
      pipeline3x(0, np, S0, S1, S2, load_rows, mul_rows);
    else
      pipeline2(0, np, S0, S1, load_rows, mul_rows);
  }

  if (cv) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = nb * 16 + 4 * g + i;
        if (t < nt)
          *reinterpret_cast<f32x4*>(part + ((size_t)c * nt + t) * d + col) =
              f32x4{acc[0][nb][i], acc[1][nb][i], acc[2][nb][i], acc[3][nb][i]};
      }
  }
}

// k_mp2: the second product with t_hi and t_lo staged in LDS (read from
// the cache once per workgroup, not once per 16-row block: at 64 tokens as
// many bytes as the p2 rows themselves).  A workgroup of 8 waves owns 128
// rows (16 per wave), walks all of k itself (one accumulator per token
// block, no cross-wave sum), and stages a piece of k steps of t_hi and t_lo
// at a time.  The p2 rows are loaded in the transposed pattern (RowStepTU:
// 256 contiguous bytes of a row per 16 lanes).  With 1-2 token blocks (up
// to 32 tokens) the pieces are kMpPiece steps and two steps of rows stay in
// flight while two are multiplied; with 3-4 blocks the pieces are 2 steps
// (so that the staged t leaves LDS for the row buffers) and each wave keeps
// the next step in flight (a whole piece in flight was slower: the staging
// loads then queue behind it).  Measured at Falcon shape against a 4-wave
// form that split k over the waves and re-read t per step (predictor,
// stand-alone call): 4 tokens 24.0 -> 22.5 us, 8 tokens 24.7 -> 22.8 us,
// 24 tokens 37.2 -> 27.7 us; 64 tokens, operand-pattern rows -> transposed,
// 41.2 -> 39.8 us.
constexpr int kMpThreads = 512;
constexpr int kMpRows = kMpThreads / kWave * 16;
constexpr int kMpPiece = 4;

template <int NB>
__global__ __launch_bounds__(kMpThreads) void k_mp2(const f16* __restrict__ p2, const float* __restrict__ c,
                                                         const f16* __restrict__ th, const f16* __restrict__ tl,
                                                         int rank, int d_ff, int nt, float theta,
                                                         uint8_t* __restrict__ mask, float* __restrict__ logits,
                                                         uint8_t* __restrict__ umask, int umask_first,
                                                         unsigned* __restrict__ status, int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ count, unsigned* __restrict__ hdr,
                                                         unsigned* __restrict__ fault) {
  constexpr int LU = 16 * NB * kMuK / 8;          // 16-byte units of one step (all token slots)
  constexpr int PC = NB <= 2 ? kMpPiece : 2;      // k-steps per staged piece
  __shared__ u32x4 th_l[PC][16 * NB * kTokStride], tl_l[PC][16 * NB * kTokStride];
  __shared__ int uni[kMpRows];                    // union over the tile's tokens
  __shared__ int wl[kMpThreads / kWave];
  if (threadIdx.x < kMpRows) uni[threadIdx.x] = 0;
  const int lane = lane_id(), wave = wave_id();
  const int g = lane >> 4, n16 = lane & 15;
  const int base = blockIdx.x * kMpRows;
  const int r0 = base + wave * 16;
  int row[1];
  bool rv[1];
  row[0] = r0 + n16;
  rv[0] = row[0] < d_ff;
  if (!rv[0]) row[0] = 0;
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ns = rank / kMuK;
  const int su = nt * (kMuK / 8);                 // units of one step of the nt real tokens
  const bool whole = ns % PC == 0;
  if (whole) {
    // Whole pieces: the unrolled branch-free pipeline of k_mup_wide.  Every
    // lane loads (rows past d_ff read row 0 and are never stored; token
    // slots past nt read a valid unit and are zeroed in LDS), and the next
    // piece's t units and first rows go out during the piece's last step.
    constexpr int XU = PC * LU / kMpThreads;   // units of t_hi (and of t_lo) per thread per piece
    u32x4 hr[XU], lr[XU];
    auto t_load = [&](int p0) {
#pragma unroll
      for (int k = 0; k < XU; ++k) {
        const int e = threadIdx.x + kMpThreads * k;
        const int q = e / LU, r = e - q * LU;
        const size_t o = (size_t)(p0 + q) * nt * kMuK + (size_t)(r < su ? r : su - 1) * 8;
        hr[k] = ld16(th + o);
        lr[k] = ld16(tl + o);
      }
    };
    auto t_store = [&]() {
#pragma unroll
      for (int k = 0; k < XU; ++k) {
        const int e = threadIdx.x + kMpThreads * k;
        const int q = e / LU, r = e - q * LU;
        const int u = (r >> 4) * kTokStride + (r & 15);
        th_l[q][u] = r < su ? hr[k] : u32x4{0, 0, 0, 0};
        tl_l[q][u] = r < su ? lr[k] : u32x4{0, 0, 0, 0};
      }
    };
    // p2 rows in the transposed pattern (256 contiguous bytes of a row per
    // 16 lanes), moved into the operand layout through this wave's LDS buffer
    // (with 3-4 token blocks the pieces are 2 k-steps, so that the staged t
    // leaves LDS for the buffers)
    constexpr bool TU = NB >= 1;   // every token count (written so that it depends on NB)
    __shared__ u32x4 w_l[TU ? kMpThreads / kWave : 1][TU ? 16 * kTStride : 1];
    int rowt[1][4];
    bool rvt[1][4];
    rows_for_load<1>(row, rv, lane, rowt, rvt);
    bool all[1] = {true};
    using Rows = typename std::conditional<TU, RowStepTU<1>, RowStep<f16, 1>>::type;
    Rows S0, S1;
    auto rows = [&](Rows& S, int st) {
      if constexpr (TU)
        S.load(p2, rowt, rank, st * kMuK, lane);
      else
        S.load(p2, 0, row, all, rank, st * kMuK, g);
    };
    auto step = [&](const Rows& S, int q) {
      u32x4 a[4];
      if constexpr (TU)
        S.operands(0, rvt, &w_l[TU ? wave : 0][0], lane, a);
      else
        S.operands(0, a);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 bh[NB], bl[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int u = (nb * 16 + n16) * kTokStride + 4 * s + g;
          bh[nb] = th_l[q][u];
          bl[nb] = tl_l[q][u];
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[nb] = mfma(a[s], bh[nb], acc[nb]);
          acc[nb] = mfma(a[s], bl[nb], acc[nb]);
        }
      }
    };
    auto piece = [&](int p0, auto has_next) {
      static_assert(PC == 4 || PC == 2, "the unrolled piece is 2 or 4 steps");
      rows(S1, p0 + 1);
      if constexpr (PC == 4) {
        step(S0, 0);
        rows(S0, p0 + 2);
        step(S1, 1);
        rows(S1, p0 + 3);
      }
      step(S0, PC - 2);
      if constexpr (decltype(has_next)::value) {
        t_load(p0 + PC);
        rows(S0, p0 + PC);
      }
      step(S1, PC - 1);
      if constexpr (decltype(has_next)::value) {
        __syncthreads();                               // every wave is done with this piece's t
        t_store();
        __syncthreads();
      }
    };
    // 1-2 token blocks (one workgroup per CU at Falcon shape, registers to
    // spare): stages of two steps, so two steps of rows are in flight while
    // two are multiplied
    Rows D0[2], D1[2];
    auto piece2 = [&](int p0, auto has_next) {
      static_assert(kMpPiece == 4, "two stages of two steps");
      rows(D1[0], p0 + 2);
      rows(D1[1], p0 + 3);
      step(D0[0], 0);
      step(D0[1], 1);
      if constexpr (decltype(has_next)::value) {
        t_load(p0 + kMpPiece);
        rows(D0[0], p0 + kMpPiece);
        rows(D0[1], p0 + kMpPiece + 1);
      }
      step(D1[0], 2);
      step(D1[1], 3);
      if constexpr (decltype(has_next)::value) {
        __syncthreads();                               // every wave is done with this piece's t
        t_store();
        __syncthreads();
      }
    };
    t_load(0);
    if constexpr (NB <= 2) {
      rows(D0[0], 0);
      rows(D0[1], 1);
    } else {
      rows(S0, 0);
    }
    t_store();
    __syncthreads();
    int p0 = 0;
    if constexpr (NB <= 2) {
      for (; p0 + kMpPiece < ns; p0 += kMpPiece) piece2(p0, std::true_type{});
      piece2(p0, std::false_type{});
    } else {
      for (; p0 + PC < ns; p0 += PC) piece(p0, std::true_type{});
      piece(p0, std::false_type{});
    }
  }
  for (int p0 = 0; p0 < ns && !whole; p0 += PC) {
    const int np = ns - p0 < PC ? ns - p0 : PC;
    RowStep<f16, 1> cur;
    cur.load(p2, 0, row, rv, rank, p0 * kMuK, g);  // the first step's rows go out before the staging
    __syncthreads();                                // the previous piece is no longer read
    for (int e = threadIdx.x; e < np * LU; e += kMpThreads) {
      const int q = e / LU, r = e - q * LU;         // token slots past nt hold zeros
      const size_t o = (size_t)(p0 + q) * nt * kMuK + (size_t)r * 8;
      const int u = (r >> 4) * kTokStride + (r & 15);
      th_l[q][u] = r < su ? ld16(th + o) : u32x4{0, 0, 0, 0};
      tl_l[q][u] = r < su ? ld16(tl + o) : u32x4{0, 0, 0, 0};
    }
    __syncthreads();
    for (int q = 0; q < np; ++q) {
      RowStep<f16, 1> nxt;
      if (q + 1 < np) nxt.load(p2, 0, row, rv, rank, (p0 + q + 1) * kMuK, g);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 bh[NB], bl[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int u = (nb * 16 + n16) * kTokStride + 4 * s + g;
          bh[nb] = th_l[q][u];
          bl[nb] = tl_l[q][u];
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[nb] = mfma(cur.v[0][s], bh[nb], acc[nb]);
          acc[nb] = mfma(cur.v[0][s], bl[nb], acc[nb]);
        }
      }
      if (q + 1 < np) cur = nxt;
    }
  }
  __syncthreads();                                  // uni[] cleared before any mark
  // lane holds rows r0 + 4g .. +3 for token nb * 16 + n16
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int j = nb * 16 + n16;
    const int r = r0 + 4 * g;
    if (j < nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (r + i < d_ff) {
          const float l = acc[nb][i] + c[r + i];
          if (mask) mask[(size_t)j * d_ff + r + i] = l > theta ? 1 : 0;
          if (logits) logits[(size_t)j * d_ff + r + i] = l;
          if (l > theta) uni[r + i - base] = 1;     // every writer stores the same value
        }
      }
    }
  }
  if (umask) {
    __syncthreads();
    const int i = threadIdx.x;
    if (i < kMpRows && base + i < d_ff) {
      const int u = uni[i] | (umask_first ? 0 : umask[base + i]);
      umask[base + i] = (uint8_t)u;
      uni[i] = u;
    }
    if (idx) {
      __syncthreads();
      list_marked<kMpThreads, kMpRows>(uni, base, d_ff, status, idx, count, wl, hdr, fault);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int kMfmaTile = kMfmaTokens;

// Columns per lane of k_mdown.  Q4_0 at up to 32 tokens: 16 (a column tile
// of 256, 512 workgroups at d = 8192 with 16 chunks); measured at Q4_0
// Falcon batch 8: 32 columns (256 workgroups) 4 us slower per layer, 8
// columns 8 us slower.
template <typename WF>
constexpr int down_cpl(int nb) {
  return std::is_same<WF, Q4>::value ? (nb <= 1 ? 16 : 8) : 8;
}

// List chunks of the down projection (partial sums per chunk): the wide
// kernel (33-64 tokens) needs 32 for 2 workgroups per CU.
// Token blocks (of 16) from which the wide kernels (k_mup_wide + k_mfin,
// k_mdown_wide) take over: 3 for fp16 rows, 2 for Q4_0 rows.
template <typename WF>
constexpr int wide_from() { return std::is_same<WF, Q4>::value ? 2 : 3; }
int wide_nb(int wtype) { return wtype == 2 ? 2 : 3; }

int mfma_chunks(int wtype, int nb) {
  if (nb >= wide_nb(wtype)) return wtype == 2 ? 32 : 16;   // fp16: k_mdown_w4, 256 columns per workgroup
  return wtype == 2 ? 16 : 8;
}

// k splits of the predictor's first product: about 4 steps of 128 per split.
int pred_splits(int d) {
  const int ns = d / kMuK;
  int sp = ns / 4;
  return sp < 1 ? 1 : (sp > 16 ? 16 : sp);
}

int ldh_of(int d_ff) { return (d_ff + kMuRows - 1) / kMuRows * kMuRows; }

size_t up256(size_t b) { return (b + 255) / 256 * 256; }

// Sparse FFN workspace of one token tile: H [64][ldh] fp16, then the
// step-major activations [d/128][nt][128] fp16, then (33-64 tokens) the
// up projection's split partial sums, up and gate, [kMxSplit][64][ldz] fp32.
size_t h_region(int d_ff, int nb) { return up256((size_t)16 * nb * ldh_of(d_ff) * sizeof(f16)); }
int ldz_of(int d_ff) { return ldh_of(d_ff); }
size_t zp_region(int d_ff) { return up256((size_t)kMxSplit * kMfmaTokens * ldz_of(d_ff) * sizeof(float)); }
size_t wide_region(int d_ff) { return 2 * zp_region(d_ff); }
size_t xs_region(int d) { return up256((size_t)kMfmaTile * d * sizeof(f16)); }

struct WideWs {
  float* zp;
  float* zg;
};
WideWs wide_ws(const SparseArgs& a) {
  char* base = reinterpret_cast<char*>(a.h) + h_region(a.d_ff, 4) + xs_region(a.d);
  return {reinterpret_cast<float*>(base), reinterpret_cast<float*>(base + zp_region(a.d_ff))};
}

template <typename WF, int ACT, int NB>
hipError_t launch_mup(const SparseArgs& a, const f16* x, int nt, f16* h, int ldh, hipStream_t s) {
  if constexpr (NB >= wide_from<WF>()) {
    const int grid = (a.max_count + kMxRows - 1) / kMxRows;
    if (grid == 0) return hipSuccess;
    const size_t so = std::is_same<WF, Q4>::value ? (size_t)a.d_ff * (a.d / 32) * 16 : 0;
    const WideWs w = wide_ws(a);
    const int ldz = ldz_of(a.d_ff);
    hipLaunchKernelGGL((k_mup_wide<WF, ACT, NB>), dim3(grid, kMxSplit), dim3(kMxThreads), 0, s, a.w_up, a.w_gate, so,
                       x, a.d, a.d_ff, nt, a.idx, a.count, a.max_count, w.zp, w.zg, ldz);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float* bias = ACT == ACT_REGLU ? a.b_gate : a.b_up;
    const int n = nt * (grid * kMxRows / 4);       // covers nt x (count rounded up to 64) / 4
    hipLaunchKernelGGL((k_mfin<ACT>), dim3((n + 255) / 256), dim3(256), 0, s, w.zp, w.zg, bias, a.idx, a.count,
                       a.max_count, a.d_ff, nt, ldz, h, ldh, a.flags);
    return hipGetLastError();
  }
  const int rows_per_wg = 16 * mup_mb<NB>();
  const int grid = (a.max_count + rows_per_wg - 1) / rows_per_wg;
  if (grid == 0) return hipSuccess;
  const float* bias = ACT == ACT_REGLU ? a.b_gate : a.b_up;
  const size_t so = std::is_same<WF, Q4>::value ? (size_t)a.d_ff * (a.d / 32) * 16 : 0;
  hipLaunchKernelGGL((k_mup<WF, ACT, NB>), dim3(grid), dim3(kMuThreads), 0, s, a.w_up, a.w_gate, so, bias, x, a.d,
                     a.d_ff, nt, a.idx, a.count, a.max_count, h, ldh, a.flags);
  return hipGetLastError();
}

template <typename WF, int NB>
hipError_t run_mtile(const SparseArgs& a, int t0, int nt, hipStream_t s) {
  const f16* x = static_cast<const f16*>(a.x) + (size_t)t0 * a.d;
  f16* h = reinterpret_cast<f16*>(a.h);
  const int ldh = ldh_of(a.d_ff);
  hipError_t e;
  if (a.xs_pre != nullptr && t0 == 0 && nt == a.n_tok) {
    x = static_cast<const f16*>(a.xs_pre);          // the predictor's step-major copy of the same tile
  } else {
    f16* xs = reinterpret_cast<f16*>(reinterpret_cast<char*>(a.h) + h_region(a.d_ff, 4));
    const int n_groups = nt * a.d / 8;
    hipLaunchKernelGGL((k_xstep<std::is_same<WF, Q4>::value>), dim3((n_groups + 255) / 256), dim3(256), 0, s, x, nt,
                       a.d, xs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    x = xs;
  }
  if (a.act == ACT_REGLU)
    e = launch_mup<WF, ACT_REGLU, NB>(a, x, nt, h, ldh, s);
  else if (a.act == ACT_RELU2)
    e = launch_mup<WF, ACT_RELU2, NB>(a, x, nt, h, ldh, s);
  else
    e = launch_mup<WF, ACT_RELU, NB>(a, x, nt, h, ldh, s);
  if (e != hipSuccess) return e;
  constexpr int CPL = down_cpl<WF>(NB);
  const int chunks = mfma_chunks(a.wtype, NB);
  const size_t so = std::is_same<WF, Q4>::value ? (size_t)a.d_ff * (a.d / 32) * 16 : 0;
  if constexpr (NB >= wide_from<WF>() && std::is_same<WF, f16>::value) {
    const int tile = kMdWaves * 16 * 4;
    const dim3 grid((a.d + tile - 1) / tile, chunks);
    hipLaunchKernelGGL((k_mdown_w4<NB>), grid, dim3(kMdThreads), 0, s, static_cast<const f16*>(a.w_down_t), a.d,
                       a.d_ff, a.idx, a.count, a.max_count, h, ldh, nt, chunks, a.part, a.rows_read,
                       a.up_rows_read);
  } else if constexpr (NB >= wide_from<WF>()) {
    const int tile = kMdWaves * 16 * CPL;
    const dim3 grid((a.d + tile - 1) / tile, chunks);
    hipLaunchKernelGGL((k_mdown_wide<WF, NB, CPL>), grid, dim3(kMdThreads), 0, s, a.w_down_t, so, a.d, a.d_ff, a.idx,
                       a.count, a.max_count, h, ldh, nt, chunks, a.part, a.rows_read,
                       a.up_rows_read);
  } else {
    const dim3 grid((a.d + 16 * CPL - 1) / (16 * CPL), chunks);
    hipLaunchKernelGGL((k_mdown<WF, NB, CPL>), grid, dim3(kMdThreads), 0, s, a.w_down_t, so, a.d, a.d_ff, a.idx,
                       a.count, a.max_count, h, ldh, nt, chunks, a.part, a.rows_read,
                       a.up_rows_read);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t yoff = (size_t)t0 * a.d * (a.ytype == 1 ? 2 : 4);
  return launch_merge(a.part, chunks, nt * a.d, static_cast<char*>(a.y) + yoff, a.ytype, a.fault, s);
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

// Workspace of one predictor token tile: the k-split partials, t_hi, t_lo
// and the step-major copy of the tokens.

// List (nullable idx): the union mask is also compacted into idx / count in
// the second product's kernel, which needs at most n_status counters.
struct PredList {
  unsigned* status;
  int n_status;
  int32_t* idx;
  int32_t* count;
  unsigned* hdr;     // workspace header: flags and the wait hooks
  unsigned* fault;   // per-call fault word of the list
};

template <int NB>
hipError_t run_ptile(const f16* p1, const f16* p2, const float* c, const f16* x, int nt, int d, int rank, int d_ff,
                     float theta, float* t, char* ws, uint8_t* mask, float* logits, uint8_t* umask, int first,
                     const PredList& pl, bool xs_block, const f16** xs_out, hipStream_t s) {
  const int splits = pred_splits(d);
  float* part = reinterpret_cast<float*>(ws);
  f16* th = reinterpret_cast<f16*>(ws + up256((size_t)splits * kMfmaTile * rank * sizeof(float)));
  f16* tl = th + (size_t)kMfmaTile * rank;
  f16* xs = tl + (size_t)kMfmaTile * rank;
  hipLaunchKernelGGL((k_mp1<NB>), dim3((rank + kMuRows - 1) / kMuRows, splits), dim3(kMuThreads), 0, s, p1, x, d,
                     rank, nt, part, xs, xs_block ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (xs_out) *xs_out = xs;
  const int grid2 = (d_ff + kMpRows - 1) / kMpRows;
  const bool list = pl.idx != nullptr && umask != nullptr;
  if (list && (pl.status == nullptr || pl.count == nullptr || pl.hdr == nullptr || pl.fault == nullptr ||
               grid2 > pl.n_status))
    return hipErrorInvalidValue;
  const int n = nt * rank;
  const int zn = list ? grid2 : 0;
  const int nz = n > zn ? n : zn;
  hipLaunchKernelGGL(k_tsplit, dim3((nz + 255) / 256), dim3(256), 0, s, part, splits, nt, rank, t, th, tl,
                     list ? pl.status : nullptr, zn, list ? pl.fault : nullptr, pl.hdr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned* st = list ? pl.status : nullptr;
  int32_t* li = list ? pl.idx : nullptr;
  int32_t* lc = list ? pl.count : nullptr;
  unsigned* fl = list ? pl.fault : nullptr;
  hipLaunchKernelGGL((k_mp2<NB>), dim3(grid2), dim3(kMpThreads), 0, s, p2, c, th, tl, rank, d_ff, nt, theta, mask,
                     logits, umask, first, st, li, lc, pl.hdr, fl);
  return hipGetLastError();
}

}  // namespace

// fp16 weights take the matrix cores from 3 tokens on (measured at Falcon
// shape, layer-tokens/s of the list path -> matrix cores: 3 tokens 26.9k ->
// 35.8k, 5 tokens 23.8k -> 47.5k, 8 tokens 23.8k -> 68.6k); Q4_0 from the
// first token count past its list-path tile.
bool mfma_path(int wtype, int d, int n_tok) {
  if (wtype != 1 && wtype != 2) return false;     // fp16 and Q4_0 weights
  if (d % kMuK != 0) return false;
  return n_tok > (wtype == 1 ? 2 : sparse_tile(wtype, d));
}

void mfma_workspace(int wtype, int d, int d_ff, int n_tok, size_t* h_bytes, size_t* part_bytes) {
  const int nt = n_tok < kMfmaTile ? n_tok : kMfmaTile;
  const int nb = (nt + 15) / 16;
  (void)nb;
  *h_bytes = h_region(d_ff, 4) + xs_region(d) + (nb >= wide_nb(wtype) ? wide_region(d_ff) : 0);
  *part_bytes = (size_t)mfma_chunks(wtype, nb) * nt * d * sizeof(float);
}

hipError_t launch_sparse_ffn_mfma(const SparseArgs& a, hipStream_t s) {
  if (a.wtype == 2) return run_mall<Q4>(a, s);
  return run_mall<f16>(a, s);
}

}  // namespace pi

namespace pi {

// From 3 tokens on, the matrix cores beat the VALU predictor (whose second
// stage re-reads t from LDS for every weight).  The choice depends only on
// the predictor and n_tok, so pi_predict and pi_layer always agree.
bool pred_mfma_path(int wtype, int d, int rank, int n_tok) {
  return wtype == 1 && d % kMuK == 0 && rank % kMuK == 0 && n_tok > 2;
}

size_t pred_mfma_part_bytes(int d, int rank, int) {
  return up256((size_t)pred_splits(d) * kMfmaTile * rank * sizeof(float)) +
         (2 * (size_t)kMfmaTile * rank + (size_t)kMfmaTile * d) * sizeof(f16);
}

hipError_t launch_predict_mfma(const void* p1, const void* p2, const float* c, const void* x, int n_tok, int d,
                               int rank, int d_ff, float theta, float* t, void* ws, uint8_t* mask, float* logits,
                               uint8_t* umask, unsigned* status, int n_status, int32_t* idx, int32_t* count,
                               unsigned* hdr, unsigned* fault, bool xs_block, const void** xs_out, hipStream_t s) {
  if (xs_out) *xs_out = nullptr;
  for (int t0 = 0; t0 < n_tok; t0 += kMfmaTile) {
    const int nt = n_tok - t0 < kMfmaTile ? n_tok - t0 : kMfmaTile;
    const bool last = t0 + nt == n_tok;
    const PredList pl{status, n_status, last ? idx : nullptr, count, hdr, fault};
    const f16* xs = nullptr;
    const f16* xt = static_cast<const f16*>(x) + (size_t)t0 * d;
    float* tt = t + (size_t)t0 * rank;
    uint8_t* mt = mask ? mask + (size_t)t0 * d_ff : nullptr;
    const int first = t0 == 0;
    float* lt = logits ? logits + (size_t)t0 * d_ff : nullptr;
    const f16* a = static_cast<const f16*>(p1);
    const f16* b = static_cast<const f16*>(p2);
    char* wsp = static_cast<char*>(ws);
    hipError_t e;
    if (nt <= 16)
      e = run_ptile<1>(a, b, c, xt, nt, d, rank, d_ff, theta, tt, wsp, mt, lt, umask, first, pl, xs_block, &xs, s);
    else if (nt <= 32)
      e = run_ptile<2>(a, b, c, xt, nt, d, rank, d_ff, theta, tt, wsp, mt, lt, umask, first, pl, xs_block, &xs, s);
    else if (nt <= 48)
      e = run_ptile<3>(a, b, c, xt, nt, d, rank, d_ff, theta, tt, wsp, mt, lt, umask, first, pl, xs_block, &xs, s);
    else
      e = run_ptile<4>(a, b, c, xt, nt, d, rank, d_ff, theta, tt, wsp, mt, lt, umask, first, pl, xs_block, &xs, s);
    if (e != hipSuccess) return e;
    if (xs_out && t0 == 0 && last) *xs_out = xs;     // one tile: its step-major copy stays valid
  }
  return hipSuccess;
}

}  // namespace pi
