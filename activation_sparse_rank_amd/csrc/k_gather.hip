// Neuron-aware sparse FFN over the active neurons (fp16 / fp32 weights).
//
// [QB] "Что такое «разреженная активация»?": only the activated neurons are
// computed; the others add nothing.  [QB] "Гибридный дизайн вывода CPU/GPU"
// and "Общая архитектура PowerInfer": the partial results of separately
// computed neuron groups are merged into the layer output.  Here the groups
// are chunks of the active-neuron list on one GPU and the merge is a
// fixed-order sum.
//
// Kernels:
//   k_up       -- list path: one wave per listed neuron; its w_up (and w_gate)
//                 row is read with 16-byte loads (1 KB per wave instruction),
//                 dotted with x, summed across the wave and activated; h is
//                 stored by neuron number.
//   k_pred_up  -- layer path: the second predictor product, the up
//                 projection and the compaction fused (see below).
//   k_down     -- a workgroup per (column slice, chunk of the list): each wave
//                 accumulates h_i * w_down_t[i] over its slice for the rows
//                 of the chunk, the 8 waves are summed in LDS in wave order,
//                 and the chunk's partial sums go to the workspace.
//   k_merge    -- y = the chunks' partial sums added in chunk order.
// No atomics take part in any sum and every sum has a fixed order, so y is
// bitwise reproducible, and the list and layer paths give identical bits.
// All kernels but the merge are bound by HBM bandwidth on the weight rows.
#include <type_traits>

#include "pi.h"
#include "predict_device.h"

namespace pi {
namespace {

template <typename W>
__device__ __forceinline__ float dotc(u32x4 w, u32x4 x, float acc);
template <>
__device__ __forceinline__ float dotc<f16>(u32x4 w, u32x4 x, float acc) { return dot8_f16(w, x, acc); }
template <>
__device__ __forceinline__ float dotc<float>(u32x4 w, u32x4 x, float acc) { return dot4_f32(w, x, acc); }

template <int ACT>
__device__ __forceinline__ float activate(float up, float gate) {
  if (ACT == ACT_REGLU) return (gate > 0.f ? gate : 0.f) * up;
  const float r = up > 0.f ? up : 0.f;
  return ACT == ACT_RELU2 ? r * r : r;
}

// Stage the token tile of x ([nt][d] elements, 16-byte chunks) into LDS.
template <typename W>
__device__ __forceinline__ void stage_x(const char* __restrict__ xb, u32x4* x_lds, int nt, int d) {
  const int tot = nt * (d / (16 / (int)sizeof(W)));
  for (int e = threadIdx.x; e < tot; e += blockDim.x) x_lds[e] = ld16(xb + (size_t)e * 16);
}

// ---------------------------------------------------------------------------
// Q4_0 rows.  A row of d weights is d/32 blocks; block b has a 16-byte code
// group (at codes + (row*nb + b)*16) and an fp16 scale (at scales +
// (row*nb + b)*2), in the repacked layout of k_q4.hip.  Word k, slot u of a
// code group holds the codes of the weight pair (8k+2u, 8k+2u+1); OR-ing the
// two 4-bit codes into the mantissas of 1024.0 and subtracting 1032.0 gives
// the exact fp16 pair (q-8, q'-8), which v_dot2_f32_f16 multiplies with the
// matching pair of activations.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x2 q4_pair(unsigned w, int u) {
  const unsigned bits = ((w >> (4 * u)) & 0x000F000Fu) | 0x64006400u;
  return as_h2(bits) - f16x2{(f16)1032.0f, (f16)1032.0f};
}

// sum over one block of (q-8) * x in fp32 (exact fp16 products); xq are the
// block's four 16-byte chunks of activations.
__device__ __forceinline__ float dot_q4(u32x4 cw, const u32x4 (&xq)[4]) {
  float acc = 0.f;
  const unsigned w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned xw[4] = {xq[k].x, xq[k].y, xq[k].z, xq[k].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_fdot2(q4_pair(w[k], u), as_h2(xw[u]), acc, false);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Row dots in a fixed order.  A row's units -- 16-byte chunks of fp16 or fp32
// weights, or Q4_0 blocks -- are split into 4 parts, part q = units
// [n*q/4, n*(q+1)/4).  In a part, lane l adds the units c_q + l, c_q + l + 64,
// ... in order; the lane sums are added over the wave (butterfly, so every
// lane holds the same bits); the 4 part sums are added in order 0..3.  The
// list path computes the 4 parts of a row in one wave; the layer path gives
// part q of every active row of a workgroup to its wave q.  Both get the same
// bits, and a workgroup with many active rows keeps all 4 waves loading.
// ---------------------------------------------------------------------------
template <typename WF>
__device__ __forceinline__ int row_units(int d) {
  return std::is_same<WF, Q4>::value ? d / 32 : d / (16 / (int)sizeof(WF));
}

struct UnitW {
  u32x4 w;
  float sc;     // Q4_0 block scale
};

template <typename WF>
__device__ __forceinline__ UnitW load_unit(const void* w, size_t scale_off, int row, int u, int d, bool ok) {
  UnitW r;
  if constexpr (std::is_same<WF, Q4>::value) {
    const size_t blk = (size_t)row * (d / 32) + u;
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    r.w = ok ? ld_nt(wb + blk * 16) : u32x4{0, 0, 0, 0};
    r.sc = ok ? (float)reinterpret_cast<const f16*>(wb + scale_off)[blk] : 0.f;
  } else {
    r.w = ok ? ld_nt(static_cast<const char*>(w) + (size_t)row * d * sizeof(WF) + (size_t)u * 16)
             : u32x4{0, 0, 0, 0};
    r.sc = 0.f;
  }
  return r;
}

// acc + unit u . x, for one token: xr is its row in global memory, xl in LDS.
template <typename WF, bool XL>
__device__ __forceinline__ float unit_dot(const UnitW& U, int u, const char* xr, const u32x4* xl, float acc) {
  if constexpr (std::is_same<WF, Q4>::value) {
    u32x4 xq[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) xq[k] = XL ? xl[4 * u + k] : ld16(xr + (size_t)(4 * u + k) * 16);
    return __builtin_fmaf(U.sc, dot_q4(U.w, xq), acc);
  } else {
    return dotc<WF>(U.w, XL ? xl[u] : ld16(xr + (size_t)u * 16), acc);
  }
}

// Units per lane per pass of a part: one pass at d = 8192 (fp16: 256 units
// per part; Q4_0: 64 blocks per part).
template <typename WF>
constexpr int part_units() { return std::is_same<WF, Q4>::value ? 1 : 4; }

// pu[s][j] = part parts[s] of row rows[s] of w_up dotted with token j, summed
// over the wave (pg: the same for w_gate).  Entries with ok[s] false give 0.
// All loads of a pass (S parts x part_units units) are in flight together.
template <typename WF, bool GATED, int NT, bool XL, int S>
__device__ __forceinline__ void part_dots(const void* w_up, const void* w_gate, size_t scale_off,
                                          const int (&rows)[S], const int (&parts)[S], const bool (&ok)[S], int d,
                                          const char* xb, const u32x4* x_lds, int nt, int lane, float (&pu)[S][NT],
                                          float (&pg)[S][NT]) {
  using X = typename FfnTraits<WF>::X;
  const int n = row_units<WF>(d);
  const int xch = d / (16 / (int)sizeof(X));   // 16-byte chunks of one token's x
  int c0[S], c1[S];
  float au[S][NT], ag[S][NT];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    c0[s] = n * parts[s] / 4;
    c1[s] = n * (parts[s] + 1) / 4;
#pragma unroll
    for (int j = 0; j < NT; ++j) au[s][j] = ag[s][j] = 0.f;
  }
  const int len = (n + 3) / 4;
  constexpr int PU = part_units<WF>();
  for (int p = 0; p < len; p += kWave * PU) {
    UnitW wu[S][PU], wg[GATED ? S : 1][PU];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int m = 0; m < PU; ++m) {
        const int u = c0[s] + p + lane + kWave * m;
        const bool v = ok[s] && u < c1[s];
        wu[s][m] = load_unit<WF>(w_up, scale_off, rows[s], u, d, v);
        if constexpr (GATED) wg[s][m] = load_unit<WF>(w_gate, scale_off, rows[s], u, d, v);
      }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j < nt) {
        const char* xr = xb + (size_t)j * d * sizeof(X);
        const u32x4* xl = x_lds + j * xch;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int m = 0; m < PU; ++m) {
            const int u = c0[s] + p + lane + kWave * m;
            if (ok[s] && u < c1[s]) {
              au[s][j] = unit_dot<WF, XL>(wu[s][m], u, xr, xl, au[s][j]);
              if constexpr (GATED) ag[s][j] = unit_dot<WF, XL>(wg[s][m], u, xr, xl, ag[s][j]);
            }
          }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      pu[s][j] = wave_sum(au[s][j]);
      pg[s][j] = GATED ? wave_sum(ag[s][j]) : 0.f;
    }
}

// h from the 4 part sums (in order) and the bias (b_up for ReLU / ReLU^2,
// b_gate for ReGLU).
template <int ACT>
__device__ __forceinline__ float combine_parts(float u0, float u1, float u2, float u3, float g0, float g1, float g2,
                                               float g3, float b) {
  const float u = ((u0 + u1) + u2) + u3;
  if (ACT == ACT_REGLU) return activate<ACT>(u, (((g0 + g1) + g2) + g3) + b);
  return activate<ACT>(u + b, 0.f);
}

// ---------------------------------------------------------------------------
// k_up: list path.  h[j][k] (by list position k) for the neuron idx[k].
// ---------------------------------------------------------------------------
constexpr int kUpThreads = 256;
constexpr int kUpWaves = kUpThreads / kWave;

template <typename WF, int ACT, int NT, bool XL>
__global__ __launch_bounds__(kUpThreads) void k_up(const void* __restrict__ w_up, const void* __restrict__ w_gate,
                                                   size_t scale_off, const float* __restrict__ bias,
                                                   const typename FfnTraits<WF>::X* __restrict__ x,
                                                   int d, int d_ff, int nt, const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ count_ptr, int max_count,
                                                   float* __restrict__ h) {
  using X = typename FfnTraits<WF>::X;
  extern __shared__ u32x4 x_lds[];   // [NT][d/E] when XL
  const int lane = lane_id();
  const int k_first = blockIdx.x * kUpWaves + wave_id();
  // idx holds max_count entries, so the first entry can be fetched while the
  // count is still in flight.
  int i_next = k_first < max_count ? idx[k_first] : -1;
  int cnt = *count_ptr;
  cnt = cnt < 0 ? 0 : (cnt < max_count ? cnt : max_count);
  const char* xb = reinterpret_cast<const char*>(x);
  if (XL) {
    stage_x<X>(xb, x_lds, nt, d);
    __syncthreads();
  }
  const int n_waves = gridDim.x * kUpWaves;
  for (int k = k_first; k < cnt; k += n_waves) {
    const int i = i_next;
    i_next = k + n_waves < cnt ? idx[k + n_waves] : -1;
    const bool valid = (unsigned)i < (unsigned)d_ff;      // a malformed entry adds nothing
    const int r = valid ? i : 0;
    const int rows[4] = {r, r, r, r}, parts[4] = {0, 1, 2, 3};
    const bool ok[4] = {valid, valid, valid, valid};
    float pu[4][NT], pg[4][NT];
    part_dots<WF, ACT == ACT_REGLU, NT, XL, 4>(w_up, w_gate, scale_off, rows, parts, ok, d, xb, x_lds, nt, lane, pu,
                                               pg);
    const float b = valid && bias ? bias[i] : 0.f;
    if (lane == 0)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        if (j < nt)
          h[(size_t)j * d_ff + k] =
              valid ? combine_parts<ACT>(pu[0][j], pu[1][j], pu[2][j], pu[3][j], pg[0][j], pg[1][j], pg[2][j],
                                         pg[3][j], b)
                    : 0.f;
  }
}

// ---------------------------------------------------------------------------
// k_pred_up: layer path.  Predictor stage 2 and the up projection fused.
// Workgroup g owns kPURows consecutive neurons (a segment):
//   A. every 16-lane group computes the logits of kPUSub neurons exactly as
//      the stand-alone predictor does (their p2 loads go out before t and x
//      are staged); a neuron is active when any token of the tile predicts it;
//   C. the active neurons are dealt round-robin to the 4 waves, each running
//      the up projection of its share (x read from LDS); results stay in LDS;
//   D. the segment's per-neuron slots are written: act[i] = i for an active
//      neuron and -1 otherwise, h[j][i] its value (0 when inactive).
// The slots are the list in place: the down projection takes whole segments
// per chunk and compacts their active neurons itself (k_down's slot form),
// so no workgroup waits on another and nothing is counted across the grid.
// ---------------------------------------------------------------------------
constexpr int kPUThreads = 256;
constexpr int kPUWaves = kPUThreads / kWave;
constexpr int kPUSub = 2;                                             // neurons per group
constexpr int kPURows = kPUThreads / kP2Group * kPUSub;               // 32 neurons per workgroup
static_assert(kPURows == PI_SEGMENT_ROWS, "the segment size pi_hot_order deals neurons over");
// Rows per phase-C batch (ReLU; ReGLU half as many).  A fp16 row part is 64
// bytes per lane, a Q4_0 row part 18: Q4_0 batches hold 3x as many rows in
// the same registers, so a segment with many active neurons needs fewer
// dependent round trips.
template <typename WF>
constexpr int pu_batch() { return std::is_same<WF, Q4>::value ? 8 : 4; }

template <typename W, typename WF, int ACT, int NT, bool XL>
__global__ __launch_bounds__(kPUThreads) void k_pred_up(const W* __restrict__ p2, const float* __restrict__ c,
                                                        const float* __restrict__ t, int rank, int d_ff,
                                                        float theta, const void* __restrict__ w_up,
                                                        const void* __restrict__ w_gate, size_t scale_off,
                                                        const float* __restrict__ bias, const W* __restrict__ x,
                                                        int d, int nt, int32_t* __restrict__ act,
                                                        float* __restrict__ h) {
  extern __shared__ float smem[];    // t tile [NT][rank], then (XL) x tile [NT][d/E] chunks
  float* t_lds = smem;
  u32x4* x_lds = reinterpret_cast<u32x4*>(smem + NT * rank);
  __shared__ int act_lds[kPURows];
  __shared__ float pu_lds[kPUWaves][kPURows][NT];                     // part sums of phase C
  __shared__ float pg_lds[ACT == ACT_REGLU ? kPUWaves : 1][kPURows][NT];
  const int lane = lane_id();
  const int wave = wave_id();
  const int g = lane & (kP2Group - 1);
  const int grp = threadIdx.x / kP2Group;                  // 0 .. 15
  const int wg = blockIdx.x;
  const int seg0 = wg * kPURows;
  const char* xb = reinterpret_cast<const char*>(x);

  // ---- A: logits ----
  int rows[kPUSub];
  bool rv[kPUSub];
#pragma unroll
  for (int s = 0; s < kPUSub; ++s) {
    rows[s] = seg0 + s * (kPUThreads / kP2Group) + grp;
    rv[s] = rows[s] < d_ff;
  }
  u32x4 w0[kPUSub][kP2Chunks];
  issue_pass<W, kPUSub>(p2, rows, rv, rank, g, 0, w0);
  stage_t<W>(t, t_lds, nt, rank);
  if (XL) stage_x<W>(xb, x_lds, nt, d);
  __syncthreads();
  float acc[kPUSub][NT];
  finish_logits<W, NT, kPUSub>(p2, rows, rv, rank, t_lds, nt, g, w0, acc);
  if (g == 0) {
#pragma unroll
    for (int s = 0; s < kPUSub; ++s) {
      bool active = false;
      if (rv[s]) {
        const float cb = c[rows[s]];
#pragma unroll
        for (int j = 0; j < NT; ++j)
          if (j < nt) active |= (acc[s][j] + cb) > theta;
      }
      act_lds[rows[s] - seg0] = active ? 1 : 0;
    }
  }
  __syncthreads();
  const unsigned long long am = __ballot(lane < kPURows && act_lds[lane < kPURows ? lane : 0] != 0);

  // ---- C: up projection of the active neurons: wave q computes part q of
  // every listed row, pu_batch rows at a time with all their loads in flight.
  // ReGLU: the gate rows first; a neuron whose gate is not positive for any
  // token has h = 0 whatever its up row holds, so only the up rows of the
  // neurons whose gate fires are read (fm).
  auto rows_pass = [&](const void* w, unsigned long long bits, float (*dst)[kPURows][NT]) {
    constexpr int S = pu_batch<WF>();
    while (bits) {                                 // the same in every wave
      int rows[S], parts[S], rr[S];
      bool ok[S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        ok[s] = bits != 0;
        rr[s] = ok[s] ? __builtin_ctzll(bits) : 0;
        bits &= bits - 1;
        rows[s] = seg0 + rr[s];
        parts[s] = wave;
      }
      float pu[S][NT], pg[S][NT];
      part_dots<WF, false, NT, XL, S>(w, w, scale_off, rows, parts, ok, d, xb, x_lds, nt, lane, pu, pg);
      if (lane == 0)
#pragma unroll
        for (int s = 0; s < S; ++s)
          if (ok[s])
#pragma unroll
            for (int j = 0; j < NT; ++j) dst[wave][rr[s]][j] = pu[s][j];
    }
  };
  unsigned long long fm = am;
  if constexpr (ACT == ACT_REGLU) {
    rows_pass(w_gate, am, pg_lds);
    __syncthreads();                               // the gate part sums are in LDS
    bool fire = false;
    if (lane < kPURows && ((am >> lane) & 1ull)) {
      const float b = bias ? bias[seg0 + lane] : 0.f;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        if (j < nt)
          fire |= (((pg_lds[0][lane][j] + pg_lds[1][lane][j]) + pg_lds[2][lane][j]) + pg_lds[3][lane][j]) + b > 0.f;
    }
    fm = __ballot(fire);                           // the same in every wave
  }
  rows_pass(w_up, fm, pu_lds);

  // ---- D: the segment's slots ----
  __syncthreads();   // the part sums of phase C are in LDS
  if (wave == 0 && lane < kPURows && seg0 + lane < d_ff) {
    const int i = seg0 + lane;
    const bool read = (fm >> lane) & 1ull;         // ReGLU: listed with a firing gate
    // the slot names the neurons whose up row was read (ReGLU: a listed
    // neuron whose gate fires for no token has h = 0 and is left out, which
    // changes nothing downstream)
    act[i] = read ? i : -1;
    const float b = read && bias ? bias[i] : 0.f;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (j < nt) {
        const bool gt = ACT == ACT_REGLU;
        const float g0 = gt ? pg_lds[0][lane][j] : 0.f, g1 = gt ? pg_lds[1][lane][j] : 0.f;
        const float g2 = gt ? pg_lds[2][lane][j] : 0.f, g3 = gt ? pg_lds[3][lane][j] : 0.f;
        h[(size_t)j * d_ff + i] = read ? combine_parts<ACT>(pu_lds[0][lane][j], pu_lds[1][lane][j],
                                                            pu_lds[2][lane][j], pu_lds[3][lane][j], g0, g1, g2, g3, b)
                                       : 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_down: part[c][j][col] = sum over the rows of chunk c (in list order) of
// h[j][row] * w_down_t[row][col].  Two forms:
//  * list (pi_sparse_ffn): chunk c covers list positions [c*cnt/C,
//    (c+1)*cnt/C), equal shares of the active rows; h is by list position.
//  * slots (pi_layer's fused path): chunk c covers the neurons of segments
//    [c*S/C, (c+1)*S/C), whose per-neuron slots (act[i] = i or -1, h by
//    neuron) the fused kernel wrote; the chunk's active neurons are compacted
//    here, in ascending order, with no count needed beforehand, so the slots
//    and the weights are two round trips, not three.
// Either way the chunk's rows and h values are staged in LDS so the row loop
// issues its weight loads with no dependent global load before them, and
// rows whose h is zero for every token are dropped while staging: ReLU
// zeroes many predicted neurons, and their rows would add nothing.  The
// workgroups of column slice 0 add the rows they kept to the workspace
// header's count.
// ---------------------------------------------------------------------------
constexpr int kDnThreads = 512;
constexpr int kDnWaves = kDnThreads / kWave;
constexpr int kDnUnroll = 8;                 // rows in flight per wave
constexpr int kDnPiece = kDnThreads;         // list entries staged per round (list form)
constexpr int kDnSlots = 2 * kDnThreads;     // neurons staged per round (slot form)

// Whether a staged row adds anything: h nonzero (or NaN) for some token.  A
// row whose h is exactly zero for every token adds +-0 to sums that start at
// +0, which changes no bit of them, so it is not read (for finite weights).
template <int NT>
__device__ __forceinline__ bool any_nonzero(const float (&hv)[NT], int nt) {
  bool nz = false;
#pragma unroll
  for (int j = 0; j < NT; ++j) nz |= j < nt && hv[j] != 0.f;
  return nz;
}

// Exclusive offset of this thread's c kept rows among the workgroup's, and
// the workgroup's total: a wave scan, then the wave totals through LDS.
// Callers pack a second count into the upper 16 bits of c (at most 2 per
// thread, so neither half carries into the other); the scan adds both.
__device__ __forceinline__ void kept_offsets(int c, int* wsum, int& pos, int& tot) {
  const int lane = lane_id(), wave = wave_id();
  int incl = c;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  pos = incl - c;
  tot = 0;
#pragma unroll
  for (int w = 0; w < kDnWaves; ++w) {
    pos += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
}

// Slot form: the active neurons among [nb0, min(nb0 + kDnSlots, n1)) with a
// nonzero h, in ascending order, into rows_l / h_l; returns how many, and
// adds the number of valid slots (neurons whose up row was read) to *n_up.
// Thread t takes neurons nb0 + 2t and nb0 + 2t + 1 (their act and h loads in
// one round trip).
template <int NT, int CAP>
__device__ __forceinline__ int stage_slots(const int32_t* __restrict__ act, const float* __restrict__ h, int d_ff,
                                           int nb0, int n1, int nt, int* rows_l, float (*h_l)[CAP], int* wsum,
                                           int* n_up) {
  const int i0 = nb0 + 2 * (int)threadIdx.x, i1 = i0 + 1;
  const int a0 = i0 < n1 ? act[i0] : -1, a1 = i1 < n1 ? act[i1] : -1;
  float h0[NT], h1[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    h0[j] = j < nt && i0 < n1 ? h[(size_t)j * d_ff + i0] : 0.f;
    h1[j] = j < nt && i1 < n1 ? h[(size_t)j * d_ff + i1] : 0.f;
  }
  const bool s0 = (unsigned)a0 < (unsigned)d_ff, s1 = (unsigned)a1 < (unsigned)d_ff;
  const bool v0 = s0 && any_nonzero<NT>(h0, nt);
  const bool v1 = s1 && any_nonzero<NT>(h1, nt);
  int pos, tot;
  kept_offsets((v0 ? 1 : 0) + (v1 ? 1 : 0) + (((s0 ? 1 : 0) + (s1 ? 1 : 0)) << 16), wsum, pos, tot);
  *n_up += tot >> 16;
  pos &= 0xFFFF;
  tot &= 0xFFFF;
  if (v0) {
    rows_l[pos] = a0;
#pragma unroll
    for (int j = 0; j < NT; ++j) h_l[j][pos] = h0[j];
    ++pos;
  }
  if (v1) {
    rows_l[pos] = a1;
#pragma unroll
    for (int j = 0; j < NT; ++j) h_l[j][pos] = h1[j];
  }
  __syncthreads();
  return tot;
}

// List form: the entries of list positions [pb, pb + n) (n <= kDnThreads)
// that name a neuron and have a nonzero h, in list order; returns how many,
// and adds the number of entries that name a neuron (the up rows the list
// path reads) to *n_up.  A malformed entry (outside [0, d_ff)) adds nothing.
template <int NT, int CAP>
__device__ __forceinline__ int stage_list(const int32_t* __restrict__ idx, const float* __restrict__ h, int d_ff,
                                          int pb, int n, int nt, int* rows_l, float (*h_l)[CAP], int* wsum,
                                          int* n_up) {
  const int k = (int)threadIdx.x;
  const int i = k < n ? idx[pb + k] : -1;
  float hv[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) hv[j] = j < nt && k < n ? h[(size_t)j * d_ff + pb + k] : 0.f;
  const bool named = (unsigned)i < (unsigned)d_ff;
  const bool v = named && any_nonzero<NT>(hv, nt);
  int pos, tot;
  kept_offsets((v ? 1 : 0) + ((named ? 1 : 0) << 16), wsum, pos, tot);
  *n_up += tot >> 16;
  pos &= 0xFFFF;
  tot &= 0xFFFF;
  if (v) {
    rows_l[pos] = i;
#pragma unroll
    for (int j = 0; j < NT; ++j) h_l[j][pos] = hv[j];
  }
  __syncthreads();
  return tot;
}

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

template <typename W, int NT, bool SLOTS>
__global__ __launch_bounds__(kDnThreads) void k_down(const W* __restrict__ w_dt, int d, int d_ff,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ count_ptr, int max_count,
                                                     const float* __restrict__ h, int nt, int n_chunks,
                                                     float* __restrict__ part,
                                                     unsigned long long* __restrict__ rows_read,
                                                     unsigned long long* __restrict__ up_rows_read) {
  // SLOTS: idx is act[d_ff], h is [nt][d_ff] by neuron, count_ptr unused
  constexpr int E = 16 / sizeof(W);
  constexpr int SW = kWave * E;               // columns per slice
  constexpr int CAP = SLOTS ? kDnSlots : kDnPiece;
  __shared__ float red[kDnWaves][SW];
  __shared__ int rows_l[CAP];
  __shared__ float h_l[NT][CAP];
  __shared__ int wsum[kDnWaves];
  const int lane = lane_id();
  const int wave = wave_id();
  const int slice = blockIdx.x;
  const int c = blockIdx.y;
  const int col = slice * SW + lane * E;
  const bool cv = col < d;
  int k0, k1;
  if constexpr (SLOTS) {
    const int n_seg = (d_ff + PI_SEGMENT_ROWS - 1) / PI_SEGMENT_ROWS;
    k0 = PI_SEGMENT_ROWS * (int)(((long long)c * n_seg) / n_chunks);
    const int e1 = PI_SEGMENT_ROWS * (int)(((long long)(c + 1) * n_seg) / n_chunks);
    k1 = e1 < d_ff ? e1 : d_ff;
  } else {
    int cnt = *count_ptr;
    cnt = cnt < 0 ? 0 : (cnt < max_count ? cnt : max_count);
    k0 = (int)(((long long)c * cnt) / n_chunks);
    k1 = (int)(((long long)(c + 1) * cnt) / n_chunks);
  }

  float acc[NT][E];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[j][e] = 0.f;

  const char* base = reinterpret_cast<const char*>(w_dt) + (size_t)col * sizeof(W);
  int n_read = 0, n_up = 0;
  for (int pb = k0; pb < k1; pb += CAP) {
    int n;
    if constexpr (SLOTS) {
      n = stage_slots<NT, CAP>(idx, h, d_ff, pb, k1, nt, rows_l, h_l, wsum, &n_up);
    } else {
      n = stage_list<NT, CAP>(idx, h, d_ff, pb, k1 - pb < kDnPiece ? k1 - pb : kDnPiece, nt, rows_l, h_l, wsum,
                              &n_up);
    }
    n_read += n;
    for (int jb = wave; jb < n; jb += kDnWaves * kDnUnroll) {
      u32x4 v[kDnUnroll];
      int rows[kDnUnroll];
#pragma unroll
      for (int u = 0; u < kDnUnroll; ++u) {
        const int jj = jb + kDnWaves * u;
        rows[u] = jj < n ? __builtin_amdgcn_readfirstlane(rows_l[jj]) : -1;
      }
#pragma unroll
      for (int u = 0; u < kDnUnroll; ++u)
        v[u] = (rows[u] >= 0 && cv) ? ld_nt(base + (size_t)rows[u] * d * sizeof(W)) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < kDnUnroll; ++u) {
        if (rows[u] >= 0) {
          const int jj = jb + kDnWaves * u;
#pragma unroll
          for (int j = 0; j < NT; ++j)
            if (j < nt) axpy_chunk<W>(acc[j], h_l[j][jj], v[u]);
        }
      }
    }
    __syncthreads();
  }

  // The column slices of a chunk read the same rows: slice 0 counts them.
  if (slice == 0 && threadIdx.x == 0) {
    if (rows_read && n_read) atomicAdd(rows_read, (unsigned long long)n_read);
    if (up_rows_read && n_up) atomicAdd(up_rows_read, (unsigned long long)n_up);
  }
  // Sum the 8 waves in wave order, one token at a time; write the partials.
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (j < nt) {
#pragma unroll
      for (int e = 0; e < E; ++e) red[wave][lane * E + e] = acc[j][e];
      __syncthreads();
      for (int o = threadIdx.x; o < SW; o += kDnThreads) {
        const int gcol = slice * SW + o;
        if (gcol < d) {
          float s = red[0][o];
#pragma unroll
          for (int w = 1; w < kDnWaves; ++w) s += red[w][o];
          part[((size_t)c * nt + j) * d + gcol] = s;
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// k_down_q4: the down projection with Q4_0 weights.  A lane owns half a block
// (16 columns, 8 bytes of codes) of each row, so a wave covers 1024 columns;
// otherwise as k_down (chunks of the list, rows staged in LDS, 8 waves summed
// in wave order).  Per row: s = h * d_block, then acc[col] += s * (q - 8).
// ---------------------------------------------------------------------------
constexpr int kDqUnroll = 16;               // rows in flight per wave
constexpr int kDqCols = 16;                 // columns per lane
constexpr int kDqSW = kWave * kDqCols;      // 1024 columns per slice

template <int NT, bool SLOTS>
__global__ __launch_bounds__(kDnThreads) void k_down_q4(const uint8_t* __restrict__ w_dt, size_t scale_off, int d,
                                                        int d_ff, const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ count_ptr, int max_count,
                                                        const float* __restrict__ h, int nt, int n_chunks,
                                                        float* __restrict__ part,
                                                        unsigned long long* __restrict__ rows_read,
                                                        unsigned long long* __restrict__ up_rows_read) {
  constexpr int CAP = SLOTS ? kDnSlots : kDnPiece;
  __shared__ float red[kDnWaves][kWave * 8];
  __shared__ int rows_l[CAP];
  __shared__ float h_l[NT][CAP];
  __shared__ int wsum[kDnWaves];
  const int lane = lane_id();
  const int wave = wave_id();
  const int slice = blockIdx.x;
  const int c = blockIdx.y;
  const int nb = d / 32;
  const int col = slice * kDqSW + lane * kDqCols;     // first of this lane's 16 columns
  const bool cv = col < d;
  const int blk = col / 32, half = (col / 16) & 1;
  const uint8_t* code_base = w_dt + (size_t)blk * 16 + half * 8;
  const f16* scale_base = reinterpret_cast<const f16*>(w_dt + scale_off) + blk;
  int k0, k1;
  if constexpr (SLOTS) {
    const int n_seg = (d_ff + PI_SEGMENT_ROWS - 1) / PI_SEGMENT_ROWS;
    k0 = PI_SEGMENT_ROWS * (int)(((long long)c * n_seg) / n_chunks);
    const int e1 = PI_SEGMENT_ROWS * (int)(((long long)(c + 1) * n_seg) / n_chunks);
    k1 = e1 < d_ff ? e1 : d_ff;
  } else {
    int cnt = *count_ptr;
    cnt = cnt < 0 ? 0 : (cnt < max_count ? cnt : max_count);
    k0 = (int)(((long long)c * cnt) / n_chunks);
    k1 = (int)(((long long)(c + 1) * cnt) / n_chunks);
  }

  float acc[NT][kDqCols];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int e = 0; e < kDqCols; ++e) acc[j][e] = 0.f;

  int n_read = 0, n_up = 0;
  for (int pb = k0; pb < k1; pb += CAP) {
    int n;
    if constexpr (SLOTS) {
      n = stage_slots<NT, CAP>(idx, h, d_ff, pb, k1, nt, rows_l, h_l, wsum, &n_up);
    } else {
      n = stage_list<NT, CAP>(idx, h, d_ff, pb, k1 - pb < kDnPiece ? k1 - pb : kDnPiece, nt, rows_l, h_l, wsum,
                              &n_up);
    }
    n_read += n;
    for (int jb = wave; jb < n; jb += kDnWaves * kDqUnroll) {
      u32x2 v[kDqUnroll];
      float dsc[kDqUnroll];
      int rows[kDqUnroll];
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const int jj = jb + kDnWaves * u;
        rows[u] = jj < n ? __builtin_amdgcn_readfirstlane(rows_l[jj]) : -1;
      }
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        const bool ok = rows[u] >= 0 && cv;
        v[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(code_base + (size_t)rows[u] * nb * 16))
                  : u32x2{0, 0};
        dsc[u] = ok ? (float)scale_base[(size_t)rows[u] * nb] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kDqUnroll; ++u) {
        if (rows[u] >= 0) {
          const int jj = jb + kDnWaves * u;
          const unsigned wd[2] = {v[u].x, v[u].y};
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            if (j < nt) {
              const float sc = h_l[j][jj] * dsc[u];
#pragma unroll
              for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const f16x2 pr = q4_pair(wd[k], q);
                  acc[j][8 * k + 2 * q] = __builtin_fmaf(sc, (float)pr.x, acc[j][8 * k + 2 * q]);
                  acc[j][8 * k + 2 * q + 1] = __builtin_fmaf(sc, (float)pr.y, acc[j][8 * k + 2 * q + 1]);
                }
            }
          }
        }
      }
    }
    __syncthreads();
  }

  if (slice == 0 && threadIdx.x == 0) {
    if (rows_read && n_read) atomicAdd(rows_read, (unsigned long long)n_read);
    if (up_rows_read && n_up) atomicAdd(up_rows_read, (unsigned long long)n_up);
  }
  // Sum the 8 waves in wave order, 8 columns per lane per round; write the partials.
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (j < nt) {
#pragma unroll
      for (int r = 0; r < kDqCols / 8; ++r) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = acc[j][8 * r + e];
        __syncthreads();
        const int o = threadIdx.x;                      // 512 entries: lane o/8, column 8r + o%8
        const int gcol = slice * kDqSW + (o / 8) * kDqCols + 8 * r + (o % 8);
        if (gcol < d) {
          float sum = red[0][o];
#pragma unroll
          for (int w = 1; w < kDnWaves; ++w) sum += red[w][o];
          part[((size_t)c * nt + j) * d + gcol] = sum;
        }
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_merge: y[j][col] = sum over chunks c = 0, 1, ... of part[c][j][col], in
// chunk order.  A workgroup owns 4*QW consecutive outputs, QW = 256 / G with
// G = n_chunks rounded up to a power of two (at most 64): thread (g, q) loads
// the 16 bytes of outputs [4q, 4q+4) of chunk g, so every load of the merge
// is in flight at once and the reads spread over n/(4*QW) workgroups (256 at
// one Falcon token with 32 chunks).  The sums then run down the chunks in LDS,
// one output per thread, in chunk order.
// ---------------------------------------------------------------------------
constexpr int kMgThreads = 256;
constexpr int kMgMaxChunks = 64;

__host__ __device__ constexpr int merge_group(int n_chunks) {
  return n_chunks <= 1 ? 1 : (n_chunks <= 2 ? 2 : (n_chunks <= 4 ? 4 : (n_chunks <= 8 ? 8 :
         (n_chunks <= 16 ? 16 : (n_chunks <= 32 ? 32 : 64)))));
}

__global__ __launch_bounds__(kMgThreads) void k_merge(const float* __restrict__ part, int n_chunks, int n,
                                                      void* __restrict__ y, int ytype,
                                                      const unsigned* __restrict__ fault) {
  __shared__ float buf[kMgThreads * 4];
  const int G = merge_group(n_chunks);
  const int QW = kMgThreads / G;                 // 16-byte quads per workgroup
  const int ncol = 4 * QW;
  const int col0 = blockIdx.x * ncol;
  const int q = threadIdx.x % QW, g = threadIdx.x / QW;
  const int col = col0 + 4 * q;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (g < n_chunks && col < n) v = *reinterpret_cast<const float4*>(part + (size_t)g * n + col);
  reinterpret_cast<float4*>(buf)[threadIdx.x] = v;   // buf[g][4q .. 4q+3]
  __syncthreads();
  const int o = threadIdx.x;
  const bool poison = fault != nullptr && *fault != 0u;
  if (o < ncol && col0 + o < n) {
    float s = 0.f;
    for (int c = 0; c < n_chunks; ++c) s += buf[c * ncol + o];
    if (poison) s = __builtin_nanf("");
    if (ytype == 1)
      static_cast<f16*>(y)[col0 + o] = (f16)s;
    else
      static_cast<float*>(y)[col0 + o] = s;
  }
}

// Zero a workspace header (one thread per word).
__global__ __launch_bounds__(kHdrWords) void k_clear_header(unsigned* __restrict__ hdr) { hdr[threadIdx.x] = 0u; }

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
template <typename WF>
constexpr int slice_cols() {
  return std::is_same<WF, Q4>::value ? kDqSW : kWave * (16 / (int)sizeof(WF));
}

template <typename WF>
size_t scale_offset(const SparseArgs& a) {
  return std::is_same<WF, Q4>::value ? (size_t)a.d_ff * (a.d / 32) * 16 : 0;
}

// slots: the fused layer path's per-neuron slots (k_pred_up) instead of a list
template <typename WF, int NT, bool SLOTS>
hipError_t launch_down_form(const SparseArgs& a, int nt, hipStream_t s) {
  const dim3 grid(a.n_slices, a.n_chunks);
  if constexpr (std::is_same<WF, Q4>::value)
    hipLaunchKernelGGL((k_down_q4<NT, SLOTS>), grid, dim3(kDnThreads), 0, s, static_cast<const uint8_t*>(a.w_down_t),
                       scale_offset<WF>(a), a.d, a.d_ff, a.idx, a.count, a.max_count, a.h, nt, a.n_chunks, a.part,
                       a.rows_read, a.up_rows_read);
  else
    hipLaunchKernelGGL((k_down<WF, NT, SLOTS>), grid, dim3(kDnThreads), 0, s, static_cast<const WF*>(a.w_down_t), a.d,
                       a.d_ff, a.idx, a.count, a.max_count, a.h, nt, a.n_chunks, a.part, a.rows_read,
                       a.up_rows_read);
  return hipGetLastError();
}

template <typename WF, int NT>
hipError_t launch_down(const SparseArgs& a, bool slots, void* y, int nt, hipStream_t s) {
  hipError_t e = slots ? launch_down_form<WF, NT, true>(a, nt, s) : launch_down_form<WF, NT, false>(a, nt, s);
  if (e != hipSuccess) return e;
  return launch_merge(a.part, a.n_chunks, nt * a.d, y, a.ytype, a.fault, s);
}

// x is staged in LDS when its token tile fits in 32 KB.
template <typename X>
bool x_in_lds(int nt_tmpl, int d) { return (size_t)nt_tmpl * d * sizeof(X) <= 32768; }

template <typename WF, int ACT, int NT>
hipError_t launch_up(const SparseArgs& a, const typename FfnTraits<WF>::X* x, int nt, hipStream_t s) {
  using X = typename FfnTraits<WF>::X;
  const int max_waves = 4096;   // 16 resident waves per CU on 256 CUs: one row per wave up to 4096 rows
  int waves = a.max_count < max_waves ? a.max_count : max_waves;
  if (waves < 1) waves = 1;
  const int grid = (waves + kUpWaves - 1) / kUpWaves;
  const float* bias = ACT == ACT_REGLU ? a.b_gate : a.b_up;
  const size_t so = scale_offset<WF>(a);
  if (x_in_lds<X>(NT, a.d)) {
    const size_t lds = (size_t)NT * a.d * sizeof(X);
    hipLaunchKernelGGL((k_up<WF, ACT, NT, true>), dim3(grid), dim3(kUpThreads), lds, s, a.w_up, a.w_gate, so, bias,
                       x, a.d, a.d_ff, nt, a.idx, a.count, a.max_count, a.h);
  } else {
    hipLaunchKernelGGL((k_up<WF, ACT, NT, false>), dim3(grid), dim3(kUpThreads), 0, s, a.w_up, a.w_gate, so, bias,
                       x, a.d, a.d_ff, nt, a.idx, a.count, a.max_count, a.h);
  }
  return hipGetLastError();
}

template <typename WF, int ACT, int NT>
hipError_t launch_pred_up(const SparseArgs& a, const LayerArgs& L, const typename FfnTraits<WF>::X* x, int nt,
                          hipStream_t s) {
  using X = typename FfnTraits<WF>::X;   // also the predictor's weight type
  const int grid = layer_segments(a.d_ff);
  const float* bias = ACT == ACT_REGLU ? a.b_gate : a.b_up;
  const X* p2 = static_cast<const X*>(L.p2);
  const size_t so = scale_offset<WF>(a);
  const size_t lds_t = (size_t)NT * L.rank * sizeof(float);
  if (x_in_lds<X>(NT, a.d)) {
    const size_t lds = lds_t + (size_t)NT * a.d * sizeof(X);
    hipLaunchKernelGGL((k_pred_up<X, WF, ACT, NT, true>), dim3(grid), dim3(kPUThreads), lds, s, p2, L.c, L.t, L.rank,
                       a.d_ff, L.theta, a.w_up, a.w_gate, so, bias, x, a.d, nt, L.act, a.h);
  } else {
    hipLaunchKernelGGL((k_pred_up<X, WF, ACT, NT, false>), dim3(grid), dim3(kPUThreads), lds_t, s, p2, L.c, L.t,
                       L.rank, a.d_ff, L.theta, a.w_up, a.w_gate, so, bias, x, a.d, nt, L.act, a.h);
  }
  return hipGetLastError();
}

template <typename WF, int NT>
hipError_t up_dispatch(const SparseArgs& a, const LayerArgs* L, const typename FfnTraits<WF>::X* x, int nt,
                       hipStream_t s) {
  if (L) {
    if (a.act == ACT_REGLU) return launch_pred_up<WF, ACT_REGLU, NT>(a, *L, x, nt, s);
    if (a.act == ACT_RELU2) return launch_pred_up<WF, ACT_RELU2, NT>(a, *L, x, nt, s);
    return launch_pred_up<WF, ACT_RELU, NT>(a, *L, x, nt, s);
  }
  if (a.act == ACT_REGLU) return launch_up<WF, ACT_REGLU, NT>(a, x, nt, s);
  if (a.act == ACT_RELU2) return launch_up<WF, ACT_RELU2, NT>(a, x, nt, s);
  return launch_up<WF, ACT_RELU, NT>(a, x, nt, s);
}

template <typename WF, int NT>
hipError_t run_tile(const SparseArgs& a, const LayerArgs* L, int t0, int nt, hipStream_t s) {
  using X = typename FfnTraits<WF>::X;
  const X* x = static_cast<const X*>(a.x) + (size_t)t0 * a.d;
  LayerArgs Lt;
  if (L) {
    Lt = *L;
    Lt.t = L->t + (size_t)t0 * L->rank;
  }
  hipError_t e = up_dispatch<WF, NT>(a, L ? &Lt : nullptr, x, nt, s);
  if (e != hipSuccess) return e;
  const size_t yoff = (size_t)t0 * a.d * (a.ytype == 1 ? 2 : 4);
  return launch_down<WF, NT>(a, L != nullptr, static_cast<char*>(a.y) + yoff, nt, s);
}

template <typename WF>
hipError_t run_all(const SparseArgs& a, const LayerArgs* L, hipStream_t s) {
  const int tile = sparse_tile(a.wtype, a.d);
  for (int t0 = 0; t0 < a.n_tok; t0 += tile) {
    const int nt = a.n_tok - t0 < tile ? a.n_tok - t0 : tile;
    hipError_t e;
    if (nt == 1)
      e = run_tile<WF, 1>(a, L, t0, nt, s);
    else if (nt == 2)
      e = run_tile<WF, 2>(a, L, t0, nt, s);
    else if (nt <= 4)
      e = run_tile<WF, 4>(a, L, t0, nt, s);
    else
      e = run_tile<WF, 8>(a, L, t0, nt, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename... Args>
hipError_t by_wtype(int wtype, const SparseArgs& a, const LayerArgs* L, hipStream_t s) {
  if (wtype == 1) return run_all<f16>(a, L, s);
  if (wtype == 2) return run_all<Q4>(a, L, s);
  return run_all<float>(a, L, s);
}

}  // namespace

int sparse_tile(int wtype, int d) {
  // Q4_0 keeps its fp16 activations in LDS: a tile of x must fit in 32 KB.
  if (wtype != 2) return kSparseTile;
  int tile = kSparseTile;
  while (tile > 1 && (size_t)tile * d * 2 > 32768) tile >>= 1;
  return tile;
}

void sparse_chunking(int wtype, int d, int* n_chunks, int* n_slices) {
  const int sw = wtype == 2 ? kDqSW : (wtype == 1 ? kWave * 8 : kWave * 4);
  const int slices = (d + sw - 1) / sw;
  // About 4096 waves (16 per CU) in the down kernel (measured at Falcon
  // batch 1: 2% faster than 2048 for fp16 and for Q4_0; 1024 is 12% slower).
  const int target_wgs = 4096 / kDnWaves;
  int c = (target_wgs + slices - 1) / slices;
  if (c < 1) c = 1;
  if (c > 64) c = 64;
  *n_chunks = c;
  *n_slices = slices;
}

int layer_segments(int d_ff) { return (d_ff + kPURows - 1) / kPURows; }

hipError_t launch_merge(const float* part, int n_chunks, int n, void* y, int ytype, const unsigned* fault,
                        hipStream_t s) {
  if (n <= 0) return hipSuccess;
  // The merge reads whole 16-byte quads of the partials.
  if (n_chunks < 1 || n_chunks > kMgMaxChunks || n % 4 != 0 || (reinterpret_cast<uintptr_t>(part) & 15) != 0)
    return hipErrorInvalidValue;
  const int ncol = 4 * (kMgThreads / merge_group(n_chunks));
  hipLaunchKernelGGL(k_merge, dim3((n + ncol - 1) / ncol), dim3(kMgThreads), 0, s, part, n_chunks, n, y, ytype,
                     fault);
  return hipGetLastError();
}

hipError_t launch_clear_header(unsigned* hdr, hipStream_t s) {
  hipLaunchKernelGGL(k_clear_header, dim3(1), dim3(kHdrWords), 0, s, hdr);
  return hipGetLastError();
}

hipError_t launch_sparse_ffn(const SparseArgs& a, hipStream_t s) {
  if (mfma_path(a.wtype, a.d, a.n_tok)) return launch_sparse_ffn_mfma(a, s);
  return by_wtype(a.wtype, a, nullptr, s);
}

hipError_t launch_layer_fused(const SparseArgs& a, const LayerArgs& L, hipStream_t s) {
  // a single token tile: the caller guarantees n_tok <= sparse_tile(wtype, d)
  return by_wtype(a.wtype, a, &L, s);
}

}  // namespace pi
