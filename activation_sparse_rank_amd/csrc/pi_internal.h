// Internal declarations shared by the libpi sources: device helpers for
// gfx950 (wave64) and the host-side launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pi.h"

namespace pi {

// ---------------------------------------------------------------------------
// Types
// ---------------------------------------------------------------------------
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Tag type for Q4_0 FFN weights (repacked layout, see k_q4.hip); the
// activations that multiply them are fp16.
struct Q4 {};
template <typename WF> struct FfnTraits { using X = WF; };
template <> struct FfnTraits<Q4> { using X = f16; };

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  // Streaming weight rows: non-temporal so they do not evict reused data.
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ f16x2 as_h2(unsigned int v) { return __builtin_bit_cast(f16x2, v); }

__device__ __forceinline__ float as_f(unsigned int v) { return __builtin_bit_cast(float, v); }

// 8 fp16 products accumulated in fp32 (v_dot2_f32_f16: exact fp16 products,
// fp32 accumulation).
__device__ __forceinline__ float dot8_f16(u32x4 w, u32x4 x, float acc) {
  acc = __builtin_amdgcn_fdot2(as_h2(w.x), as_h2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(w.y), as_h2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(w.z), as_h2(x.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(w.w), as_h2(x.w), acc, false);
  return acc;
}

// 4 fp32 products accumulated in fp32.
__device__ __forceinline__ float dot4_f32(u32x4 w, u32x4 x, float acc) {
  acc = __builtin_fmaf(as_f(w.x), as_f(x.x), acc);
  acc = __builtin_fmaf(as_f(w.y), as_f(x.y), acc);
  acc = __builtin_fmaf(as_f(w.z), as_f(x.z), acc);
  acc = __builtin_fmaf(as_f(w.w), as_f(x.w), acc);
  return acc;
}

// Butterfly sum over the 64 lanes of a wave; every lane ends with the same
// bits (each step adds the same two values in either order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Butterfly sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Activation codes (match pi_act).
enum : int { ACT_RELU = 0, ACT_REGLU = 1, ACT_RELU2 = 2 };

// ---------------------------------------------------------------------------
// Fault reporting (the workspace header of pi.h).  hdr points at the header:
// hdr[0] collects sticky flag bits, hdr[1] and hdr[2] are the test hooks of
// the in-kernel waits.  A per-call fault word (cleared by an earlier kernel
// of the same call) tells the merge to write NaN.
// ---------------------------------------------------------------------------
constexpr int kHdrWords = PI_WS_HEADER_BYTES / 4;
constexpr int kDefaultWaitPolls = 1 << 16;

__device__ __forceinline__ void raise_flag(unsigned* word, unsigned bits) {
  if (word != nullptr) __hip_atomic_fetch_or(word, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True when v is not finite after rounding to fp16 (the value a matrix-core
// operand holds).
__device__ __forceinline__ bool fp16_overflows(float v) {
  const float r = (float)(_Float16)v;
  return !(__builtin_fabsf(r) <= 65504.f);
}

// Raise bits in *word once per wave when any lane's cond holds.
__device__ __forceinline__ void raise_flag_if_any(unsigned* word, bool cond, unsigned bits) {
  if (__ballot(cond) != 0ull && (threadIdx.x & 63) == 0) raise_flag(word, bits);
}

// ---------------------------------------------------------------------------
// Host launchers (each returns the hipError_t of its launch)
// ---------------------------------------------------------------------------

// t[n][r] = p1[r] . x[n]  (fp32 out).  Block 0 also zeroes zero_n words at
// zero_ptr (NULL: none), for counters a later kernel of the same call uses.
hipError_t launch_predict_stage1(int wtype, const void* p1, const void* x, int n_tok, int d,
                                 int rank, float* t, unsigned* zero_ptr, int zero_n, hipStream_t s);
// l[n][i] = p2[i] . t[n] + c[i];  mask[n][i] = l > theta
hipError_t launch_predict_stage2(int wtype, const void* p2, const float* c, const float* t,
                                 int n_tok, int rank, int d_ff, float theta, uint8_t* mask,
                                 float* logits, hipStream_t s);
// Tokens per pass of the predictor's second stage (a tile of t fits in LDS).
int pred_tile(int rank);
// ascending list of neurons marked by any token
hipError_t launch_compact(const uint8_t* mask, int n_tok, int d_ff, int32_t* idx, int32_t* count,
                          hipStream_t s);

// Sparse FFN (one call = all launches for n_tok tokens, in tiles of
// sparse_tile(wtype, d) <= kSparseTile tokens).
constexpr int kSparseTile = 8;
int sparse_tile(int wtype, int d);

struct SparseArgs {
  int wtype, act, d, d_ff, n_tok, max_count;
  const void* w_up;
  const void* w_gate;
  const void* w_down_t;
  const float* b_up;
  const float* b_gate;
  const void* x;
  const int32_t* idx;       // list of active neurons (at least max_count entries)
  const int32_t* count;     // device count of valid list entries
  void* y;
  int ytype;
  float* h;                 // workspace [tile][d_ff] fp32, by list position
  float* part;              // workspace [n_chunks][tile][d] fp32
  int n_chunks, n_slices;
  // Matrix-core path, one token tile: x already copied step-major
  // ([d/128][n_tok][128] fp16; for Q4_0 weights in block order, as
  // launch_predict_mfma writes it with xs_block) by the predictor; NULL:
  // copy it.
  const void* xs_pre = nullptr;
  // Sticky flags word (PI_FLAG_FP16_RANGE from the matrix-core H); nullable.
  unsigned* flags = nullptr;
  // Per-call fault word of the list's producer; nonzero makes the merge
  // write NaN.  NULL when the list came from no waiting kernel.
  const unsigned* fault = nullptr;
  // The header's 64-bit count of down-projection rows read; nullable.
  unsigned long long* rows_read = nullptr;
  // The header's 64-bit count of w_up rows read; nullable.
  unsigned long long* up_rows_read = nullptr;
};
hipError_t launch_sparse_ffn(const SparseArgs& a, hipStream_t s);

// Predictor operands of the fused layer path (one token tile): stage 2 of
// the predictor and the up projection run as one kernel that writes
// per-neuron slots -- act[i] = i for an active neuron, else -1, and h by
// neuron -- which the down projection reads in its slot form.
struct LayerArgs {
  const void* p2;
  const float* c;
  const float* t;           // [n_tok][rank] from stage 1
  int rank;
  float theta;
  int32_t* act;             // workspace [d_ff]
};
// n_tok <= min(sparse_tile(wtype, d), pred_tile(rank)); a.idx must be L.act and
// a.h the slots' h ([n_tok][d_ff], by neuron).
hipError_t launch_layer_fused(const SparseArgs& a, const LayerArgs& L, hipStream_t s);
// Number of neuron segments (workgroups) of the fused kernel.
int layer_segments(int d_ff);

// How the down projection splits the active list (n_chunks chunks) and the
// columns (n_slices slices); sizes the workspace.
void sparse_chunking(int wtype, int d, int* n_chunks, int* n_slices);

// Multi-token path on the matrix cores (fp16 / Q4_0 weights, d % 128 == 0,
// more tokens than one pass of the list path takes): used by
// launch_sparse_ffn when mfma_path() says so.  Workspace: H [16*ceil(nt/16)]
// [d_ff rounded up to 64] fp16 in a.h, partials [chunks][nt][d] fp32 in a.part
// (nt = min(n_tok, 64)).
bool mfma_path(int wtype, int d, int n_tok);
void mfma_workspace(int wtype, int d, int d_ff, int n_tok, size_t* h_bytes, size_t* part_bytes);
hipError_t launch_sparse_ffn_mfma(const SparseArgs& a, hipStream_t s);

// Predictor for many tokens on the matrix cores (fp16 predictor, d and rank
// multiples of 128, more tokens than one pass of the list path's predictor
// takes).  t: [n_tok][rank] fp32 out; ws: pred_mfma_part_bytes() of
// workspace (256-byte aligned); mask/logits as launch_predict_stage2, either
// may be NULL; umask (nullable): [d_ff], 1 where any token is active.
// With umask and idx given, the union is also listed (ascending) into idx
// and count, using status[n_status] as counters (cleared in the call).
// xs_out (nullable) receives the step-major token copy when n_tok <= 64; with
// xs_block its 16-byte groups are in the block order Q4_0 rows meet.
bool pred_mfma_path(int wtype, int d, int rank, int n_tok);
size_t pred_mfma_part_bytes(int d, int rank, int n_tok);
// hdr: the workspace header (flags; the wait hooks when listing); fault: the
// per-call fault word of the list (cleared in the call), nullable when not
// listing.
hipError_t launch_predict_mfma(const void* p1, const void* p2, const float* c, const void* x, int n_tok, int d,
                               int rank, int d_ff, float theta, float* t, void* ws, uint8_t* mask, float* logits,
                               uint8_t* umask, unsigned* status, int n_status, int32_t* idx, int32_t* count,
                               unsigned* hdr, unsigned* fault, bool xs_block, const void** xs_out, hipStream_t s);

// y = sum over c of part[c][0 .. n), in chunk order (fp32 or fp16 out); NaN
// everywhere when fault (nullable) holds a nonzero word.
hipError_t launch_merge(const float* part, int n_chunks, int n, void* y, int ytype, const unsigned* fault,
                        hipStream_t s);

// Zero the kHdrWords words of a workspace header (pi_clear_flags).
hipError_t launch_clear_header(unsigned* hdr, hipStream_t s);

hipError_t launch_q4_0_repack(const void* src, int rows, int cols, void* dst, hipStream_t s);

// Neuron placement (k_place.hip): firing counts from masks, the placement
// order from the counts (host), and a row permutation dst[k] = src[perm[k]].
hipError_t launch_count_active(const uint8_t* mask, int n_tok, int d_ff, uint32_t* counts, hipStream_t s);
void hot_order(const uint32_t* counts, int d_ff, int seg, int32_t* perm);
hipError_t launch_permute_rows(const void* src, int rows, int row_bytes, const int32_t* perm, void* dst,
                               hipStream_t s);

// Streaming read of bytes of src by blocks workgroups; out[b] = XOR of the
// 32-bit words workgroup b read (k_stream.hip).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t s);
// Gathered read of the rows listed in rows[0 .. min(*count, max_count)) of a
// [n_rows][row_bytes] matrix; out[b] = XOR of the words workgroup b read.
hipError_t launch_gather_read(const void* src, int n_rows, int row_bytes, const int32_t* rows, const int32_t* count,
                              int max_count, uint32_t* out, int blocks, hipStream_t s);

}  // namespace pi
