// The C ABI of libpi (declared in include/pi.h): host-side validation,
// workspace layout and the launch sequence of each entry point.  Every
// argument check happens before the first launch, so a rejected call has no
// effect on the device.
#include <math.h>
#include <string.h>

#include <mutex>
#include <string>

#include "pi.h"
#include "pi_internal.h"

namespace {

thread_local std::string g_last_error;

pi_status hip_fail(hipError_t e) {
  g_last_error = hipGetErrorString(e);
  return PI_E_HIP;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

int elems_per_chunk(int wtype) { return wtype == PI_F16 ? 8 : (wtype == PI_F32 ? 4 : 32); }

pi_status check_pred(const pi_predictor* p) {
  if (!p) return PI_E_NULL;
  if (p->wtype != PI_F16 && p->wtype != PI_F32) return PI_E_DTYPE;
  if (p->d_model <= 0 || p->rank <= 0 || p->d_ff <= 0) return PI_E_SHAPE;
  if (p->rank % 8 || p->rank > 4096) return PI_E_SHAPE;
  if (p->d_model % elems_per_chunk(p->wtype)) return PI_E_SHAPE;
  if (!p->p1 || !p->p2 || !p->c) return PI_E_NULL;
  if (!al16(p->p1) || !al16(p->p2) || !al16(p->c)) return PI_E_ALIGN;
  return PI_OK;
}

pi_status check_ffn(const pi_ffn* f) {
  if (!f) return PI_E_NULL;
  if (f->wtype != PI_F16 && f->wtype != PI_F32 && f->wtype != PI_Q4_0) return PI_E_DTYPE;
  if (f->act != PI_RELU && f->act != PI_REGLU && f->act != PI_RELU2) return PI_E_DTYPE;
  if (f->d_model <= 0 || f->d_ff <= 0) return PI_E_SHAPE;
  if (f->d_model % elems_per_chunk(f->wtype)) return PI_E_SHAPE;
  if (!f->w_up || !f->w_down_t) return PI_E_NULL;
  if (f->act == PI_REGLU && !f->w_gate) return PI_E_NULL;
  if (!al16(f->w_up) || !al16(f->w_down_t)) return PI_E_ALIGN;
  if (f->act == PI_REGLU && !al16(f->w_gate)) return PI_E_ALIGN;
  if (f->b_up && !al16(f->b_up)) return PI_E_ALIGN;
  if (f->b_gate && !al16(f->b_gate)) return PI_E_ALIGN;
  return PI_OK;
}

int x_type_of(const pi_ffn* f) { return f->wtype == PI_Q4_0 ? PI_F16 : f->wtype; }

// Workspace: the header (pi.h), then only the sections the entry point uses,
// in this order, every section 256-byte aligned.  The status section holds
// one counter per segment of the in-kernel list and, after them, the
// per-call fault word.
struct Layout {
  size_t t = 0, tpart = 0, mask = 0, idx = 0, count = 0, status = 0, h = 0, part = 0;
  size_t total = 0;
  int n_chunks = 0, n_slices = 0, n_segments = 0;
};

Layout layout(const pi_predictor* pred, const pi_ffn* ffn, int n_tok) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up256(bytes);
    return o;
  };
  take(PI_WS_HEADER_BYTES);
  if (pred) {
    L.t = take((size_t)n_tok * pred->rank * sizeof(float));
    if (pi::pred_mfma_path(pred->wtype, pred->d_model, pred->rank, n_tok))
      L.tpart = take(pi::pred_mfma_part_bytes(pred->d_model, pred->rank, n_tok));
  }
  if (pred && ffn) {
    L.mask = take((size_t)n_tok * ffn->d_ff);
    L.idx = take((size_t)ffn->d_ff * sizeof(int32_t));
    L.count = take(sizeof(int32_t));
    L.n_segments = pi::layer_segments(ffn->d_ff);
    L.status = take(((size_t)L.n_segments + 1) * sizeof(unsigned));
  }
  if (ffn) {
    const int tile = pi::sparse_tile(ffn->wtype, ffn->d_model);
    const int nt = n_tok < tile ? n_tok : tile;
    pi::sparse_chunking(ffn->wtype, ffn->d_model, &L.n_chunks, &L.n_slices);
    size_t hb = (size_t)nt * ffn->d_ff * sizeof(float);
    size_t pb = (size_t)L.n_chunks * nt * ffn->d_model * sizeof(float);
    if (pi::mfma_path(ffn->wtype, ffn->d_model, n_tok)) {
      size_t mh, mp;
      pi::mfma_workspace(ffn->wtype, ffn->d_model, ffn->d_ff, n_tok, &mh, &mp);
      hb = hb > mh ? hb : mh;
      pb = pb > mp ? pb : mp;
    }
    L.h = take(hb);
    L.part = take(pb);
  }
  L.total = off;
  return L;
}

pi_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return PI_E_WORKSPACE;
  if (!al16(ws)) return PI_E_ALIGN;
  if (ws_bytes < need) return PI_E_WORKSPACE;
  return PI_OK;
}

pi_status check_tau(float tau) {
  if (!(tau > 0.0f && tau < 1.0f)) return PI_E_RANGE;   // also rejects NaN
  return PI_OK;
}

float theta_of(float tau) {
  const double t = (double)tau;
  return (float)log(t / (1.0 - t));
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Masks (and optional logits) of n_tok tokens: the matrix-core predictor for
// many fp16 tokens, else the two predictor stages.
hipError_t predict_any(const pi_predictor* pred, const void* x, int n_tok, float theta, float* t, char* ws,
                       const Layout& L, uint8_t* mask, float* logits, hipStream_t s) {
  if (pi::pred_mfma_path(pred->wtype, pred->d_model, pred->rank, n_tok))
    return pi::launch_predict_mfma(pred->p1, pred->p2, pred->c, x, n_tok, pred->d_model, pred->rank, pred->d_ff,
                                   theta, t, ws + L.tpart, mask, logits, nullptr, nullptr, 0, nullptr, nullptr,
                                   reinterpret_cast<unsigned*>(ws), nullptr, false, nullptr, s);
  hipError_t e = pi::launch_predict_stage1(pred->wtype, pred->p1, x, n_tok, pred->d_model, pred->rank, t, nullptr,
                                           0, s);
  if (e != hipSuccess) return e;
  return pi::launch_predict_stage2(pred->wtype, pred->p2, pred->c, t, n_tok, pred->rank, pred->d_ff, theta, mask,
                                   logits, s);
}

pi::SparseArgs sparse_args(const pi_ffn* f, const void* x, int n_tok, const int32_t* idx, const int32_t* count,
                           int max_count, void* y, int ytype, char* ws, const Layout& L) {
  pi::SparseArgs a;
  a.wtype = f->wtype;
  a.act = f->act;
  a.d = f->d_model;
  a.d_ff = f->d_ff;
  a.n_tok = n_tok;
  a.max_count = max_count;
  a.w_up = f->w_up;
  a.w_gate = f->act == PI_REGLU ? f->w_gate : nullptr;
  a.w_down_t = f->w_down_t;
  a.b_up = f->b_up;
  a.b_gate = f->b_gate;
  a.x = x;
  a.idx = idx;
  a.count = count;
  a.y = y;
  a.ytype = ytype;
  a.h = reinterpret_cast<float*>(ws + L.h);
  a.part = reinterpret_cast<float*>(ws + L.part);
  a.n_chunks = L.n_chunks;
  a.n_slices = L.n_slices;
  a.flags = reinterpret_cast<unsigned*>(ws);     // the header's flags word
  a.rows_read = reinterpret_cast<unsigned long long*>(reinterpret_cast<unsigned*>(ws) + PI_WS_DOWN_ROWS);
  a.up_rows_read = reinterpret_cast<unsigned long long*>(reinterpret_cast<unsigned*>(ws) + PI_WS_UP_ROWS);
  a.fault = nullptr;
  return a;
}

pi_status check_layer(const pi_predictor* pred, const pi_ffn* ffn, const void* x, int32_t xtype, int32_t n_tok,
                      float tau, const void* y, int32_t ytype) {
  pi_status st = check_pred(pred);
  if (st != PI_OK) return st;
  if ((st = check_ffn(ffn)) != PI_OK) return st;
  if (pred->d_model != ffn->d_model || pred->d_ff != ffn->d_ff) return PI_E_SHAPE;
  if (!x || !y) return PI_E_NULL;
  if (n_tok < 1) return PI_E_SHAPE;
  if (xtype != pred->wtype || xtype != x_type_of(ffn)) return PI_E_DTYPE;
  if (ytype != PI_F32 && ytype != PI_F16) return PI_E_DTYPE;
  if (!al16(x) || !al16(y)) return PI_E_ALIGN;
  return check_tau(tau);
}

// The launch sequence of one layer on workspace w (laid out as L).
pi_status run_layer(const pi_predictor* pred, const pi_ffn* ffn, const void* x, int n_tok, float tau, void* y,
                    int ytype, char* w, const Layout& L, hipStream_t s) {
  float* t = reinterpret_cast<float*>(w + L.t);
  uint8_t* mask = reinterpret_cast<uint8_t*>(w + L.mask);
  int32_t* idx = reinterpret_cast<int32_t*>(w + L.idx);
  int32_t* count = reinterpret_cast<int32_t*>(w + L.count);
  unsigned* status = reinterpret_cast<unsigned*>(w + L.status);
  unsigned* fault = status + L.n_segments;
  unsigned* hdr = reinterpret_cast<unsigned*>(w);
  pi::SparseArgs a = sparse_args(ffn, x, n_tok, idx, count, ffn->d_ff, y, ytype, w, L);
  // The fused path takes one token tile of the list path; where either
  // stand-alone call would take the matrix cores, the layer does too.  Off the
  // fused path pi_layer equals pi_predict + pi_compact + pi_sparse_ffn bit for
  // bit; on it the up rows and H are the same, but the down projection walks
  // per-neuron slots in neuron ranges instead of list pieces, so y differs
  // from the separate calls by the order of its fp32 sums only.
  const bool fused = n_tok <= pi::sparse_tile(ffn->wtype, ffn->d_model) && n_tok <= pi::pred_tile(pred->rank) &&
                     !pi::pred_mfma_path(pred->wtype, pred->d_model, pred->rank, n_tok) &&
                     !pi::mfma_path(ffn->wtype, ffn->d_model, n_tok);
  hipError_t e;
  if (fused) {
    e = pi::launch_predict_stage1(pred->wtype, pred->p1, x, n_tok, pred->d_model, pred->rank, t, nullptr, 0, s);
    if (e != hipSuccess) return hip_fail(e);
    pi::LayerArgs la;
    la.p2 = pred->p2;
    la.c = pred->c;
    la.t = t;
    la.rank = pred->rank;
    la.theta = theta_of(tau);
    la.act = idx;            // the list section holds the per-neuron slots
    e = pi::launch_layer_fused(a, la, s);
    if (e != hipSuccess) return hip_fail(e);
    return PI_OK;
  }
  // Many tokens: predict every token, take the union list, then the list path.
  if (pi::pred_mfma_path(pred->wtype, pred->d_model, pred->rank, n_tok)) {
    // The matrix-core predictor writes the union mask and lists it (idx,
    // count) in its last kernel; the FFN reuses its step-major copy of a
    // single token tile (in block order for Q4_0 rows).
    const void* xs = nullptr;
    e = pi::launch_predict_mfma(pred->p1, pred->p2, pred->c, x, n_tok, pred->d_model, pred->rank, pred->d_ff,
                                theta_of(tau), t, w + L.tpart, nullptr, nullptr, mask, status, L.n_segments, idx,
                                count, hdr, fault, ffn->wtype == PI_Q4_0, &xs, s);
    a.xs_pre = xs;
    a.fault = fault;
  } else {
    e = predict_any(pred, x, n_tok, theta_of(tau), t, w, L, mask, nullptr, s);
    if (e != hipSuccess) return hip_fail(e);
    e = pi::launch_compact(mask, n_tok, ffn->d_ff, idx, count, s);
  }
  if (e != hipSuccess) return hip_fail(e);
  e = pi::launch_sparse_ffn(a, s);
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}


// Scratch of pi_layer_noalloc: one static array per GPU, held until the
// process ends.  Host code never uses the symbol's name as an address (on the
// host it names a stand-in, not device memory): each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current,
// and only that pointer reaches kernels.
static __device__ __align__(256) unsigned char scratch[PI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
char* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address; the first call on a device takes it
// and clears the scratch's header (a kernel on s, like pi_clear_flags).
hipError_t static_scratch(hipStream_t s, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0) return hipErrorInvalidSymbol;
    e = pi::launch_clear_header(static_cast<unsigned*>(ptr), s);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t pi_workspace_bytes(const pi_predictor* pred, const pi_ffn* ffn, int32_t n_tok) {
  if (n_tok < 1) return 0;
  if (pred && check_pred(pred) != PI_OK) return 0;
  if (ffn && check_ffn(ffn) != PI_OK) return 0;
  if (!pred && !ffn) return 0;
  return layout(pred, ffn, n_tok).total;
}

pi_status pi_predict(const pi_predictor* pred, const void* x, int32_t xtype, int32_t n_tok, float tau,
                     uint8_t* mask, float* logits, void* ws, size_t ws_bytes, void* stream) {
  pi_status st = check_pred(pred);
  if (st != PI_OK) return st;
  if (!x || !mask) return PI_E_NULL;
  if (n_tok < 1) return PI_E_SHAPE;
  if (xtype != pred->wtype) return PI_E_DTYPE;
  if (!al16(x) || !al16(mask) || (logits && !al16(logits))) return PI_E_ALIGN;
  if ((st = check_tau(tau)) != PI_OK) return st;
  const Layout L = layout(pred, nullptr, n_tok);
  if ((st = check_ws(ws, ws_bytes, L.total)) != PI_OK) return st;
  float* t = reinterpret_cast<float*>(static_cast<char*>(ws) + L.t);
  const hipError_t e = predict_any(pred, x, n_tok, theta_of(tau), t, static_cast<char*>(ws), L, mask, logits,
                                   as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_compact(const uint8_t* mask, int32_t n_tok, int32_t d_ff, int32_t* idx, int32_t* count,
                     void* stream) {
  if (!mask || !idx || !count) return PI_E_NULL;
  if (n_tok < 1 || d_ff < 1) return PI_E_SHAPE;
  if (!al16(mask) || !al16(idx) || (reinterpret_cast<uintptr_t>(count) & 3u)) return PI_E_ALIGN;
  const hipError_t e = pi::launch_compact(mask, n_tok, d_ff, idx, count, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_sparse_ffn(const pi_ffn* ffn, const void* x, int32_t xtype, int32_t n_tok, const int32_t* idx,
                        const int32_t* count, int32_t max_count, void* y, int32_t ytype, void* ws,
                        size_t ws_bytes, void* stream) {
  pi_status st = check_ffn(ffn);
  if (st != PI_OK) return st;
  if (!x || !idx || !count || !y) return PI_E_NULL;
  if (n_tok < 1) return PI_E_SHAPE;
  if (xtype != x_type_of(ffn)) return PI_E_DTYPE;
  if (ytype != PI_F32 && ytype != PI_F16) return PI_E_DTYPE;
  if (max_count < 0 || max_count > ffn->d_ff) return PI_E_RANGE;
  if (!al16(x) || !al16(idx) || !al16(y) || (reinterpret_cast<uintptr_t>(count) & 3u)) return PI_E_ALIGN;
  const Layout L = layout(nullptr, ffn, n_tok);
  if ((st = check_ws(ws, ws_bytes, L.total)) != PI_OK) return st;
  const pi::SparseArgs a =
      sparse_args(ffn, x, n_tok, idx, count, max_count, y, ytype, static_cast<char*>(ws), L);
  const hipError_t e = pi::launch_sparse_ffn(a, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_layer(const pi_predictor* pred, const pi_ffn* ffn, const void* x, int32_t xtype, int32_t n_tok,
                   float tau, void* y, int32_t ytype, void* ws, size_t ws_bytes, void* stream) {
  pi_status st = check_layer(pred, ffn, x, xtype, n_tok, tau, y, ytype);
  if (st != PI_OK) return st;
  const Layout L = layout(pred, ffn, n_tok);
  if ((st = check_ws(ws, ws_bytes, L.total)) != PI_OK) return st;
  return run_layer(pred, ffn, x, n_tok, tau, y, ytype, static_cast<char*>(ws), L, as_stream(stream));
}

pi_status pi_layer_noalloc(const pi_predictor* pred, const pi_ffn* ffn, const void* x, int32_t xtype,
                           int32_t n_tok, float tau, void* y, int32_t ytype, void* stream) {
  pi_status st = check_layer(pred, ffn, x, xtype, n_tok, tau, y, ytype);
  if (st != PI_OK) return st;
  const Layout L = layout(pred, ffn, n_tok);
  if (L.total > (size_t)PI_NOALLOC_SCRATCH_BYTES) {
    g_last_error = "pi_layer_noalloc: this layer and token count need " + std::to_string(L.total) +
                   " bytes of scratch; the library's static scratch holds " +
                   std::to_string((size_t)PI_NOALLOC_SCRATCH_BYTES) + " (use pi_layer with a workspace)";
    return PI_E_WORKSPACE;
  }
  const hipStream_t s = as_stream(stream);
  char* w = nullptr;
  const hipError_t e = static_scratch(s, &w);
  if (e != hipSuccess) return hip_fail(e);
  return run_layer(pred, ffn, x, n_tok, tau, y, ytype, w, L, s);
}

pi_status pi_q4_0_repack(const void* src, int32_t rows, int32_t cols, void* dst, void* stream) {
  if (!src || !dst) return PI_E_NULL;
  if (rows < 1 || cols < 32 || cols % 32) return PI_E_SHAPE;
  const size_t bytes = (size_t)rows * (cols / 32) * 18;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return PI_E_RANGE;   // overlapping buffers
  if (!al16(dst)) return PI_E_ALIGN;
  const hipError_t e = pi::launch_q4_0_repack(src, rows, cols, dst, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_count_active(const uint8_t* mask, int32_t n_tok, int32_t d_ff, uint32_t* counts, void* stream) {
  if (!mask || !counts) return PI_E_NULL;
  if (n_tok < 1 || d_ff < 1) return PI_E_SHAPE;
  const hipError_t e = pi::launch_count_active(mask, n_tok, d_ff, counts, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_hot_order(const uint32_t* counts, int32_t d_ff, int32_t* perm) {
  if (!counts || !perm) return PI_E_NULL;
  if (d_ff < 1) return PI_E_SHAPE;
  pi::hot_order(counts, d_ff, PI_SEGMENT_ROWS, perm);
  return PI_OK;
}

pi_status pi_rank_order(const uint32_t* counts, int32_t d_ff, int32_t* perm) {
  if (!counts || !perm) return PI_E_NULL;
  if (d_ff < 1) return PI_E_SHAPE;
  pi::hot_order(counts, d_ff, 1, perm);     // dealing over segments of one row: the sorted order
  return PI_OK;
}

pi_status pi_permute_rows(const void* src, int32_t rows, int32_t row_bytes, const int32_t* perm, void* dst,
                          void* stream) {
  if (!src || !dst || !perm) return PI_E_NULL;
  if (rows < 1 || row_bytes < 4 || row_bytes % 4) return PI_E_SHAPE;
  if (!al16(src) || !al16(dst)) return PI_E_ALIGN;
  const size_t bytes = (size_t)rows * (size_t)row_bytes;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return PI_E_RANGE;   // overlapping buffers
  const hipError_t e = pi::launch_permute_rows(src, rows, row_bytes, perm, dst, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_stream_read(const void* src, size_t bytes, uint32_t* out, void* stream) {
  if (!src || !out) return PI_E_NULL;
  if (bytes == 0 || bytes % 16) return PI_E_SHAPE;
  if (!al16(src)) return PI_E_ALIGN;
  const hipError_t e = pi::launch_stream_read(src, bytes, out, PI_STREAM_BLOCKS, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_clear_flags(void* ws, void* stream) {
  if (!ws) return PI_E_NULL;
  if (!al16(ws)) return PI_E_ALIGN;
  const hipError_t e = pi::launch_clear_header(static_cast<unsigned*>(ws), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_read_flags(const void* ws, uint32_t* flags, void* stream) {
  if (!ws || !flags) return PI_E_NULL;
  if (!al16(ws)) return PI_E_ALIGN;
  const hipStream_t s = as_stream(stream);
  hipError_t e = hipMemcpyAsync(flags, static_cast<const unsigned*>(ws) + PI_WS_FLAGS, sizeof(uint32_t),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_read_down_rows(const void* ws, uint64_t* rows, void* stream) {
  if (!ws || !rows) return PI_E_NULL;
  if (!al16(ws)) return PI_E_ALIGN;
  const hipStream_t s = as_stream(stream);
  hipError_t e = hipMemcpyAsync(rows, static_cast<const unsigned*>(ws) + PI_WS_DOWN_ROWS, sizeof(uint64_t),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_read_up_rows(const void* ws, uint64_t* rows, void* stream) {
  if (!ws || !rows) return PI_E_NULL;
  if (!al16(ws)) return PI_E_ALIGN;
  const hipStream_t s = as_stream(stream);
  hipError_t e = hipMemcpyAsync(rows, static_cast<const unsigned*>(ws) + PI_WS_UP_ROWS, sizeof(uint64_t),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

pi_status pi_gather_read(const void* src, int32_t n_rows, int32_t row_bytes, const int32_t* rows,
                         const int32_t* count, int32_t max_count, uint32_t* out, void* stream) {
  if (!src || !rows || !count || !out) return PI_E_NULL;
  if (n_rows < 1 || row_bytes < 16 || row_bytes % 16) return PI_E_SHAPE;
  if (max_count < 0) return PI_E_RANGE;
  if (!al16(src) || (reinterpret_cast<uintptr_t>(rows) & 3u) || (reinterpret_cast<uintptr_t>(count) & 3u))
    return PI_E_ALIGN;
  const hipError_t e =
      pi::launch_gather_read(src, n_rows, row_bytes, rows, count, max_count, out, PI_STREAM_BLOCKS, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e);
  return PI_OK;
}

const char* pi_status_str(pi_status s) {
  switch (s) {
    case PI_OK: return "ok";
    case PI_E_NULL: return "a required pointer is NULL";
    case PI_E_SHAPE: return "a size is out of range or sizes disagree";
    case PI_E_DTYPE: return "unsupported dtype or dtype/activation combination";
    case PI_E_ALIGN: return "a pointer is not 16-byte aligned";
    case PI_E_RANGE: return "a value is out of range (tau, max_count, overlap)";
    case PI_E_WORKSPACE: return "workspace missing or too small";
    case PI_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* pi_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
