/*
 * pi.h -- C ABI of libpi: a predictor-gated, neuron-aware sparse FFN for one
 * AMD MI355X (gfx950).
 *
 * The method (PowerInfer, as three web pages describe it):
 *  - [QB] QbitAI article on r-manual.ru, "2080 Ti может запускать большие
 *    модели 70B ...", sections "Что такое «разреженная активация»?",
 *    "Гибридный дизайн вывода CPU/GPU" (worked example: the predictor names
 *    neurons 3, 4 and 5; each is computed where its weights live; the partial
 *    results are merged) and "Общая архитектура PowerInfer".
 *  - [GN] GeekNews, vi.news.hada.io topic 12458, sections "Cách suy luận lai
 *    CPU/GPU" (adaptive predictor, neuron-aware sparse operators) and "Lượng
 *    tử hóa và tương thích" (INT4 Q4_0).
 *  - [AB] aibars.net profile "SJTU-IPADS/PowerInfer", sections "Componentes
 *    Principais" and "Aprofundamento nos Princípios Técnicos".
 *
 * One decode layer: a small per-layer predictor guesses which FFN neurons an
 * input activates (pi_predict), the guess becomes an ordered neuron list
 * (pi_compact), and only those neurons' weight rows are read and computed
 * (pi_sparse_ffn); pi_layer runs the three in sequence.  Every neuron stays
 * resident in device memory: there is no host/device split of neurons.
 *
 * Conventions for every entry point:
 *  - Ownership: every array pointer is DEVICE memory owned by the caller.  The
 *    library allocates and frees nothing; scratch space comes from the
 *    caller's workspace `ws` (see pi_workspace_bytes), or for
 *    pi_layer_noalloc from a static array inside the library.  Descriptor structs
 *    are host memory, read during the call only.  The library keeps no
 *    mutable global state beyond the per-device address of
 *    pi_layer_noalloc's static scratch.
 *  - Streams: calls are asynchronous and ordered on `stream` (a hipStream_t;
 *    NULL = the default stream).  No call but pi_read_flags synchronises
 *    the host or copies device->host, so every other call may be captured
 *    into a HIP graph.
 *  - Errors: arguments are validated on the host BEFORE anything is
 *    launched; on any error the call returns a status and launches nothing.
 *    A failed launch returns PI_E_HIP (pi_last_error() gives the HIP message,
 *    per host thread).  Faults inside kernels surface at the caller's next
 *    synchronisation of the stream.  No C++ exception crosses this ABI.
 *  - Layout: matrices are row-major with one row per neuron.  Activations are
 *    [n_tok][d_model].  All array pointers must be 16-byte aligned.
 *  - Determinism: identical inputs give bitwise identical outputs on every
 *    run (no atomics in any reduction; every sum has a fixed order).
 *  - Fault flags: every workspace starts with a 256-byte header whose first
 *    32-bit word collects PI_FLAG_* bits (see pi_read_flags).
 */
#ifndef PI_H_
#define PI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pi_status {
  PI_OK = 0,
  PI_E_NULL = 1,      /* a required pointer is NULL */
  PI_E_SHAPE = 2,     /* a size is out of range or sizes disagree */
  PI_E_DTYPE = 3,     /* unsupported dtype, or dtype/activation combination */
  PI_E_ALIGN = 4,     /* a pointer is not 16-byte aligned */
  PI_E_RANGE = 5,     /* tau outside (0, 1), max_count outside [0, d_ff], or overlapping buffers */
  PI_E_WORKSPACE = 6, /* ws is NULL or smaller than required */
  PI_E_HIP = 7        /* the HIP runtime refused a launch */
} pi_status;

typedef enum pi_dtype {
  PI_F32 = 0,
  PI_F16 = 1,
  PI_Q4_0 = 2 /* 4-bit weights, 32 per block with one fp16 scale; see pi_q4_0_repack */
} pi_dtype;

typedef enum pi_act {
  PI_RELU = 0,  /* h = max(w_up.x + b_up, 0)                       */
  PI_REGLU = 1, /* h = max(w_gate.x + b_gate, 0) * (w_up.x)        */
  PI_RELU2 = 2  /* h = max(w_up.x + b_up, 0)^2  (squared ReLU)     */
} pi_act;

/* Low-rank activation predictor of one layer ([QB] "Что такое «разреженная
 * активация»?": a small model per layer, trained offline, predicts the
 * neurons an input will activate).  Reading used: t = p1 x; logit
 * l_i = p2_i . t + c_i; neuron i predicted active iff sigmoid(l_i) > tau.  */
typedef struct pi_predictor {
  int32_t d_model;   /* input width d                                   */
  int32_t rank;      /* r; must be a multiple of 8                       */
  int32_t d_ff;      /* number of neurons                                */
  int32_t wtype;     /* PI_F16 or PI_F32                                 */
  const void* p1;    /* [rank][d_model]                                  */
  const void* p2;    /* [d_ff][rank]                                     */
  const float* c;    /* [d_ff] logit bias                                */
} pi_predictor;

/* FFN weights of one layer.  Row i of w_down_t holds the weights neuron i
 * adds into every output (the transposed down projection).  */
typedef struct pi_ffn {
  int32_t d_model;        /* multiple of 8 (F16), 4 (F32), 32 (Q4_0)      */
  int32_t d_ff;
  int32_t act;            /* pi_act                                        */
  int32_t wtype;          /* PI_F32, PI_F16, or PI_Q4_0 (repacked layout)  */
  const void* w_up;       /* [d_ff][d_model]                               */
  const void* w_gate;     /* [d_ff][d_model] for PI_REGLU, else ignored    */
  const void* w_down_t;   /* [d_ff][d_model]                               */
  const float* b_up;      /* [d_ff] for RELU / RELU2; NULL = no bias       */
  const float* b_gate;    /* [d_ff] for REGLU; NULL = no bias              */
} pi_ffn;

/* Bytes of workspace any call with these descriptors and n_tok tokens needs
 * (the most any entry point asks for; pi_layer needs all of it).  Either
 * descriptor may be NULL when the calls that need it are not made.  Returns
 * 0 for invalid descriptors.  */
size_t pi_workspace_bytes(const pi_predictor* pred, const pi_ffn* ffn, int32_t n_tok);

/* ---- Workspace header and fault flags -----------------------------------
 * The first PI_WS_HEADER_BYTES of every workspace are a header of 32-bit
 * words; the sections a call uses follow it.
 *   word PI_WS_FLAGS: sticky fault flags.  Kernels only OR PI_FLAG_* bits
 *     into it; nothing in the library clears it except pi_clear_flags.  A
 *     zero-filled new workspace starts with no flags.
 *   word PI_WS_WAIT_POLLS: test hook, the bound on the polls of each
 *     in-kernel wait for another workgroup's count (0 = the built-in bound,
 *     65536 polls of about 128 clock cycles each).
 *   word PI_WS_SKIP_PUBLISH: test hook, 1 + the index of one workgroup of an
 *     in-kernel list that leaves its count unpublished, so the waits of the
 *     workgroups after it give up (0 = none).
 * Both hooks exist to force the give-up path from the host; leave them 0.
 *   words PI_WS_DOWN_ROWS, PI_WS_DOWN_ROWS + 1: a 64-bit count (low word
 *     first) of the w_down_t rows that the down projections of calls on this
 *     workspace have read, summed over calls; read it with pi_read_down_rows.
 *     The list-path down projection (one or two tokens; Q4_0's tile of two)
 *     reads only the listed rows whose h is nonzero for at least one token:
 *     a row whose h is exactly zero for every token adds nothing to y, so
 *     leaving it out changes no result (for finite weights).  The
 *     matrix-core down projection reads, and counts, every listed row once
 *     per token tile.
 *   words PI_WS_UP_ROWS, PI_WS_UP_ROWS + 1: the same for the w_up rows the
 *     up projections have read (pi_read_up_rows).  Every path reads the up
 *     row of every listed neuron (the matrix cores once per token tile),
 *     except pi_layer's fused kernel with ReGLU: it reads each listed
 *     neuron's gate row first and its up row only when the gate is positive
 *     for some token, since otherwise h = relu(gate) * up is zero whatever
 *     the up row holds (again for finite weights).  A ReGLU call reads every
 *     listed neuron's w_gate row.
 *
 * With one or two tokens pi_layer needs no list: the kernel that decides a
 * neuron writes a per-neuron slot (its index, or -1), and the down
 * projection compacts slots in LDS; nothing waits.  Where pi_layer takes the
 * matrix cores (many tokens), the predictor's last kernel lists the union of
 * the predicted neurons itself: each workgroup publishes its count and waits,
 * a bounded number of polls, for the counts of the workgroups with smaller
 * indices.  That relies on the workgroups of one launch being dispatched in
 * increasing index order (as the GPU's dispatcher does), never on
 * co-residency.  If a wait runs out anyway, the call raises
 * PI_FLAG_WAIT_EXPIRED and writes NaN to every element of its y, so a wrong
 * list never passes as a result.  */
#define PI_WS_HEADER_BYTES 256
#define PI_WS_FLAGS 0
#define PI_WS_WAIT_POLLS 1
#define PI_WS_SKIP_PUBLISH 2
#define PI_WS_DOWN_ROWS 4
#define PI_WS_UP_ROWS 6
#define PI_FLAG_WAIT_EXPIRED 1u /* an in-kernel wait gave up; that call's y is all NaN            */
#define PI_FLAG_FP16_RANGE 2u   /* a value the matrix-core path keeps in fp16 (the FFN's H, or the
                                   predictor's t) was not finite after rounding to fp16; the
                                   affected outputs are inf or NaN                              */

/* Zero the header of ws (flags, test hooks, row count).  Asynchronous on stream, a
 * kernel (no memset), so it may be captured into a graph.
 * Errors: NULL ws, ws not 16-byte aligned.  */
pi_status pi_clear_flags(void* ws, void* stream);

/* Read the flags word of ws into *flags (host memory).  One of the two
 * SYNCHRONOUS calls of this library (with pi_read_down_rows and
 * pi_read_up_rows): it waits for
 * the work queued on stream before it returns, so the flags of every earlier
 * call on that stream are included.
 * Errors: NULL pointers, ws not 16-byte aligned, PI_E_HIP.  */
pi_status pi_read_flags(const void* ws, uint32_t* flags, void* stream);

/* Read the header's count of down-projection rows read (PI_WS_DOWN_ROWS)
 * into *rows (host memory).  SYNCHRONOUS, like pi_read_flags.
 * Errors: NULL pointers, ws not 16-byte aligned, PI_E_HIP.  */
pi_status pi_read_down_rows(const void* ws, uint64_t* rows, void* stream);

/* The same for the count of w_up rows read (PI_WS_UP_ROWS).  SYNCHRONOUS.
 * Errors: NULL pointers, ws not 16-byte aligned, PI_E_HIP.  */
pi_status pi_read_up_rows(const void* ws, uint64_t* rows, void* stream);

/* Predict which neurons each token activates.
 *   x:      [n_tok][d_model], dtype xtype == pred->wtype
 *   tau:    probability threshold in (0, 1); compared as l_i > ln(tau/(1-tau))
 *           in fp32 (a NaN logit is inactive)
 *   mask:   out [n_tok][d_ff] uint8, 1 = predicted active, 0 = not
 *   logits: optional out [n_tok][d_ff] fp32 (may be NULL)
 *   ws:     workspace (the first rank*n_tok*4 bytes are used)
 * Cited passage: [QB] "Гибридный дизайн вывода CPU/GPU" (the prediction step
 * of the worked example) and [GN] "Cách suy luận lai CPU/GPU".  */
pi_status pi_predict(const pi_predictor* pred, const void* x, int32_t xtype, int32_t n_tok,
                     float tau, uint8_t* mask, float* logits,
                     void* ws, size_t ws_bytes, void* stream);

/* Turn masks into the ascending list of marked neurons.
 *   mask:  [n_tok][d_ff] uint8; an entry marks its neuron when nonzero; with
 *          n_tok > 1 the list is the union over tokens
 *   idx:   out [d_ff] int32; entries [0, *count) are written, ascending
 *   count: out, ONE int32 in device memory (never copied to the host)
 * Cited passage: [QB] "Гибридный дизайн вывода CPU/GPU" (the predicted set
 * {3, 4, 5}).  */
pi_status pi_compact(const uint8_t* mask, int32_t n_tok, int32_t d_ff,
                     int32_t* idx, int32_t* count, void* stream);

/* FFN over listed neurons only; unlisted neurons contribute exactly zero.
 *   x:         [n_tok][d_model]; xtype == ffn->wtype, or PI_F16 for Q4_0
 *   idx:       device int32 list, strictly increasing, values in [0, d_ff)
 *              (as pi_compact writes it); duplicates are undefined.  The
 *              buffer must hold max_count entries: entries past *count may
 *              be read (and ignored).  An entry outside [0, d_ff) adds
 *              nothing.
 *   count:     device int32: number of valid entries of idx
 *   max_count: host bound on *count, in [0, d_ff]; sizes the launch (pass
 *              d_ff when unknown).  A device count above max_count is clamped
 *              to max_count.
 *   y:         out [n_tok][d_model], ytype PI_F32 or PI_F16 (round to nearest
 *              even); every token evaluates every listed neuron
 * Cited passage: [QB] "Что такое «разреженная активация»?" (only the
 * activated neurons are computed) and "Общая архитектура PowerInfer" (partial
 * results merged into the output).  */
pi_status pi_sparse_ffn(const pi_ffn* ffn, const void* x, int32_t xtype, int32_t n_tok,
                        const int32_t* idx, const int32_t* count, int32_t max_count,
                        void* y, int32_t ytype, void* ws, size_t ws_bytes, void* stream);

/* One layer: pi_predict, pi_compact, pi_sparse_ffn on the same x.  The
 * predictor and FFN must agree on d_model and d_ff.  Mask, list and count
 * live in ws.  y is all NaN when the call raised PI_FLAG_WAIT_EXPIRED (see
 * the workspace header above).  Cited passage: [QB] "Общая архитектура
 * PowerInfer".  */
pi_status pi_layer(const pi_predictor* pred, const pi_ffn* ffn, const void* x, int32_t xtype,
                   int32_t n_tok, float tau, void* y, int32_t ytype,
                   void* ws, size_t ws_bytes, void* stream);

/* ---- A layer call that allocates nothing --------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same call and result as pi_layer (bit for bit), with its
 * scratch in a static device array of PI_NOALLOC_SCRATCH_BYTES inside the
 * library: one per GPU, held until the process ends, its address taken once
 * per device on the first call there (with that device current).  The call
 * itself allocates nothing and calls no allocating routine.
 *   x, y, descriptors, n_tok, tau, xtype, ytype, stream: as pi_layer; the
 *   stream must belong to the current device.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents: calls that overlap on one GPU (different streams, or
 * different host threads) race and give wrong results; order them.  Each
 * call clears the counters it waits on itself.  The scratch's fault flags
 * cannot be read; a call whose in-kernel wait gave up still writes NaN to y.
 * Errors: as pi_layer; PI_E_WORKSPACE (with a pi_last_error() message) when
 * pi_workspace_bytes(pred, ffn, n_tok) exceeds PI_NOALLOC_SCRATCH_BYTES --
 * up to 32 tokens per call fit for fp16 layers of the Falcon-40B / Llama2-70B
 * shapes, 16 for Q4_0.  */
#define PI_NOALLOC_SCRATCH_BYTES (32u << 20)
pi_status pi_layer_noalloc(const pi_predictor* pred, const pi_ffn* ffn, const void* x, int32_t xtype,
                           int32_t n_tok, float tau, void* y, int32_t ytype, void* stream);

/* Convert canonical Q4_0 blocks into the layout the kernels read.
 *   src: [rows][cols/32] blocks of 18 bytes (little-endian fp16 scale d, then
 *        16 bytes; byte j holds code j in its low nibble and code j+16 in its
 *        high nibble; code q means weight d*(q-8))
 *   dst: rows*cols/32*18 bytes: all rows' 16-byte code groups first
 *        ([rows][cols/32][16]), then all scales ([rows][cols/32] fp16).
 *        Inside a code group, 32-bit word k (k = 0..3, little-endian) holds
 *        weight pairs p = 4k+u (u = 0..3): code 2p in bits [4u, 4u+4) and
 *        code 2p+1 in bits [16+4u, 20+4u).
 * cols must be a multiple of 32.  src and dst must not overlap.
 * Cited passage: [GN] "Lượng tử hóa và tương thích" (INT4 Q4_0).  */
pi_status pi_q4_0_repack(const void* src, int32_t rows, int32_t cols, void* dst, void* stream);

/* ---- Neuron placement by hotness (offline, at load time) ----------------
 * Cited passages: [QB] "Локальность вывода, вызванная редкой активацией"
 * (firing follows a power law: a small share of neurons carries most
 * activations) and "Гибридный дизайн вывода CPU/GPU" (each neuron's hot or
 * cold character is analysed in advance and decides its placement).  Here
 * placement is a neuron's row inside its layer: pi_layer's fused kernel
 * gives each workgroup a segment of PI_SEGMENT_ROWS consecutive neurons, and
 * dealing hot neurons evenly over the segments evens out the active rows per
 * workgroup.  Applying one permutation to every per-neuron array of a layer
 * (rows of w_up, w_gate, w_down_t and p2; entries of c, b_up, b_gate) renames
 * its neurons: the layer computes the same y up to summation order, and
 * masks and lists then refer to the new row numbers.  */
#define PI_SEGMENT_ROWS 32

/* Firing counts of calibration tokens:
 *   mask:   [n_tok][d_ff] u8, nonzero = active (as pi_predict writes)
 *   counts: [d_ff] u32, device; counts[i] += number of tokens t with
 *           mask[t][i] != 0 (accumulates over calls; the caller zeroes it).
 * Errors: NULL pointers, n_tok < 1, d_ff < 1.  */
pi_status pi_count_active(const uint8_t* mask, int32_t n_tok, int32_t d_ff, uint32_t* counts, void* stream);

/* Placement order from firing counts.  HOST memory, synchronous, no device
 * work: counts [d_ff], perm [d_ff] out.  perm[k] = the neuron placed at row k.
 * Neurons sorted by count, highest first (ties: lower neuron number first),
 * are dealt over n_seg = ceil(d_ff / PI_SEGMENT_ROWS) segments: the k-th one
 * takes slot k / n_seg of segment k % n_seg, segments walked forward on even
 * slots and backward on odd slots; positions past d_ff are skipped.
 * Errors: NULL pointers, d_ff < 1.  */
pi_status pi_hot_order(const uint32_t* counts, int32_t d_ff, int32_t* perm);

/* Placement order by rank: perm[k] = the neuron with the k-th highest count
 * (ties: lower neuron number first), so the always-firing neurons take the
 * first rows, contiguous.  HOST memory, synchronous, no device work.  The
 * alternative to pi_hot_order's dealing, for locality of the hot rows rather
 * than balance over segments.  Errors: NULL pointers, d_ff < 1.  */
pi_status pi_rank_order(const uint32_t* counts, int32_t d_ff, int32_t* perm);

/* Row permutation: dst row k = src row perm[k], k < rows.
 *   src, dst: rows * row_bytes bytes each, device, must not overlap;
 *             16-byte aligned
 *   perm:     [rows] i32, device; should be a permutation of [0, rows) (an
 *             entry outside that range gives a zero row, never a read out of
 *             bounds)
 *   row_bytes: a multiple of 4 (4 for a per-neuron fp32 vector).  Q4_0
 *             weights are permuted as canonical blocks (row_bytes =
 *             cols / 32 * 18) before pi_q4_0_repack.
 * Errors: NULL pointers, rows < 1, row_bytes < 4 or not a multiple of 4,
 * misaligned pointers, overlapping buffers.  */
pi_status pi_permute_rows(const void* src, int32_t rows, int32_t row_bytes, const int32_t* perm, void* dst,
                          void* stream);

/* ---- Measurement aid ----------------------------------------------------
 * Not an operation of the method: a plain streaming read of a device buffer,
 * the achievable HBM read bandwidth against which the path's own streams and
 * gathers are reported.
 *   src:   bytes of device memory, 16-byte aligned; bytes a positive
 *          multiple of 16
 *   out:   [PI_STREAM_BLOCKS] u32, device; out[b] = XOR of the 32-bit words
 *          that workgroup b read, so the XOR over out[] is the XOR of every
 *          32-bit word of src (a check that every byte was read).
 * Errors: NULL pointers, bytes 0 or not a multiple of 16, misaligned src.  */
#define PI_STREAM_BLOCKS 2048
pi_status pi_stream_read(const void* src, size_t bytes, uint32_t* out, void* stream);

/* The same read restricted to listed rows: the rows rows[0 .. n) of a
 * [n_rows][row_bytes] matrix, n = min(*count, max_count), each read whole
 * (one wave per row, 16-byte loads), in list order across the grid.  This
 * is the access pattern of the sparse FFN's weight gathers without their
 * arithmetic, the ceiling such a gather can reach.
 *   src:   n_rows * row_bytes bytes, device, 16-byte aligned
 *   rows:  device int32 list (at least max_count entries readable); an
 *          entry outside [0, n_rows) reads nothing
 *   count: device int32
 *   out:   [PI_STREAM_BLOCKS] u32, device; the XOR over out[] is the XOR of
 *          every 32-bit word of the listed rows (a row listed twice cancels)
 * Errors: NULL pointers, n_rows < 1, row_bytes not a positive multiple of
 * 16, max_count < 0, misaligned pointers.  */
pi_status pi_gather_read(const void* src, int32_t n_rows, int32_t row_bytes, const int32_t* rows,
                         const int32_t* count, int32_t max_count, uint32_t* out, void* stream);

/* Static text for a status code.  */
const char* pi_status_str(pi_status s);

/* Text of the last PI_E_HIP error, or of pi_layer_noalloc's PI_E_WORKSPACE,
 * on this host thread ("" if none).  */
const char* pi_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PI_H_ */
