/*
 * sparse_ffn.h -- C ABI of the activation-sparse FFN decode library (MI355X, gfx950).
 *
 * One FFN layer at decode time: a low-rank predictor scores every neuron, the scores are
 * thresholded and compacted into an ascending list of active neurons, and only those
 * neurons' rows are read: the ReLU-input rows (W_up, or W_gate and W_up in the ReLU-fied
 * gated form) and the matching rows of W_down transposed.
 *
 * Sources (web pages; no page states an API, so the calls below follow from what the
 * method does):
 *  - predict the active neurons and skip the rest: unite.ai PowerInfer overview,
 *    "Fase en línea" and "Predictores de espacialidad adaptativa"; novita.ai
 *    activation-sparsity article, sections 單層計算優化 and 自適應稀疏預測器;
 *  - operate on individual row/column vectors with no sparse-format conversion at run
 *    time: unite.ai overview, "Operador consciente de neuronas";
 *  - ReLU between up and down makes skipped rows contribute exactly zero: novita.ai
 *    article, section 激活稀疏性的可行性; ReLU on the gate for gated FFNs: section 第一階段;
 *  - gate/up of neuron i co-activate, so they are stored as one bundle: PowerInfer-2
 *    article, section 4.4 Neuron-Cluster-Level Pipeline;
 *  - offline activation profile, hot neurons first, and a neuron table back to original
 *    positions: unite.ai overview, "Fase fuera de línea" and "Colocación y gestión de
 *    neuronas";
 *  - batch: each token has its own active set; the union decides which rows are read:
 *    novita.ai article, section 批次大小影響.
 *
 * Conventions
 *  - Every pointer named *_dev or documented "device" is HIP device memory owned by the
 *    caller. Host pointers are documented "host".
 *  - `stream` is a hipStream_t passed as void*. Every device call is enqueued on it and
 *    nothing synchronizes; results are ready when the caller synchronizes the stream.
 *  - Errors: arguments are validated on the host before anything is enqueued. A rejected
 *    call returns SFFN_ERR_INVALID (or SFFN_ERR_UNSUPPORTED) and enqueues nothing. A
 *    launch failure returns SFFN_ERR_HIP. Faults inside kernels surface at the caller's
 *    next synchronization. No C++ exception crosses this interface.
 *  - Index space: indices are positions in the (packed) row order the weights are stored
 *    in. The original neuron id of packed position p is perm[p] (sparse_ffn_permutation).
 *  - Layout: all matrices are row-major with one row per neuron, rows contiguous:
 *      plain  w_act:    [d_ffn][d]        row i = W_up row of neuron i
 *      gated  w_act:    [d_ffn][2][d]     neuron i's gate row followed by its up row
 *      w_down_t:        [d_ffn][d]        row i = neuron i's column of W_down
 *      p1:              [rank][d]         predictor stage 1
 *      p2:              [d_ffn][rank]     predictor stage 2, one row per neuron
 *      x:               [B][d] fp32       tokens;  y: [B][d] fp32
 *      scores:          [B][d_ffn] fp32
 *  - Arithmetic: weights are read as stored (fp16 or fp32) and widened to fp32; every
 *    accumulation is fp32. Index lists, counts and token bits are always bit-identical
 *    from run to run; y is too when the descriptor asks for it (`deterministic`),
 *    otherwise the down projection's row splits add into y with float atomics and its
 *    last bits may vary between runs.
 *  - Range limit of the matrix-core path (2 or more tokens, fp16 weights, d a multiple of
 *    256): there each fp32 token value and each fp32 activation h is carried as a pair of
 *    fp16 halves (hi + lo, about 22 significant bits) and multiplied on the matrix cores.
 *    Every |x| and |h| must therefore stay below 65504, the largest finite fp16 value; a
 *    larger one becomes inf and its token's y is not finite. The single-token path and
 *    fp32 weights have no such limit (fp32 throughout).
 */
#ifndef SPARSE_FFN_H
#define SPARSE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SFFN_OK = 0,
  SFFN_ERR_INVALID = -1,      /* bad argument; nothing was enqueued */
  SFFN_ERR_UNSUPPORTED = -2,  /* valid but no kernel for this dtype/shape */
  SFFN_ERR_HIP = -3,          /* a HIP call failed (device query or launch) */
  SFFN_ERR_TOO_LARGE = -4     /* sparse_ffn_decode_static: the call needs more scratch than
                                 SFFN_STATIC_SCRATCH_BYTES; nothing was enqueued */
};

typedef enum { SFFN_F32 = 0, SFFN_F16 = 1 } sffn_dtype;

/* Weight layouts (sffn_desc.layout).
 * SFFN_LAYOUT_SPLIT:  w_act and w_down_t are separate arrays, as described above.
 * SFFN_LAYOUT_BUNDLE: each neuron's rows are stored together, as one bundle: w_act is
 *   [d_ffn][m][d] with m = 2 (plain: up row, down row) or 3 (gated: gate row, up row, down
 *   row), and w_down_t is NULL. Gate, up and down rows of a neuron are used together, so
 *   PowerInfer-2 stores them together and reads them in one I/O (PowerInfer-2 article,
 *   section 4.4 Neuron-Cluster-Level Pipeline). Every entry point accepts either layout
 *   with the same results; the single-pass decode (sffn_desc.single_pass) reads a neuron's
 *   bundle in one batch of loads. */
typedef enum { SFFN_LAYOUT_SPLIT = 0, SFFN_LAYOUT_BUNDLE = 1 } sffn_layout;

/* Largest batch: one bit per token in the 64-bit membership words. */
#define SFFN_MAX_BATCH 64

/* Size of the static per-device scratch array behind sparse_ffn_decode_static (16 MiB). */
#define SFFN_STATIC_SCRATCH_BYTES (16u << 20)

typedef struct sparse_ffn_s* sparse_ffn_t;

/* Layer descriptor. The handle borrows every pointer: weights and workspace must outlive
 * the handle. d and rank must be multiples of 8 (16-byte aligned fp16 rows; fp32 rows are
 * then 32-byte aligned), all device pointers 16-byte aligned. */
typedef struct {
  int32_t d;          /* model dimension */
  int32_t d_ffn;      /* number of FFN neurons */
  int32_t rank;       /* predictor rank r */
  int32_t max_batch;  /* 1 .. SFFN_MAX_BATCH; sizes the workspace */
  int32_t gated;      /* 0: h = relu(W_up x + b);  1: h = relu(W_gate x + b) * (W_up x) */
  int32_t w_dtype;    /* sffn_dtype of w_act and w_down_t */
  int32_t p_dtype;    /* sffn_dtype of p1 and p2 */
  float threshold;    /* tau: neuron i is active for a token iff its score > tau (strict; NaN inactive) */
  const void* w_act;     /* device, see layout above */
  const void* w_down_t;  /* device, [d_ffn][d]; NULL in the bundle layout */
  const float* b_act;    /* device [d_ffn]: bias inside the ReLU (b_up, or b_gate); NULL = 0 */
  const float* b_out;    /* device [d]: output bias; NULL = 0 */
  const void* p1;        /* device [rank][d] */
  const void* p2;        /* device [d_ffn][rank] */
  const float* p_bias;   /* device [d_ffn]: predictor bias c; NULL = 0 */
  void* workspace;       /* device scratch of at least sparse_ffn_workspace_bytes(); or NULL
                            with workspace_bytes 0: the handle then serves only
                            sparse_ffn_decode_static (every other call on it returns
                            SFFN_ERR_INVALID) */
  size_t workspace_bytes;
  const float* neuron_freq; /* host [d_ffn], optional: expected activation frequency of each
                               neuron (e.g. profile counts / profile tokens). Read only by
                               sparse_ffn_create, to cut the neurons into contiguous ranges
                               of about equal expected work. NULL = every neuron equal. */
  int32_t deterministic;    /* 1 (recommended; the Python layer's default): y is bitwise
                               reproducible from run to run. The down projection's row
                               splits are summed in a fixed order: two add into a zeroed y
                               (exact in either order), more hand their sums to the
                               column block's last-arriving workgroup, which adds them in
                               split order. 0: the splits add into y with float atomics
                               (a few percent faster; the last bits of y can vary between
                               runs). Index lists, counts and token bits are bit-exact
                               either way. */
  int32_t layout;           /* sffn_layout: SFFN_LAYOUT_SPLIT (0) or SFFN_LAYOUT_BUNDLE (1) */
  int32_t single_pass;      /* 1: the single-token decode (sparse_ffn_decode at B = 1, and its
                               static form) gathers each active neuron's input rows and down
                               row in one pass, keeps a partial output per workgroup and adds
                               the partials in a fixed order in a second launch (no float
                               atomics: y is bitwise reproducible whatever `deterministic`
                               says), where the layer's shape allows (weights and predictor
                               of one type, rank 64 to 512 in fp16 or 32 to 256 in fp32,
                               d <= 4096 in fp16 or 2048 in fp32; otherwise the three-launch
                               path runs). The workspace then also holds the partials (about
                               d * 4 bytes per four neuron ranges). 0: the three-launch path
                               (middle kernel, then a down projection that finds the active
                               rows again). Lists, counts, token bits and scores are the same
                               either way; y agrees to rounding. Operator fusion: novita.ai
                               activation-sparsity article, section 工程影響. */
  float dense_union;        /* 0: never. In (0, 1]: sparse_ffn_decode computes every neuron
                               for every token (the dense FFN; the predictor is skipped and
                               the published list is every neuron with every token's bit)
                               from the smallest batch size whose expected union of the
                               tokens' predicted sets, 1 - mean_i (1 - f_i)^B over the
                               neurons' neuron_freq values f_i (tokens independent), exceeds
                               this fraction. The choice depends on B only and is fixed at
                               create (needs neuron_freq). As the union grows with the batch,
                               the sparse path stops paying (novita.ai article, section
                               批次大小影響; PowerInfer-2 article, section 4.1.1 NPU-Centric
                               Prefill runs prefill dense). */
} sffn_desc;

/* Bytes of device workspace a descriptor needs (0 if the descriptor is invalid). The
 * workspace holds predictor intermediates, per-neuron activations, compaction state,
 * partial sums of tiles and of down-projection splits that workgroups hand to each other,
 * a small table of neuron ranges that sparse_ffn_create writes and every later call reads,
 * and arrival counters that sparse_ffn_create zeroes and every call leaves at zero (both
 * synchronously, at create). The size depends on the current device's compute-unit count
 * (it sets how many splits the down projection takes): query it with the device current
 * that the handle will be created on; with no device it covers any. Give each handle its
 * own workspace, and order the calls on one handle (a call that overlaps another on the
 * same workspace races with it). */
size_t sparse_ffn_workspace_bytes(const sffn_desc* desc);

/* Validate `desc` and create a handle (host metadata only). Queries the current HIP device
 * and writes the range table into the workspace with one synchronous copy. The handle is
 * bound to that device. *out is set only on SFFN_OK. */
int sparse_ffn_create(const sffn_desc* desc, sparse_ffn_t* out);

/* Free the handle's host metadata. Borrowed memory is untouched. NULL is accepted. */
int sparse_ffn_destroy(sparse_ffn_t h);

/* Predictor (both stages): scores[b][i] = P2[i] . (P1 x_b) + c[i], fp32.
 * x: device [B][d] fp32; scores: device [B][d_ffn] fp32; 1 <= B <= max_batch. */
int sparse_ffn_predict(sparse_ffn_t h, const float* x, int32_t B, float* scores, void* stream);

/* Threshold and compaction: idx = ascending list of neurons whose score exceeds tau for at
 * least one of the B tokens; *count (device int32) = its length; tokmask[k] bit b = token b
 * has neuron idx[k] active. idx: device [d_ffn] int32; count: device [1] int32; tokmask:
 * device [d_ffn] uint64, may be NULL only when B == 1. Integer results are bit-exact given
 * the scores. */
int sparse_ffn_compact(sparse_ffn_t h, const float* scores, int32_t B, int32_t* idx,
                       int32_t* count, uint64_t* tokmask, void* stream);

/* Forward over a given active list (device idx/count/tokmask as produced by
 * sparse_ffn_compact; tokmask NULL = every token uses every listed neuron):
 *   h_{k,b} = relu(w_act[idx_k] . x_b + b_act) (gated: times w_up[idx_k] . x_b), zero when
 *   bit b of tokmask[k] is 0;  y_b = sum_k h_{k,b} w_down_t[idx_k] + b_out.
 * y: device [B][d] fp32, fully overwritten (count == 0 gives y = b_out). The count is read
 * on the device; launches have fixed sizes, so the call can be captured in a HIP graph. */
int sparse_ffn_forward(sparse_ffn_t h, const float* x, int32_t B, const int32_t* idx,
                       const int32_t* count, const uint64_t* tokmask, float* y, void* stream);

/* The whole decode step for one layer with the fewest launches: predict, threshold,
 * compact and forward. Outputs y as sparse_ffn_forward would for the list that
 * sparse_ffn_compact would produce from sparse_ffn_predict's scores, and also writes that
 * list: idx, count and (if non-NULL) tokmask, same meaning as above. scores, if non-NULL,
 * receives the predictor scores. */
int sparse_ffn_decode(sparse_ffn_t h, const float* x, int32_t B, float* y, int32_t* idx,
                      int32_t* count, uint64_t* tokmask, float* scores, void* stream);

/* Dense FFN over every neuron for B tokens, any B >= 1 (prefill): y_b = sum_i
 * h_i(x_b) w_down_t[i] + b_out with h as in sparse_ffn_forward, i.e. sparse_ffn_forward over
 * the list of all d_ffn neurons with every token's bit set. No predictor. Tokens go through
 * in chunks of the handle's max_batch (the workspace's size), so B may exceed
 * SFFN_MAX_BATCH. x: device [B][d] fp32; y: device [B][d] fp32, fully overwritten. The
 * dense prefill of PowerInfer-2 (PowerInfer-2 article, section 4.1.1 NPU-Centric Prefill);
 * the sparse path pays only while the active set is a small part of the layer (novita.ai
 * activation-sparsity article, section 批次大小影響). */
int sparse_ffn_dense(sparse_ffn_t h, const float* x, int32_t B, float* y, void* stream);

/* Look-ahead decode, one token (the asynchronous predictor of the novita.ai
 * activation-sparsity article, section 上下文稀疏性: the next layer's active neurons are
 * predicted from the current layer's input, beside the current layer's weight reads).
 *
 * sparse_ffn_lookahead_begin(first, x) predicts first's active set from x (first's own
 * input, as sparse_ffn_decode would) and keeps it in first's workspace.
 * sparse_ffn_decode_lookahead(cur, next, x) then runs layer cur on its input x over the
 * set held in cur's workspace (from begin, or from the previous call, which named cur as
 * its next), writing y, idx, count and, if non-NULL, tokmask as sparse_ffn_decode does at
 * B = 1; and, when next is non-NULL, predicts next's set from this same x and keeps it in
 * next's workspace. A stack of layers 0..L-1 is: begin(h0, x0); then for each l,
 * decode_lookahead(h_l, h_{l+1} or NULL for the last, x_l). Layer l >= 1 thus uses the set
 * its own predictor gives for x_{l-1}. Below rank 512 its list is bit-exact with
 * sparse_ffn_decode's on x_{l-1} (same summation order); from rank 512 sparse_ffn_decode
 * sums stage 1 in another order, so the lists may differ for scores within rounding of the
 * threshold. y is the single-token decode's output on x_l over that list (bitwise so in
 * the deterministic mode).
 * Two launches per layer, and no wait between the launches' workgroups. x: device [1][d]
 * fp32; y: device [1][d] fp32. Both layers need weights and predictor of one type (both
 * fp16 or both fp32, the same in both layers), a predictor row of 8 to 128 16-byte chunks
 * (a power of two: rank 64 to 1024 in fp16, 32 to 512 in fp32), an input row of at most
 * 1024 chunks (plain layers: 1536; d <= 8192 or 12288 in fp16), the same d, and workspaces
 * that do not overlap (SFFN_ERR_UNSUPPORTED / SFFN_ERR_INVALID otherwise).
 * Calls on the layers involved must be ordered on one stream. The held set lives in the
 * layer's workspace: other calls on that layer may overwrite it (sparse_ffn_decode at one
 * token leaves the set of its own input); a layer never predicted holds the empty set. */
int sparse_ffn_lookahead_begin(sparse_ffn_t first, const float* x, void* stream);
int sparse_ffn_decode_lookahead(sparse_ffn_t cur, sparse_ffn_t next, const float* x, float* y,
                                int32_t* idx, int32_t* count, uint64_t* tokmask, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sparse_ffn_decode with the same
 * arguments, results and kernels, but every per-call intermediate (predictor output,
 * activations, token bits, union and range words, split tokens, tile partial sums and
 * counters, and a copy of the handle's range table) lives in a static array of
 * SFFN_STATIC_SCRATCH_BYTES that the library holds on each device it runs on until the
 * process ends; the handle's workspace is not touched (it may be NULL, see sffn_desc).
 * It allocates nothing: no hipMalloc, no hipFree, no memset; one small kernel writes the
 * range table and zeroes the counters at the start of every call.
 * Limits: the scratch the call needs is sparse_ffn_workspace_bytes() of the descriptor
 * with max_batch = B; above SFFN_STATIC_SCRATCH_BYTES it returns SFFN_ERR_TOO_LARGE and
 * enqueues nothing (16 MiB covers d_ffn = 16384, rank 256, d = 4096 up to 64 tokens, and
 * d_ffn = 49152, rank 1024, d = 12288 up to 32). The handle must have been created on the
 * device whose stream is passed. Every call on a device shares that device's one array
 * and leaves its contents behind: two calls on one device that overlap in time (on
 * different streams, or from different threads, on any handles) race with each other and
 * give wrong results; order them on one stream. The look-ahead entry points keep their
 * state in the workspace and have no static form. */
int sparse_ffn_decode_static(sparse_ffn_t h, const float* x, int32_t B, float* y, int32_t* idx,
                             int32_t* count, uint64_t* tokmask, float* scores, void* stream);

/* Measurement hook. events: NULL (off) or an array of six hipEvent_t (passed as void*)
 * created by the caller. While set, every sparse_ffn_decode on this handle launches its
 * three kernels so that each dispatch stamps a pair of events with its own start and end
 * time: events[0..1] the predictor stage-1 kernel, events[2..3] the fused middle kernel
 * (stage 2, threshold, compaction, gather), events[4..5] the down projection. Then
 * hipEventElapsedTime(events[2k], events[2k+1]) is that kernel's execution time, the same
 * interval a kernel-trace profiler reports. Use it outside graph capture. The events are
 * borrowed; the handle only stores the six values. Returns SFFN_ERR_INVALID for a NULL
 * handle or a NULL entry. */
int sparse_ffn_set_timing_events(sparse_ffn_t h, void* const* events);

/* Measurement helper, not a step of the method: enqueue a plain read stream over bytes of
 * device memory at buf (16-byte aligned; bytes a positive multiple of 16), 16-byte loads,
 * non-temporal, by `workgroups` workgroups of 256 threads (0 = 8 per compute unit). Timed
 * by the caller (events around the call), it gives the read bandwidth this device
 * achieves, the practical ceiling of every weight stream of the decode path, reported
 * beside the nominal HBM peak. sink: device uint32 [workgroups] the kernel may write (it
 * practically never does; the possible store keeps the loads from being removed). Nothing
 * is read from sink. Returns SFFN_ERR_INVALID on a bad argument. */
int sparse_ffn_read_probe(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                          void* stream);

/* Dense prefill on the matrix cores: y_b = the dense FFN of x_b over every neuron (as
 * sparse_ffn_dense), for any number of tokens B >= 1, with the two products blocked for
 * reuse (each weight tile is read once per 128 tokens). The pages run prefill dense
 * (PowerInfer-2 article, section 4.1.1 NPU-Centric Prefill). Arithmetic as on the
 * matrix-core decode path: fp16 weights, fp32 activations as fp16 hi + lo pairs (same
 * range limit), fp32 accumulation; y is bitwise reproducible. Requires fp16 weights and d
 * a multiple of 128 (else SFFN_ERR_UNSUPPORTED; sparse_ffn_dense covers every shape).
 * x: device [B][d] fp32; y: device [B][d] fp32, fully overwritten. work: device scratch,
 * 256-byte aligned, of work_bytes >= sparse_ffn_prefill_work_bytes(h, 128); the tokens are
 * processed in chunks of the largest multiple of 128 whose scratch fits work_bytes. The
 * handle's workspace is not used. sparse_ffn_prefill_work_bytes returns the scratch for
 * chunks of chunk_tokens (rounded up to 128), or 0 for a NULL handle, chunk_tokens < 1 or
 * an unsupported layer. */
size_t sparse_ffn_prefill_work_bytes(sparse_ffn_t h, int32_t chunk_tokens);
int sparse_ffn_prefill(sparse_ffn_t h, const float* x, int32_t B, float* y, void* work,
                       size_t work_bytes, void* stream);

/* sparse_ffn_prefill with flags (0: exactly sparse_ffn_prefill). SFFN_PREFILL_FP16_ACT
 * rounds the activations to fp16 once, x before the up products and h before the down
 * product (round to nearest even; the same |x|, |h| < 65504 limit), and runs each product
 * once instead of as a hi + lo pair: half the matrix-core work and activation traffic, at
 * fp16 activation precision (about 11 significant bits per activation; the weights, the
 * fp32 accumulation and the bitwise reproducibility are unchanged). Same arguments,
 * scratch and errors as sparse_ffn_prefill; other flag bits give SFFN_ERR_INVALID. */
#define SFFN_PREFILL_FP16_ACT 1
int sparse_ffn_prefill_ex(sparse_ffn_t h, const float* x, int32_t B, float* y, void* work,
                          size_t work_bytes, int32_t flags, void* stream);

/* Input-sparse up projection probe: a measurement, not a step of the decode path. The
 * second ReLU-fication stage puts a ReLU after RMSNorm, so about half of the up
 * projection's input x is zero (novita.ai activation-sparsity article, section 第二階段).
 * The decode path gathers whole rows of W_u for the listed neurons, where a zero inside a
 * row's 128-byte line saves no bytes; this probe computes the same products from a
 * column-major copy of W_u, which can skip the zero inputs, so the two can be timed
 * against each other. One token, fp16 weights, fp32 x and u, fp32 accumulation.
 *   layout SFFN_UP_ROWS: w_up [d_ffn][d] (the path's row layout); idx, count: device list
 *     of neuron ids (count <= d_ffn; ids outside [0, d_ffn) read row 0); u[k] = w_up[idx[k]]
 *     . x for k < *count (device, at least d_ffn floats). words, work unused (may be NULL).
 *   layout SFFN_UP_COLUMNS: w_up [d][d_ffn] (W_u transposed); words: device uint64
 *     [ceil(d_ffn / 64)], bit i % 64 of word i / 64 = neuron i listed (d_ffn % 8 == 0); u[i]
 *     (device [d_ffn]) = sum over j with x[j] != 0 of w_up[j][i] x[j] for each neuron i of a
 *     16-byte piece (8 neurons) that holds a listed neuron, 0 for the others; inputs and
 *     pieces that are skipped are not read. work: device scratch of at least
 *     sparse_ffn_up_probe_work_bytes(d_ffn) bytes. idx, count unused.
 * d % 8 == 0, d <= 16384; w_up and x 16-byte aligned. Returns SFFN_ERR_INVALID on a bad
 * argument (nothing enqueued). */
enum { SFFN_UP_ROWS = 0, SFFN_UP_COLUMNS = 1 };
size_t sparse_ffn_up_probe_work_bytes(int32_t d_ffn);
int sparse_ffn_up_probe(const void* w_up, int32_t layout, int32_t d, int32_t d_ffn,
                        const float* x, const int32_t* idx, const int32_t* count,
                        const uint64_t* words, float* u, void* work, size_t work_bytes,
                        void* stream);

/* Human-readable text for a status code (static storage). */
const char* sparse_ffn_status_string(int status);

/* ---- offline helpers: run once per layer before sparse_ffn_create ---- */

/* Activation profile: counts[i] (device int64, overwritten) = number of the N tokens x
 * (device [N][d] fp32) for which neuron i's ReLU input w_act[i] . x + b_act[i] is > 0
 * (the gate row for gated layers, whose row stride is 2*d). Computed in fp32. */
int sparse_ffn_profile_counts(const void* w_act, int32_t w_dtype, int32_t gated,
                              const float* b_act, int32_t d, int32_t d_ffn, const float* x,
                              int32_t N, int64_t* counts, void* stream);

/* Hot-first permutation (host, pure): perm[new] = old. The n_hot neurons with the largest
 * counts come first, by count descending and original index ascending on ties; the rest
 * follow in ascending original index. counts, perm: host arrays of d_ffn. */
int sparse_ffn_permutation(const int64_t* counts, int32_t d_ffn, int32_t n_hot,
                           int32_t* perm_new_to_old);

/* Row gather copy (device): the row_bytes bytes at dst + i*dst_stride_bytes become source
 * row perm[i] (source rows are contiguous, row_bytes apart). row_bytes and
 * dst_stride_bytes are multiples of 4; dst_stride_bytes = 0 means row_bytes. A stride
 * larger than the row interleaves matrices, e.g. the gated [d_ffn][2][d] bundle is two
 * calls with stride 2*d*elem, the second at dst + d*elem. src, dst: device; perm: device
 * int32 [rows], values in 0..rows-1 (bounds-checked on the device: an out-of-range entry
 * leaves that destination row untouched). */
int sparse_ffn_pack_rows(const void* src, const int32_t* perm, void* dst, int32_t rows,
                         int64_t row_bytes, int64_t dst_stride_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_FFN_H */
