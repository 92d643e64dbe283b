// Internal interface between the C-ABI host code (sffn_api.hip), the host dispatch
// (sffn_dispatch.hip) and the kernel translation units. Not installed; the public
// interface is include/sparse_ffn.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sffn {

constexpr int G_MID_MAX = 2048;   // most workgroups the fused middle kernel may use
constexpr int MID_RANGE_MAX = 64;  // most neurons one middle workgroup may own (one 64-bit
                                   // activity word per range)
// Neuron ranges of the middle kernel passed by value in the kernel arguments, so that a
// workgroup's first weight loads do not wait on a table load (the table and the other
// arguments fit the 4 KB argument block).
constexpr int RS_ARG_MAX = 952;
struct RangeArg {
  int32_t r[RS_ARG_MAX + 1];
};
// Row splits of the decode down projection: split k covers middle-kernel ranges
// [s[k], s[k+1]), cut so that the splits expect about equal numbers of active neurons.
constexpr int KS_MAX = 16;
// rows one workgroup of the single-token down projection gathers in one batch (32 row
// slots x 16 rows in flight each)
constexpr int DOWN_B1_BATCH = 512;
// most splits the single-token down projection's fixed-order join takes
constexpr int KS_JOIN_MAX = 8;
struct SplitArg {
  int32_t s[KS_MAX + 1];
};

// Device-side view of one layer plus the workspace carve-up.
struct LayerDev {
  int d, n, r;
  int gated;
  int w_f16, p_f16;  // 1 = fp16 storage, 0 = fp32
  float tau;
  const void* w_act;
  const void* w_down_t;
  int act_ld;   // 16-byte chunks from one neuron's ReLU-input row(s) to the next neuron's
  int down_ld;  // the same for the rows of w_down_t (both larger in the bundle layout)
  const float* b_act;
  const float* b_out;
  const void* p1;
  const void* p2;
  const float* p_bias;
  // workspace regions
  float* q;            // [max_batch][r] predictor stage-1 output
  float* h_buf;        // [n][B] activations: by list position (forward) or neuron (decode)
  uint64_t* tok_full;  // [n] token bits by neuron (compaction, decode)
  int32_t* rs;         // [g_mid + 1] neuron ranges of the fused middle kernel (set at create)
  uint64_t* words;     // [ceil(n/64)] union bit words (compaction)
  void* x_hl;          // tokens split into fp16 hi/lo for the matrix-core up projection:
                       // 2 x [d/8 chunks][B token slots] x 16 bytes (sized for max_batch)
  uint64_t* wbits;     // [G_MID_MAX] activity word of each middle-kernel range (decode)
  float* part;         // single-pass decode: partial outputs of its workgroups (null: unused)
  float* sk_part;      // stream-K up projection: two part slots per workgroup (null: unused)
  int32_t* sk_cnt;     // [ceil(n/16) + 1] arrival counters of its tiles (zero between calls)
  // launch geometry fixed at create time
  int g_mid;     // workgroups of the fused middle kernel (<= G_MID_MAX)
  int n_tiles;   // compaction tiles of 256 neurons
  int g_gather;  // workgroups of the balanced gather
  int n_cus;     // compute units on the device
  int ks_down;   // row splits of the down projection (1 = plain stores; 2 keeps y bitwise
                 // reproducible; more adds float atomics in a varying order)
  bool join_b1;  // the single-token down projection's splits meet in a fixed-order join
                 // (dn_part, dn_cnt) instead of float atomics
  float* dn_part;   // split sums of the down projections' joins (dn_part_bytes)
  int32_t* dn_cnt;  // [ceil(d / 32) + 2] its arrival counters (zero between calls)
  int ks_tile;   // the same for the batch (matrix-core) down projection
  bool join_tile;  // its splits meet in the fixed-order join (deterministic mode, ks_tile > 2)
  int ldh;       // row stride of token-major activations hT [B][ldh] (d_ffn rounded up to 64, plus 64)
  int g_up;      // workgroups of the batch up projection (each loops over row tiles)
  int up_half_b;  // up to this batch size (0: none) its tiles take 8 listed rows, not 16
  int g_sk;      // workgroups of its stream-K form (at most SK_G_MAX)
  bool rs_in_arg;  // the range table travels in the middle kernel's arguments (ra)
  RangeArg ra;     // copy of the range table (valid entries 0..g_mid when rs_in_arg)
  SplitArg sa;     // decode down projection: range splits, ks_down of them
  int split_upt;   // most ranges of one split per thread of the down kernel (1, 2, 4, 8)
  bool b1_ok;      // the single-token kernels cover this layer (else one token takes the
                   // vector path)
  int ks_vec;      // the same three for the vector down projection (batches, and one token
  SplitArg sa_vec; // where the single-token kernels do not apply), which joins its splits
  int upt_vec;     // with float atomics only: at most two in the deterministic mode
  int la_occ;      // workgroups per compute unit of the look-ahead down launch (0: unknown)
  bool single_pass;  // single-token decode through the bundle pass (sffn_bundle.hip)
  int max_batch;     // tokens the workspace is sized for
  int dense_from_b;  // decode computes every neuron from this many tokens on (65: never)
  int32_t* dense_idx;  // [n + 1]: the identity list and its count, for the dense route
};

// workspace sizing (bytes) for a layer shape; mirrors the carve-up in carve_workspace
// (single_pass: also the partial outputs of the single-pass decode)
// (n_cus: compute units of the device, which sets the matrix-core down projection's
// splits; 0 sizes for any device). carve_workspace reads L.n_cus.
size_t workspace_bytes(int d, int n, int r, int max_batch, bool single_pass, int n_cus);
void carve_workspace(LayerDev& L, void* ws, int max_batch, bool single_pass);
// row splits of the matrix-core down projection for a width d on n_cus compute units
int tile_split(int d, int n_cus);
// 128-byte column blocks of the down projection, and the row split it should use
int down_blocks(const LayerDev& L);
int down_split(const LayerDev& L, bool deterministic);
int tile_split(const LayerDev& L);
// whether kernels exist for this shape (fused = the single-call decode path)
bool shape_supported(const LayerDev& L, bool fused);
// middle-kernel workgroups that can be resident at once (all CUs), for batches up to max_batch
int mid_resident_groups(const LayerDev& L, int max_batch);

// Stream-K up projection: most workgroups, and the bytes of their part slots (two slots of
// 2 matrices x 2 token tiles x 64 lanes x 4 floats each)
constexpr int SK_G_MAX = 512;
constexpr size_t SK_PART_BYTES = (size_t)2 * SK_G_MAX * 2 * 2 * 64 * 4 * 4;

// From this many tokens on (fp16 weights, d a multiple of 128) the decode and forward
// entry points run the gathered-tile matrix-core kernels.
constexpr int TILE_MIN_B = 2;

// Kernel-family entry points (one translation unit each; tev: an optional start/end event
// pair stamped by the dispatch).
// sffn_stage1.hip: predictor stage 1 (y0/ny: output zeroed for the split-k down
// projection; split_x (2+ tokens): extra workgroups write the tokens' fp16 hi/lo split into
// x_hl for the up tile kernel). sffn_decode_b1.hip: the batch-1 middle kernel (false when no
// kernel exists for the shape) and down projection.
void run_stage1(const LayerDev& L, const float* x, int B, hipStream_t s, const hipEvent_t* tev,
                float* y0, int ny, bool split_x);
bool run_mid_b1(const LayerDev& L, const float* x, float* scores, hipStream_t s,
                const hipEvent_t* tev);
int occ_down_b1(const LayerDev& L);  // workgroups per CU of the single-token down kernel
int occ_mid_b1(const LayerDev& L);  // workgroups per CU, -1 when no batch-1 kernel applies
// look-ahead decode (one token): which layers its kernels cover; begin (stage 1 and the
// scores of layer Nx on x, leaving Nx's range words); one layer C on x over its held set,
// predicting Nx's set from x when Nx is given (ev: optional six timing events, of which
// pairs 1 and 2 stamp the two launches)
bool lookahead_layer_ok(const LayerDev& L);
int lookahead_down_occ(const LayerDev& L);  // for the launch with this layer as both roles' shape
hipError_t run_lookahead_begin(const LayerDev& Nx, const float* x, hipStream_t s);
hipError_t run_lookahead(const LayerDev& C, const LayerDev* Nx, const float* x, float* y,
                         int32_t* idx, int32_t* count, uint64_t* tok, hipStream_t s,
                         const hipEvent_t* ev);
void run_down_b1(const LayerDev& L, int32_t* idx_out, int32_t* count_out, uint64_t* tok_out,
                 float* y, hipStream_t s, const hipEvent_t* tev);
// sffn_batch.hip: the middle kernel for any batch (small-batch kernel for 2..8 tokens,
// otherwise the general fused one), the down projection (bits: the decode step's list from
// the range activity words; otherwise the given idx/count), and the forward's gather.
void run_mid_batch(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s,
                   const hipEvent_t* tev);
int occ_mid_batch(const LayerDev& L, int B);
void run_down(const LayerDev& L, int B, bool bits, const int32_t* idx, const int32_t* count,
              int32_t* idx_out, int32_t* count_out, uint64_t* tok_out, float* y, hipStream_t s,
              const hipEvent_t* tev);
void run_gather(const LayerDev& L, const float* x, int B, const int32_t* idx, const int32_t* count,
                const uint64_t* tokmask, float* y0, hipStream_t s);
// sffn_mid_bt_{h,f}{4,8}.hip: the small-batch middle kernel for fp16 (h) or fp32 (f)
// weights and up to 4 or 8 tokens (false / -1 when no kernel exists for the shape)
bool run_mid_bt_h4(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s, const hipEvent_t* tev);
bool run_mid_bt_h8(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s, const hipEvent_t* tev);
bool run_mid_bt_f4(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s, const hipEvent_t* tev);
bool run_mid_bt_f8(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s, const hipEvent_t* tev);
int occ_mid_bt_h4(const LayerDev& L);
int occ_mid_bt_h8(const LayerDev& L);
int occ_mid_bt_f4(const LayerDev& L);
int occ_mid_bt_f8(const LayerDev& L);
// sffn_tiles.hip: predictor stage 2 scores, and the matrix-core forward (zero_y: clear y
// first when the down projection splits rows)
hipError_t run_scores(const LayerDev& L, int B, float* scores, hipStream_t s);
// scores, threshold and the union words in one matrix-core kernel (scores may be null),
// when q fits in LDS; then launch_scatter writes the ascending list from the words
constexpr size_t SCORE_Q_LDS = 64 * 1024;
bool score_tiles_ok(const LayerDev& L, int B);
hipError_t run_score_tiles(const LayerDev& L, int B, float* scores, hipStream_t s);
hipError_t launch_scatter(const LayerDev& L, int32_t* idx, int32_t* count, uint64_t* tokmask,
                          hipStream_t s);
// from_words: the up kernel lists the union itself from the words and token bits of
// run_score_tiles (writing idx, count and tokmask; needs union_in_up_ok) instead of
// reading them. Otherwise it reads idx and count, and each listed neuron's token bits from
// tokmask (by list position) or, when tokmask is null, from tok_by_neuron (by neuron, as
// the compaction leaves them in tok_full); both null: every token uses every listed neuron.
bool union_in_up_ok(const LayerDev& L);
void run_forward_tiles(const LayerDev& L, const float* x, int B, const int32_t* idx,
                       const int32_t* count, const uint64_t* tokmask,
                       const uint64_t* tok_by_neuron, float* y, bool zero_y, bool from_words,
                       hipStream_t s, const hipEvent_t* t_up, const hipEvent_t* t_down);

// launchers; each returns hipGetLastError() after enqueueing
hipError_t launch_predict(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s);
hipError_t launch_compact(const LayerDev& L, const float* scores, int B, int32_t* idx,
                          int32_t* count, uint64_t* tokmask, hipStream_t s);
hipError_t launch_forward(const LayerDev& L, const float* x, int B, const int32_t* idx,
                          const int32_t* count, const uint64_t* tokmask, float* y, hipStream_t s);
// ev: optional six events, a start/end pair stamped by each of the three kernel dispatches
hipError_t launch_decode(const LayerDev& L, const float* x, int B, float* y, int32_t* idx,
                         int32_t* count, uint64_t* tokmask, float* scores, hipStream_t s,
                         const hipEvent_t* ev);
hipError_t launch_profile_counts(const void* w_act, int w_f16, int gated, const float* b_act,
                                 int d, int n, const float* x, int N, int64_t* counts,
                                 hipStream_t s);
hipError_t launch_pack_rows(const void* src, const int32_t* perm, void* dst, int rows,
                            int64_t row_bytes, int64_t dst_stride_bytes, hipStream_t s);
// sffn_static.hip: the decode step over a static per-device scratch array of
// STATIC_SCRATCH_BYTES (see sparse_ffn_decode_static). setup: look the array's address up
// on device dev (current), once; ptr: that address (null before setup). run: carve the
// per-call regions of H's workspace layout for B tokens out of base, write the range table
// (g + 1 entries from the host) and zero the tile counters with a small kernel, then the
// decode step's kernels.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)16 << 20;
bool static_scratch_setup(int dev);
void* static_scratch_ptr(int dev);
hipError_t run_decode_static(const LayerDev& H, const int32_t* rs_host, int g, void* base,
                             const float* x, int B, float* y, int32_t* idx, int32_t* count,
                             uint64_t* tokmask, float* scores, hipStream_t s);
// sffn_bundle.hip: the single-token decode in one pass over each active neuron's bundle
// (input rows and down row together), then a fixed-order reduction of the workgroups'
// partial outputs that also publishes the list. ok: kernels exist for the shape; run:
// after stage 1, false when they do not (t_pass, t_reduce: optional event pairs).
constexpr int BUNDLE_RANGES_PER_GROUP = 4;
bool bundle_ok(const LayerDev& L);
bool run_bundle_b1(const LayerDev& L, const float* x, float* y, int32_t* idx, int32_t* count,
                   uint64_t* tok, float* scores, hipStream_t s, const hipEvent_t* t_pass,
                   const hipEvent_t* t_reduce);
size_t bundle_part_bytes(int d, int n);
// the dense route (sparse_ffn_dense, and decode above its union crossover): every neuron,
// no predictor; tokens in chunks of at most max_batch (and 64). idx/count/tok: where the
// identity list goes (tok may be null; B bits set per entry), or the workspace's own copy
hipError_t launch_fill_list(const LayerDev& L, int B, int32_t* idx, int32_t* count,
                            uint64_t* tok, hipStream_t s);
hipError_t launch_dense(const LayerDev& L, const float* x, int B, float* y, hipStream_t s);
// sffn_measure.hip: a plain read stream of bytes (a multiple of 16) over buf by the given
// number of workgroups; sink [workgroups] is written only in a practically impossible case
// dense prefill on the matrix cores (sffn_prefill.hip): fp16 weights, d a multiple of 128;
// scratch bytes for chunks of up to `chunk` tokens, the chunk a scratch holds, and the run
bool prefill_ok(const LayerDev& L);
size_t prefill_work_bytes(const LayerDev& L, int chunk);
int prefill_chunk(const LayerDev& L, size_t work_bytes);
hipError_t run_prefill(const LayerDev& L, const float* x, int B, float* y, void* work,
                       size_t work_bytes, bool fp16_act, hipStream_t s);
// input-sparse up projection probe: layout 0 rows [n][d], 1 columns [d][n] (fp16)
size_t up_probe_work_bytes(int n);
hipError_t launch_up_probe(const void* w, int layout, int d, int n, const float* x,
                           const int32_t* idx, const int32_t* count, const uint64_t* words,
                           float* u, void* work, hipStream_t s);
hipError_t launch_read_probe(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                             hipStream_t s);

}  // namespace sffn
