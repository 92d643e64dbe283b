// Host dispatch of the activation-sparse FFN decode library: workspace carve-up, launch
// geometry, and which kernels run for each entry point and batch size.
#include "sffn_device.h"

namespace sffn {
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static size_t x_hl_bytes(int d, int max_batch) { return (size_t)2 * (d / 8) * max_batch * 16; }
static size_t sk_part_bytes(int max_batch) { return max_batch >= TILE_MIN_B ? SK_PART_BYTES : 0; }
static size_t sk_cnt_bytes(int n) { return (size_t)((n + 15) / 16 + 1) * 4; }

int tile_split(int d, int n_cus) {
  const int ncb = (d + 63) / 64;
  return std::max(1, std::min(KS_JOIN_MAX, (n_cus + ncb / 2) / ncb));
}

// the down projections' join slots: up to KS_JOIN_MAX per column block of 64 outputs
// (single token: blocks of 32 or 64 columns), and for the matrix-core down projection,
// when it joins (more than two splits), one slot of 64 columns x 16 tokens per token tile
// for each of its workgroups (n_cus 0: the most splits any device could take)
size_t dn_part_bytes(int d, int max_batch, int n_cus) {
  const size_t b1 = (size_t)(d / 32 + 1) * KS_JOIN_MAX * 64 * 4;
  size_t tiles = 0;
  if (max_batch >= TILE_MIN_B) {
    const int ks = n_cus > 0 ? tile_split(d, n_cus) : KS_JOIN_MAX;
    const size_t nt = (size_t)(std::min(max_batch, MAXB) + 15) / 16;
    if (ks > 2) tiles = (size_t)((d + 63) / 64) * ks * nt * 1024 * 4;
  }
  return std::max(b1, tiles);
}

size_t workspace_bytes(int d, int n, int r, int max_batch, bool single_pass, int n_cus) {
  size_t b = 0;
  b += align256((size_t)max_batch * r * 4);      // q
  b += align256((size_t)((n + 63) / 64 * 64 + 64) * max_batch * 4);  // h_buf ([n][B], or [B][ldh])
  b += align256((size_t)n * 8);                  // tok_full
  b += align256((size_t)(G_MID_MAX + 1) * 4);    // rs (range table, written at create)
  b += align256((size_t)((n + 63) / 64) * 8);    // words
  b += align256((size_t)G_MID_MAX * 8);          // wbits
  b += align256(x_hl_bytes(d, max_batch));       // x_hl
  b += align256(sk_part_bytes(max_batch));       // sk_part
  b += align256(sk_cnt_bytes(n));                // sk_cnt
  if (single_pass) b += align256(bundle_part_bytes(d, n));  // part
  b += align256((size_t)(n + 1) * 4);            // dense_idx
  b += align256(dn_part_bytes(d, max_batch, n_cus));  // dn_part
  b += align256((size_t)(d / 32 + 2) * 4);       // dn_cnt
  return b;
}

void carve_workspace(LayerDev& L, void* ws, int max_batch, bool single_pass) {
  char* p = static_cast<char*>(ws);
  const int n = L.n;
  const int n_tiles = (n + TPB - 1) / TPB;
  auto take = [&](size_t bytes) { char* q = p; p += align256(bytes); return q; };
  L.q = reinterpret_cast<float*>(take((size_t)max_batch * L.r * 4));
  L.ldh = (n + 63) / 64 * 64 + 64;  // 64 spare slots: the down tile kernel reads past the list end
  L.h_buf = reinterpret_cast<float*>(take((size_t)L.ldh * max_batch * 4));
  L.tok_full = reinterpret_cast<uint64_t*>(take((size_t)n * 8));
  L.rs = reinterpret_cast<int32_t*>(take((size_t)(G_MID_MAX + 1) * 4));
  L.words = reinterpret_cast<uint64_t*>(take((size_t)((n + 63) / 64) * 8));
  L.wbits = reinterpret_cast<uint64_t*>(take((size_t)G_MID_MAX * 8));
  L.x_hl = take(x_hl_bytes(L.d, max_batch));
  L.sk_part = sk_part_bytes(max_batch) ? reinterpret_cast<float*>(take(sk_part_bytes(max_batch))) : nullptr;
  L.sk_cnt = reinterpret_cast<int32_t*>(take(sk_cnt_bytes(n)));
  L.part = single_pass ? reinterpret_cast<float*>(take(bundle_part_bytes(L.d, n))) : nullptr;
  L.dense_idx = reinterpret_cast<int32_t*>(take((size_t)(n + 1) * 4));
  L.dn_part = reinterpret_cast<float*>(take(dn_part_bytes(L.d, max_batch, L.n_cus)));
  L.dn_cnt = reinterpret_cast<int32_t*>(take((size_t)(L.d / 32 + 2) * 4));
  L.n_tiles = n_tiles;
}

namespace {

// the matrix-core path: fp16 weights, and each quarter of the input width a whole number
// of 64-input step pairs
bool tile_ok(const LayerDev& L, int B) {
  return B >= TILE_MIN_B && L.w_f16 && L.d % 256 == 0 && B <= MAXB;
}

}  // namespace

int down_blocks(const LayerDev& L) {
  const int nch = L.d / (L.w_f16 ? 8 : 4);
  return (nch + CB_LANES - 1) / CB_LANES;
}

int tile_split(const LayerDev& L) { return tile_split(L.d, L.n_cus); }

int down_split(const LayerDev& L, bool deterministic) {
  const int ncb = down_blocks(L);
  // at least one workgroup per compute unit (a wide layer has more column blocks than
  // half the compute units but fewer than all of them)
  int ks = std::max(1, std::min(8, (L.n_cus + ncb - 1) / ncb));
  if (deterministic) ks = std::min(ks, 2);
  return ks;
}

int mid_resident_groups(const LayerDev& L, int max_batch) {
  if (pick_cpt(row_chunks(L)) == 0 || L.w_f16 != L.p_f16) return 0;
  int occ1 = occ_mid_b1(L);
  if (occ1 < 0) occ1 = occ_mid_batch(L, 1);
  const int occb = max_batch > 1 ? occ_mid_batch(L, std::min(max_batch, TILE_MIN_B - 1)) : occ1;
  return std::min(occ1, occb) * L.n_cus;
}

bool shape_supported(const LayerDev& L, bool fused) {
  if (pick_cpt(row_chunks(L)) == 0) return false;
  const int nchp = L.r / (L.p_f16 ? 8 : 4);
  if (nchp > 256) return false;
  const int epc_p = L.p_f16 ? 8 : 4;
  if (L.d / epc_p > 8 * TPB) return false;  // stage 1 register budget
  if (fused) {
    if (L.w_f16 != L.p_f16) return false;
    if (nchp > 128 || (nchp & (nchp - 1)) != 0) return false;  // P2 row = power-of-two chunks
    if (L.g_mid < 1 || L.g_mid > G_MID_MAX) return false;
    if (L.split_upt < 1 || L.split_upt > 8) return false;  // the down kernel's word registers
    if (L.ks_down < 1 || L.ks_down > KS_MAX) return false;
    if (L.upt_vec < 1 || L.upt_vec > 8 || L.ks_vec < 1 || L.ks_vec > KS_MAX) return false;
  }
  return true;
}

hipError_t launch_predict(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s) {
  run_stage1(L, x, B, s, nullptr, nullptr, 0, false);
  // the same scores kernel the decode step runs at this batch, so both give equal scores
  if (tile_ok(L, B) && score_tiles_ok(L, B)) return run_score_tiles(L, B, scores, s);
  return run_scores(L, B, scores, s);
}

hipError_t launch_forward(const LayerDev& L, const float* x, int B, const int32_t* idx,
                          const int32_t* count, const uint64_t* tokmask, float* y, hipStream_t s) {
  if (tile_ok(L, B)) {
    run_forward_tiles(L, x, B, idx, count, tokmask, nullptr, y, true, false, s, nullptr, nullptr);
    return hipGetLastError();
  }
  run_gather(L, x, B, idx, count, tokmask, y, s);
  run_down(L, B, false, idx, count, nullptr, nullptr, nullptr, y, s, nullptr);
  return hipGetLastError();
}

// Every neuron of the layer for B tokens (any B): the identity list, then the forward
// entry point's kernels over it, in chunks of the tokens the workspace holds.
hipError_t launch_dense(const LayerDev& L, const float* x, int B, float* y, hipStream_t s) {
  hipError_t e = launch_fill_list(L, 0, L.dense_idx, L.dense_idx + L.n, nullptr, s);
  if (e != hipSuccess) return e;
  const int chunk = std::min(L.max_batch, MAXB);
  for (int b0 = 0; b0 < B; b0 += chunk) {
    const int bc = std::min(chunk, B - b0);
    e = launch_forward(L, x + (size_t)b0 * L.d, bc, L.dense_idx, L.dense_idx + L.n, nullptr,
                       y + (size_t)b0 * L.d, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_decode(const LayerDev& L, const float* x, int B, float* y, int32_t* idx,
                         int32_t* count, uint64_t* tokmask, float* scores, hipStream_t s,
                         const hipEvent_t* ev) {
  if (B >= L.dense_from_b) {
    // above the crossover: every neuron for every token (the published list says so); the
    // predictor runs only when its scores are asked for
    if (scores) {
      hipError_t e = launch_predict(L, x, B, scores, s);
      if (e != hipSuccess) return e;
    }
    hipError_t e = launch_fill_list(L, B, idx, count, tokmask, s);
    if (e != hipSuccess) return e;
    return launch_forward(L, x, B, idx, count, tokmask, y, s);
  }
  const hipEvent_t* t1 = ev ? ev + 0 : nullptr;
  const hipEvent_t* t2 = ev ? ev + 2 : nullptr;
  const hipEvent_t* t3 = ev ? ev + 4 : nullptr;
  if (tile_ok(L, B)) {
    // stage 1; scores, threshold and union words in one matrix-core kernel, with the up
    // tile kernel listing the union itself from those words (or a scatter pass when the
    // words do not fit its LDS); else scores and two compaction passes, the scores going
    // to the caller's buffer or, when none is given, to the activation buffer, which the
    // up projection only overwrites after compaction has read them; then the tiles
    run_stage1(L, x, B, s, t1, y, L.ks_tile > 1 && !L.join_tile ? B * L.d : 0, true);
    hipError_t e;
    bool fw = false;
    if (score_tiles_ok(L, B)) {
      e = run_score_tiles(L, B, scores, s);
      if (e != hipSuccess) return e;
      fw = union_in_up_ok(L);
      if (!fw) e = launch_scatter(L, idx, count, tokmask, s);
    } else {
      float* sc = scores ? scores : L.h_buf;
      e = run_scores(L, B, sc, s);
      if (e != hipSuccess) return e;
      e = launch_compact(L, sc, B, idx, count, tokmask, s);
    }
    if (e != hipSuccess) return e;
    // a caller that wants no token bits still gets per-token activations: the up kernel
    // then takes each listed neuron's bits from the compaction's by-neuron words
    run_forward_tiles(L, x, B, idx, count, tokmask, tokmask ? nullptr : L.tok_full, y, false,
                      fw, s, t2, t3);
    return hipGetLastError();
  }
  if (B == 1 && L.single_pass && bundle_ok(L)) {
    // one pass over the active neurons' bundles writes partial outputs; the reduction
    // writes all of y, so stage 1 clears nothing
    run_stage1(L, x, 1, s, t1, nullptr, 0, false);
    if (run_bundle_b1(L, x, y, idx, count, tokmask, scores, s, t2, t3)) return hipGetLastError();
  }
  // stage 1 clears y where the down projection adds its splits into it
  if (B == 1 && L.b1_ok) {
    run_stage1(L, x, 1, s, t1, y, L.ks_down > 1 && !L.join_b1 ? L.d : 0, false);
    run_mid_b1(L, x, scores, s, t2);
    run_down_b1(L, idx, count, tokmask, y, s, t3);
    return hipGetLastError();
  }
  run_stage1(L, x, B, s, t1, y, L.ks_vec > 1 ? B * L.d : 0, false);
  run_mid_batch(L, x, B, scores, s, t2);
  run_down(L, B, true, nullptr, nullptr, idx, count, tokmask, y, s, t3);
  return hipGetLastError();
}

}  // namespace sffn
