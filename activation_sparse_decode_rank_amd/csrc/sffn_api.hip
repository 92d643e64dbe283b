// C-ABI host code of the activation-sparse FFN decode library: argument validation,
// handle creation, workspace carve-up, load-balanced neuron ranges, and the offline
// helpers. Every check happens before anything is enqueued; no C++ exception escapes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "../../include/sparse_ffn.h"
#include "sffn_host.h"
#include "sffn_internal.h"

struct sparse_ffn_s {
  sffn_desc desc;
  sffn::LayerDev L;
  int max_batch;
  hipEvent_t ev[6];
  bool timing;
  bool has_ws;                  // false: created without a workspace (static decode only)
  int device;                   // the HIP device current at creation
  std::vector<int32_t> rs_host;  // the range table (g_mid + 1 entries), for the static decode
};

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int t) { return t == SFFN_F32 || t == SFFN_F16; }

// Shape and pointer checks shared by workspace sizing and create (no HIP calls).
int check_desc(const sffn_desc* d) {
  if (!d) return SFFN_ERR_INVALID;
  if (d->d <= 0 || d->d_ffn <= 0 || d->rank <= 0) return SFFN_ERR_INVALID;
  if (d->max_batch < 1 || d->max_batch > SFFN_MAX_BATCH) return SFFN_ERR_INVALID;
  if (d->gated != 0 && d->gated != 1) return SFFN_ERR_INVALID;
  if (!dtype_ok(d->w_dtype) || !dtype_ok(d->p_dtype)) return SFFN_ERR_INVALID;
  if (d->d % 8 != 0 || d->rank % 8 != 0) return SFFN_ERR_INVALID;
  if (d->d_ffn > (1 << 24)) return SFFN_ERR_UNSUPPORTED;
  if (d->layout != SFFN_LAYOUT_SPLIT && d->layout != SFFN_LAYOUT_BUNDLE) return SFFN_ERR_INVALID;
  if (d->single_pass != 0 && d->single_pass != 1) return SFFN_ERR_INVALID;
  if (!(d->dense_union >= 0.f && d->dense_union <= 1.f)) return SFFN_ERR_INVALID;
  return SFFN_OK;
}

// workspace may be NULL with workspace_bytes 0: a handle for sparse_ffn_decode_static only
// bundle layout: the down rows sit inside w_act's bundles and w_down_t must be NULL
int check_ptrs(const sffn_desc* d) {
  if (!d->w_act || !d->p1 || !d->p2) return SFFN_ERR_INVALID;
  if ((d->layout == SFFN_LAYOUT_BUNDLE) != (d->w_down_t == nullptr)) return SFFN_ERR_INVALID;
  if (!d->workspace && d->workspace_bytes != 0) return SFFN_ERR_INVALID;
  if (!aligned16(d->w_act) || !aligned16(d->w_down_t) || !aligned16(d->p1) ||
      !aligned16(d->p2) || !aligned16(d->workspace))
    return SFFN_ERR_INVALID;
  if (d->b_out && !aligned16(d->b_out)) return SFFN_ERR_INVALID;
  return SFFN_OK;
}

// the down projection's splits into the kernel argument
void split_ranges(const std::vector<int32_t>& rs, const float* freq, int ks, sffn::SplitArg& sa,
                  int& upt) {
  const std::vector<int32_t> s = sffn::host::split_ranges(rs, freq, ks, upt);
  sa = sffn::SplitArg{};
  std::copy(s.begin(), s.end(), sa.s);
}

// compute units of the current device; 0 when there is none (sizes then cover any device)
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

}  // namespace

extern "C" {

const char* sparse_ffn_status_string(int status) {
  switch (status) {
    case SFFN_OK: return "ok";
    case SFFN_ERR_INVALID: return "invalid argument";
    case SFFN_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case SFFN_ERR_HIP: return "HIP call failed";
    case SFFN_ERR_TOO_LARGE:
      return "workspace needed exceeds the static scratch buffer (SFFN_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t sparse_ffn_workspace_bytes(const sffn_desc* desc) {
  if (check_desc(desc) != SFFN_OK) return 0;
  return sffn::workspace_bytes(desc->d, desc->d_ffn, desc->rank, desc->max_batch,
                               desc->single_pass != 0, device_cus());
}

int sparse_ffn_create(const sffn_desc* desc, sparse_ffn_t* out) {
  try {
    if (!out) return SFFN_ERR_INVALID;
    int rc = check_desc(desc);
    if (rc != SFFN_OK) return rc;
    rc = check_ptrs(desc);
    if (rc != SFFN_OK) return rc;
    const bool has_ws = desc->workspace != nullptr;
    const size_t need = sffn::workspace_bytes(desc->d, desc->d_ffn, desc->rank, desc->max_batch,
                                              desc->single_pass != 0, device_cus());
    if (has_ws && desc->workspace_bytes < need) return SFFN_ERR_INVALID;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SFFN_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return SFFN_ERR_HIP;

    sffn::LayerDev L{};
    L.d = desc->d;
    L.n = desc->d_ffn;
    L.r = desc->rank;
    L.gated = desc->gated;
    L.w_f16 = desc->w_dtype == SFFN_F16;
    L.p_f16 = desc->p_dtype == SFFN_F16;
    L.tau = desc->threshold;
    L.w_act = desc->w_act;
    L.w_down_t = desc->w_down_t;
    {
      // row strides in 16-byte chunks; in the bundle layout neuron i's rows (gate,) up and
      // down follow each other, and the down rows start after the first bundle's input rows
      const int nch = desc->d / (desc->w_dtype == SFFN_F16 ? 8 : 4);
      const int m_in = desc->gated ? 2 : 1;
      if (desc->layout == SFFN_LAYOUT_BUNDLE) {
        L.act_ld = L.down_ld = (m_in + 1) * nch;
        L.w_down_t = static_cast<const char*>(desc->w_act) + (size_t)m_in * nch * 16;
      } else {
        L.act_ld = m_in * nch;
        L.down_ld = nch;
      }
    }
    L.single_pass = desc->single_pass != 0;
    L.max_batch = desc->max_batch;
    // the dense route from the smallest batch whose expected union of predicted sets (the
    // neurons' profile frequencies f_i, tokens independent: 1 - mean_i (1 - f_i)^B) exceeds
    // dense_union; 0 (or no frequencies) = never
    L.dense_from_b = sffn::host::dense_from_batch(desc->neuron_freq, desc->d_ffn,
                                                  desc->dense_union, desc->max_batch,
                                                  SFFN_MAX_BATCH + 1);
    L.b_act = desc->b_act;
    L.b_out = desc->b_out;
    L.p1 = desc->p1;
    L.p2 = desc->p2;
    L.p_bias = desc->p_bias;
    L.n_cus = cus;
    sffn::carve_workspace(L, desc->workspace, desc->max_batch, L.single_pass);
    if (!sffn::shape_supported(L, false)) return SFFN_ERR_UNSUPPORTED;

    // the static scratch array's address on this device (looked up once per device); a
    // handle without a workspace has no other device memory to run on
    if (!sffn::static_scratch_setup(dev) && !has_ws) return SFFN_ERR_HIP;
    L.g_gather = std::max(1, 2 * cus);
    L.ks_down = sffn::down_split(L, desc->deterministic != 0);
    L.ks_tile = sffn::tile_split(L);
    // deterministic mode: two splits add into y exactly in either order; more meet in the
    // fixed-order join
    L.join_tile = desc->deterministic && L.ks_tile > 2;
    L.g_up = std::max(1, std::min((desc->d_ffn + 7) / 8, 4 * cus));
    // Up tiles of 8 listed rows (twice the workgroups) while the expected union would keep
    // at most half the compute units busy with 16-row tiles: on the gated Llama-7B shape
    // 28.5 against 30.4 us a layer at 2 tokens (16% union); at 4 and 8 tokens (25%, 39%)
    // they measured slower (35.9 against 34.1, 46.5 against 45.0).
    L.up_half_b = sffn::host::union_within_batch(desc->neuron_freq, desc->d_ffn, 8.0 * cus,
                                                 std::min(desc->max_batch, 15));
    // stream-K up projection: two workgroups per compute unit, and enough that one
    // range touches at most 13 tiles of the largest list
    L.g_sk = std::min(sffn::SK_G_MAX, std::max(2 * cus, ((desc->d_ffn + 15) / 16 + 12) / 13));
    if (has_ws && hipMemset(L.dn_cnt, 0, (size_t)(desc->d / 32 + 2) * 4) != hipSuccess)
      return SFFN_ERR_HIP;
    if (has_ws && L.sk_part) {
      // its arrival counters start at zero; every call leaves them zero
      if (hipMemset(L.sk_cnt, 0, (size_t)((desc->d_ffn + 15) / 16 + 1) * 4) != hipSuccess)
        return SFFN_ERR_HIP;
    }
    // range activity words start empty, so a look-ahead decode run before any prediction
    // sees an empty set
    if (has_ws && (hipMemset(L.wbits, 0, (size_t)sffn::G_MID_MAX * 8) != hipSuccess ||
                   hipStreamSynchronize(nullptr) != hipSuccess))
      return SFFN_ERR_HIP;

    // the middle kernel reads the predictor row of every neuron and the ReLU-input row(s)
    // of the active ones; as many ranges as can be resident at once, at most G_MID_MAX
    const double wb = desc->w_dtype == SFFN_F16 ? 2.0 : 4.0;
    const double pb = desc->p_dtype == SFFN_F16 ? 2.0 : 4.0;
    const double act_row = wb * desc->d * (desc->gated ? 2.0 : 1.0);
    int resident = sffn::mid_resident_groups(L, desc->max_batch);
    if (resident <= 0) resident = 2 * cus;
    // up to RS_ARG_MAX ranges travel in the kernel arguments
    const int min_groups = (desc->d_ffn + sffn::MID_RANGE_MAX - 1) / sffn::MID_RANGE_MAX;
    const int target = std::max(std::min(resident, sffn::RS_ARG_MAX), min_groups);
    std::vector<int32_t> rs = sffn::host::balanced_ranges(
        desc->d_ffn, desc->neuron_freq, pb * desc->rank, act_row, target, sffn::MID_RANGE_MAX);
    // When the 64-neuron cap alone fixes the layout (a wide layer whose resident workgroups
    // number about n/64), the hot prefix lands in a few full ranges whose gathers run long.
    // More ranges than are resident at once then pay off: up to RS_ARG_MAX in the kernel
    // arguments, or twice the minimum (table in memory) when even that is not more. Kept
    // when the costliest range's expected bytes at least halve.
    const int wide = min_groups < sffn::RS_ARG_MAX ? sffn::RS_ARG_MAX
                                                   : std::min(2 * min_groups, sffn::G_MID_MAX);
    if (!rs.empty() && target == min_groups && wide > (int)rs.size() - 1) {
      std::vector<int32_t> rs2 = sffn::host::balanced_ranges(
          desc->d_ffn, desc->neuron_freq, pb * desc->rank, act_row, wide, sffn::MID_RANGE_MAX);
      if (!rs2.empty() &&
          sffn::host::max_range_cost(rs2, desc->neuron_freq, pb * desc->rank, act_row) <
              0.5 * sffn::host::max_range_cost(rs, desc->neuron_freq, pb * desc->rank, act_row))
        rs.swap(rs2);
    }
    L.g_mid = rs.empty() ? 0 : (int)rs.size() - 1;
    // the workspace holds a range table and activity words for at most G_MID_MAX ranges
    // (d_ffn up to 131072 at 64 neurons a range); a wider layer keeps g_mid out of range,
    // so the decode entry points return SFFN_ERR_UNSUPPORTED and nothing reads the table
    if (L.g_mid > 0 && L.g_mid <= sffn::G_MID_MAX) {
      if (has_ws && hipMemcpy(L.rs, rs.data(), rs.size() * sizeof(int32_t),
                              hipMemcpyHostToDevice) != hipSuccess)
        return SFFN_ERR_HIP;
      L.rs_in_arg = L.g_mid <= sffn::RS_ARG_MAX;
      if (L.rs_in_arg) std::copy(rs.begin(), rs.end(), L.ra.r);
      // Each down workgroup gathers its split's rows in batches of DOWN_B1_BATCH, one
      // round trip each, and the batches do not overlap. When the expected active rows
      // (from the profile) would give a split more than one batch, more splits are cut
      // instead, up to 8 in the fast mode. The OPT-175B shape at 5% expects 2458 rows:
      // 5 splits rather than 2 took its down kernel from 20.2 to 18.4 us (7 splits, all
      // 1344 workgroups not resident at once, measured the same).
      double ea = 0.0;  // expected active neurons per token
      if (desc->neuron_freq)
        for (int i = 0; i < desc->d_ffn; ++i) ea += sffn::host::clamp_freq(desc->neuron_freq[i]);
      if (desc->neuron_freq && !desc->deterministic) {
        const int want = (int)std::ceil(ea / sffn::DOWN_B1_BATCH);
        L.ks_down = std::min(std::max(L.ks_down, want), std::min(8, sffn::KS_MAX));
      }
      // joined splits: no more than keep every split's workgroup resident at once (on the
      // OPT-175B slice 4 splits instead of 5: 60.1 against 60.6 us a layer, and the
      // look-ahead decode 56.9 against 59.6; the fast mode's atomics measured better with
      // 5, 57.5 against 59.8)
      const int occ_dn = sffn::occ_down_b1(L);
      const int ks_resident = occ_dn > 0 ? std::max(1, occ_dn * cus / sffn::down_blocks(L)) : 8;
      // Deterministic mode: at most two splits add into y (two addends into a zeroed y give
      // the same sum in either order). When the expected rows need more splits than two
      // (more than two batches), the fast mode's splits meet in a fixed-order join instead:
      // at 10% activity on the OPT-6.7B shape 20.2 us a layer against 22.7 with two splits
      // and 19.0 with atomics.
      L.b1_ok = sffn::occ_mid_b1(L) >= 0;
      if (desc->deterministic && L.b1_ok) {
        const int want = desc->neuron_freq ? (int)std::ceil(ea / sffn::DOWN_B1_BATCH) : 0;
        const int ks = (L.n_cus + sffn::down_blocks(L) - 1) / sffn::down_blocks(L);
        const int kj = std::min(std::max(ks, std::min(want, ks_resident)), sffn::KS_JOIN_MAX);
        if (want > 2 && kj > 2) {
          L.ks_down = kj;
          L.join_b1 = true;
        }
      }
      split_ranges(rs, desc->neuron_freq, L.ks_down, L.sa, L.split_upt);
      L.ks_vec = L.ks_down;
      L.sa_vec = L.sa;
      L.upt_vec = L.split_upt;
      if (L.join_b1) {
        L.ks_vec = 2;
        split_ranges(rs, desc->neuron_freq, L.ks_vec, L.sa_vec, L.upt_vec);
      }
    }
    // workgroups per compute unit of this layer's look-ahead down launch (set once here:
    // the launch order depends on it, and graph capture may be running at call time)
    L.la_occ = sffn::lookahead_layer_ok(L) ? sffn::lookahead_down_occ(L) : 0;
    sparse_ffn_s* h = new (std::nothrow) sparse_ffn_s;
    if (!h) return SFFN_ERR_HIP;
    h->desc = *desc;
    h->desc.neuron_freq = nullptr;  // host array is only read here
    h->L = L;
    h->max_batch = desc->max_batch;
    for (auto& e : h->ev) e = nullptr;
    h->timing = false;
    h->has_ws = has_ws;
    h->device = dev;
    if (L.g_mid > 0 && L.g_mid <= sffn::G_MID_MAX) h->rs_host = rs;
    *out = h;
    return SFFN_OK;
  } catch (...) {
    return SFFN_ERR_HIP;
  }
}

int sparse_ffn_destroy(sparse_ffn_t h) {
  delete h;
  return SFFN_OK;
}

int sparse_ffn_predict(sparse_ffn_t h, const float* x, int32_t B, float* scores, void* stream) {
  if (!h || !x || !scores || B < 1 || B > h->max_batch) return SFFN_ERR_INVALID;
  if (!h->has_ws) return SFFN_ERR_INVALID;
  if (!aligned16(x) || !aligned16(scores)) return SFFN_ERR_INVALID;
  return sffn::launch_predict(h->L, x, B, scores, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

int sparse_ffn_compact(sparse_ffn_t h, const float* scores, int32_t B, int32_t* idx,
                       int32_t* count, uint64_t* tokmask, void* stream) {
  if (!h || !scores || !idx || !count || B < 1 || B > h->max_batch) return SFFN_ERR_INVALID;
  if (!h->has_ws) return SFFN_ERR_INVALID;
  if (B > 1 && !tokmask) return SFFN_ERR_INVALID;
  return sffn::launch_compact(h->L, scores, B, idx, count, tokmask,
                              static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

int sparse_ffn_forward(sparse_ffn_t h, const float* x, int32_t B, const int32_t* idx,
                       const int32_t* count, const uint64_t* tokmask, float* y, void* stream) {
  if (!h || !x || !idx || !count || !y || B < 1 || B > h->max_batch) return SFFN_ERR_INVALID;
  if (!h->has_ws) return SFFN_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y)) return SFFN_ERR_INVALID;
  return sffn::launch_forward(h->L, x, B, idx, count, tokmask, y,
                              static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

int sparse_ffn_decode(sparse_ffn_t h, const float* x, int32_t B, float* y, int32_t* idx,
                      int32_t* count, uint64_t* tokmask, float* scores, void* stream) {
  if (!h || !x || !y || !idx || !count || B < 1 || B > h->max_batch) return SFFN_ERR_INVALID;
  if (!h->has_ws) return SFFN_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y)) return SFFN_ERR_INVALID;
  if (!sffn::shape_supported(h->L, true)) return SFFN_ERR_UNSUPPORTED;
  return sffn::launch_decode(h->L, x, B, y, idx, count, tokmask, scores,
                             static_cast<hipStream_t>(stream), h->timing ? h->ev : nullptr) ==
                 hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

namespace {
bool lookahead_ok(sparse_ffn_t h) {
  return sffn::shape_supported(h->L, true) && sffn::lookahead_layer_ok(h->L);
}
bool overlap(const sffn_desc& a, const sffn_desc& b) {
  const char* a0 = static_cast<const char*>(a.workspace);
  const char* b0 = static_cast<const char*>(b.workspace);
  return a0 < b0 + b.workspace_bytes && b0 < a0 + a.workspace_bytes;
}
}  // namespace

int sparse_ffn_lookahead_begin(sparse_ffn_t first, const float* x, void* stream) {
  if (!first || !x || !aligned16(x) || !first->has_ws) return SFFN_ERR_INVALID;
  if (!lookahead_ok(first)) return SFFN_ERR_UNSUPPORTED;
  return sffn::run_lookahead_begin(first->L, x, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

int sparse_ffn_decode_lookahead(sparse_ffn_t cur, sparse_ffn_t next, const float* x, float* y,
                                int32_t* idx, int32_t* count, uint64_t* tokmask, void* stream) {
  if (!cur || !x || !y || !idx || !count || cur == next) return SFFN_ERR_INVALID;
  if (!cur->has_ws || (next && !next->has_ws)) return SFFN_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y)) return SFFN_ERR_INVALID;
  if (next && (next->L.d != cur->L.d || overlap(cur->desc, next->desc))) return SFFN_ERR_INVALID;
  if (!lookahead_ok(cur) || (next && !lookahead_ok(next))) return SFFN_ERR_UNSUPPORTED;
  if (next && next->L.w_f16 != cur->L.w_f16) return SFFN_ERR_UNSUPPORTED;  // one launch, one type
  return sffn::run_lookahead(cur->L, next ? &next->L : nullptr, x, y, idx, count, tokmask,
                             static_cast<hipStream_t>(stream), cur->timing ? cur->ev : nullptr) ==
                 hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

int sparse_ffn_dense(sparse_ffn_t h, const float* x, int32_t B, float* y, void* stream) {
  if (!h || !x || !y || B < 1) return SFFN_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y)) return SFFN_ERR_INVALID;
  if (!h->has_ws) return SFFN_ERR_INVALID;
  return sffn::launch_dense(h->L, x, B, y, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

size_t sparse_ffn_prefill_work_bytes(sparse_ffn_t h, int32_t chunk_tokens) {
  if (!h || chunk_tokens < 1 || !sffn::prefill_ok(h->L)) return 0;
  return sffn::prefill_work_bytes(h->L, chunk_tokens);
}

int sparse_ffn_prefill_ex(sparse_ffn_t h, const float* x, int32_t B, float* y, void* work,
                          size_t work_bytes, int32_t flags, void* stream) {
  if (!h || !x || !y || !work || B < 1) return SFFN_ERR_INVALID;
  if ((flags & ~SFFN_PREFILL_FP16_ACT) != 0) return SFFN_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y) || (reinterpret_cast<uintptr_t>(work) & 255u))
    return SFFN_ERR_INVALID;
  if (!sffn::prefill_ok(h->L)) return SFFN_ERR_UNSUPPORTED;
  if (sffn::prefill_chunk(h->L, work_bytes) < 1) return SFFN_ERR_INVALID;
  return sffn::run_prefill(h->L, x, B, y, work, work_bytes, (flags & SFFN_PREFILL_FP16_ACT) != 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

int sparse_ffn_prefill(sparse_ffn_t h, const float* x, int32_t B, float* y, void* work,
                       size_t work_bytes, void* stream) {
  return sparse_ffn_prefill_ex(h, x, B, y, work, work_bytes, 0, stream);
}

int sparse_ffn_decode_static(sparse_ffn_t h, const float* x, int32_t B, float* y, int32_t* idx,
                             int32_t* count, uint64_t* tokmask, float* scores, void* stream) {
  if (!h || !x || !y || !idx || !count || B < 1 || B > h->max_batch) return SFFN_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y)) return SFFN_ERR_INVALID;
  if (!sffn::shape_supported(h->L, true) || h->rs_host.empty()) return SFFN_ERR_UNSUPPORTED;
  if (sffn::workspace_bytes(h->L.d, h->L.n, h->L.r, B, h->L.single_pass, h->L.n_cus) >
      sffn::STATIC_SCRATCH_BYTES)
    return SFFN_ERR_TOO_LARGE;
  void* base = sffn::static_scratch_ptr(h->device);
  if (!base) return SFFN_ERR_HIP;
  return sffn::run_decode_static(h->L, h->rs_host.data(), h->L.g_mid, base, x, B, y, idx, count,
                                 tokmask, scores, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

int sparse_ffn_set_timing_events(sparse_ffn_t h, void* const* events) {
  if (!h) return SFFN_ERR_INVALID;
  if (!events) {
    h->timing = false;
    return SFFN_OK;
  }
  for (int k = 0; k < 6; ++k)
    if (!events[k]) return SFFN_ERR_INVALID;
  for (int k = 0; k < 6; ++k) h->ev[k] = static_cast<hipEvent_t>(events[k]);
  h->timing = true;
  return SFFN_OK;
}

int sparse_ffn_profile_counts(const void* w_act, int32_t w_dtype, int32_t gated,
                              const float* b_act, int32_t d, int32_t d_ffn, const float* x,
                              int32_t N, int64_t* counts, void* stream) {
  if (!w_act || !x || !counts || d <= 0 || d_ffn <= 0 || N <= 0) return SFFN_ERR_INVALID;
  if (!dtype_ok(w_dtype) || (gated != 0 && gated != 1)) return SFFN_ERR_INVALID;
  return sffn::launch_profile_counts(w_act, w_dtype == SFFN_F16, gated, b_act, d, d_ffn, x, N,
                                     counts, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

int sparse_ffn_permutation(const int64_t* counts, int32_t d_ffn, int32_t n_hot,
                           int32_t* perm_new_to_old) {
  if (!counts || !perm_new_to_old || d_ffn <= 0 || n_hot < 0 || n_hot > d_ffn)
    return SFFN_ERR_INVALID;
  try {
    sffn::host::hot_first_permutation(counts, d_ffn, n_hot, perm_new_to_old);
    return SFFN_OK;
  } catch (...) {
    return SFFN_ERR_HIP;
  }
}

int sparse_ffn_pack_rows(const void* src, const int32_t* perm, void* dst, int32_t rows,
                         int64_t row_bytes, int64_t dst_stride_bytes, void* stream) {
  if (dst_stride_bytes == 0) dst_stride_bytes = row_bytes;
  if (!src || !perm || !dst || rows <= 0 || row_bytes <= 0 || row_bytes % 4 != 0 ||
      dst_stride_bytes < row_bytes || dst_stride_bytes % 4 != 0)
    return SFFN_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(src) & 3u) || (reinterpret_cast<uintptr_t>(dst) & 3u))
    return SFFN_ERR_INVALID;
  return sffn::launch_pack_rows(src, perm, dst, rows, row_bytes, dst_stride_bytes,
                                static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

size_t sparse_ffn_up_probe_work_bytes(int32_t d_ffn) {
  return d_ffn > 0 ? sffn::up_probe_work_bytes(d_ffn) : 0;
}

int sparse_ffn_up_probe(const void* w_up, int32_t layout, int32_t d, int32_t d_ffn,
                        const float* x, const int32_t* idx, const int32_t* count,
                        const uint64_t* words, float* u, void* work, size_t work_bytes,
                        void* stream) {
  if (!w_up || !x || !u || d <= 0 || d_ffn <= 0 || d % 8 != 0 || d > 16384) return SFFN_ERR_INVALID;
  if (!aligned16(w_up) || !aligned16(x)) return SFFN_ERR_INVALID;
  if (layout == SFFN_UP_ROWS) {
    if (!idx || !count) return SFFN_ERR_INVALID;
  } else if (layout == SFFN_UP_COLUMNS) {
    if (!words || !work || d_ffn % 8 != 0 || work_bytes < sffn::up_probe_work_bytes(d_ffn))
      return SFFN_ERR_INVALID;
  } else {
    return SFFN_ERR_INVALID;
  }
  return sffn::launch_up_probe(w_up, layout, d, d_ffn, x, idx, count, words, u, work,
                               static_cast<hipStream_t>(stream)) == hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

int sparse_ffn_read_probe(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                          void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || workgroups < 0) return SFFN_ERR_INVALID;
  if (!aligned16(buf)) return SFFN_ERR_INVALID;
  int g = workgroups;
  if (g == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return SFFN_ERR_HIP;
    g = 8 * std::max(cus, 1);
  }
  return sffn::launch_read_probe(buf, bytes, g, sink, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? SFFN_OK
             : SFFN_ERR_HIP;
}

}  // extern "C"
