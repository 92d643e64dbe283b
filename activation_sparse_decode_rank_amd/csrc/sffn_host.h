// Host-side planning of the activation-sparse FFN decode library: pure C++ with no HIP
// dependency, so that it can also be built and checked on its own (the CPU sanitizer test
// compiles it with AddressSanitizer and UndefinedBehaviorSanitizer).
//  - neuron ranges of the middle kernel, cut for equal expected cost from the profile
//    frequencies, and the down projection's splits of those ranges;
//  - the hot-first neuron permutation (unite.ai PowerInfer overview, "Fase fuera de línea"
//    and "Colocación y gestión de neuronas": the offline profile orders neurons by how
//    often they activate);
//  - the batch size from which the decode step computes every neuron (the union of the
//    tokens' active sets grows with the batch: novita.ai activation-sparsity article,
//    section 批次大小影響);
//  - the dense prefill's plan: its up-projection tile, the down projection's neuron
//    splits and the layout of the caller's scratch.
#pragma once
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

namespace sffn {
namespace host {

// an expected frequency clamped to [0, 1]; NaN and negatives count as 0
inline double clamp_freq(float f) {
  const double v = (double)f;
  if (!(v >= 0.0)) return 0.0;
  return v > 1.0 ? 1.0 : v;
}

// Split neurons [0, n) into contiguous ranges of at most max_len neurons whose expected
// costs (predictor row bytes plus expected activation frequency times the bytes of the
// neuron's ReLU-input row(s)) are about equal, at most target_groups of them (the cost per
// range is raised until the cut fits). With no frequencies every neuron costs the same.
// Returns the g + 1 range starts (the last = n), or an empty vector when no cut fits. The
// greedy cut is deterministic.
inline std::vector<int32_t> balanced_ranges(int n, const float* freq, double p2_row_bytes,
                                            double act_row_bytes, int target_groups, int max_len) {
  std::vector<double> cost(n > 0 ? n : 0);
  for (int i = 0; i < n; ++i)
    cost[i] = p2_row_bytes + (freq ? clamp_freq(freq[i]) : 0.0) * act_row_bytes;
  const double total = std::accumulate(cost.begin(), cost.end(), 0.0);
  double target = total / std::max(1, target_groups);
  for (int attempt = 0; attempt < 64; ++attempt) {
    std::vector<int32_t> rs{0};
    double acc = 0.0;
    int len = 0;
    for (int i = 0; i < n; ++i) {
      if (len > 0 && (len == max_len || acc + cost[i] > target)) {
        rs.push_back(i);
        acc = 0.0;
        len = 0;
      }
      acc += cost[i];
      ++len;
    }
    rs.push_back(n);
    if ((int)rs.size() - 1 <= std::max(target_groups, 1)) return rs;
    target *= 1.25;
  }
  return {};
}

// the largest expected cost (bytes) of one range: its predictor rows plus each neuron's
// ReLU-input row(s) weighted by its activation frequency
inline double max_range_cost(const std::vector<int32_t>& rs, const float* freq,
                             double p2_row_bytes, double act_row_bytes) {
  double worst = 0.0;
  for (size_t u = 0; u + 1 < rs.size(); ++u) {
    double c = 0.0;
    for (int i = rs[u]; i < rs[u + 1]; ++i)
      c += p2_row_bytes + (freq ? clamp_freq(freq[i]) : 0.0) * act_row_bytes;
    worst = std::max(worst, c);
  }
  return worst;
}

// Cut the g ranges (starts rs, g + 1 entries) into ks contiguous splits of about equal
// expected active neurons (the sum of the neurons' frequencies; every neuron counts 1
// without frequencies), for the down projection. Returns the ks + 1 split bounds (range
// indices: split k owns ranges [s[k], s[k + 1])); upt = ranges per thread the widest split
// needs with 256 threads (1, 2, 4, 8, 16).
inline std::vector<int32_t> split_ranges(const std::vector<int32_t>& rs, const float* freq,
                                         int ks, int& upt) {
  const int g = (int)rs.size() - 1;
  std::vector<double> cum(g + 1, 0.0);
  for (int u = 0; u < g; ++u) {
    double e = 0.0;
    for (int i = rs[u]; i < rs[u + 1]; ++i) e += freq ? clamp_freq(freq[i]) : 1.0;
    cum[u + 1] = cum[u] + e;
  }
  std::vector<int32_t> s(ks + 1, 0);
  int u = 0;
  for (int k = 1; k < ks; ++k) {
    const double goal = cum[g] * k / ks;
    while (u < g && cum[u] < goal) ++u;
    s[k] = u;
  }
  s[ks] = g;
  int widest = 0;
  for (int k = 0; k < ks; ++k) widest = std::max(widest, s[k + 1] - s[k]);
  upt = 1;
  while (upt * 256 < widest && upt < 16) upt *= 2;
  return s;
}

// Hot-first permutation, perm[new] = old: the n_hot neurons with the largest counts first,
// by count descending and original index ascending on ties; the rest follow in ascending
// original index. Requires 0 <= n_hot <= n.
inline void hot_first_permutation(const int64_t* counts, int n, int n_hot, int32_t* perm) {
  std::vector<int32_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::partial_sort(order.begin(), order.begin() + n_hot, order.end(),
                    [counts](int32_t a, int32_t b) {
                      return counts[a] != counts[b] ? counts[a] > counts[b] : a < b;
                    });
  std::vector<char> hot(n, 0);
  for (int k = 0; k < n_hot; ++k) {
    perm[k] = order[k];
    hot[order[k]] = 1;
  }
  int k = n_hot;
  for (int i = 0; i < n; ++i)
    if (!hot[i]) perm[k++] = i;
}

// The smallest batch size b <= max_batch whose expected union of the tokens' predicted
// sets, 1 - mean_i (1 - f_i)^b with the neurons' frequencies f_i and independent tokens,
// exceeds the fraction dense_union; `never` when there is none (or dense_union <= 0).
inline int dense_from_batch(const float* freq, int n, double dense_union, int max_batch,
                            int never) {
  if (!(dense_union > 0.0) || !freq || n <= 0) return never;
  for (int b = 1; b <= max_batch; ++b) {
    double u = 0.0;
    for (int i = 0; i < n; ++i) u += 1.0 - std::pow(1.0 - clamp_freq(freq[i]), (double)b);
    if (u / n > dense_union) return b;
  }
  return never;
}

// The largest batch size b in [2, max_b] (0: none) up to which the expected union of the
// tokens' predicted sets, sum_i 1 - (1 - f_i)^b (independent tokens), stays within
// max_rows; with no frequencies the union is bounded by n. The union grows with b, so
// every smaller batch from 2 on qualifies as well.
inline int union_within_batch(const float* freq, int n, double max_rows, int max_b) {
  int best = 0;
  for (int b = 2; b <= max_b; ++b) {
    double u = 0.0;
    if (freq) {
      for (int i = 0; i < n; ++i) u += 1.0 - std::pow(1.0 - clamp_freq(freq[i]), (double)b);
    } else {
      u = (double)n;
    }
    if (!(u <= max_rows)) break;
    best = b;
  }
  return best;
}

// ---- dense prefill plan
constexpr int kPfTile = 128;      // tokens per tile, and output columns per down tile
constexpr int kPfMaxSplits = 16;  // most neuron splits of the down projection

inline size_t pf_align(size_t v) { return (v + 255) & ~(size_t)255; }

// H row length the scratch holds: d_ffn rounded up to every neuron tile (64 to 192)
inline size_t pf_rows(int n) { return (size_t)(n + 383) / 384 * 384; }

// H row length of a run with up tiles of 32 it neurons: whole tiles
inline int pf_np(int n, int it) { return (n + 32 * it - 1) / (32 * it) * (32 * it); }

// Up tile (32 it neurons) for nbt token tiles. Gated layers take it = 3, plain ones 4 or 6,
// whichever finishes first with one tile a compute unit at a time (rounds of tiles x the
// tile's size; ties: 4). it = 2 replaces either when it needs fewer rounds over the compute
// units x rows staged per workgroup (weight rows plus one or two token blocks), the measure
// the kernel's times follow: with few token tiles the larger tiles leave units idle.
inline int pf_up_it(int n, bool gated, bool lo, int nbt, int n_cus) {
  auto cost = [&](int mr) {
    const long long tiles = (long long)((n + mr - 1) / mr) * nbt;
    return (tiles + n_cus - 1) / n_cus * mr;
  };
  auto staged = [&](int it) {
    const long long tiles = (long long)((n + 32 * it - 1) / (32 * it)) * nbt;
    const long long rows = (gated ? 2 : 1) * 32 * it + (lo ? 2 : 1) * kPfTile;
    return (tiles + n_cus - 1) / n_cus * rows;
  };
  int it = gated ? 3 : (cost(192) < cost(128) ? 6 : 4);
  if (staged(2) < staged(it)) it = 2;
  return it;
}

// Neuron splits of the down projection for nbt token tiles and H rows of np: doubled until
// two workgroups a compute unit, keeping at least 8 stages of 32 neurons a split. Never
// smaller for a larger np, never larger for more token tiles.
inline int pf_splits(int d, int n_cus, int nbt, size_t np) {
  const long long tiles = (long long)(d / kPfTile) * nbt;
  int S = 1;
  while (S < kPfMaxSplits && tiles * S < 2LL * n_cus && np / 32 >= (size_t)16 * S) S *= 2;
  return S;
}

// Partial-sum scratch for chunks of up to Bp tokens: the largest splits x tokens of any
// chunk size up to Bp, at the largest H row length (the scan ends at the first size that
// needs no split).
inline size_t pf_part_bytes(int d, int n, int n_cus, size_t Bp) {
  size_t m = 0;
  for (size_t t = kPfTile; t <= Bp; t += kPfTile) {
    const int S = pf_splits(d, n_cus, (int)(t / kPfTile), pf_rows(n));
    if (S == 1) break;
    m = std::max(m, (size_t)S * t * (size_t)d * 4);
  }
  return m;
}

// Layout of the scratch for a chunk of Bp tokens (byte offsets, 256-byte aligned): x's fp16
// hi and lo rows [Bp][d], h's hi and lo rows [Bp][pf_rows(n)], the split partial sums;
// end = the bytes it spans.
struct PfCarve {
  size_t xh, xl, hh, hl, part, end;
};
inline PfCarve pf_carve(int d, int n, int n_cus, size_t Bp) {
  PfCarve c;
  size_t p = 0;
  c.xh = p;
  p += pf_align(Bp * (size_t)d * 2);
  c.xl = p;
  p += pf_align(Bp * (size_t)d * 2);
  c.hh = p;
  p += pf_align(Bp * pf_rows(n) * 2);
  c.hl = p;
  p += pf_align(Bp * pf_rows(n) * 2);
  c.part = p;
  p += pf_align(pf_part_bytes(d, n, n_cus, Bp));
  c.end = p;
  return c;
}

// Scratch for chunks of up to chunk tokens (rounded up to a whole tile); 0 for chunk < 1
inline size_t pf_work_bytes(int d, int n, int n_cus, int chunk) {
  if (chunk < 1) return 0;
  const size_t Bp = (size_t)(chunk + kPfTile - 1) / kPfTile * kPfTile;
  return pf_carve(d, n, n_cus, Bp).end;
}

// Tokens a scratch of work_bytes holds per chunk: the largest multiple of the tile, up to
// 2^20 tokens, whose scratch fits (0 when not even one tile fits). pf_work_bytes never
// falls as the chunk grows, so a binary search over the tile counts finds it.
inline int pf_chunk_tokens(int d, int n, int n_cus, size_t work_bytes) {
  int lo = 0, hi = (1 << 20) / kPfTile;  // tiles: lo fits (0 trivially), answer in [lo, hi]
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (pf_work_bytes(d, n, n_cus, mid * kPfTile) <= work_bytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo * kPfTile;
}


}  // namespace host
}  // namespace sffn
