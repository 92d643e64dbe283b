// Single-token decode in one pass over each active neuron's bundle (gfx950): the neuron's
// ReLU-input row(s) and its down-projection row are requested together, so the down
// projection needs no launch of its own that first finds the active rows again. The pages
// motivate it: gate, up and down rows of a neuron are used together, so PowerInfer-2 stores
// them as one bundle and reads it in one I/O (PowerInfer-2 article, section 4.4
// Neuron-Cluster-Level Pipeline), and operator fusion cuts memory round trips (novita.ai
// activation-sparsity article, section 工程影響). The method itself is the same as the other
// paths (predictor, threshold, ascending list, gather + ReLU, down projection); see the top
// of sffn_device.h.
//
// Two launches after predictor stage 1:
//  - k_bundle_b1: BSG neuron ranges per workgroup (one per group of 256 threads, ranges
//    gridDim.x apart). Each
//    range is scored, thresholded and compacted exactly as by the three-launch path's
//    middle kernel (same arithmetic, so the same scores, list and activations h); each
//    active neuron's down row arrives with its input rows, and the group accumulates
//    y_part += h * W_down^T[i] over its rows in ascending order. The groups' sums are added
//    in LDS in group order and stored as the workgroup's partial output.
//  - k_bundle_reduce: y = sum of the partials in a fixed order, + b_out; it also publishes
//    the ascending list, the count and the token bits from the ranges' activity words.
// No float atomics: y is bitwise reproducible. The partials cost d * 4 bytes per
// workgroup each way (3.9 MB at d = 4096 with 952 ranges), which is why each workgroup
// takes several ranges.
#include "sffn_device.h"

namespace sffn {
namespace {

constexpr int BSG = BUNDLE_RANGES_PER_GROUP;  // ranges per workgroup
constexpr int BCW = 32;                        // columns of one partial block (128 bytes)

template <bool F16, bool GATED, int CPT, int CPD, int NCHP>
__global__ __launch_bounds__(TPB * BSG) void k_bundle_b1(
    const void* __restrict__ p2, const float* __restrict__ pbias, const float* __restrict__ q,
    const void* __restrict__ w_act, int ld_act, const void* __restrict__ w_down_t, int ld_down,
    const float* __restrict__ b_act, const float* __restrict__ x, int d, float tau, int g,
    const int32_t* __restrict__ rs, uint64_t* __restrict__ wbits, float* __restrict__ part,
    float* __restrict__ scores, const RangeArg ra) {
  constexpr int EPC = Elt<F16>::EPC;
  constexpr int RMAX = MID_RANGE_MAX;
  constexpr int NV = GATED ? 2 : 1;
  constexpr int RB = 16 / (CPT + CPD) > 0 ? 16 / (CPT + CPD) : 1;  // rows in flight
  constexpr int GRP = NCHP < 64 ? NCHP : 64;
  constexpr int RPP = TPB / NCHP;  // predictor rows per slot of a group
  constexpr int PL = 8;            // slots in flight per thread
  static_assert(NCHP >= 8 && NCHP <= 64 && (NCHP & (NCHP - 1)) == 0, "predictor row within a wave");
  __shared__ float s_pb[BSG][RMAX];
  __shared__ float s_ba[BSG][RMAX];
  __shared__ float s_bias[BSG][RMAX];
  __shared__ uint8_t s_act[BSG][RMAX];
  __shared__ int32_t s_rows[BSG][RMAX];
  __shared__ int s_wcnt[BSG][TPB / 64];
  __shared__ float s_red[BSG][TPB / 64][RB][NV];
  __shared__ float s_h[BSG][RB];
  extern __shared__ float4_t s_dyn4[];
  float* s_part = reinterpret_cast<float*>(s_dyn4);  // [d]

  touch_kernargs<2>();
  const int tid = threadIdx.x, sg = tid / TPB, lt = tid % TPB, lane = tid & 63, wv = lt >> 6;
  // this group's range: groups take ranges gridDim.x apart, so that the hot prefix (short
  // ranges with many active rows) spreads over workgroups instead of filling the first few
  const int u = sg * (int)gridDim.x + (int)blockIdx.x;
  const bool has = u < g;
  const int r0 = has ? (rs ? rs[u] : ra.r[u]) : 0;
  const int nown = has ? (rs ? rs[u + 1] : ra.r[u + 1]) - r0 : 0;  // 0..RMAX

  // ---- predictor stage 2 and threshold, as mid_scores_b1 (rows that fit one wave)
  const int pos = lt & (NCHP - 1), rsub = lt / NCHP;
  const int nslots = (nown + RPP - 1) / RPP;
  const size_t blk0 = (size_t)r0 * NCHP;
  const int jmax = max(nown - 1, 0);
  u32x4 pv[PL];
#pragma unroll
  for (int m = 0; m < PL; ++m) pv[m] = ld_chunk(p2, blk0 + (size_t)min(m * RPP + rsub, jmax) * NCHP + pos);
  float qs[EPC];
  load_x<EPC>(q + (size_t)pos * EPC, qs);
  const float pb = (lt < nown && pbias) ? pbias[r0 + lt] : 0.f;
  const float ba = (lt < nown && b_act) ? b_act[r0 + lt] : 0.f;
  if (lt < RMAX) s_act[sg][lt] = 0;
  if (lt < nown) {
    s_pb[sg][lt] = pb;
    s_ba[sg][lt] = ba;
  }
  __syncthreads();
  for (int s0 = 0; s0 < nslots; s0 += PL) {  // no barrier inside: uniform or not, it is safe
    const int mlim = min(PL, nslots - s0);
    if (s0 > 0) {
#pragma unroll
      for (int m = 0; m < PL; ++m)
        pv[m] = ld_chunk(p2, blk0 + (size_t)min((s0 + m) * RPP + rsub, jmax) * NCHP + pos);
    }
    float acc[PL];
#pragma unroll
    for (int m = 0; m < PL; ++m) acc[m] = m < mlim ? dot_chunk<F16>(pv[m], qs, 0.f) : 0.f;
#pragma unroll
    for (int m = 0; m < PL; ++m)
      if (m < mlim) acc[m] = group_sum<GRP>(acc[m]);
#pragma unroll
    for (int m = 0; m < PL; ++m) {
      const int j = (s0 + m) * RPP + rsub;
      if (j < nown && (lane & (GRP - 1)) == group_leader(GRP)) {
        const float sc = acc[m] + s_pb[sg][j];
        if (scores) scores[r0 + j] = sc;
        s_act[sg][j] = sc > tau ? 1 : 0;
      }
    }
  }
  __syncthreads();

  // ---- compaction of each range: the range fits in its group's first wave
  const bool act = lt < nown && s_act[sg][lt];
  const uint64_t word = __ballot(act);
  if (lane == 0) s_wcnt[sg][wv] = __popcll(word);
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int v = 0; v < TPB / 64; ++v) before += v < wv ? s_wcnt[sg][v] : 0;
  int nact = 0, nmax = 0;
#pragma unroll
  for (int s2 = 0; s2 < BSG; ++s2) {
    int c = 0;
#pragma unroll
    for (int v = 0; v < TPB / 64; ++v) c += s_wcnt[s2][v];
    if (s2 == sg) nact = c;
    nmax = max(nmax, c);
  }
  if (act) {
    const uint64_t lower = lane ? (word & ((~(uint64_t)0) >> (64 - lane))) : 0;
    const int k = before + __popcll(lower);
    s_rows[sg][k] = r0 + lt;
    s_bias[sg][k] = s_ba[sg][lt];
  }
  if (has && lt == 0) wbits[u] = word;
  __syncthreads();

  // ---- gather: each active neuron's input row(s) and down row in one batch of loads
  const int nch = d / EPC;
  const int rowch = GATED ? 2 * nch : nch;
  float xs[CPT][EPC];
  if (nmax > 0) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int c = lt + m * TPB;
      const bool up = GATED && c >= nch;
      load_x<EPC>(x + (size_t)min(up ? c - nch : c, nch - 1) * EPC, xs[m]);
    }
  }
  float yp[CPD][EPC];
#pragma unroll
  for (int m = 0; m < CPD; ++m)
#pragma unroll
    for (int e = 0; e < EPC; ++e) yp[m][e] = 0.f;
  for (int base = 0; base < nmax; base += RB) {  // the same count in every group
    const int nb = max(0, min(RB, nact - base));  // uniform within the group
    u32x4 gv[RB][CPT], dv[RB][CPD];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      if (rr < nb) {
        const size_t row = (size_t)s_rows[sg][base + rr];
#pragma unroll
        for (int m = 0; m < CPT; ++m) gv[rr][m] = ld_stream(w_act, row * ld_act + min(lt + m * TPB, rowch - 1));
#pragma unroll
        for (int m = 0; m < CPD; ++m) dv[rr][m] = ld_stream(w_down_t, row * ld_down + min(lt + m * TPB, nch - 1));
      }
    }
    float acc[RB][NV];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[rr][v] = 0.f;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int c = lt + m * TPB;
      const bool cv = c < rowch;
      const bool up = GATED && c >= nch;
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        if (rr < nb) {
          const float dt = dot_chunk<F16>(gv[rr][m], xs[m], 0.f);
          const float add = cv ? dt : 0.f;
          if (GATED && up) acc[rr][NV - 1] += add;
          else acc[rr][0] += add;
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int v = 0; v < NV; ++v)
        if (rr < nb) acc[rr][v] = wave_sum(acc[rr][v]);
    if (lane == WAVE_SUM_LANE) {
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (rr < nb) s_red[sg][wv][rr][v] = acc[rr][v];
    }
    __syncthreads();
    if (lt < nb) {
      // h exactly as the three-launch middle kernel forms it
      float a = s_red[sg][0][lt][0];
      a += s_red[sg][1][lt][0];
      a += s_red[sg][2][lt][0];
      a += s_red[sg][3][lt][0];
      a += s_bias[sg][base + lt];
      float h = a > 0.f ? a : 0.f;
      if (GATED) {
        float uu = s_red[sg][0][lt][NV - 1];
        uu += s_red[sg][1][lt][NV - 1];
        uu += s_red[sg][2][lt][NV - 1];
        uu += s_red[sg][3][lt][NV - 1];
        h = h * uu;
      }
      s_h[sg][lt] = h;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      if (rr < nb) {
        const float h = s_h[sg][rr];
#pragma unroll
        for (int m = 0; m < CPD; ++m) {
          float f[EPC];
          unpack<F16>(dv[rr][m], f);
#pragma unroll
          for (int e = 0; e < EPC; ++e) yp[m][e] = fmaf(h, f[e], yp[m][e]);
        }
      }
    }
  }

  // ---- the groups' sums, added in group order ((g0 + g1) + g2) + g3 in one d-long LDS
  // row, out as this workgroup's partial
#pragma unroll
  for (int s2 = 0; s2 < BSG; ++s2) {
    if (sg == s2) {
#pragma unroll
      for (int m = 0; m < CPD; ++m) {
        const int c = lt + m * TPB;
        if (c < nch) {
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            float* p = s_part + c * EPC + e;
            *p = s2 == 0 ? yp[m][e] : *p + yp[m][e];
          }
        }
      }
    }
    __syncthreads();
  }
  const int np = gridDim.x;
  for (int col = tid; col < d; col += TPB * BSG)
    part[((size_t)(col / BCW) * np + blockIdx.x) * BCW + col % BCW] = s_part[col];
}

// Workgroup cb: output columns [32 cb, 32 cb + 32) from the np partials (block cb of each,
// contiguous), every load issued at once; thread t adds the partials t / 8, t / 8 + 32, ...
// of column quad t % 8 in that order, then the 32 threads of each quad are added by a
// butterfly (the same total in every lane) and the four waves in order; + b_out. It also
// publishes the list: the ranges' activity words are prefix-summed (each thread a
// contiguous run of UPT words), and workgroup cb writes the entries of the ranges u with
// u % gridDim.x == cb, each at its global position; workgroup 0 writes the count.
template <int UPT>
__global__ __launch_bounds__(TPB) void k_bundle_reduce(
    const float* __restrict__ part, int np, int d, const float* __restrict__ b_out,
    float* __restrict__ y, const uint64_t* __restrict__ wbits, const int32_t* __restrict__ rs,
    int g, int32_t* __restrict__ idx_out, int32_t* __restrict__ count_out,
    uint64_t* __restrict__ tokmask_out) {
  constexpr int PMAX = (G_MID_MAX / BSG) * (BCW / 4) / TPB;  // float4 loads per thread
  __shared__ float4_t s_sum[TPB / 64][BCW / 4];
  __shared__ int s_wsum[TPB / 64];
  touch_kernargs<2>();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, cb = blockIdx.x;
  // list words first (their loads overlap the partials')
  uint64_t wd[UPT];
  int rb[UPT];
#pragma unroll
  for (int v = 0; v < UPT; ++v) {
    const int uu = tid * UPT + v;
    wd[v] = uu < g ? wbits[uu] : 0;
    rb[v] = uu < g ? rs[uu] : 0;
  }
  const float4_t* pp = reinterpret_cast<const float4_t*>(part) + (size_t)cb * np * (BCW / 4);
  const int nq = np * (BCW / 4);
  float4_t pv[PMAX];
#pragma unroll
  for (int k = 0; k < PMAX; ++k) {
    const int p = tid + k * TPB;
    pv[k] = p < nq ? pp[p] : float4_t{0.f, 0.f, 0.f, 0.f};
  }
  float4_t s = pv[0];
#pragma unroll
  for (int k = 1; k < PMAX; ++k) s += pv[k];
#pragma unroll
  for (int m = 8; m < 64; m <<= 1) {
    s[0] += __shfl_xor(s[0], m);
    s[1] += __shfl_xor(s[1], m);
    s[2] += __shfl_xor(s[2], m);
    s[3] += __shfl_xor(s[3], m);
  }
  if (lane < BCW / 4) s_sum[wave][lane] = s;
  // the list: exclusive prefix of the words' popcounts over threads
  int c = 0;
#pragma unroll
  for (int v = 0; v < UPT; ++v) c += __popcll(wd[v]);
  const int incl = wave_incl_scan(c);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  if (tid < BCW / 4) {
    float4_t t = s_sum[0][tid];
#pragma unroll
    for (int w2 = 1; w2 < TPB / 64; ++w2) t += s_sum[w2][tid];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = cb * BCW + tid * 4 + e;
      if (col < d) y[col] = t[e] + (b_out ? b_out[col] : 0.f);
    }
  }
  int before = 0, total = 0;
#pragma unroll
  for (int v = 0; v < TPB / 64; ++v) {
    before += v < wave ? s_wsum[v] : 0;
    total += s_wsum[v];
  }
  int at = before + incl - c;
#pragma unroll
  for (int v = 0; v < UPT; ++v) {
    const int uu = tid * UPT + v;
    uint64_t m = wd[v];
    if (uu % (int)gridDim.x == cb && idx_out) {
      while (m) {
        idx_out[at] = rb[v] + (__ffsll((unsigned long long)m) - 1);
        if (tokmask_out) tokmask_out[at] = 1;
        ++at;
        m &= m - 1;
      }
    } else {
      at += __popcll(m);
    }
  }
  if (cb == 0 && tid == 0 && count_out) *count_out = total;
}

template <bool F16, bool GATED, int CPT, int CPD, int NCHP>
void bundle_launch(const LayerDev& L, const float* x, float* scores, hipStream_t s,
                   const hipEvent_t* tev) {
  const int np = (L.g_mid + BSG - 1) / BSG;
  launch(k_bundle_b1<F16, GATED, CPT, CPD, NCHP>, dim3(np), dim3(TPB * BSG), (size_t)L.d * 4, s,
         tev, L.p2, L.p_bias, L.q, L.w_act, L.act_ld, L.w_down_t,
         L.down_ld, L.b_act, x, L.d, L.tau, L.g_mid, L.rs_in_arg ? nullptr : L.rs, L.wbits,
         L.part, scores, L.ra);
}

template <bool F16, bool GATED, int CPT, int CPD>
bool bundle_nchp(const LayerDev& L, const float* x, float* scores, hipStream_t s,
                 const hipEvent_t* tev) {
  switch (L.r / (F16 ? 8 : 4)) {
    case 8: bundle_launch<F16, GATED, CPT, CPD, 8>(L, x, scores, s, tev); return true;
    case 16: bundle_launch<F16, GATED, CPT, CPD, 16>(L, x, scores, s, tev); return true;
    case 32: bundle_launch<F16, GATED, CPT, CPD, 32>(L, x, scores, s, tev); return true;
    case 64: bundle_launch<F16, GATED, CPT, CPD, 64>(L, x, scores, s, tev); return true;
    default: return false;
  }
}

// chunks per thread of a row's input part (CPT: 1, 2, 4) and of its down row (CPD: 1, 2)
inline int bundle_cpt(const LayerDev& L) {
  const int nch = L.d / (L.w_f16 ? 8 : 4), rowch = (L.gated ? 2 : 1) * nch;
  return rowch <= TPB ? 1 : rowch <= 2 * TPB ? 2 : rowch <= 4 * TPB ? 4 : 0;
}
inline int bundle_cpd(const LayerDev& L) {
  const int nch = L.d / (L.w_f16 ? 8 : 4);
  return nch <= TPB ? 1 : nch <= 2 * TPB ? 2 : 0;
}

template <bool F16, bool GATED>
bool bundle_any(const LayerDev& L, const float* x, float* scores, hipStream_t s,
                const hipEvent_t* tev) {
  const int cpt = bundle_cpt(L), cpd = bundle_cpd(L);
#define SFFN_BF(CP, CD) \
  if (cpt == CP && cpd == CD) return bundle_nchp<F16, GATED, CP, CD>(L, x, scores, s, tev);
  if constexpr (GATED) {
    SFFN_BF(1, 1) SFFN_BF(2, 1) SFFN_BF(4, 2)
  } else {
    SFFN_BF(1, 1) SFFN_BF(2, 2)
  }
#undef SFFN_BF
  return false;
}

template <int UPT>
void reduce_launch(const LayerDev& L, float* y, int32_t* idx, int32_t* count, uint64_t* tok,
                   hipStream_t s, const hipEvent_t* tev) {
  const int np = (L.g_mid + BSG - 1) / BSG;
  launch(k_bundle_reduce<UPT>, dim3((L.d + BCW - 1) / BCW), dim3(TPB), 0, s, tev,
         (const float*)L.part, np, L.d, L.b_out, y, (const uint64_t*)L.wbits, (const int32_t*)L.rs,
         L.g_mid, idx, count, tok);
}

}  // namespace

// A layer the single-pass kernels cover: weights and predictor of one type, a predictor row
// of 8 to 64 chunks (rank 64 to 512 in fp16, 32 to 256 in fp32), an input row of at most
// 512 chunks (d <= 4096 in fp16, 2048 in fp32) and the single-token path's ranges.
bool bundle_ok(const LayerDev& L) {
  if (L.w_f16 != L.p_f16 || !L.part) return false;
  const int nchp = L.r / (L.p_f16 ? 8 : 4);
  if (L.r % (L.p_f16 ? 8 : 4) != 0 || nchp < 8 || nchp > 64 || (nchp & (nchp - 1)) != 0)
    return false;
  if (bundle_cpt(L) == 0 || bundle_cpd(L) == 0) return false;
  return L.g_mid >= 1 && L.g_mid <= G_MID_MAX;
}

bool run_bundle_b1(const LayerDev& L, const float* x, float* y, int32_t* idx, int32_t* count,
                   uint64_t* tok, float* scores, hipStream_t s, const hipEvent_t* t_pass,
                   const hipEvent_t* t_reduce) {
  if (!bundle_ok(L)) return false;
  const bool ok = L.w_f16 ? (L.gated ? bundle_any<true, true>(L, x, scores, s, t_pass)
                                     : bundle_any<true, false>(L, x, scores, s, t_pass))
                          : (L.gated ? bundle_any<false, true>(L, x, scores, s, t_pass)
                                     : bundle_any<false, false>(L, x, scores, s, t_pass));
  if (!ok) return false;
  const int upt = (L.g_mid + TPB - 1) / TPB;
  if (upt <= 1) reduce_launch<1>(L, y, idx, count, tok, s, t_reduce);
  else if (upt <= 2) reduce_launch<2>(L, y, idx, count, tok, s, t_reduce);
  else if (upt <= 4) reduce_launch<4>(L, y, idx, count, tok, s, t_reduce);
  else reduce_launch<8>(L, y, idx, count, tok, s, t_reduce);
  return true;
}

size_t bundle_part_bytes(int d, int n) {
  const int min_groups = (n + MID_RANGE_MAX - 1) / MID_RANGE_MAX;
  const int gmax = std::min(G_MID_MAX, std::max(RS_ARG_MAX, 2 * min_groups));
  const int np = (gmax + BSG - 1) / BSG;
  return (size_t)np * ((d + BCW - 1) / BCW) * BCW * 4;
}

}  // namespace sffn
