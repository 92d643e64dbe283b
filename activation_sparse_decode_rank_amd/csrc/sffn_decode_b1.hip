// Batch-1 decode kernels (gfx950): the fused middle kernel (predictor stage 2, threshold,
// per-range compaction, gather-GEMV + ReLU) and the single-token down projection. The method is
// described at the top of sffn_device.h.
#include "sffn_device.h"

namespace sffn {
namespace {

// ---------------------------------------------------------------------------- B = 1
// The two halves of the single-token middle kernel, as device functions: the fused kernel
// runs both in one workgroup, the look-ahead decode runs them in different launches.

// Predictor stage 2 and threshold over one range's neurons [r0, r0 + nown) (1 <= nown <=
// MID_RANGE_MAX): s_act[j] = (P2[r0 + j] . q + c[r0 + j] > tau), the score also stored when
// scores is given. Specialized on NCHP (chunks per predictor row) so that the lane-group
// reductions are straight-line DPP code; addresses of unused slots are clamped into the
// owned block instead of branching per lane. extra() runs after the predictor loads are
// issued and before the first barrier. Returns after a barrier, with s_act complete.
template <bool F16, int NCHP, typename Extra>
__device__ __forceinline__ void mid_scores_b1(const void* __restrict__ p2,
                                              const float* __restrict__ pbias,
                                              const float* __restrict__ q, int r0, int nown,
                                              float tau, float* __restrict__ scores,
                                              uint8_t* s_act, Extra extra) {
  constexpr int EPC = Elt<F16>::EPC;
  constexpr int GRP = NCHP < 64 ? NCHP : 64;   // lanes holding one predictor row in a wave
  constexpr int WPR = NCHP > 64 ? NCHP / 64 : 1;  // waves per predictor row
  constexpr int RPP = TPB / NCHP;              // predictor rows per slot of the workgroup
  constexpr int PL = 8;                        // slots in flight per thread
  constexpr int RMAX = MID_RANGE_MAX;
  static_assert(NCHP >= 1 && NCHP <= 128 && (NCHP & (NCHP - 1)) == 0, "NCHP");
  __shared__ float s_part[WPR > 1 ? RMAX * WPR : 1];
  __shared__ float s_pb[RMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pos = tid & (NCHP - 1);
  const int rsub = tid / NCHP;
  const int nslots = (nown + RPP - 1) / RPP;
  const size_t blk0 = (size_t)r0 * NCHP;

  // every score-independent load first: P2 (first PL slots), q, the predictor biases.
  // Slots beyond the range (m >= mlim, uniform) re-read its last row and are not computed.
  // (Guarding these loads instead makes the compiler keep far more registers live.)
  u32x4 wv[PL];
  int mlim = min(PL, nslots);
#pragma unroll
  for (int m = 0; m < PL; ++m) {
    const int j = min(m * RPP + rsub, nown - 1);
    wv[m] = ld_chunk(p2, blk0 + (size_t)j * NCHP + pos);
  }
  float qs[EPC];
  load_x<EPC>(q + (size_t)pos * EPC, qs);
  const float pb = (tid < nown && pbias) ? pbias[r0 + tid] : 0.f;
  extra();
  if (tid < RMAX) s_act[tid] = 0;
  if (tid < nown) s_pb[tid] = pb;
  __syncthreads();

  for (int s0 = 0; s0 < nslots; s0 += PL) {
    if (s0 > 0) {
      mlim = min(PL, nslots - s0);
#pragma unroll
      for (int m = 0; m < PL; ++m) {
        const int j = min((s0 + m) * RPP + rsub, nown - 1);
        wv[m] = ld_chunk(p2, blk0 + (size_t)j * NCHP + pos);
      }
    }
    float acc[PL];
#pragma unroll
    for (int m = 0; m < PL; ++m) acc[m] = m < mlim ? dot_chunk<F16>(wv[m], qs, 0.f) : 0.f;
#pragma unroll
    for (int m = 0; m < PL; ++m)
      if (m < mlim) acc[m] = group_sum<GRP>(acc[m]);
#pragma unroll
    for (int m = 0; m < PL; ++m) {
      const int j = (s0 + m) * RPP + rsub;
      if (j < nown && (lane & (GRP - 1)) == group_leader(GRP)) {
        if (WPR == 1) {
          const float sc = acc[m] + s_pb[j];
          if (scores) scores[r0 + j] = sc;
          s_act[j] = sc > tau ? 1 : 0;
        } else {
          s_part[j * WPR + (wave & (WPR - 1))] = acc[m];
        }
      }
    }
    if (WPR > 1) {
      __syncthreads();
      const int jlo = s0 * RPP, jhi = min(nown, (s0 + PL) * RPP);
      if (tid >= jlo && tid < jhi) {
        float sc = s_part[tid * WPR];
#pragma unroll
        for (int u = 1; u < WPR; ++u) sc += s_part[tid * WPR + u];
        sc += s_pb[tid];
        if (scores) scores[r0 + tid] = sc;
        s_act[tid] = sc > tau ? 1 : 0;
      }
      __syncthreads();
    }
  }
  __syncthreads();
}

// Gather-GEMV + ReLU over the nact active rows listed in s_rows (their activation biases in
// s_bias), RB rows in flight, against the input chunks xs the caller loaded (chunk tid + m
// TPB of the row; for the gated bundle the second half maps onto the same input):
// h_g[row] = ReLU(W_a[row] . x + b), gated: times W_u[row] . x. first() runs exactly once:
// after the first rows' loads are issued, or at once when no row is active.
template <bool F16, bool GATED, int CPT, typename First>
__device__ __forceinline__ void mid_gather_b1(const void* __restrict__ w_act, int ld, int d, int nact,
                                              const int32_t* s_rows, const float* s_bias,
                                              const float (&xs)[CPT][Elt<F16>::EPC],
                                              float* __restrict__ h_g, First first) {
  constexpr int EPC = Elt<F16>::EPC;
  constexpr int RB = (16 / CPT) > 0 ? (16 / CPT) : 1;  // gathered rows in flight
  constexpr int NV = GATED ? 2 : 1;
  __shared__ float s_red[4 * RB * NV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = d / EPC;
  const int rowch = GATED ? 2 * nch : nch;
  if (nact == 0) first();
  for (int base = 0; base < nact; base += RB) {
    const int nb = min(RB, nact - base);  // uniform
    u32x4 gv[RB][CPT];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      if (rr < nb) {
        const size_t row0 = (size_t)s_rows[base + rr] * ld;
#pragma unroll
        for (int m = 0; m < CPT; ++m) gv[rr][m] = ld_stream(w_act, row0 + min(tid + m * TPB, rowch - 1));
      }
    }
    if (base == 0) first();

    float acc[RB][NV];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[rr][v] = 0.f;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int c = tid + m * TPB;
      const bool cv = c < rowch;
      const bool up = GATED && c >= nch;
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        if (rr < nb) {
          const float dv = dot_chunk<F16>(gv[rr][m], xs[m], 0.f);
          const float add = cv ? dv : 0.f;
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
          if (rr < nb) s_red[(wave * RB + rr) * NV + v] = acc[rr][v];
    }
    __syncthreads();
    if (tid < nb) {
      const int rr = tid;
      float a = s_red[(0 * RB + rr) * NV];
      a += s_red[(1 * RB + rr) * NV];
      a += s_red[(2 * RB + rr) * NV];
      a += s_red[(3 * RB + rr) * NV];
      a += s_bias[base + rr];
      float h = a > 0.f ? a : 0.f;
      if (GATED) {
        float u = s_red[(0 * RB + rr) * NV + 1];
        u += s_red[(1 * RB + rr) * NV + 1];
        u += s_red[(2 * RB + rr) * NV + 1];
        u += s_red[(3 * RB + rr) * NV + 1];
        h = h * u;
      }
      h_g[s_rows[base + rr]] = h;
    }
    __syncthreads();
  }
}

// The single-token middle kernel: predictor stage 2, threshold, compaction of the owned
// range and the gather over its active rows, in one workgroup per range. Outputs as in
// k_fused_mid with B = 1: the range's activity word and h_g[i] for every active neuron i
// (no token bits: with one token every listed neuron is active for it).
template <bool F16, bool GATED, int CPT, int NCHP>
__global__ __launch_bounds__(TPB) void k_mid_b1(
    const void* __restrict__ p2, const float* __restrict__ pbias, const float* __restrict__ q,
    const void* __restrict__ w_act, int ld_act, const float* __restrict__ b_act,
    const float* __restrict__ x, int d, int n, float tau, const int32_t* __restrict__ rs,
    uint64_t* __restrict__ wbits, float* __restrict__ h_g, float* __restrict__ scores,
    const RangeArg ra) {
  constexpr int EPC = Elt<F16>::EPC;
  constexpr int RMAX = MID_RANGE_MAX;
  __shared__ uint8_t s_act[RMAX];
  __shared__ int32_t s_rows[RMAX];
  __shared__ float s_bias[RMAX];
  __shared__ float s_ba[RMAX];
  __shared__ int s_wcnt[TPB / 64];

  touch_kernargs<2>();
  const int w = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = rs ? rs[w] : ra.r[w], r1 = rs ? rs[w + 1] : ra.r[w + 1];
  const int nown = r1 - r0;  // 1..RMAX

  mid_scores_b1<F16, NCHP>(p2, pbias, q, r0, nown, tau, scores, s_act, [&]() {
    const float ba = (tid < nown && b_act) ? b_act[r0 + tid] : 0.f;
    if (tid < nown) s_ba[tid] = ba;
  });
  // ---- compaction of the owned range: ballot per wave, prefix over the four waves
  const bool act = tid < nown && s_act[tid];
  const uint64_t word = __ballot(act);
  if (lane == 0) s_wcnt[wave] = __popcll(word);
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int v = 0; v < TPB / 64; ++v) before += v < wave ? s_wcnt[v] : 0;
  const int nact = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
  if (act) {
    const uint64_t lower = lane ? (word & ((~(uint64_t)0) >> (64 - lane))) : 0;
    const int k = before + __popcll(lower);
    s_rows[k] = r0 + tid;
    s_bias[k] = s_ba[tid];
  }
  __syncthreads();

  // ---- gather-GEMV + ReLU over the active rows. The input chunks this thread multiplies
  // are loaded into registers once, with the first rows' loads.
  const int nch = d / EPC;
  float xs[CPT][EPC];
  if (nact > 0) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int c = tid + m * TPB;
      const bool up = GATED && c >= nch;
      load_x<EPC>(x + (size_t)min(up ? c - nch : c, nch - 1) * EPC, xs[m]);
    }
  }
  mid_gather_b1<F16, GATED, CPT>(w_act, ld_act, d, nact, s_rows, s_bias, xs, h_g, []() {});
  // The range's activity word (the range fits in wave 0's 64 lanes) is stored last: the
  // wait that follows a store and a barrier would hold back the gather's loads.
  if (tid == 0) wbits[w] = word;
}

// Single-token decode form of the down projection (list from the middle kernel's activity
// words, one token). Same column blocks, range splits and fixed-order reduction as k_down,
// written for a short dependent chain of instructions: these workgroups run one wave per
// SIMD, so every instruction on the path to the weight loads adds its full latency. The
// split's own words are scanned first; the words of earlier ranges (needed only for the
// list's global positions, which are published last) are loaded in the same round but
// summed after the sums have been issued. Neuron ids expand into LDS without bound checks
// when the split fits one window (the usual case), and no barrier precedes that window.
template <bool WF16>
__device__ __forceinline__ void down_rows_b1(const void* __restrict__ w_down_t,
                                             const float* __restrict__ h_in, int n,
                                             unsigned ld, unsigned chunk, int rsl,
                                             const int32_t* s_list, int wl,
                                             float (&acc)[Elt<WF16>::EPC]) {
  constexpr int EPC = Elt<WF16>::EPC;
  constexpr int LD = 16;
  static_assert(RSD * LD == DOWN_B1_BATCH, "batch size the split count is chosen for");
  for (int kb0 = 0; kb0 < wl; kb0 += RSD * LD) {
    int ii[LD];
#pragma unroll
    for (int u = 0; u < LD; ++u) ii[u] = min(s_list[min(kb0 + u * RSD + rsl, wl - 1)], n - 1);
    float hv[LD];
#pragma unroll
    for (int u = 0; u < LD; ++u) hv[u] = h_in[ii[u]];
    u32x4 wv[LD];
#pragma unroll
    for (int u = 0; u < LD; ++u) wv[u] = ld_stream(w_down_t, (size_t)ii[u] * ld + chunk);
#pragma unroll
    for (int u = 0; u < LD; ++u) {
      const float h = kb0 + u * RSD + rsl < wl ? hv[u] : 0.f;
      float f[EPC];
      unpack<WF16>(wv[u], f);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] = fmaf(h, f[e], acc[e]);
    }
  }
}

// The body of one workgroup (index bid) of the single-token down projection; the kernel
// below runs it on every workgroup, and the look-ahead decode on the first ones of a launch
// it shares with the next layer's scores.
template <bool WF16, int UPT, bool JOIN>
__device__ __forceinline__ void down_b1_body(
    int bid, const void* __restrict__ w_down_t, int ld_down, const float* __restrict__ b_out,
    const float* __restrict__ h_in, int d, int n, const uint64_t* __restrict__ wbits,
    const int32_t* __restrict__ rs, int KS, int ncb, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, uint64_t* __restrict__ tokmask_out,
    float* __restrict__ y, const SplitArg& sa, float* __restrict__ dn_part = nullptr,
    int32_t* __restrict__ dn_cnt = nullptr) {
  constexpr int EPC = Elt<WF16>::EPC;
  constexpr int COLS = CB_LANES * EPC;
  constexpr int PFX = G_MID_MAX / TPB;  // earlier-range words per thread
  static_assert(UPT >= 1 && UPT * TPB <= G_MID_MAX, "UPT");
  extern __shared__ float4_t s_dyn4[];
  int32_t* s_list = reinterpret_cast<int32_t*>(s_dyn4);  // LIST_CAP entries
  __shared__ int s_wsum[TPB / 64];
  __shared__ int s_psum[TPB / 64];
  __shared__ float s_red[TPB / 64][4][CB_LANES][EPC];  // [wave][16-lane row][chunk][value]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned nch = d / EPC;
  const int cb = bid % ncb, kq = bid / ncb;
  const int li = tid & (CB_LANES - 1), rsl = tid / CB_LANES;
  const unsigned chunk = min((unsigned)(cb * CB_LANES + li), nch - 1);  // partial last block
  const int u0 = sa.s[kq], u1 = sa.s[kq + 1];

  uint64_t wd[UPT];
  int rb[UPT];
  int c = 0;
#pragma unroll
  for (int v = 0; v < UPT; ++v) {
    const int u = u0 + tid * UPT + v;
    wd[v] = u < u1 ? wbits[u] : 0;
    rb[v] = u < u1 ? rs[u] : 0;
  }
  uint64_t pw[PFX];
#pragma unroll
  for (int v = 0; v < PFX; ++v) pw[v] = tid + v * TPB < u0 ? wbits[tid + v * TPB] : 0;
#pragma unroll
  for (int v = 0; v < UPT; ++v) c += __popcll(wd[v]);
  const int incl = wave_incl_scan(c);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int v = 0; v < TPB / 64; ++v) before += v < wave ? s_wsum[v] : 0;
  const int total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];  // rows of this split
  const int off = before + incl - c;  // local position of this thread's first set bit

  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  int gbase = -1;  // global list position of the split's first row, once known
  if (total <= LIST_CAP) {
    int pos = off;
#pragma unroll
    for (int v = 0; v < UPT; ++v) {
      uint64_t m = wd[v];
      while (m) {
        s_list[pos++] = rb[v] + (__ffsll((unsigned long long)m) - 1);
        m &= m - 1;
      }
    }
    __syncthreads();
    down_rows_b1<WF16>(w_down_t, h_in, n, ld_down, chunk, rsl, s_list, total, acc);
  } else {
    // long split: windows of LIST_CAP, each published as it is expanded (global offset first)
    int pc = 0;
#pragma unroll
    for (int v = 0; v < PFX; ++v) pc += __popcll(pw[v]);
    const int pincl = wave_incl_scan(pc);
    if (lane == 63) s_psum[wave] = pincl;
    for (int wb = 0; wb < total; wb += LIST_CAP) {
      const int wl = min(LIST_CAP, total - wb);
      __syncthreads();
      gbase = s_psum[0] + s_psum[1] + s_psum[2] + s_psum[3];
      int pos = off;
#pragma unroll
      for (int v = 0; v < UPT; ++v) {
        uint64_t m = wd[v];
        while (m) {
          if (pos >= wb && pos < wb + wl) s_list[pos - wb] = rb[v] + (__ffsll((unsigned long long)m) - 1);
          m &= m - 1;
          ++pos;
        }
      }
      __syncthreads();
      if (idx_out) {
        for (int k = cb + tid * ncb; k < wl; k += TPB * ncb) {
          idx_out[gbase + wb + k] = s_list[k];
          if (tokmask_out) tokmask_out[gbase + wb + k] = 1;
        }
      }
      down_rows_b1<WF16>(w_down_t, h_in, n, ld_down, chunk, rsl, s_list, wl, acc);
    }
  }
  // fixed-order reduction of the 32 row slots: lanes l and l+8 of each 16-lane row (DPP,
  // complete in lanes 8..15), then the 4 rows of each wave and the 4 waves in order
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = dpp_add<dpp_shr(8)>(acc[e]);
  if ((lane & 15) >= 8) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) s_red[wave][lane >> 4][li][e] = acc[e];
  }
  __syncthreads();
  // the list: this split's rows sit at global positions gbase + k (gbase = active neurons
  // of all earlier ranges); workgroup cb publishes the positions k with k % ncb == cb
  auto publish_list = [&]() {
    if (gbase >= 0) return;  // published window by window above
    int pc = 0;
#pragma unroll
    for (int v = 0; v < PFX; ++v) pc += __popcll(pw[v]);
    const int pincl = wave_incl_scan(pc);
    if (lane == 63) s_psum[wave] = pincl;
    __syncthreads();
    gbase = s_psum[0] + s_psum[1] + s_psum[2] + s_psum[3];
    if (idx_out) {
      for (int k = cb + tid * ncb; k < total; k += TPB * ncb) {
        idx_out[gbase + k] = s_list[k];
        if (tokmask_out) tokmask_out[gbase + k] = 1;
      }
    }
  };
  const int c_li = tid / EPC, e_c = tid % EPC;
  const int col = (cb * CB_LANES + c_li) * EPC + e_c;
  float sum = 0.f;
  if (tid < COLS) {
#pragma unroll
    for (int w2 = 0; w2 < TPB / 64; ++w2)
#pragma unroll
      for (int row = 0; row < 4; ++row) sum += s_red[w2][row][c_li][e_c];
    if (kq == 0 && b_out && col < d) sum += b_out[col];
  }
  if (JOIN && KS > 1) {
    // Fixed-order join of the KS splits of column block cb, in place of float atomics
    // into y: every split stores its sums in its own slot with device-coherent stores,
    // publishes its part of the list while they land, waits for them, then takes a ticket
    // from the block's counter. The split that arrives last reads the other slots back
    // with device-coherent loads, writes y as the sum of all slots in split order and
    // resets the counter for the next call.
    __shared__ int s_last;
    float* slot = dn_part + (size_t)cb * KS * COLS + tid;
    if (tid < COLS) __hip_atomic_store(slot + kq * COLS, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    publish_list();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(dn_cnt + cb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == KS - 1;
    __syncthreads();
    if (s_last) {
      asm volatile("" ::: "memory");
      if (tid < COLS) {
        float pv[KS_JOIN_MAX];
#pragma unroll
        for (int q = 0; q < KS_JOIN_MAX; ++q)
          pv[q] = q < KS && q != kq ? __hip_atomic_load(slot + q * COLS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                    : sum;
        float a = pv[0];
#pragma unroll
        for (int q = 1; q < KS_JOIN_MAX; ++q)
          if (q < KS) a += pv[q];
        if (col < d) y[col] = a;
      }
      if (tid == 0) __hip_atomic_store(dn_cnt + cb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    if (tid < COLS && col < d && (kq == 0 || total > 0)) {
      if (KS == 1)
        y[col] = sum;
      else
        atomicAdd(y + col, sum);
    }
    publish_list();
  }
  if (kq == KS - 1 && cb == 0 && tid == 0 && count_out) *count_out = gbase + total;
}

template <bool WF16, int UPT, bool JOIN>
__global__ __launch_bounds__(TPB) void k_down_b1(
    const void* __restrict__ w_down_t, int ld_down, const float* __restrict__ b_out,
    const float* __restrict__ h_in, int d, int n, const uint64_t* __restrict__ wbits,
    const int32_t* __restrict__ rs, int KS, int ncb, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, uint64_t* __restrict__ tokmask_out,
    float* __restrict__ y, const SplitArg sa, float* __restrict__ dn_part,
    int32_t* __restrict__ dn_cnt) {
  touch_kernargs<2>();
  down_b1_body<WF16, UPT, JOIN>(blockIdx.x, w_down_t, ld_down, b_out, h_in, d, n, wbits,
                                        rs, KS, ncb, idx_out, count_out, tokmask_out, y, sa,
                                        dn_part, dn_cnt);
}


// ------------------------------------------------------------ look-ahead decode (B = 1)
// The asynchronous predictor of the novita.ai activation-sparsity article (section
// 上下文稀疏性): the next layer's active set is predicted from the current layer's input,
// so that its prediction runs beside the current layer's weight streams instead of before
// them. A layer then takes two launches, each holding two independent roles (no wait
// between workgroups inside a launch):
//   k_la_gather: this layer's gather-GEMV + ReLU over the set chosen earlier (its range
//                activity words), and stage 1 of the next layer's predictor on this input;
//   k_la_down:   this layer's down projection, and the next layer's stage 2 + threshold,
//                which leave that layer's range activity words.
// Both roles run the same code, in the same summation order, as the single-token decode
// kernels, so a layer's list equals the one its own decode step would make from the
// previous layer's input, and y equals that step's output under that list.

// Workgroup w gathers middle range w of this layer (w < gm) and, for w < rn, computes row w
// of the next layer's stage 1 (qn[w] = P1n[w] . x, in k_pred_stage1's order for one token)
// between issuing its first weight loads and using them; the grid is max(gm, rn), and
// workgroups past the ranges compute their stage-1 row only. The first workgroups also
// clear y (ny floats) for the down projection's split sums. F16: fp16 weights and predictor
// (else fp32).
// Up to four chunks a gathered row, the registers are capped so that four workgroups fit a
// compute unit: every range is then resident at once, as in the single-token middle kernel.
template <bool F16, bool GATED, int CPT, int NCPT>
__global__ __attribute__((amdgpu_flat_work_group_size(1, TPB),
                          amdgpu_waves_per_eu(CPT <= 4 ? 4 : 1))) void k_la_gather(
    const void* __restrict__ w_act, int ld_act, const float* __restrict__ b_act,
    const float* __restrict__ x, int d, int gm, const int32_t* __restrict__ rs,
    const uint64_t* __restrict__ wbits,
    float* __restrict__ h_g, float* __restrict__ y0, int ny, const void* __restrict__ p1n,
    int rn, float* __restrict__ qn, const RangeArg ra) {
  constexpr int EPC = Elt<F16>::EPC;
  constexpr int RMAX = MID_RANGE_MAX;
  __shared__ int32_t s_rows[RMAX];
  __shared__ float s_bias[RMAX];
  __shared__ float s_q[TPB / 64];
  touch_kernargs<2>();
  const int w = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool owns = w < gm;  // uniform
  const int r0 = owns ? (rs ? rs[w] : ra.r[w]) : 0;
  const int nown = owns ? (rs ? rs[w + 1] : ra.r[w + 1]) - r0 : 0;  // 1..RMAX, or 0
  const uint64_t word =
      owns ? wbits[w] & (nown >= 64 ? ~(uint64_t)0 : (((uint64_t)1) << nown) - 1) : 0;
  const float ba = (tid < nown && b_act) ? b_act[r0 + tid] : 0.f;
  const int nch = d / EPC;
  const bool s1 = w < rn;  // uniform
  // the stage-1 row's chunks are chunks tid + m TPB (m < NCPT <= CPT) of x, which the
  // gather's input registers xs[m] already hold wherever the chunk exists
  static_assert(NCPT <= CPT, "stage-1 chunks within the gather's input chunks");
  u32x4 pv[NCPT];
  if (s1) {
#pragma unroll
    for (int m = 0; m < NCPT; ++m) {
      const int c = tid + m * TPB;
      if (c < nch) pv[m] = ld_stream(p1n, (size_t)w * nch + c);
    }
  }
  float xs[CPT][EPC];
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int c = tid + m * TPB;
    const bool up = GATED && c >= nch;
    load_x<EPC>(x + (size_t)min(up ? c - nch : c, nch - 1) * EPC, xs[m]);
  }
  for (int i = w * TPB + tid; i < ny; i += gridDim.x * TPB) y0[i] = 0.f;
  // the range's active rows in ascending order, from its word (the range fits in 64 lanes)
  const int nact = __popcll(word);
  if (tid < nown && ((word >> tid) & 1)) {
    const int k = __popcll(word & ((((uint64_t)1) << tid) - 1));
    s_rows[k] = r0 + tid;
    s_bias[k] = ba;
  }
  __syncthreads();
  auto stage1 = [&]() {
    if (!s1) return;
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < NCPT; ++m) {
      const int c = tid + m * TPB;
      if (c < nch) {
        float f[EPC];
        unpack<F16>(pv[m], f);
#pragma unroll
        for (int e2 = 0; e2 < EPC; ++e2) acc = fmaf(f[e2], xs[m][e2], acc);
      }
    }
    acc = wave_sum(acc);
    if (lane == WAVE_SUM_LANE) s_q[wave] = acc;
    __syncthreads();
    if (tid == 0) qn[w] = ((s_q[0] + s_q[1]) + s_q[2]) + s_q[3];
  };
  mid_gather_b1<F16, GATED, CPT>(w_act, ld_act, d, nact, s_rows, s_bias, xs, h_g, stage1);
}

// ndown workgroups run this layer's down projection (as k_down_b1, which also publishes the
// list, count and token bits); scoring workgroup i scores the next layer's ranges LA_RPW i
// onwards (of gn; bounds from its range table rsn) against qn and stores each range's
// activity word in wbits_n. The down workgroups come first, unless sfirst: when the launch
// does not fit the GPU at once, the scoring workgroups go first so that the next layer's
// predictor stream starts with the down projection's instead of after it. Two ranges a
// workgroup keep every workgroup of the launch resident at once where it fits; the second
// range's predictor rows are pulled into cache while the first is scored (one load per
// 128-byte line, values discarded). F16: fp16 weights and predictor (else fp32).
// next-layer ranges scored per workgroup: two halve the scoring workgroups at the cost of
// one more serial score pass; three or four make that serial tail the longer role
constexpr int LA_RPW = 2;
template <bool F16, int UPT, int NCHP, bool JOIN>
__global__ __launch_bounds__(TPB) void k_la_down(
    const void* __restrict__ w_down_t, int ld_down, const float* __restrict__ b_out,
    const float* __restrict__ h_in, int d, int n, const uint64_t* __restrict__ wbits,
    const int32_t* __restrict__ rs, int KS, int ncb, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, uint64_t* __restrict__ tokmask_out, float* __restrict__ y,
    int ndown, const void* __restrict__ p2n, const float* __restrict__ pbn,
    const float* __restrict__ qn, float taun, const int32_t* __restrict__ rsn, int gn,
    uint64_t* __restrict__ wbits_n, int sfirst, const SplitArg sa, float* __restrict__ dn_part,
    int32_t* __restrict__ dn_cnt) {
  __shared__ uint8_t s_act[MID_RANGE_MAX];
  touch_kernargs<2>();
  const int nsc = (gn + LA_RPW - 1) / LA_RPW, bid = blockIdx.x;
  if (sfirst ? bid >= nsc : bid < ndown) {
    down_b1_body<F16, UPT, JOIN>(sfirst ? bid - nsc : bid, w_down_t, ld_down, b_out, h_in, d, n,
                                 wbits, rs, KS, ncb, idx_out, count_out, tokmask_out, y, sa,
                                 dn_part, dn_cnt);
    return;
  }
  constexpr int ROW_BYTES = NCHP * 16;
  constexpr int PF_ITERS = (MID_RANGE_MAX * ROW_BYTES + TPB * 128 - 1) / (TPB * 128);
  const int w0 = LA_RPW * (sfirst ? bid : bid - ndown), tid = threadIdx.x;
  const int nr = min(LA_RPW, gn - w0);  // uniform, >= 1
  int rb[LA_RPW + 1];
#pragma unroll
  for (int k = 0; k <= LA_RPW; ++k) rb[k] = rsn[w0 + min(k, nr)];
  uint32_t sink = 0;
  mid_scores_b1<F16, NCHP>(p2n, pbn, qn, rb[0], rb[1] - rb[0], taun, nullptr, s_act, [&]() {
#pragma unroll
    for (int k = 1; k < LA_RPW; ++k) {
      if (k >= nr) break;
      const char* base = static_cast<const char*>(p2n) + (size_t)rb[k] * ROW_BYTES;
      const int bytes = (rb[k + 1] - rb[k]) * ROW_BYTES;
#pragma unroll
      for (int v = 0; v < PF_ITERS; ++v) {
        const int off = min((tid + v * TPB) * 128, bytes - 4);
        sink ^= *reinterpret_cast<const uint32_t*>(base + off);
      }
      if (tid < rb[k + 1] - rb[k] && pbn) sink ^= __float_as_uint(pbn[rb[k] + tid]);
    }
  });
  {
    const uint64_t word = __ballot(tid < rb[1] - rb[0] && s_act[tid]);
    if (tid == 0) wbits_n[w0] = word;
  }
#pragma unroll
  for (int k = 1; k < LA_RPW; ++k) {
    if (k >= nr) break;
    const int nk = rb[k + 1] - rb[k];
    mid_scores_b1<F16, NCHP>(p2n, pbn, qn, rb[k], nk, taun, nullptr, s_act, []() {});
    const uint64_t word = __ballot(tid < nk && s_act[tid]);
    if (tid == 0) wbits_n[w0 + k] = word;
  }
  asm volatile("" ::"v"(sink));
}


template <bool F16, bool GATED, int CPT, int NCHP>
void mid_b1_launch(const LayerDev& L, const float* x, float* scores, hipStream_t s,
                   const hipEvent_t* tev) {
  launch(k_mid_b1<F16, GATED, CPT, NCHP>, dim3(L.g_mid), dim3(TPB), 0, s, tev, L.p2,
         L.p_bias, L.q, L.w_act, L.act_ld, L.b_act, x, L.d, L.n, L.tau, L.rs_in_arg ? nullptr : L.rs,
         L.wbits, L.h_buf, scores, L.ra);
}

template <bool F16, bool GATED, int CPT>
bool mid_b1_dispatch(const LayerDev& L, const float* x, float* scores, hipStream_t s,
                     const hipEvent_t* tev) {
  switch (L.r / (F16 ? 8 : 4)) {
    case 8: mid_b1_launch<F16, GATED, CPT, 8>(L, x, scores, s, tev); return true;
    case 16: mid_b1_launch<F16, GATED, CPT, 16>(L, x, scores, s, tev); return true;
    case 32: mid_b1_launch<F16, GATED, CPT, 32>(L, x, scores, s, tev); return true;
    case 64: mid_b1_launch<F16, GATED, CPT, 64>(L, x, scores, s, tev); return true;
    case 128: mid_b1_launch<F16, GATED, CPT, 128>(L, x, scores, s, tev); return true;
    default: return false;
  }
}

template <bool F16, bool GATED, int CPT, int NCHP>
int mid_b1_occ(size_t lds) {
  int a = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, k_mid_b1<F16, GATED, CPT, NCHP>, TPB, lds) != hipSuccess) a = 0;
  return a;
}

// chunks per thread of a gathered row: as pick_cpt, plus 6 for rows of 1281-1536 chunks
// (the OPT-175B width), which saves the registers of two unused chunks per row and input
// and keeps four workgroups resident per compute unit
inline int pick_cpt_b1(int rowch) {
  const int c = pick_cpt(rowch);
  return c == 8 && rowch <= 6 * TPB ? 6 : c;
}

template <bool F16, bool GATED>
bool mid_b1_any(const LayerDev& L, const float* x, float* scores, hipStream_t s,
                const hipEvent_t* tev) {
  switch (pick_cpt_b1(row_chunks(L))) {
    case 1: return mid_b1_dispatch<F16, GATED, 1>(L, x, scores, s, tev);
    case 2: return mid_b1_dispatch<F16, GATED, 2>(L, x, scores, s, tev);
    case 4: return mid_b1_dispatch<F16, GATED, 4>(L, x, scores, s, tev);
    case 6: return mid_b1_dispatch<F16, GATED, 6>(L, x, scores, s, tev);
    case 8: return mid_b1_dispatch<F16, GATED, 8>(L, x, scores, s, tev);
    default: return false;
  }
}

template <bool F16, bool GATED, int CPT>
int mid_b1_occ_nchp(const LayerDev& L) {
  switch (L.r / (F16 ? 8 : 4)) {
    case 8: return mid_b1_occ<F16, GATED, CPT, 8>(0);
    case 16: return mid_b1_occ<F16, GATED, CPT, 16>(0);
    case 32: return mid_b1_occ<F16, GATED, CPT, 32>(0);
    case 64: return mid_b1_occ<F16, GATED, CPT, 64>(0);
    case 128: return mid_b1_occ<F16, GATED, CPT, 128>(0);
    default: return -1;
  }
}

template <bool F16, bool GATED>
int mid_b1_occ_any(const LayerDev& L) {
  switch (pick_cpt_b1(row_chunks(L))) {
    case 1: return mid_b1_occ_nchp<F16, GATED, 1>(L);
    case 2: return mid_b1_occ_nchp<F16, GATED, 2>(L);
    case 4: return mid_b1_occ_nchp<F16, GATED, 4>(L);
    case 6: return mid_b1_occ_nchp<F16, GATED, 6>(L);
    case 8: return mid_b1_occ_nchp<F16, GATED, 8>(L);
    default: return -1;
  }
}

template <bool F16, int UPT>
void down_b1_launch(const LayerDev& L, int32_t* idx_out, int32_t* count_out, uint64_t* tok_out,
                    float* y, hipStream_t s, const hipEvent_t* tev) {
  const int ncb = down_blocks(L);
  if (L.join_b1)
    launch(k_down_b1<F16, UPT, true>, dim3(ncb * L.ks_down), dim3(TPB),
           (size_t)LIST_CAP * 4, s, tev, L.w_down_t, L.down_ld, L.b_out, L.h_buf, L.d, L.n,
           L.wbits, L.rs, L.ks_down, ncb, idx_out, count_out, tok_out, y, L.sa, L.dn_part,
           L.dn_cnt);
  else
    launch(k_down_b1<F16, UPT, false>, dim3(ncb * L.ks_down), dim3(TPB),
           (size_t)LIST_CAP * 4, s, tev, L.w_down_t, L.down_ld, L.b_out, L.h_buf, L.d, L.n,
           L.wbits, L.rs, L.ks_down, ncb, idx_out, count_out, tok_out, y, L.sa, nullptr,
           nullptr);
}

template <bool F16>
void down_b1_any(const LayerDev& L, int32_t* idx_out, int32_t* count_out, uint64_t* tok_out,
                 float* y, hipStream_t s, const hipEvent_t* tev) {
  switch (L.split_upt) {
    case 1: down_b1_launch<F16, 1>(L, idx_out, count_out, tok_out, y, s, tev); break;
    case 2: down_b1_launch<F16, 2>(L, idx_out, count_out, tok_out, y, s, tev); break;
    case 4: down_b1_launch<F16, 4>(L, idx_out, count_out, tok_out, y, s, tev); break;
    default: down_b1_launch<F16, 8>(L, idx_out, count_out, tok_out, y, s, tev); break;
  }
}


// ---- look-ahead launches
// chunks per thread of the folded stage-1 row (d / 8 chunks of fp16, d / 4 of fp32): 1, 2,
// 4 or 6, else 0
inline int la_ncpt(int d, bool f16) {
  const int nch = d / (f16 ? 8 : 4);
  return nch <= TPB ? 1 : nch <= 2 * TPB ? 2 : nch <= 4 * TPB ? 4 : nch <= 6 * TPB ? 6 : 0;
}

template <bool F16, bool GATED, int CPT, int NCPT>
void la_gather_launch(const LayerDev& C, const LayerDev* Nx, const float* x, float* y,
                      hipStream_t s, const hipEvent_t* tev) {
  const int ny = C.ks_down > 1 ? C.d : 0;
  const int grid = std::max(C.g_mid, Nx ? Nx->r : 0);
  launch(k_la_gather<F16, GATED, CPT, NCPT>, dim3(grid), dim3(TPB), 0, s, tev, C.w_act, C.act_ld, C.b_act,
         x, C.d, C.g_mid, C.rs_in_arg ? nullptr : C.rs, C.wbits, C.h_buf, y, ny,
         Nx ? Nx->p1 : nullptr, Nx ? Nx->r : 0, Nx ? Nx->q : nullptr, C.ra);
}

// the (gated, chunks per gathered row, chunks per stage-1 row) forms instantiated below:
// those that occur up to 1024 input chunks (d <= 8192 in fp16), and plain layers up to 1536
// (d = 12288); both counts follow from d
inline bool la_form_ok(bool gated, int cpt, int ncpt) {
  if (gated)
    return (cpt == 1 && ncpt == 1) || (cpt == 2 && ncpt == 1) || (cpt == 4 && ncpt == 2) ||
           (cpt == 6 && ncpt == 4) || (cpt == 8 && ncpt == 4);
  return (cpt == 1 && ncpt == 1) || (cpt == 2 && ncpt == 2) || (cpt == 4 && ncpt == 4) ||
         (cpt == 6 && ncpt == 6);
}

template <bool F16, bool GATED>
bool la_gather_any(const LayerDev& C, const LayerDev* Nx, const float* x, float* y,
                   hipStream_t s, const hipEvent_t* tev) {
  const int cpt = pick_cpt_b1(row_chunks(C)), ncpt = la_ncpt(C.d, F16);
#define SFFN_LA(CP, NC)                                           \
  if (cpt == CP && ncpt == NC) {                                  \
    la_gather_launch<F16, GATED, CP, NC>(C, Nx, x, y, s, tev);    \
    return true;                                                  \
  }
  if constexpr (GATED) {
    SFFN_LA(1, 1) SFFN_LA(2, 1) SFFN_LA(4, 2) SFFN_LA(6, 4) SFFN_LA(8, 4)
  } else {
    SFFN_LA(1, 1) SFFN_LA(2, 2) SFFN_LA(4, 4) SFFN_LA(6, 6)
  }
#undef SFFN_LA
  return false;
}

template <bool F16, int UPT, int NCHP, bool JOIN>
void la_down_launch(const LayerDev* C, const LayerDev* Nx, int32_t* idx, int32_t* count,
                    uint64_t* tok, float* y, hipStream_t s, const hipEvent_t* tev) {
  const int ncb = C ? down_blocks(*C) : 1;
  const int ndown = C ? ncb * C->ks_down : 0;
  const int nscore = Nx ? (Nx->g_mid + LA_RPW - 1) / LA_RPW : 0;
  SplitArg none{};
  const int sfirst = C && nscore > 0 && ndown + nscore > C->la_occ * C->n_cus ? 1 : 0;
  launch(k_la_down<F16, UPT, NCHP, JOIN>, dim3(ndown + nscore), dim3(TPB), (size_t)LIST_CAP * 4, s, tev,
         C ? C->w_down_t : nullptr, C ? C->down_ld : 0, C ? C->b_out : nullptr,
         C ? C->h_buf : nullptr,
         C ? C->d : 0, C ? C->n : 0, C ? C->wbits : nullptr, C ? C->rs : nullptr,
         C ? C->ks_down : 1, ncb, idx, count, tok, y, ndown, Nx ? Nx->p2 : nullptr,
         Nx ? Nx->p_bias : nullptr, Nx ? Nx->q : nullptr, Nx ? Nx->tau : 0.f,
         Nx ? Nx->rs : nullptr, Nx ? Nx->g_mid : 0, Nx ? Nx->wbits : nullptr, sfirst,
         C ? C->sa : none, C ? C->dn_part : nullptr, C ? C->dn_cnt : nullptr);
}

template <bool F16, int UPT, bool JOIN>
bool la_down_nchp(const LayerDev* C, const LayerDev* Nx, int32_t* idx, int32_t* count,
                  uint64_t* tok, float* y, hipStream_t s, const hipEvent_t* tev) {
  switch (Nx ? Nx->r / (F16 ? 8 : 4) : 32) {
    case 8: la_down_launch<F16, UPT, 8, JOIN>(C, Nx, idx, count, tok, y, s, tev); return true;
    case 16: la_down_launch<F16, UPT, 16, JOIN>(C, Nx, idx, count, tok, y, s, tev); return true;
    case 32: la_down_launch<F16, UPT, 32, JOIN>(C, Nx, idx, count, tok, y, s, tev); return true;
    case 64: la_down_launch<F16, UPT, 64, JOIN>(C, Nx, idx, count, tok, y, s, tev); return true;
    case 128: la_down_launch<F16, UPT, 128, JOIN>(C, Nx, idx, count, tok, y, s, tev); return true;
    default: return false;
  }
}

template <bool F16, int UPT, int NCHP>
int la_down_occ() {
  // the join adds no registers or LDS that change the residency
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_la_down<F16, UPT, NCHP, false>, TPB,
                                                   (size_t)LIST_CAP * 4) != hipSuccess)
    occ = 0;
  return occ;
}

template <bool F16, int UPT>
int la_down_occ_nchp(int nchp) {
  switch (nchp) {
    case 8: return la_down_occ<F16, UPT, 8>();
    case 16: return la_down_occ<F16, UPT, 16>();
    case 32: return la_down_occ<F16, UPT, 32>();
    case 64: return la_down_occ<F16, UPT, 64>();
    default: return la_down_occ<F16, UPT, 128>();
  }
}

template <bool F16, bool JOIN>
bool la_down_upt(const LayerDev* C, const LayerDev* Nx, int32_t* idx, int32_t* count,
                 uint64_t* tok, float* y, hipStream_t s, const hipEvent_t* tev) {
  switch (C ? C->split_upt : 1) {
    case 1: return la_down_nchp<F16, 1, JOIN>(C, Nx, idx, count, tok, y, s, tev);
    case 2: return la_down_nchp<F16, 2, JOIN>(C, Nx, idx, count, tok, y, s, tev);
    case 4: return la_down_nchp<F16, 4, JOIN>(C, Nx, idx, count, tok, y, s, tev);
    default: return la_down_nchp<F16, 8, JOIN>(C, Nx, idx, count, tok, y, s, tev);
  }
}

// both roles share the weight type (checked by the caller)
bool la_down_any(const LayerDev* C, const LayerDev* Nx, int32_t* idx, int32_t* count,
                 uint64_t* tok, float* y, hipStream_t s, const hipEvent_t* tev) {
  // the down role joins its splits as the layer's decode step does, so that its y is the
  // decode step's
  const bool f16 = C ? C->w_f16 : Nx->w_f16;
  if (C && C->join_b1)
    return f16 ? la_down_upt<true, true>(C, Nx, idx, count, tok, y, s, tev)
               : la_down_upt<false, true>(C, Nx, idx, count, tok, y, s, tev);
  return f16 ? la_down_upt<true, false>(C, Nx, idx, count, tok, y, s, tev)
             : la_down_upt<false, false>(C, Nx, idx, count, tok, y, s, tev);
}

}  // namespace


bool run_mid_b1(const LayerDev& L, const float* x, float* scores, hipStream_t s,
                const hipEvent_t* tev) {
  if (L.w_f16 != L.p_f16) return false;
  if (L.w_f16) return L.gated ? mid_b1_any<true, true>(L, x, scores, s, tev) : mid_b1_any<true, false>(L, x, scores, s, tev);
  return L.gated ? mid_b1_any<false, true>(L, x, scores, s, tev) : mid_b1_any<false, false>(L, x, scores, s, tev);
}

template <bool F16>
int down_b1_occ() {
  // the widest form (eight ranges a thread) bounds the others' registers
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_down_b1<F16, 8, true>, TPB,
                                                   (size_t)LIST_CAP * 4) != hipSuccess)
    occ = 0;
  return occ;
}

int occ_down_b1(const LayerDev& L) { return L.w_f16 ? down_b1_occ<true>() : down_b1_occ<false>(); }

int occ_mid_b1(const LayerDev& L) {
  if (L.w_f16 != L.p_f16) return -1;
  if (L.w_f16) return L.gated ? mid_b1_occ_any<true, true>(L) : mid_b1_occ_any<true, false>(L);
  return L.gated ? mid_b1_occ_any<false, true>(L) : mid_b1_occ_any<false, false>(L);
}

void run_down_b1(const LayerDev& L, int32_t* idx_out, int32_t* count_out, uint64_t* tok_out,
                 float* y, hipStream_t s, const hipEvent_t* tev) {
  if (L.w_f16)
    down_b1_any<true>(L, idx_out, count_out, tok_out, y, s, tev);
  else
    down_b1_any<false>(L, idx_out, count_out, tok_out, y, s, tev);
}

// A layer the look-ahead kernels cover: weights and predictor of one type (fp16 or fp32),
// 8 to 128 chunks a predictor row (a power of two: rank 64 to 1024 in fp16, 32 to 512 in
// fp32), at most 1024 chunks a row of the input (1536 for plain layers: d <= 8192 and
// 12288 in fp16), and the single-token decode's own conditions.
bool lookahead_layer_ok(const LayerDev& L) {
  if (L.w_f16 != L.p_f16) return false;
  const int epc = L.w_f16 ? 8 : 4;
  const int nchp = L.r / epc;
  if (L.r % epc != 0 || nchp < 8 || nchp > 128 || (nchp & (nchp - 1)) != 0) return false;
  if (la_ncpt(L.d, L.w_f16) == 0 || L.d % epc != 0) return false;
  const int cpt = pick_cpt_b1(row_chunks(L)), ncpt = la_ncpt(L.d, L.w_f16);
  return la_form_ok(L.gated, cpt, ncpt) && occ_mid_b1(L) > 0;
}

hipError_t run_lookahead_begin(const LayerDev& Nx, const float* x, hipStream_t s) {
  run_stage1(Nx, x, 1, s, nullptr, nullptr, 0, false);
  if (!la_down_any(nullptr, &Nx, nullptr, nullptr, nullptr, nullptr, s, nullptr))
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t run_lookahead(const LayerDev& C, const LayerDev* Nx, const float* x, float* y,
                         int32_t* idx, int32_t* count, uint64_t* tok, hipStream_t s,
                         const hipEvent_t* ev) {
  const hipEvent_t* t1 = ev ? ev + 2 : nullptr;
  const bool ok = C.w_f16 ? (C.gated ? la_gather_any<true, true>(C, Nx, x, y, s, t1)
                                     : la_gather_any<true, false>(C, Nx, x, y, s, t1))
                          : (C.gated ? la_gather_any<false, true>(C, Nx, x, y, s, t1)
                                     : la_gather_any<false, false>(C, Nx, x, y, s, t1));
  if (!ok) return hipErrorInvalidValue;
  if (!la_down_any(&C, Nx, idx, count, tok, y, s, ev ? ev + 4 : nullptr))
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <bool F16>
int lookahead_down_occ_t(const LayerDev& L) {
  const int nchp = L.r / (F16 ? 8 : 4);
  switch (L.split_upt) {
    case 1: return la_down_occ_nchp<F16, 1>(nchp);
    case 2: return la_down_occ_nchp<F16, 2>(nchp);
    case 4: return la_down_occ_nchp<F16, 4>(nchp);
    default: return la_down_occ_nchp<F16, 8>(nchp);
  }
}

int lookahead_down_occ(const LayerDev& L) {
  return L.w_f16 ? lookahead_down_occ_t<true>(L) : lookahead_down_occ_t<false>(L);
}

}  // namespace sffn
