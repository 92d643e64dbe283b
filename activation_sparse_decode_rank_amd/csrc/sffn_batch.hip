// Batch and general kernels (gfx950): the general fused middle kernel (the small-batch
// one lives in sffn_mid_bt.h), the down projection for batches and for a given list, and
// the balanced gather of the forward entry point.
#include "sffn_device.h"

namespace sffn {
namespace {

// ============================================================================ gather
// Workgroup-cooperative gather-GEMV + ReLU over a list of active rows. All 256 threads
// share every row: thread t reads chunks t, t+256, ... of each row (16-byte loads, so a
// wave reads 1 KB contiguous per instruction), and up to RB rows' loads are in flight at
// once however many rows the workgroup owns. Each chunk is widened once per group of TBG
// tokens. Per-row partial dots are reduced in a fixed order (wave shuffle tree, then the
// four waves in order).
//   plain: h = relu(w[i] . x + b[i]);  gated (row = [gate | up]): h = relu(g . x + b) * (u . x)
// Inputs are LDS arrays per listed row: neuron id (-1 = skip), token bits, bias, and the
// output position p: h_out[p*B + b] receives h for every token (0 where the bit is clear).
template <bool WF16, bool GATED, int CPT, int TBG>
struct Gather {
  static constexpr int EPC = Elt<WF16>::EPC;
  static constexpr int LOADS_G = 8;
  static constexpr int RB = (LOADS_G / CPT) > 0 ? (LOADS_G / CPT) : 1;  // rows per batch
  static constexpr int NV = GATED ? 2 : 1;
  static constexpr int RED_FLOATS = 4 * RB * TBG * NV;

  __device__ static void run(const void* __restrict__ w_act, int ld, const float* xsrc, int d, int n,
                             int B, const int32_t* rows, const uint64_t* bits, const float* bias,
                             const int32_t* outpos, int nrows, float* __restrict__ h_out,
                             float* s_red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nch = d / EPC;                  // chunks per matrix row
    const int rowch = GATED ? 2 * nch : nch;  // chunks per stored row
    for (int base = 0; base < nrows; base += RB) {
      const int nb = min(RB, nrows - base);
      u32x4 wv[RB][CPT];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const int ri = rr < nb ? rows[base + rr] : -1;
        if (ri >= 0 && ri < n) {
          const size_t row0 = (size_t)ri * ld;
#pragma unroll
          for (int m = 0; m < CPT; ++m) {
            const int c = tid + m * TPB;
            if (c < rowch) wv[rr][m] = ld_chunk(w_act, row0 + c);
          }
        }
      }
      for (int b0 = 0; b0 < B; b0 += TBG) {
        float acc[RB][TBG][NV];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
#pragma unroll
          for (int b = 0; b < TBG; ++b)
#pragma unroll
            for (int v = 0; v < NV; ++v) acc[rr][b][v] = 0.f;
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
          const int c = tid + m * TPB;
          if (c < rowch) {
            const bool up = GATED && c >= nch;
            const int xc = up ? c - nch : c;
            float xs[TBG][EPC];
#pragma unroll
            for (int b = 0; b < TBG; ++b)
              if (b0 + b < B) load_x<EPC>(xsrc + (size_t)(b0 + b) * d + (size_t)xc * EPC, xs[b]);
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
              if (rr < nb) {
                float f[EPC];
                unpack<WF16>(wv[rr][m], f);
#pragma unroll
                for (int b = 0; b < TBG; ++b) {
                  if (b0 + b < B) {
                    float a = acc[rr][b][up ? NV - 1 : 0];
#pragma unroll
                    for (int e = 0; e < EPC; ++e) a = fmaf(f[e], xs[b][e], a);
                    acc[rr][b][up ? NV - 1 : 0] = a;
                  }
                }
              }
            }
          }
        }
        // wave reductions, independent chains interleaved
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
#pragma unroll
          for (int b = 0; b < TBG; ++b)
#pragma unroll
            for (int v = 0; v < NV; ++v) acc[rr][b][v] = wave_sum(acc[rr][b][v]);
        if (lane == WAVE_SUM_LANE) {
#pragma unroll
          for (int rr = 0; rr < RB; ++rr)
#pragma unroll
            for (int b = 0; b < TBG; ++b)
#pragma unroll
              for (int v = 0; v < NV; ++v) s_red[((wave * RB + rr) * TBG + b) * NV + v] = acc[rr][b][v];
        }
        __syncthreads();
        if (tid < nb * TBG) {
          const int rr = tid / TBG, b = tid % TBG;
          const int i = rows[base + rr];
          if (b0 + b < B && i >= 0 && i < n) {
            const bool on = (bits[base + rr] >> (b0 + b)) & 1;
            float h = 0.f;
            if (on) {
              float a = s_red[((0 * RB + rr) * TBG + b) * NV];
              a += s_red[((1 * RB + rr) * TBG + b) * NV];
              a += s_red[((2 * RB + rr) * TBG + b) * NV];
              a += s_red[((3 * RB + rr) * TBG + b) * NV];
              a += bias[base + rr];
              h = a > 0.f ? a : 0.f;
              if (GATED) {
                float u = s_red[((0 * RB + rr) * TBG + b) * NV + 1];
                u += s_red[((1 * RB + rr) * TBG + b) * NV + 1];
                u += s_red[((2 * RB + rr) * TBG + b) * NV + 1];
                u += s_red[((3 * RB + rr) * TBG + b) * NV + 1];
                h = h * u;
              }
            }
            h_out[(size_t)outpos[base + rr] * B + b0 + b] = h;
          }
        }
        __syncthreads();
      }
    }
  }
};

// Balanced gather for the forward entry point: workgroup w takes the contiguous slice
// [w*per, (w+1)*per) of the given list (per = ceil(count / grid)); h of list position k
// goes to h_pos[k*B + b].
template <bool WF16, bool GATED, int CPT, int TBG>
__global__ __launch_bounds__(TPB) void k_gather(const void* __restrict__ w_act, int ld_act,
                                                const float* __restrict__ b_act,
                                                const float* __restrict__ x, int d, int n, int B,
                                                const int32_t* __restrict__ idx,
                                                const int32_t* __restrict__ count,
                                                const uint64_t* __restrict__ tokmask,
                                                float* __restrict__ h_pos, int x_lds,
                                                float* __restrict__ y0, int ny) {
  using G = Gather<WF16, GATED, CPT, TBG>;
  zero_grid(y0, ny);
  constexpr int RCAP = 512;
  extern __shared__ float4_t s_dyn4[];
  float* s_x = reinterpret_cast<float*>(s_dyn4);
  __shared__ int32_t s_rows[RCAP];
  __shared__ uint64_t s_bits[RCAP];
  __shared__ float s_bias[RCAP];
  __shared__ int32_t s_pos[RCAP];
  __shared__ float s_red[G::RED_FLOATS];
  const int cnt = min(max(*count, 0), n);  // a count beyond the list is clamped
  const int per = (cnt + gridDim.x - 1) / gridDim.x;
  const int k0 = min(cnt, (int)blockIdx.x * per), k1 = min(cnt, k0 + per);
  if (k0 >= k1) return;
  if (x_lds) stage_x(s_x, x, B * d);
  const float* xsrc = x_lds ? s_x : x;
  for (int kb = k0; kb < k1; kb += RCAP) {
    const int nr = min(RCAP, k1 - kb);
    __syncthreads();
    for (int u = threadIdx.x; u < nr; u += TPB) {
      const int i = idx[kb + u];
      const bool ok = i >= 0 && i < n;
      s_rows[u] = ok ? i : -1;
      s_bits[u] = tokmask ? tokmask[kb + u] : ~(uint64_t)0;
      s_bias[u] = (ok && b_act) ? b_act[i] : 0.f;
      s_pos[u] = kb + u;
    }
    __syncthreads();
    G::run(w_act, ld_act, xsrc, d, n, B, s_rows, s_bits, s_bias, s_pos, nr, h_pos, s_red);
  }
}

// ============================================================================ fused middle
// One kernel for predictor stage 2, threshold, per-workgroup compaction and the gather.
// Workgroup w owns the contiguous neuron range [rs[w], rs[w+1]) (1..MID_RANGE_MAX neurons;
// the ranges are balanced offline by expected cost, so the hot prefix is split into short
// ranges). Its P2 rows form one contiguous block, read linearly (thread t takes chunks t,
// t+256, ...); with NCHP = chunks per P2 row a power of two, a row's chunks sit in NCHP
// consecutive lanes (above 64, in consecutive waves). Every load that does not depend on
// the scores (P2 block, q, biases, x) is issued before the first wait.
// Outputs: wbits[w], the range's activity word (bit j = neuron rs[w] + j is active for at
// least one token; ranges hold at most 64 neurons), written every call with a plain store;
// and for each active neuron i its token bits tok_full[i] and activations h_g[i*B + b] (0
// for tokens whose bit is clear). Other neurons' entries are not written. scores is
// written when non-null.
template <bool F16, bool GATED, int CPT, int TBG>
__global__ __launch_bounds__(TPB) void k_fused_mid(
    const void* __restrict__ p2, const float* __restrict__ pbias, const float* __restrict__ q,
    int r, const void* __restrict__ w_act, int ld_act, const float* __restrict__ b_act,
    const float* __restrict__ x, int d, int n, int B, float tau, const int32_t* __restrict__ rs,
    uint64_t* __restrict__ wbits, uint64_t* __restrict__ tok_full, float* __restrict__ h_g,
    float* __restrict__ scores, int x_lds, const RangeArg ra) {
  constexpr int EPC = Elt<F16>::EPC;
  constexpr int PL = 16;  // P2 chunks a thread keeps in flight
  constexpr int RMAX = MID_RANGE_MAX;
  using G = Gather<F16, GATED, CPT, TBG>;
  extern __shared__ float4_t s_dyn4[];
  float* s_x = reinterpret_cast<float*>(s_dyn4);
  __shared__ uint64_t s_tok[RMAX];
  __shared__ int32_t s_rows[RMAX];
  __shared__ uint64_t s_bits[RMAX];
  __shared__ float s_bias[RMAX];
  __shared__ int32_t s_pos[RMAX];
  __shared__ float s_part[RMAX * 2];  // per-row partial scores from up to 2 waves
  __shared__ float s_pb[RMAX];
  __shared__ float s_ba[RMAX];
  __shared__ int s_wcnt[TPB / 64];
  __shared__ float s_red[G::RED_FLOATS];

  touch_kernargs<2>();
  const int w = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = rs ? rs[w] : ra.r[w], r1 = rs ? rs[w + 1] : ra.r[w + 1];
  const int nown = r1 - r0;  // 1..RMAX
  const int nchp = r / EPC;  // power of two, <= 128
  const int lg = 31 - __clz(nchp);
  const int total = nown * nchp;
  const int grp = nchp < 64 ? nchp : 64;      // lanes of one row inside a wave
  const int wpr = nchp > 64 ? nchp / 64 : 1;  // waves per row (1 or 2)
  const size_t blk0 = (size_t)r0 * nchp;
  const int pos = tid & (nchp - 1);  // this thread's chunk within its row (256 % nchp == 0)

  // ---- every score-independent load first
  u32x4 wv[PL];
#pragma unroll
  for (int m = 0; m < PL; ++m) {
    const int f = tid + m * TPB;
    if (f < total) wv[m] = ld_chunk(p2, blk0 + f);
  }
  float qs[EPC];
  load_x<EPC>(q + (size_t)pos * EPC, qs);
  float pb = 0.f, ba = 0.f;
  if (tid < nown) {
    pb = pbias ? pbias[r0 + tid] : 0.f;
    ba = b_act ? b_act[r0 + tid] : 0.f;
  }
  if (tid < RMAX) s_tok[tid] = 0;
  if (x_lds) stage_x(s_x, x, B * d);
  if (tid < nown) {
    s_pb[tid] = pb;
    s_ba[tid] = ba;
  }
  __syncthreads();

  // ---- predictor stage 2 and threshold
  for (int c0 = 0; c0 < total; c0 += PL * TPB) {
    if (c0 > 0) {  // rows beyond the first PL*256 chunks: next block (rare)
      __syncthreads();
#pragma unroll
      for (int m = 0; m < PL; ++m) {
        const int f = c0 + tid + m * TPB;
        if (f < total) wv[m] = ld_chunk(p2, blk0 + f);
      }
    }
    for (int b = 0; b < B; ++b) {
      if (b > 0 || c0 > 0) load_x<EPC>(q + (size_t)b * r + (size_t)pos * EPC, qs);
      const int mlim = min(PL, (total - c0 + TPB - 1) / TPB);  // chunk slots in use (uniform)
      float acc[PL];
#pragma unroll
      for (int m = 0; m < PL; ++m) {
        acc[m] = 0.f;
        if (m < mlim) {
          const int f = c0 + tid + m * TPB;
          if (f < total) acc[m] = dot_chunk<F16>(wv[m], qs, 0.f);
        }
      }
      // group sums over grp lanes (uniform branches; the PL chains interleave)
      if (grp >= 2) {
#pragma unroll
        for (int m = 0; m < PL; ++m)
          if (m < mlim) acc[m] = dpp_add<DPP_QP_XOR1>(acc[m]);
      }
      if (grp >= 4) {
#pragma unroll
        for (int m = 0; m < PL; ++m)
          if (m < mlim) acc[m] = dpp_add<DPP_QP_XOR2>(acc[m]);
      }
      if (grp >= 8) {
#pragma unroll
        for (int m = 0; m < PL; ++m)
          if (m < mlim) acc[m] = dpp_add<DPP_HALF_MIRROR>(acc[m]);
      }
      if (grp >= 16) {
#pragma unroll
        for (int m = 0; m < PL; ++m)
          if (m < mlim) acc[m] = dpp_add<DPP_MIRROR>(acc[m]);
      }
      if (grp >= 32) {
#pragma unroll
        for (int m = 0; m < PL; ++m)
          if (m < mlim) acc[m] = dpp_add<DPP_BCAST15, 0xA>(acc[m]);
      }
      if (grp >= 64) {
#pragma unroll
        for (int m = 0; m < PL; ++m)
          if (m < mlim) acc[m] = dpp_add<DPP_BCAST31, 0xC>(acc[m]);
      }
      const int leader = group_leader(grp);
#pragma unroll
      for (int m = 0; m < PL; ++m) {
        const int f = c0 + tid + m * TPB;
        if (m < mlim && f < total && (lane & (grp - 1)) == leader)
          s_part[(f >> lg) * 2 + (wpr > 1 ? (wave & 1) : 0)] = acc[m];
      }
      __syncthreads();
      if (tid < nown && tid * nchp >= c0 && tid * nchp < c0 + PL * TPB) {
        float s = s_part[tid * 2];
        if (wpr > 1) s += s_part[tid * 2 + 1];
        s += s_pb[tid];
        if (scores) scores[(size_t)b * n + r0 + tid] = s;
        if (s > tau) s_tok[tid] |= (uint64_t)1 << b;
      }
      __syncthreads();
    }
  }
  // ---- compaction of the owned range: ballot per wave, prefix over the four waves
  const uint64_t bits = (tid < nown) ? s_tok[tid] : 0;
  const bool act = bits != 0;
  const uint64_t word = __ballot(act);
  if (lane == 0) s_wcnt[wave] = __popcll(word);
  __syncthreads();
  int before = 0;
  for (int v = 0; v < wave; ++v) before += s_wcnt[v];
  const int nact = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
  if (act) {
    const uint64_t lower = lane ? (word & ((~(uint64_t)0) >> (64 - lane))) : 0;
    const int k = before + __popcll(lower);
    const int i = r0 + tid;
    s_rows[k] = i;
    s_bits[k] = bits;
    s_bias[k] = s_ba[tid];
    s_pos[k] = i;
  }
  __syncthreads();
  // ---- gather + ReLU over the owned active rows
  G::run(w_act, ld_act, x_lds ? s_x : x, d, n, B, s_rows, s_bits, s_bias, s_pos, nact, h_g, s_red);
  // token bits and the range's activity word (the range fits in wave 0's 64 lanes) are
  // stored last: the wait that follows a store and a barrier would hold back the gather
  if (tid < nact) tok_full[s_rows[tid]] = s_bits[tid];
  if (tid == 0) wbits[w] = word;
}

// ============================================================================ down
// Down projection y_b = sum_k h_{k,b} W_down^T[idx_k] + b_out, split two ways:
//  - columns: workgroup (cb, kq) owns the 128-byte column block cb (8 chunks = 8*EPC output
//    columns), so every weight read is a whole 128-byte line of a row;
//  - rows (split-k): it owns split kq of the active rows.
// Inside the workgroup, thread t handles chunk t&7 of the block and row slot t>>3 (32
// slots); per batch the row ids and activations are loaded first, then LOADS_D weight
// chunks per thread, then the FMAs. The 32 slots are reduced in a fixed order (DPP within
// 16-lane rows, then LDS across rows and waves). The workgroup's sums are added into y,
// which an earlier kernel of the same call has zeroed: a plain store when KS == 1, else a
// float atomic add, b_out riding on kq == 0's sum. With KS == 2 the result is still
// bitwise reproducible (two addends onto +0 commute exactly); KS > 2 trades that for
// speed.
// BITS (decode): the active rows come from the middle kernel's per-range activity words
// (bit j of wbits[u] = neuron rs[u] + j; ranges ascending and contiguous) and activations
// are indexed by neuron, h_in[i*B + b]. Split kq owns the ranges [sa.s[kq], sa.s[kq+1])
// (cut offline for equal expected activity). In one round of loads each thread reads its
// UPT ranges' words and starts and the words of every earlier range (their popcount is
// the split's first list position); a workgroup-local scan then places the split's set
// bits into an LDS list, so each thread expands only its own few bits. The kernel also
// writes idx, count and tokmask (if non-null) for the whole list, each workgroup a share
// of its split's positions, after its sums (a store followed by a barrier would stall).
// Otherwise (list mode) the list is idx_in[0..*count), split by position, with
// activations indexed by list position, h_in[k*B + b].
template <int TB>
struct DownCfg {
  static constexpr int LOADS_D = TB == 1 ? 16 : 8;  // weight rows a thread keeps in flight
};

template <bool WF16, bool BITS, int TB, int UPT>
__global__ __launch_bounds__(TPB) void k_down(
    const void* __restrict__ w_down_t, int ld_down, const float* __restrict__ b_out,
    const float* __restrict__ h_in, int d, int n, int B, const int32_t* __restrict__ idx_in,
    const int32_t* __restrict__ count_in, const uint64_t* __restrict__ wbits,
    const int32_t* __restrict__ rs, const SplitArg sa, const uint64_t* __restrict__ tok_full,
    int KS, int ncb, int32_t* __restrict__ idx_out, int32_t* __restrict__ count_out,
    uint64_t* __restrict__ tokmask_out, float* __restrict__ y) {
  constexpr int EPC = Elt<WF16>::EPC;
  constexpr int COLS = CB_LANES * EPC;
  constexpr int LD = DownCfg<TB>::LOADS_D;
  constexpr int PFX = G_MID_MAX / TPB;  // earlier-range words per thread
  static_assert(UPT >= 1 && UPT * TPB <= G_MID_MAX, "UPT");
  extern __shared__ float4_t s_dyn4[];
  int32_t* s_list = reinterpret_cast<int32_t*>(s_dyn4);  // LIST_CAP entries (BITS)
  __shared__ int s_wsum[TPB / 64];
  __shared__ int s_psum[TPB / 64];
  __shared__ float s_red[TPB / 64][4][CB_LANES][TB * EPC];  // [wave][16-lane row][chunk][value]

  touch_kernargs<4>();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = d / EPC;
  const int cb = blockIdx.x % ncb, kq = blockIdx.x / ncb;
  const int li = tid & (CB_LANES - 1), rsl = tid / CB_LANES;
  const int chunk = min(cb * CB_LANES + li, nch - 1);  // a partial last block re-reads; unused

  // p0..p1: this workgroup's positions (BITS: local to the split); gbase: global position
  // of local position 0
  int p0, p1, gbase = 0;
  uint64_t wd[UPT];
  int rb[UPT];
  int woff = 0;  // BITS: local position of this thread's first set bit
  if (BITS) {
    const int u0 = sa.s[kq], u1 = sa.s[kq + 1];
    int c = 0;
#pragma unroll
    for (int v = 0; v < UPT; ++v) {
      const int u = u0 + tid * UPT + v;
      wd[v] = u < u1 ? wbits[u] : 0;
      rb[v] = u < u1 ? rs[u] : 0;
      c += __popcll(wd[v]);
    }
    int pc = 0;
#pragma unroll
    for (int v = 0; v < PFX; ++v) {
      const int u = tid + v * TPB;
      if (u < u0) pc += __popcll(wbits[u]);
    }
    const int incl = wave_incl_scan(c);
    const int pincl = wave_incl_scan(pc);
    if (lane == 63) {
      s_wsum[wave] = incl;
      s_psum[wave] = pincl;
    }
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int v = 0; v < TPB / 64; ++v) before += v < wave ? s_wsum[v] : 0;
    p0 = 0;
    p1 = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    gbase = s_psum[0] + s_psum[1] + s_psum[2] + s_psum[3];
    woff = before + incl - c;
  } else {
    const int total = min(max(*count_in, 0), n);  // a count beyond the list is clamped
    const int per = (total + KS - 1) / KS;
    p0 = min(total, kq * per);
    p1 = min(total, p0 + per);
  }

  float acc[TB][EPC];
  const int ntg = (B + TB - 1) / TB;
  for (int tg = 0; tg < ntg; ++tg) {
    const int b0 = tg * TB;
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[b][e] = 0.f;
    for (int wb = p0; wb < p1; wb += LIST_CAP) {
      const int wl = min(LIST_CAP, p1 - wb);
      // BITS: expand the split's set bits at local positions [wb, wb + wl) into s_list
      // (once, when the whole split fits one window)
      if (BITS && (tg == 0 || p1 - p0 > LIST_CAP)) {
        __syncthreads();
        int pos = woff;
#pragma unroll
        for (int v = 0; v < UPT; ++v) {
          uint64_t m = wd[v];
          const int c = __popcll(m);
          if (pos < wb + wl && pos + c > wb) {
            while (m) {
              const int bit = __ffsll((unsigned long long)m) - 1;
              m &= m - 1;
              if (pos >= wb && pos < wb + wl) s_list[pos - wb] = rb[v] + bit;
              ++pos;
            }
          } else {
            pos += c;
          }
        }
        __syncthreads();
        // a list longer than one window is published window by window, here
        if (p1 - p0 > LIST_CAP && tg == 0 && idx_out) {
          for (int k = tid; k < wl; k += TPB) {
            if (k % ncb != cb) continue;
            const int i = s_list[k];
            idx_out[gbase + wb + k] = i;
            if (tokmask_out) tokmask_out[gbase + wb + k] = B == 1 ? (uint64_t)1 : tok_full[i];
          }
        }
      }
      // Per batch: every row id and activation load first, then every weight load, then
      // the FMAs. Slots past the end re-read the last position and add 0.
      for (int kb0 = 0; kb0 < wl; kb0 += RSD * LD) {
        int ii[LD];
#pragma unroll
        for (int u = 0; u < LD; ++u) {
          const int kc = min(kb0 + u * RSD + rsl, wl - 1);
          ii[u] = BITS ? s_list[kc] : idx_in[wb + kc];
        }
        float hv[LD][TB];
#pragma unroll
        for (int u = 0; u < LD; ++u) {
          const int kc = min(kb0 + u * RSD + rsl, wl - 1);
          const int hr = BITS ? ((ii[u] >= 0 && ii[u] < n) ? ii[u] : 0) : wb + kc;
#pragma unroll
          for (int b = 0; b < TB; ++b) hv[u][b] = h_in[(size_t)hr * B + min(b0 + b, B - 1)];
        }
        u32x4 wv[LD];
#pragma unroll
        for (int u = 0; u < LD; ++u) {
          const int ic = (ii[u] >= 0 && ii[u] < n) ? ii[u] : 0;  // out-of-range entries add 0
          wv[u] = ld_stream(w_down_t, (size_t)ic * ld_down + chunk);
        }
#pragma unroll
        for (int u = 0; u < LD; ++u) {
          const int k = kb0 + u * RSD + rsl;
          const bool ok = k < wl && ii[u] >= 0 && ii[u] < n;
          float f[EPC];
          unpack<WF16>(wv[u], f);
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            const float h = (ok && b0 + b < B) ? hv[u][b] : 0.f;
#pragma unroll
            for (int e2 = 0; e2 < EPC; ++e2) acc[b][e2] = fmaf(h, f[e2], acc[b][e2]);
          }
        }
      }
    }
    // fixed-order reduction of the 32 row slots: lanes l and l+8 of each 16-lane row
    // (DPP, complete in lanes 8..15), then the 4 rows of each wave and the 4 waves in order
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[b][e] = dpp_add<dpp_shr(8)>(acc[b][e]);
    if ((lane & 15) >= 8) {
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int e = 0; e < EPC; ++e) s_red[wave][(lane >> 4)][li][b * EPC + e] = acc[b][e];
    }
    __syncthreads();
    for (int o = tid; o < TB * COLS; o += TPB) {  // TB * COLS may exceed the workgroup
      const int b = o / COLS, cc = o % COLS;
      const int c_li = cc / EPC, e = cc % EPC;
      const int col = (cb * CB_LANES + c_li) * EPC + e;
      if (b0 + b < B && col < d && (kq == 0 || p1 > p0)) {
        float sum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < TPB / 64; ++w2)
#pragma unroll
          for (int row = 0; row < 4; ++row) sum += s_red[w2][row][c_li][b * EPC + e];
        if (kq == 0 && b_out) sum += b_out[col];
        float* dst = y + (size_t)(b0 + b) * d + col;
        if (KS == 1)
          *dst = sum;
        else
          atomicAdd(dst, sum);
      }
    }
    __syncthreads();
  }
  if (BITS) {
    // the list of this split (held whole in s_list when it fits one window): workgroup cb
    // publishes local positions k with k % ncb == cb; the last split's workgroup 0 knows
    // the total
    if (idx_out && p1 - p0 <= LIST_CAP) {
      for (int k = cb + tid * ncb; k < p1; k += TPB * ncb) {
        const int i = s_list[k];
        idx_out[gbase + k] = i;
        if (tokmask_out) tokmask_out[gbase + k] = B == 1 ? (uint64_t)1 : tok_full[i];
      }
    }
    if (kq == KS - 1 && cb == 0 && tid == 0 && count_out) *count_out = gbase + p1;
  }
}

template <bool F16, bool GATED, int CPT>
void gather_launch(const LayerDev& L, const float* x, int B, const int32_t* idx,
                   const int32_t* count, const uint64_t* tokmask, float* y0, hipStream_t s) {
  const bool xl = x_in_lds(B, L.d);
  const size_t lds = xl ? (size_t)B * L.d * 4 : 0;
  const int ny = L.ks_vec > 1 ? B * L.d : 0;
  if (B == 1)
    hipLaunchKernelGGL((k_gather<F16, GATED, CPT, 1>), dim3(L.g_gather), dim3(TPB), lds, s,
                       L.w_act, L.act_ld, L.b_act, x, L.d, L.n, B, idx, count, tokmask, L.h_buf, xl ? 1 : 0,
                       y0, ny);
  else
    hipLaunchKernelGGL((k_gather<F16, GATED, CPT, 4>), dim3(L.g_gather), dim3(TPB), lds, s,
                       L.w_act, L.act_ld, L.b_act, x, L.d, L.n, B, idx, count, tokmask, L.h_buf, xl ? 1 : 0,
                       y0, ny);
}

template <bool F16, bool GATED>
void gather_dispatch(const LayerDev& L, const float* x, int B, const int32_t* idx,
                     const int32_t* count, const uint64_t* tokmask, float* y0, hipStream_t s) {
  switch (pick_cpt(row_chunks(L))) {
    case 1: gather_launch<F16, GATED, 1>(L, x, B, idx, count, tokmask, y0, s); break;
    case 2: gather_launch<F16, GATED, 2>(L, x, B, idx, count, tokmask, y0, s); break;
    case 4: gather_launch<F16, GATED, 4>(L, x, B, idx, count, tokmask, y0, s); break;
    default: gather_launch<F16, GATED, 8>(L, x, B, idx, count, tokmask, y0, s); break;
  }
}

template <bool F16, bool BITS, int TB, int UPT>
void down_launch_t(const LayerDev& L, int B, const int32_t* idx, const int32_t* count,
                   int32_t* idx_out, int32_t* count_out, uint64_t* tok_out, float* y,
                   hipStream_t s, const hipEvent_t* tev) {
  const int grid = down_blocks(L) * L.ks_vec;
  const size_t lds = BITS ? (size_t)LIST_CAP * 4 : 0;
  launch(k_down<F16, BITS, TB, UPT>, dim3(grid), dim3(TPB), lds, s, tev, L.w_down_t, L.down_ld, L.b_out,
         L.h_buf, L.d, L.n, B, idx, count, L.wbits, L.rs, L.sa_vec, L.tok_full, L.ks_vec,
         down_blocks(L), idx_out, count_out, tok_out, y);
}

// the general fused middle kernel (any batch up to 64; also the batch-1 fallback)
template <bool F16, bool GATED, int CPT>
void fused_launch(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s,
                  const hipEvent_t* tev) {
  const bool xl = x_in_lds(B, L.d);
  const size_t lds = xl ? (size_t)B * L.d * 4 : 0;
  if (B == 1)
    launch(k_fused_mid<F16, GATED, CPT, 1>, dim3(L.g_mid), dim3(TPB), lds, s, tev, L.p2,
           L.p_bias, L.q, L.r, L.w_act, L.act_ld, L.b_act, x, L.d, L.n, B, L.tau,
           L.rs_in_arg ? nullptr : L.rs, L.wbits, L.tok_full, L.h_buf, scores, xl ? 1 : 0, L.ra);
  else
    launch(k_fused_mid<F16, GATED, CPT, 4>, dim3(L.g_mid), dim3(TPB), lds, s, tev, L.p2,
           L.p_bias, L.q, L.r, L.w_act, L.act_ld, L.b_act, x, L.d, L.n, B, L.tau,
           L.rs_in_arg ? nullptr : L.rs, L.wbits, L.tok_full, L.h_buf, scores, xl ? 1 : 0, L.ra);
}

template <bool F16, bool GATED, int CPT>
int fused_occ(const LayerDev& L, int B) {
  const size_t lds = x_in_lds(B, L.d) ? (size_t)B * L.d * 4 : 0;
  int a = 0;
  hipError_t e = B == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, k_fused_mid<F16, GATED, CPT, 1>, TPB, lds)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, k_fused_mid<F16, GATED, CPT, 4>, TPB, lds);
  return e == hipSuccess ? a : 0;
}

template <bool F16, bool GATED>
void mid_batch_any(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s,
                   const hipEvent_t* tev) {
  if (B >= 2 && B <= 4 && (F16 ? run_mid_bt_h4 : run_mid_bt_f4)(L, x, B, scores, s, tev)) return;
  if (B >= 5 && B <= 8 && (F16 ? run_mid_bt_h8 : run_mid_bt_f8)(L, x, B, scores, s, tev)) return;
  switch (pick_cpt(row_chunks(L))) {
    case 1: fused_launch<F16, GATED, 1>(L, x, B, scores, s, tev); break;
    case 2: fused_launch<F16, GATED, 2>(L, x, B, scores, s, tev); break;
    case 4: fused_launch<F16, GATED, 4>(L, x, B, scores, s, tev); break;
    default: fused_launch<F16, GATED, 8>(L, x, B, scores, s, tev); break;
  }
}

template <bool F16, bool GATED>
int mid_batch_occ(const LayerDev& L, int B) {
  if (B >= 2 && B <= 8) {
    const int o = B <= 4 ? (F16 ? occ_mid_bt_h4 : occ_mid_bt_f4)(L) : (F16 ? occ_mid_bt_h8 : occ_mid_bt_f8)(L);
    if (o >= 0) return o;
  }
  switch (pick_cpt(row_chunks(L))) {
    case 1: return fused_occ<F16, GATED, 1>(L, B);
    case 2: return fused_occ<F16, GATED, 2>(L, B);
    case 4: return fused_occ<F16, GATED, 4>(L, B);
    default: return fused_occ<F16, GATED, 8>(L, B);
  }
}

template <bool F16, bool BITS>
void down_any(const LayerDev& L, int B, const int32_t* idx, const int32_t* count,
              int32_t* idx_out, int32_t* count_out, uint64_t* tok_out, float* y, hipStream_t s,
              const hipEvent_t* tev) {
  if (!BITS) {
    if (B == 1) down_launch_t<F16, false, 1, 1>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev);
    else if (B <= 4) down_launch_t<F16, false, 4, 1>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev);
    else down_launch_t<F16, false, 8, 1>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev);
    return;
  }
#define DOWN_BITS(TB)                                                                          \
  switch (L.upt_vec) {                                                                         \
    case 1: down_launch_t<F16, true, TB, 1>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev); break; \
    case 2: down_launch_t<F16, true, TB, 2>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev); break; \
    case 4: down_launch_t<F16, true, TB, 4>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev); break; \
    default: down_launch_t<F16, true, TB, 8>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev); break; \
  }
  if (B <= 4) {
    DOWN_BITS(4)
  } else {
    DOWN_BITS(8)
  }
#undef DOWN_BITS
}

}  // namespace

void run_mid_batch(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s,
                   const hipEvent_t* tev) {
  if (L.w_f16) {
    if (L.gated) mid_batch_any<true, true>(L, x, B, scores, s, tev);
    else mid_batch_any<true, false>(L, x, B, scores, s, tev);
  } else {
    if (L.gated) mid_batch_any<false, true>(L, x, B, scores, s, tev);
    else mid_batch_any<false, false>(L, x, B, scores, s, tev);
  }
}

int occ_mid_batch(const LayerDev& L, int B) {
  if (L.w_f16) return L.gated ? mid_batch_occ<true, true>(L, B) : mid_batch_occ<true, false>(L, B);
  return L.gated ? mid_batch_occ<false, true>(L, B) : mid_batch_occ<false, false>(L, B);
}

void run_down(const LayerDev& L, int B, bool bits, const int32_t* idx, const int32_t* count,
              int32_t* idx_out, int32_t* count_out, uint64_t* tok_out, float* y, hipStream_t s,
              const hipEvent_t* tev) {
  if (L.w_f16) {
    if (bits) down_any<true, true>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev);
    else down_any<true, false>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev);
  } else {
    if (bits) down_any<false, true>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev);
    else down_any<false, false>(L, B, idx, count, idx_out, count_out, tok_out, y, s, tev);
  }
}

void run_gather(const LayerDev& L, const float* x, int B, const int32_t* idx, const int32_t* count,
                const uint64_t* tokmask, float* y0, hipStream_t s) {
  if (L.w_f16) {
    if (L.gated) gather_dispatch<true, true>(L, x, B, idx, count, tokmask, y0, s);
    else gather_dispatch<true, false>(L, x, B, idx, count, tokmask, y0, s);
  } else {
    if (L.gated) gather_dispatch<false, true>(L, x, B, idx, count, tokmask, y0, s);
    else gather_dispatch<false, false>(L, x, B, idx, count, tokmask, y0, s);
  }
}

}  // namespace sffn
