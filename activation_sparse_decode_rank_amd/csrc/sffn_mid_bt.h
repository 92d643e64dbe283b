// The small-batch middle kernel (2..8 tokens) and its launch helpers. Included by the
// translation units that instantiate it for fp16 or fp32 weights and up to 4 or 8 tokens
// (each exports run_mid_bt_* and occ_mid_bt_*, declared in sffn_internal.h).
#pragma once
#include "sffn_device.h"

namespace sffn {
namespace {

// ---------------------------------------------------------------------------- small batch
// The middle kernel for 2 .. BT tokens (BT = 4 or 8): the batch-1 form with every
// predictor chunk and every gathered row reused for all tokens. Each (neuron, token) score
// is thresholded into the neuron's token bits; the range's union of active neurons is
// compacted, and each union row's activations are formed for every token (0 where the
// token's bit is clear). Outputs as k_fused_mid: wbits[w], tok_full[i], h_g[i*B + b].
// Thread t multiplies input chunks t, t + 256, ... (CX of them): the plain row's chunk,
// or the gate row's and the up row's chunk at the same position, so each input chunk is
// held once per token. Predictor rows fit one wave (NCHP <= 64).
template <bool F16, bool GATED, int CX, int NCHP, int BT>
__global__ __launch_bounds__(TPB) void k_mid_bt(
    const void* __restrict__ p2, const float* __restrict__ pbias, const float* __restrict__ q,
    const void* __restrict__ w_act, int ld_act, const float* __restrict__ b_act,
    const float* __restrict__ x, int d, int n, int B, float tau, const int32_t* __restrict__ rs,
    uint64_t* __restrict__ wbits,
    uint64_t* __restrict__ tok_full, float* __restrict__ h_g, float* __restrict__ scores,
    const RangeArg ra) {
  constexpr int EPC = Elt<F16>::EPC;
  constexpr int R = NCHP * EPC;       // predictor rank
  constexpr int RPP = TPB / NCHP;     // predictor rows per slot of the workgroup
  constexpr int PL = 8;               // slots in flight per thread
  constexpr int RMAX = MID_RANGE_MAX;
  constexpr int NV = GATED ? 2 : 1;
  constexpr int RB = (BT == 4 && !GATED) ? 4 : 2;  // gathered rows per batch
  static_assert(NCHP >= 1 && NCHP <= 64 && (NCHP & (NCHP - 1)) == 0, "NCHP");
  static_assert(BT == 4 || BT == 8, "BT");
  __shared__ uint64_t s_tok[RMAX];
  __shared__ int32_t s_rows[RMAX];
  __shared__ uint64_t s_bits[RMAX];
  __shared__ float s_bias[RMAX];
  __shared__ float s_pb[RMAX];
  __shared__ float s_ba[RMAX];
  __shared__ int s_wcnt[TPB / 64];
  __shared__ float s_red[TPB / 64][RB][BT][NV];

  touch_kernargs<2>();
  const int w = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = rs ? rs[w] : ra.r[w], r1 = rs ? rs[w + 1] : ra.r[w + 1];
  const int nown = r1 - r0;  // 1..RMAX
  const int pos = tid & (NCHP - 1);
  const int rsub = tid / NCHP;
  const int nslots = (nown + RPP - 1) / RPP;
  const size_t blk0 = (size_t)r0 * NCHP;

  // ---- every score-independent load first: P2 (first PL slots), q of every token, biases
  u32x4 wv[PL];
  int mlim = min(PL, nslots);
#pragma unroll
  for (int m = 0; m < PL; ++m) wv[m] = ld_chunk(p2, blk0 + (size_t)min(m * RPP + rsub, nown - 1) * NCHP + pos);
  float qs[BT][EPC];
#pragma unroll
  for (int b = 0; b < BT; ++b) load_x<EPC>(q + (size_t)min(b, B - 1) * R + (size_t)pos * EPC, qs[b]);
  if (tid < nown) {
    s_pb[tid] = pbias ? pbias[r0 + tid] : 0.f;
    s_ba[tid] = b_act ? b_act[r0 + tid] : 0.f;
  }
  if (tid < RMAX) s_tok[tid] = 0;
  __syncthreads();

  // ---- predictor stage 2 and threshold, token by token on the same predictor chunks
  for (int s0 = 0; s0 < nslots; s0 += PL) {
    if (s0 > 0) {
      mlim = min(PL, nslots - s0);
#pragma unroll
      for (int m = 0; m < PL; ++m)
        wv[m] = ld_chunk(p2, blk0 + (size_t)min((s0 + m) * RPP + rsub, nown - 1) * NCHP + pos);
    }
#pragma unroll
    for (int m = 0; m < PL; ++m) {
      if (m < mlim) {
        const int j = (s0 + m) * RPP + rsub;
        uint64_t bits = 0;
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (b < B) {
            const float acc = group_sum<NCHP>(dot_chunk<F16>(wv[m], qs[b], 0.f));
            if (j < nown && (lane & (NCHP - 1)) == group_leader(NCHP)) {
              const float sc = acc + s_pb[j];
              if (scores) scores[(size_t)b * n + r0 + j] = sc;
              if (sc > tau) bits |= (uint64_t)1 << b;  // NaN compares false
            }
          }
        }
        if (j < nown && (lane & (NCHP - 1)) == group_leader(NCHP)) s_tok[j] = bits;
      }
    }
  }
  __syncthreads();
  // ---- union compaction of the owned range: ballot per wave, prefix over the four waves
  const uint64_t tbits = tid < nown ? s_tok[tid] : 0;
  const bool act = tbits != 0;
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
    s_bits[k] = tbits;
    s_bias[k] = s_ba[tid];
  }
  __syncthreads();

  // ---- gather-GEMV + ReLU over the union rows, every token, RB rows per batch
  const int nch = d / EPC;
  float xs[CX][BT][EPC];
  if (nact > 0) {
#pragma unroll
    for (int m = 0; m < CX; ++m)
#pragma unroll
      for (int b = 0; b < BT; ++b)
        load_x<EPC>(x + (size_t)min(b, B - 1) * d + (size_t)min(tid + m * TPB, nch - 1) * EPC, xs[m][b]);
  }
  for (int base = 0; base < nact; base += RB) {
    const int nb = min(RB, nact - base);  // uniform
    u32x4 gv[RB][CX][NV];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      if (rr < nb) {
        const size_t row0 = (size_t)s_rows[base + rr] * ld_act;
#pragma unroll
        for (int m = 0; m < CX; ++m) {
          const int c = min(tid + m * TPB, nch - 1);
#pragma unroll
          for (int v = 0; v < NV; ++v) gv[rr][m][v] = ld_stream(w_act, row0 + v * nch + c);
        }
      }
    }
    float acc[RB][BT][NV];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int b = 0; b < BT; ++b)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[rr][b][v] = 0.f;
#pragma unroll
    for (int m = 0; m < CX; ++m) {
      const bool cv = tid + m * TPB < nch;
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        if (rr < nb) {
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            float f[EPC];
            unpack<F16>(gv[rr][m][v], f);
#pragma unroll
            for (int b = 0; b < BT; ++b) {
              float a = 0.f;
#pragma unroll
              for (int e = 0; e < EPC; ++e) a = fmaf(f[e], xs[m][b][e], a);
              acc[rr][b][v] += cv ? a : 0.f;
            }
          }
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int b = 0; b < BT; ++b)
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (rr < nb && b < B) acc[rr][b][v] = wave_sum(acc[rr][b][v]);
    if (lane == WAVE_SUM_LANE) {
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
#pragma unroll
        for (int b = 0; b < BT; ++b)
#pragma unroll
          for (int v = 0; v < NV; ++v) s_red[wave][rr][b][v] = acc[rr][b][v];
    }
    __syncthreads();
    if (tid < nb * BT) {
      const int rr = tid / BT, b = tid % BT;
      if (b < B) {
        float a = ((s_red[0][rr][b][0] + s_red[1][rr][b][0]) + s_red[2][rr][b][0]) + s_red[3][rr][b][0];
        a += s_bias[base + rr];
        float h = a > 0.f ? a : 0.f;
        if (GATED)
          h *= ((s_red[0][rr][b][NV - 1] + s_red[1][rr][b][NV - 1]) + s_red[2][rr][b][NV - 1]) +
               s_red[3][rr][b][NV - 1];
        const bool on = (s_bits[base + rr] >> b) & 1;
        h_g[(size_t)s_rows[base + rr] * B + b] = on ? h : 0.f;
      }
    }
    __syncthreads();
  }
  // token bits and the range's activity word (the range fits in wave 0's 64 lanes) are
  // stored last: the wait that follows a store and a barrier would hold back the gather
  if (tid < nact) tok_full[s_rows[tid]] = s_bits[tid];
  if (tid == 0) wbits[w] = word;
}

// small batches (2 .. 8 tokens) with predictor rows of at most 64 chunks
template <bool F16, bool GATED, int CX, int NCHP, int BT>
void mid_bt_launch(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s,
                   const hipEvent_t* tev) {
  launch(k_mid_bt<F16, GATED, CX, NCHP, BT>, dim3(L.g_mid), dim3(TPB), 0, s, tev, L.p2, L.p_bias,
         L.q, L.w_act, L.act_ld, L.b_act, x, L.d, L.n, B, L.tau, L.rs_in_arg ? nullptr : L.rs, L.wbits,
         L.tok_full, L.h_buf, scores, L.ra);
}

template <bool F16, bool GATED, int CX, int BT>
bool mid_bt_dispatch_nchp(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s,
                          const hipEvent_t* tev) {
  switch (L.r / (F16 ? 8 : 4)) {
    case 8: mid_bt_launch<F16, GATED, CX, 8, BT>(L, x, B, scores, s, tev); return true;
    case 16: mid_bt_launch<F16, GATED, CX, 16, BT>(L, x, B, scores, s, tev); return true;
    case 32: mid_bt_launch<F16, GATED, CX, 32, BT>(L, x, B, scores, s, tev); return true;
    case 64: mid_bt_launch<F16, GATED, CX, 64, BT>(L, x, B, scores, s, tev); return true;
    default: return false;
  }
}

template <bool F16, bool GATED, int BT>
bool mid_bt_dispatch(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s,
                     const hipEvent_t* tev) {
  switch (pick_cpt(L.d / (F16 ? 8 : 4))) {
    case 1: return mid_bt_dispatch_nchp<F16, GATED, 1, BT>(L, x, B, scores, s, tev);
    case 2: return mid_bt_dispatch_nchp<F16, GATED, 2, BT>(L, x, B, scores, s, tev);
    case 4: return mid_bt_dispatch_nchp<F16, GATED, 4, BT>(L, x, B, scores, s, tev);
    case 8: return mid_bt_dispatch_nchp<F16, GATED, 8, BT>(L, x, B, scores, s, tev);
    default: return false;
  }
}

template <bool F16, bool GATED, int CX, int BT>
int mid_bt_occ_cx(const LayerDev& L) {
  int a = 0;
  hipError_t e;
  switch (L.r / (F16 ? 8 : 4)) {
    case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, k_mid_bt<F16, GATED, CX, 8, BT>, TPB, 0); break;
    case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, k_mid_bt<F16, GATED, CX, 16, BT>, TPB, 0); break;
    case 32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, k_mid_bt<F16, GATED, CX, 32, BT>, TPB, 0); break;
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, k_mid_bt<F16, GATED, CX, 64, BT>, TPB, 0); break;
    default: return -1;  // no small-batch kernel for this predictor width
  }
  return e == hipSuccess ? a : 0;
}

// occupancy of the small-batch middle kernel for up to BT tokens, -1 when it does not apply
template <bool F16, bool GATED, int BT>
int mid_bt_occ(const LayerDev& L) {
  switch (pick_cpt(L.d / (F16 ? 8 : 4))) {
    case 1: return mid_bt_occ_cx<F16, GATED, 1, BT>(L);
    case 2: return mid_bt_occ_cx<F16, GATED, 2, BT>(L);
    case 4: return mid_bt_occ_cx<F16, GATED, 4, BT>(L);
    case 8: return mid_bt_occ_cx<F16, GATED, 8, BT>(L);
    default: return -1;
  }
}

}  // namespace
}  // namespace sffn

// Defines run_<NAME> (launch for 2..BT tokens; false when no kernel exists for the shape)
// and occ_<NAME> (workgroups per CU, -1 when no kernel applies) for weights of F16.
#define SFFN_MID_BT_ENTRY(F16, BT, NAME)                                                       \
  namespace sffn {                                                                             \
  bool run_##NAME(const LayerDev& L, const float* x, int B, float* scores, hipStream_t s,      \
                  const hipEvent_t* tev) {                                                     \
    return L.gated ? mid_bt_dispatch<F16, true, BT>(L, x, B, scores, s, tev)                   \
                   : mid_bt_dispatch<F16, false, BT>(L, x, B, scores, s, tev);                 \
  }                                                                                            \
  int occ_##NAME(const LayerDev& L) {                                                          \
    return L.gated ? mid_bt_occ<F16, true, BT>(L) : mid_bt_occ<F16, false, BT>(L);             \
  }                                                                                            \
  }
