// Predictor stage 1 (gfx950): q = P1 x for one token or several. The method is described at
// the top of sffn_device.h; the predictor is the first half of the low-rank score map (unite.ai PowerInfer overview,
// "Predictores de espacialidad adaptativa"; novita.ai activation-sparsity article, section
// 自適應稀疏預測器).
#include "sffn_device.h"

namespace sffn {
namespace {

// ============================================================================ predictor
// Stage 1: q[b][j] = P1[j] . x_b. Workgroup j < r owns predictor row j; each thread holds
// NCPT chunks of the row in registers and reuses them for every token group of TBG. In the
// decode step these workgroups also clear y (ny floats), which the down projection later
// adds its split-k sums into.
template <bool PF16, int TBG, int NCPT>
__global__ __launch_bounds__(TPB) void k_pred_stage1(const void* __restrict__ p1,
                                                     const float* __restrict__ x, int d, int r,
                                                     int B, float* __restrict__ q,
                                                     float* __restrict__ y0, int ny) {
  constexpr int EPC = Elt<PF16>::EPC;
  touch_kernargs<1>();
  const int j = blockIdx.x, tid = threadIdx.x;
  for (int i = j * TPB + tid; i < ny; i += r * TPB) y0[i] = 0.f;
  const int nch = d / EPC;
  const size_t row0 = (size_t)j * nch;
  __shared__ float red[TPB / 64][MAXB];
  u32x4 wv[NCPT];
#pragma unroll
  for (int m = 0; m < NCPT; ++m) {
    const int c = tid + m * TPB;
    if (c < nch) wv[m] = ld_stream(p1, row0 + c);
  }
  for (int b0 = 0; b0 < B; b0 += TBG) {
    float acc[TBG];
#pragma unroll
    for (int b = 0; b < TBG; ++b) acc[b] = 0.f;
#pragma unroll
    for (int m = 0; m < NCPT; ++m) {
      const int c = tid + m * TPB;
      if (c < nch) {
        float f[EPC];
        unpack<PF16>(wv[m], f);
#pragma unroll
        for (int b = 0; b < TBG; ++b) {
          if (b0 + b < B) {
            float xs[EPC];
            load_x<EPC>(x + (size_t)(b0 + b) * d + (size_t)c * EPC, xs);
#pragma unroll
            for (int e2 = 0; e2 < EPC; ++e2) acc[b] = fmaf(f[e2], xs[e2], acc[b]);
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < TBG; ++b) acc[b] = wave_sum(acc[b]);
#pragma unroll
    for (int b = 0; b < TBG; ++b)
      if ((tid & 63) == WAVE_SUM_LANE && b0 + b < B) red[tid >> 6][b0 + b] = acc[b];
  }
  __syncthreads();
  if (tid < B) q[(size_t)tid * r + j] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// Sum each of V values (V a power of two, at most 64) over the 64 lanes of a wave, as a
// reduce-scatter: every butterfly step halves the set a lane carries, keeping the half
// its lane bit selects and adding the partner lane's copy of that half. Afterwards lane l
// holds the wave's total of value l >> (6 - log2 V), in 64 / V lanes each. Fixed order, so
// the sums are bitwise reproducible; 2V - 1 + log2(64 / V) shuffles in place of V full
// reductions.
template <int V>
__device__ __forceinline__ float wave_reduce_scatter(float (&a)[V]) {
  constexpr int K = __builtin_ctz(V);
  static_assert((V & (V - 1)) == 0 && V >= 1 && V <= 64, "V");
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < K; ++s) {
    const int mask = 32 >> s;
    const int half = V >> (s + 1);
    const bool up = (lane & mask) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      // the empty asm makes lo and hi plain register values, so the selects stay two
      // v_cndmask instead of becoming one dynamically indexed read of the whole array
      float lo = a[i], hi = a[i + half];
      asm("" : "+v"(lo), "+v"(hi));
      const float keep = up ? hi : lo;
      const float send = up ? lo : hi;
      a[i] = keep + __shfl_xor(send, mask);
    }
  }
  float v = a[0];
#pragma unroll
  for (int mask = 32 >> K; mask >= 1; mask >>= 1) v += __shfl_xor(v, mask);
  return v;
}

// Stage 1 for several tokens: workgroup (row tile, token group) computes q[b][j] = P1[j] . x_b
// for MT predictor rows and BT tokens. Each thread takes the same 16-byte column chunks of
// all MT rows and BT tokens, so every P1 row is read ceil(B / BT) times in all and every
// token r / MT times (the single-row form reads each token r times, which dominates from
// a few tokens on). Row tile = id mod (rows / MT): with rows / MT a multiple of 8 a row
// tile stays on one XCD, whose L2 then serves its rows to every token group. The nsplit
// workgroups from nmain on split the tokens into x_hl for the matrix-core up projection
// (see split_x_items; tbp token slots). The first nmain workgroups also clear y0[0..ny).
template <bool PF16, int MT, int BT>
__global__ __launch_bounds__(TPB) void k_pred_stage1_mt(
    const void* __restrict__ p1, const float* __restrict__ x, int d, int r, int B,
    float* __restrict__ q, float* __restrict__ y0, int ny, int nrt, int nmain,
    u32x4* __restrict__ x_hl, int tbp, int nsplit) {
  constexpr int EPC = Elt<PF16>::EPC;
  constexpr int V = MT * BT;
  constexpr int SPAN = 64 / V;  // lanes holding each reduced value
  touch_kernargs<2>();
  const int g = blockIdx.x, tid = threadIdx.x;
  if (g >= nmain) {
    split_x_items(x, B, d, tbp, x_hl, (g - nmain) * TPB + tid, nsplit * TPB);
    return;
  }
  for (int i = g * TPB + tid; i < ny; i += nmain * TPB) y0[i] = 0.f;
  const int j0 = (g % nrt) * MT, b0 = (g / nrt) * BT;
  if (j0 >= r || b0 >= B) return;  // padding workgroup (uniform, before any barrier)
  const int nch = d / EPC;
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
#pragma unroll 2
  for (int c = tid; c < nch; c += TPB) {
    u32x4 wv[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) wv[i] = ld_stream(p1, (size_t)min(j0 + i, r - 1) * nch + c);
    float xs[BT][EPC];
#pragma unroll
    for (int b = 0; b < BT; ++b)
      load_x<EPC>(x + (size_t)min(b0 + b, B - 1) * d + (size_t)c * EPC, xs[b]);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float f[EPC];
      unpack<PF16>(wv[i], f);
#pragma unroll
      for (int b = 0; b < BT; ++b)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[i * BT + b] = fmaf(f[e], xs[b][e], acc[i * BT + b]);
    }
  }
  const float v = wave_reduce_scatter<V>(acc);
  __shared__ float red[TPB / 64][V];
  const int lane = tid & 63;
  if ((lane & (SPAN - 1)) == 0) red[tid >> 6][lane / SPAN] = v;
  __syncthreads();
  if (tid < V) {
    const int i = tid / BT, b = tid % BT;
    if (j0 + i < r && b0 + b < B)
      q[(size_t)(b0 + b) * r + j0 + i] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
  }
}

// y0: output of ny floats the down projection will add into (zeroed here), or null
template <bool F16, int NCPT>
void stage1_launch_t(const LayerDev& L, const float* x, int B, hipStream_t s,
                     const hipEvent_t* tev, float* y0, int ny) {
  launch(k_pred_stage1<F16, 1, NCPT>, dim3(L.r), dim3(TPB), 0, s, tev, L.p1, x, L.d, L.r, B, L.q,
         y0, ny);
}

template <bool F16, int MT, int BT>
void stage1_mt_launch(const LayerDev& L, const float* x, int B, hipStream_t s,
                      const hipEvent_t* tev, float* y0, int ny, bool split_x) {
  const int nrt = (L.r + MT - 1) / MT;
  const int nmain = (nrt * ((B + BT - 1) / BT) + 7) / 8 * 8;
  const int tbp = B;  // token slots per chunk in x_hl
  const int nsplit = split_x ? (L.d / 8 * tbp + 4 * TPB - 1) / (4 * TPB) : 0;  // 4 items a thread
  launch(k_pred_stage1_mt<F16, MT, BT>, dim3(nmain + nsplit), dim3(TPB), 0, s, tev, L.p1, x, L.d,
         L.r, B, L.q, y0, ny, nrt, nmain, static_cast<u32x4*>(L.x_hl), tbp, nsplit);
}

// Several tokens: BT = 2 tokens per workgroup up to 8 tokens, 4 beyond; MT the largest row
// tile that still leaves at least 256 workgroups (one per compute unit).
template <bool F16>
void stage1_mt_dispatch(const LayerDev& L, const float* x, int B, hipStream_t s,
                        const hipEvent_t* tev, float* y0, int ny, bool split_x) {
  const int bt = B <= 8 ? 2 : 4;
  const int ntg = (B + bt - 1) / bt;
  int mt = 1;
  for (int m = 8; m >= 2; m /= 2)
    if ((L.r / m) * ntg >= 256) { mt = m; break; }
#define SFFN_S1(M, T) stage1_mt_launch<F16, M, T>(L, x, B, s, tev, y0, ny, split_x)
  if (bt == 2) {
    if (mt == 8) SFFN_S1(8, 2); else if (mt == 4) SFFN_S1(4, 2); else if (mt == 2) SFFN_S1(2, 2); else SFFN_S1(1, 2);
  } else {
    if (mt == 8) SFFN_S1(8, 4); else if (mt == 4) SFFN_S1(4, 4); else if (mt == 2) SFFN_S1(2, 4); else SFFN_S1(1, 4);
  }
#undef SFFN_S1
}

template <bool F16>
void stage1_launch(const LayerDev& L, const float* x, int B, hipStream_t s, const hipEvent_t* tev,
                   float* y0, int ny, bool split_x) {
  if (!y0) ny = 0;
  if (B > 1) {
    stage1_mt_dispatch<F16>(L, x, B, s, tev, y0, ny, split_x);
    return;
  }
  // one token, rank 512 and up (e.g. the OPT-175B slice: 1024 rows of 12288): four rows per
  // workgroup, so the token is read from L2 a quarter as often (every single-row workgroup
  // reads all of it, twice the bytes of its own row)
  if (L.r >= 512) {
    stage1_mt_launch<F16, 4, 1>(L, x, B, s, tev, y0, ny, split_x);
    return;
  }
  const int ncpt = (L.d / (F16 ? 8 : 4) + TPB - 1) / TPB;
  if (ncpt <= 1) stage1_launch_t<F16, 1>(L, x, B, s, tev, y0, ny);
  else if (ncpt <= 2) stage1_launch_t<F16, 2>(L, x, B, s, tev, y0, ny);
  else if (ncpt <= 4) stage1_launch_t<F16, 4>(L, x, B, s, tev, y0, ny);
  else stage1_launch_t<F16, 8>(L, x, B, s, tev, y0, ny);
}

}  // namespace

void run_stage1(const LayerDev& L, const float* x, int B, hipStream_t s, const hipEvent_t* tev,
                float* y0, int ny, bool split_x) {
  if (L.p_f16)
    stage1_launch<true>(L, x, B, s, tev, y0, ny, split_x);
  else
    stage1_launch<false>(L, x, B, s, tev, y0, ny, split_x);
}

}  // namespace sffn
