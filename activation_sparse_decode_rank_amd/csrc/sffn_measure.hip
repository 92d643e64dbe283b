// Measurement helpers (gfx950), not steps of the method: a plain read stream over device
// memory, the achievable-peak denominator reported beside the nominal HBM bandwidth (every
// kernel of the decode path is bound by how fast it can read weight rows, so the rate this
// stream reaches is the ceiling those kernels are measured against); and the input-sparse
// up projection probe below.
#include "sffn_device.h"

namespace sffn {
namespace {

// Each thread reads 16-byte chunks i, i + S, i + 2S, ... (S = all threads of the grid), 8
// in flight at a time, non-temporal like the weight streams. The values are folded into
// one register; the store behind an (almost never true) test keeps every load live.
constexpr int PROBE_INFLIGHT = 8;
__global__ __launch_bounds__(TPB) void k_read_probe(const u32x4* __restrict__ buf, size_t nchunks,
                                                    uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * TPB;
  size_t i = (size_t)blockIdx.x * TPB + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (PROBE_INFLIGHT - 1) * stride < nchunks; i += PROBE_INFLIGHT * stride) {
    u32x4 v[PROBE_INFLIGHT];
#pragma unroll
    for (int u = 0; u < PROBE_INFLIGHT; ++u) v[u] = ld_stream(buf, i + u * stride);
#pragma unroll
    for (int u = 0; u < PROBE_INFLIGHT; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < nchunks; i += stride) {
    const u32x4 v = ld_stream(buf, i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// ---------------------------------------------------------------- input-sparse up probe
// Two ways to compute u_k = W_u[i_k] . x for the listed neurons i_k of one token whose input
// x is about half zeros (the ReLU after RMSNorm of the second ReLU-fication stage: novita.ai
// activation-sparsity article, section 第二階段). They exist to measure whether a
// column-major copy of W_u, which can skip the zero inputs, beats gathering the listed rows
// (which cannot: a zero inside a row's 128-byte line saves no bytes). Not a step of the
// decode path.

// Rows ([n][d] fp16): one wave per listed row, M chunks per lane (d / 8 chunks of 8 fp16),
// all of the row's loads issued before any is used; the sum over lanes in fixed order.
template <int M>
__global__ __launch_bounds__(TPB) void k_upp_rows(const void* __restrict__ w, int d, int n,
                                                  const float* __restrict__ x,
                                                  const int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ count,
                                                  float* __restrict__ u) {
  const int lane = threadIdx.x & 63;
  const int nch = d / 8;
  const int cnt = min(max(*count, 0), n);
  float xs[M][8];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = lane + 64 * m;
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[m][e] = 0.f;
    if (c < nch) load_x<8>(x + (size_t)c * 8, xs[m]);
  }
  const int nw = gridDim.x * (TPB / 64);
  for (int k = blockIdx.x * (TPB / 64) + (threadIdx.x >> 6); k < cnt; k += nw) {
    const int i = idx[k];
    const size_t row = (size_t)(i >= 0 && i < n ? i : 0) * nch;  // out-of-range entries read row 0
    u32x4 wv[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int c = lane + 64 * m;
      wv[m] = c < nch ? ld_stream(w, row + c) : u32x4{0u, 0u, 0u, 0u};
    }
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m) acc = dot_chunk<true>(wv[m], xs[m], acc);
    acc = wave_sum(acc);
    if (lane == WAVE_SUM_LANE) u[k] = acc;
  }
}

// Columns ([d][n] fp16, W_u transposed): workgroup (tile, s) owns neurons [512 tile, +512)
// (lane l of every wave holds the 16-byte piece of neurons 512 tile + 8l .. +7) and inputs
// [s cps, (s + 1) cps), cps <= 1024. The workgroup first lists its nonzero inputs (and their
// values) in LDS, so that no weight load waits on an input load; wave w then takes list
// entries w, w + 4, ..., 16 loads in flight at a time. A piece none of whose neurons is
// listed (words: the neurons' list bits) loads nothing. The 4 waves' sums are added in
// wave order into part[s][n]; k_upp_sum adds the UPP_S splits in order.
constexpr int UPP_S = 16;
constexpr int UPP_INFLIGHT = 16;
__global__ __launch_bounds__(TPB) void k_upp_cols(const void* __restrict__ w, int d, int n,
                                                  const float* __restrict__ x,
                                                  const uint64_t* __restrict__ words,
                                                  float* __restrict__ part) {
  __shared__ float s_red[TPB / 64][64][8];
  constexpr int CPS_MAX = 16384 / UPP_S;
  __shared__ int s_j[CPS_MAX];
  __shared__ float s_x[CPS_MAX];
  __shared__ int s_wc[TPB / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntile = (n + 511) / 512;
  const int tile = blockIdx.x % ntile, s = blockIdx.x / ntile;
  const int npc = n / 8;                  // pieces per column
  const int p = tile * 64 + lane;         // this lane's piece
  const bool live = p < npc && ((words[p >> 3] >> ((p & 7) * 8)) & 0xFFu) != 0;
  const int cps = (d + UPP_S - 1) / UPP_S;  // <= CPS_MAX (d <= 16384)
  const int j0 = s * cps, j1 = min(d, j0 + cps);
  // the nonzero inputs of [j0, j1), in order, TPB inputs a pass
  int nnz = 0;
  for (int jb = j0; jb < j1; jb += TPB) {
    const int j = jb + tid;
    const float xj = j < j1 ? x[j] : 0.f;
    const uint64_t m = __ballot(xj != 0.f);
    if (lane == 0) s_wc[wave] = __popcll(m);
    __syncthreads();
    int before = nnz;
#pragma unroll
    for (int v = 0; v < TPB / 64; ++v) before += v < wave ? s_wc[v] : 0;
    if (xj != 0.f) {
      const int pos = before + __popcll(m & ((1ull << lane) - 1));
      s_j[pos] = j;
      s_x[pos] = xj;
    }
    nnz += s_wc[0] + s_wc[1] + s_wc[2] + s_wc[3];
    __syncthreads();
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int q0 = wave; q0 < nnz; q0 += 4 * UPP_INFLIGHT) {
    float xv[UPP_INFLIGHT];
    u32x4 wv[UPP_INFLIGHT];
#pragma unroll
    for (int t = 0; t < UPP_INFLIGHT; ++t) {
      const int q = q0 + 4 * t;
      const bool ok = q < nnz;
      const int jj = ok ? s_j[q] : 0;
      xv[t] = ok ? s_x[q] : 0.f;
      wv[t] = (ok && live) ? ld_stream(w, (size_t)jj * npc + p) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int t = 0; t < UPP_INFLIGHT; ++t) {
      float f[8];
      unpack<true>(wv[t], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(f[e], xv[t], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_red[wave][lane][e] = acc[e];
  __syncthreads();
  for (int o = tid; o < 512; o += TPB) {
    const int l = o >> 3, e = o & 7;
    const int i = tile * 512 + o;
    if (i < n)
      part[(size_t)s * n + i] = ((s_red[0][l][e] + s_red[1][l][e]) + s_red[2][l][e]) + s_red[3][l][e];
  }
}

__global__ __launch_bounds__(TPB) void k_upp_sum(const float* __restrict__ part, int n,
                                                 float* __restrict__ u) {
  const int i = blockIdx.x * TPB + threadIdx.x;
  if (i >= n) return;
  float a = part[i];
#pragma unroll
  for (int s = 1; s < UPP_S; ++s) a += part[(size_t)s * n + i];
  u[i] = a;
}

}  // namespace

size_t up_probe_work_bytes(int n) { return (size_t)UPP_S * n * 4; }

hipError_t launch_up_probe(const void* w, int layout, int d, int n, const float* x,
                           const int32_t* idx, const int32_t* count, const uint64_t* words,
                           float* u, void* work, hipStream_t s) {
  if (layout == 0) {
    const int m = (d / 8 + 63) / 64;
    const dim3 grid(512);
    if (m <= 1) hipLaunchKernelGGL(k_upp_rows<1>, grid, dim3(TPB), 0, s, w, d, n, x, idx, count, u);
    else if (m <= 2) hipLaunchKernelGGL(k_upp_rows<2>, grid, dim3(TPB), 0, s, w, d, n, x, idx, count, u);
    else if (m <= 4) hipLaunchKernelGGL(k_upp_rows<4>, grid, dim3(TPB), 0, s, w, d, n, x, idx, count, u);
    else if (m <= 8) hipLaunchKernelGGL(k_upp_rows<8>, grid, dim3(TPB), 0, s, w, d, n, x, idx, count, u);
    else if (m <= 16) hipLaunchKernelGGL(k_upp_rows<16>, grid, dim3(TPB), 0, s, w, d, n, x, idx, count, u);
    else hipLaunchKernelGGL(k_upp_rows<32>, grid, dim3(TPB), 0, s, w, d, n, x, idx, count, u);  // d <= 16384
  } else {
    float* part = static_cast<float*>(work);
    const int ntile = (n + 511) / 512;
    hipLaunchKernelGGL(k_upp_cols, dim3(ntile * UPP_S), dim3(TPB), 0, s, w, d, n, x, words, part);
    hipLaunchKernelGGL(k_upp_sum, dim3((n + TPB - 1) / TPB), dim3(TPB), 0, s, part, n, u);
  }
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_read_probe, dim3(workgroups), dim3(TPB), 0, s,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace sffn
