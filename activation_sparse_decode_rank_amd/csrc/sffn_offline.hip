// Offline helpers (gfx950): activation profile counts over profiling tokens and the
// row-gather copy that packs weights in hot-first order.
#include "sffn_device.h"

namespace sffn {
namespace {

// ============================================================================ offline
// Activation profile: counts[i] = #{tokens t : w_act[i] . x_t + b_act[i] > 0}. A plain
// LDS-tiled fp32 product: workgroup owns 64 neurons and walks every token in tiles of 64;
// a thread computes a 4x4 block. Integer counts per neuron stay in the owner thread.
template <bool WF16>
__global__ __launch_bounds__(TPB) void k_profile(const void* __restrict__ w_act, int row_elems,
                                                 const float* __restrict__ b_act,
                                                 const float* __restrict__ x, int d, int n,
                                                 int N, int64_t* __restrict__ counts) {
  constexpr int TK = 32;
  __shared__ float s_w[TK][64 + 1];
  __shared__ float s_xt[TK][64 + 1];
  __shared__ int s_cnt[16][64];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int i0 = blockIdx.x * 64;
  int cnt[4] = {0, 0, 0, 0};
  for (int t0 = 0; t0 < N; t0 += 64) {
    float acc[4][4] = {};
    for (int k0 = 0; k0 < d; k0 += TK) {
      for (int u = tid; u < 64 * TK; u += TPB) {
        const int rr = u / TK, kk = u % TK;
        const int i = i0 + rr, t = t0 + rr, k = k0 + kk;
        float wvv = 0.f, xv = 0.f;
        if (i < n && k < d) {
          if (WF16)
            wvv = (float)reinterpret_cast<const _Float16*>(w_act)[(size_t)i * row_elems + k];
          else
            wvv = reinterpret_cast<const float*>(w_act)[(size_t)i * row_elems + k];
        }
        if (t < N && k < d) xv = x[(size_t)t * d + k];
        s_w[kk][rr] = wvv;
        s_xt[kk][rr] = xv;
      }
      __syncthreads();
#pragma unroll 8
      for (int kk = 0; kk < TK; ++kk) {
        float a[4], bb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[u] = s_w[kk][ty * 4 + u];
          bb[u] = s_xt[kk][tx * 4 + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], bb[v], acc[u][v]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + ty * 4 + u;
      const float bias = (i < n && b_act) ? b_act[i] : 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + tx * 4 + v;
        if (i < n && t < N && acc[u][v] + bias > 0.f) ++cnt[u];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) s_cnt[tx][ty * 4 + u] = cnt[u];
  __syncthreads();
  if (tid < 64 && i0 + tid < n) {
    int sum = 0;
    for (int u = 0; u < 16; ++u) sum += s_cnt[u][tid];
    counts[i0 + tid] = sum;
  }
}

// dst row i (at word offset i*dst_wstride) = src row perm[i]; 4-byte words, grid-stride;
// out-of-range perm entries leave their destination row untouched.
__global__ __launch_bounds__(TPB) void k_pack_rows(const uint32_t* __restrict__ src,
                                                   const int32_t* __restrict__ perm,
                                                   uint32_t* __restrict__ dst, int rows,
                                                   int64_t wpr, int64_t dst_wstride) {
  const int64_t total = (int64_t)rows * wpr;
  for (int64_t u = blockIdx.x * (int64_t)TPB + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * TPB) {
    const int64_t rr = u / wpr, ww = u % wpr;
    const int p = perm[rr];
    if (p >= 0 && p < rows) dst[rr * dst_wstride + ww] = src[(int64_t)p * wpr + ww];
  }
}

// The identity list of the dense route: idx[k] = k, *count = n, and (tok non-null) every
// entry's token bits set for B tokens.
__global__ __launch_bounds__(TPB) void k_fill_list(int n, int B, int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ count,
                                                   uint64_t* __restrict__ tok) {
  const uint64_t bits = B >= 64 ? ~(uint64_t)0 : (((uint64_t)1) << B) - 1;
  for (int k = blockIdx.x * TPB + threadIdx.x; k < n; k += gridDim.x * TPB) {
    idx[k] = k;
    if (tok) tok[k] = bits;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *count = n;
}

}  // namespace

hipError_t launch_fill_list(const LayerDev& L, int B, int32_t* idx, int32_t* count,
                            uint64_t* tok, hipStream_t s) {
  const int grid = std::max(1, std::min((L.n + TPB - 1) / TPB, 4 * L.n_cus));
  hipLaunchKernelGGL(k_fill_list, dim3(grid), dim3(TPB), 0, s, L.n, B, idx, count, tok);
  return hipGetLastError();
}

hipError_t launch_profile_counts(const void* w_act, int w_f16, int gated, const float* b_act,
                                 int d, int n, const float* x, int N, int64_t* counts,
                                 hipStream_t s) {
  const int row_elems = gated ? 2 * d : d;
  const dim3 grid((n + 63) / 64);
  if (w_f16)
    hipLaunchKernelGGL(k_profile<true>, grid, dim3(TPB), 0, s, w_act, row_elems, b_act, x, d, n, N, counts);
  else
    hipLaunchKernelGGL(k_profile<false>, grid, dim3(TPB), 0, s, w_act, row_elems, b_act, x, d, n, N, counts);
  return hipGetLastError();
}

hipError_t launch_pack_rows(const void* src, const int32_t* perm, void* dst, int rows,
                            int64_t row_bytes, int64_t dst_stride_bytes, hipStream_t s) {
  const int64_t wpr = row_bytes / 4;
  const int64_t total = (int64_t)rows * wpr;
  int64_t blocks = (total + TPB - 1) / TPB;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_pack_rows, dim3((unsigned)blocks), dim3(TPB), 0, s,
                     static_cast<const uint32_t*>(src), perm, static_cast<uint32_t*>(dst), rows, wpr,
                     dst_stride_bytes / 4);
  return hipGetLastError();
}

}  // namespace sffn
