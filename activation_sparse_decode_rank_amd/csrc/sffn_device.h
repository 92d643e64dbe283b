// Device helpers shared by the kernel translation units of the activation-sparse FFN
// decode library, written for gfx950 (CDNA4):
// 64-lane wavefronts, 256-thread workgroups, 16-byte vector loads, LDS staging.
//
// The method (what is computed) comes from the pages:
//  - a predictor scores every neuron and only the predicted-active ones are computed
//    (unite.ai PowerInfer overview, "Fase en línea"; novita.ai activation-sparsity
//    article, section 單層計算優化);
//  - neuron-aware operators touch whole rows of the up matrix and whole rows of the
//    transposed down matrix, with no sparse-format conversion (unite.ai overview,
//    "Operador consciente de neuronas");
//  - ReLU between up and down (novita.ai article, section 激活稀疏性的可行性), on the gate in
//    the ReLU-fied gated FFN (section 第一階段); gate and up rows of one neuron are stored
//    together because they co-activate (PowerInfer-2 article, section 4.4);
//  - memory is read in whole coalesced blocks and operators are fused (novita.ai article,
//    section 工程影響).
// How it is computed here is specific to this chip: kernel boundaries are the only
// grid-wide synchronization (inside a HIP graph the next kernel starts as the previous one
// drains; a hand-off between workgroups of one launch through a device-coherent counter
// measured slower, since same-address atomics and polls serialize at the coherent level).
// Global atomics are few: the down projections may add up to KS split-k sums per output
// element with float atomics (bitwise reproducible for KS <= 2), and the stream-K up
// kernel counts the parts of each split tile. Every other reduction has a fixed order.
#pragma once
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

#include "sffn_internal.h"

namespace sffn {
namespace {

constexpr int TPB = 256;        // threads per workgroup for every kernel here
constexpr int MAXB = 64;        // tokens per call (one bit each in a 64-bit word)
constexpr int X_LDS_MAX = 48 * 1024;  // tokens are staged in LDS when they fit in this

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));   // LDS transpose-read result
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

// Buffer resources for the raw buffer load/store builtins: word 3 of the descriptor for
// the gfx9 family (untyped 32-bit data, no swizzle), and the cache-policy bit that makes an
// access device-coherent (sc1: what agent-scope atomic loads and stores use on this part).
constexpr int BUF_RSRC_WORD3 = 0x00020000;
constexpr int CPOL_SC1 = 16;

// A "chunk" is 16 bytes of weights: 8 fp16 or 4 fp32 elements.
template <bool F16>
struct Elt {
  static constexpr int EPC = F16 ? 8 : 4;
};

__device__ __forceinline__ u32x4 ld_chunk(const void* base, size_t chunk) {
  return reinterpret_cast<const u32x4*>(base)[chunk];
}
// Weight rows read once per step: non-temporal, so that streaming them does not evict
// what the step reuses from the caches (kernel code, the token, predictor outputs,
// activations).
__device__ __forceinline__ u32x4 ld_stream(const void* base, size_t chunk) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + chunk);
}

template <bool F16>
__device__ __forceinline__ void unpack(const u32x4& v, float* f) {
  if constexpr (F16) {
    half8_t h = __builtin_bit_cast(half8_t, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
  } else {
    float4_t g = __builtin_bit_cast(float4_t, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = g[e];
  }
}

// acc + sum_e w[e] * x[e], e ascending
template <bool F16>
__device__ __forceinline__ float dot_chunk(const u32x4& v, const float* x, float acc) {
  float f[Elt<F16>::EPC];
  unpack<F16>(v, f);
#pragma unroll
  for (int e = 0; e < Elt<F16>::EPC; ++e) acc = fmaf(f[e], x[e], acc);
  return acc;
}

template <int EPC>
__device__ __forceinline__ void load_x(const float* p, float* xs) {
  const float4_t* q = reinterpret_cast<const float4_t*>(p);
#pragma unroll
  for (int u = 0; u < EPC / 4; ++u) {
    float4_t v = q[u];
    xs[4 * u + 0] = v[0];
    xs[4 * u + 1] = v[1];
    xs[4 * u + 2] = v[2];
    xs[4 * u + 3] = v[3];
  }
}

// Read one word of each of the first LINES 64-byte lines of this kernel's explicit
// arguments at entry, all loads issued before one wait. The compiler otherwise loads
// arguments next to their first use, spread through the kernel, and each argument line
// touched for the first time costs a memory round trip; after this every such load hits
// the scalar cache. Large by-value tables go last in the argument list, past LINES.
template <int LINES>
__device__ __forceinline__ void touch_kernargs() {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef const uint32_t __attribute__((address_space(4)))* karg_ptr;
  const karg_ptr ka = (karg_ptr)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t v = 0;
#pragma unroll
  for (int l = 0; l < LINES; ++l) v ^= ka[16 * l];
  asm volatile("" ::"s"(v));
#endif
}

// Cross-lane adds through DPP: VALU operations that read a neighbouring lane's register
// directly, with no LDS round trip. Lanes whose source is outside the pattern, or whose
// 16-lane row is masked off, add 0. Patterns used (each adds the value of lane src(l)):
//   QP_XOR1 / QP_XOR2   quad permutations l^1 and l^2
//   HALF_MIRROR         l -> 7-l within each 8 lanes; MIRROR: l -> 15-l within each row
//   SHR(k)              l -> l-k within the row
//   BCAST15 (rows 1,3)  += lane 15 of the previous row; BCAST31 (rows 2,3) += lane 31
constexpr int DPP_QP_XOR1 = 0xB1, DPP_QP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141,
              DPP_MIRROR = 0x140, DPP_BCAST15 = 0x142, DPP_BCAST31 = 0x143;
constexpr int dpp_shr(int k) { return 0x110 + k; }

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_add_i(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}

// Sum over all 64 lanes; the total is complete in lanes 48..63.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<DPP_QP_XOR1>(v);
  v = dpp_add<DPP_QP_XOR2>(v);
  v = dpp_add<DPP_HALF_MIRROR>(v);
  v = dpp_add<DPP_MIRROR>(v);
  v = dpp_add<DPP_BCAST15, 0xA>(v);
  return dpp_add<DPP_BCAST31, 0xC>(v);
}
constexpr int WAVE_SUM_LANE = 63;

// Inclusive prefix sum over the 64 lanes (lane order).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v = dpp_add_i<dpp_shr(1)>(v);
  v = dpp_add_i<dpp_shr(2)>(v);
  v = dpp_add_i<dpp_shr(4)>(v);
  v = dpp_add_i<dpp_shr(8)>(v);
  v = dpp_add_i<DPP_BCAST15, 0xA>(v);
  return dpp_add_i<DPP_BCAST31, 0xC>(v);
}

// Sum over aligned groups of L lanes (L = 1, 2, 4, ..., 64). The group's sum is complete in
// its lane group_leader(L): the first lane for L <= 16 (every lane, in fact), the last lane
// for L = 32 and 64.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if (L >= 2) v = dpp_add<DPP_QP_XOR1>(v);
  if (L >= 4) v = dpp_add<DPP_QP_XOR2>(v);
  if (L >= 8) v = dpp_add<DPP_HALF_MIRROR>(v);
  if (L >= 16) v = dpp_add<DPP_MIRROR>(v);
  if (L >= 32) v = dpp_add<DPP_BCAST15, 0xA>(v);
  if (L >= 64) v = dpp_add<DPP_BCAST31, 0xC>(v);
  return v;
}
__host__ __device__ constexpr int group_leader(int L) { return L <= 16 ? 0 : L - 1; }

// y[0..ny) = 0 over the whole grid: the down projection adds its split-k sums into y.
__device__ __forceinline__ void zero_grid(float* __restrict__ y, int ny) {
  for (int i = blockIdx.x * TPB + threadIdx.x; i < ny; i += gridDim.x * TPB) y[i] = 0.f;
}
// Cooperative copy of x [B][d] fp32 into LDS.
__device__ __forceinline__ void stage_x(float* s_x, const float* x, int n_floats) {
  const float4_t* src = reinterpret_cast<const float4_t*>(x);
  float4_t* dst = reinterpret_cast<float4_t*>(s_x);
  for (int u = threadIdx.x; u < n_floats / 4; u += TPB) dst[u] = src[u];
}

// fp32 -> (hi, lo) fp16 pair with v = hi + lo to about 22 significant bits: the matrix-core
// kernels multiply fp16 weights by both halves of an fp32 activation.
__device__ __forceinline__ void split_hi_lo(const float4_t& a, const float4_t& b, half8_t& hi,
                                            half8_t& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const _Float16 ha = (_Float16)a[e], hb = (_Float16)b[e];
    hi[e] = ha;
    hi[4 + e] = hb;
    lo[e] = (_Float16)(a[e] - (float)ha);
    lo[4 + e] = (_Float16)(b[e] - (float)hb);
  }
}

// Token split for the matrix-core up projection. x_hl holds, for every 8-input chunk c of
// the d inputs and every token slot b < tbp (tbp >= B; the library uses tbp = B), the hi
// halves of x_b[8c .. 8c+7] at x_hl[c * tbp + b] and the lo halves at
// x_hl[(d/8 + c) * tbp + b] (16 bytes each; slots b >= B hold zeros). With the token
// fastest, all tokens of 4 consecutive chunks are one contiguous run. Item u in
// [u0, nitems) step ustride is the pair (c = u / tbp, b = u % tbp). A thread's items go in
// batches of 4 whose loads are all issued before any is used (the tokens come cold from
// HBM; one round trip per batch, not per item). Items past the end repeat the last item,
// the same value to the same place, so no store is conditional.
__device__ __forceinline__ void split_x_items(const float* __restrict__ x, int B, int d, int tbp,
                                              u32x4* __restrict__ x_hl, int u0, int ustride) {
  constexpr int IPT = 4;
  const int nch = d / 8, nitems = nch * tbp;
  for (int ub = u0; ub < nitems; ub += IPT * ustride) {
    float4_t a[IPT], e[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int u = min(ub + i * ustride, nitems - 1);
      const int c = u / tbp, b = min(u % tbp, B - 1);
      const float4_t* p = reinterpret_cast<const float4_t*>(x + (size_t)b * d + (size_t)c * 8);
      a[i] = p[0];
      e[i] = p[1];
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int u = min(ub + i * ustride, nitems - 1);
      const int c = u / tbp, b = u % tbp;
      if (b >= B) a[i] = e[i] = float4_t{0.f, 0.f, 0.f, 0.f};
      half8_t hi, lo;
      split_hi_lo(a[i], e[i], hi, lo);
      x_hl[(size_t)c * tbp + b] = __builtin_bit_cast(u32x4, hi);
      x_hl[(size_t)(nch + c) * tbp + b] = __builtin_bit_cast(u32x4, lo);
    }
  }
}

// Orders LDS accesses of one wave: stores before it are visible to the wave's loads after
// it (a wave's LDS operations execute in order; the fences keep the compiler from moving
// them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int LIST_CAP = 8192;            // split-list window held in LDS (BITS)
constexpr int CB_LANES = 8;               // 16-byte chunks per column block (128 bytes)
constexpr int RSD = TPB / CB_LANES;       // row slots per workgroup

// ---------------------------------------------------------------------------- host helpers
// chunks per stored row (gated rows hold gate and up)
inline int row_chunks(const LayerDev& L) {
  const int epc = L.w_f16 ? 8 : 4;
  return (L.gated ? 2 : 1) * (L.d / epc);
}
inline int pick_cpt(int rowch) {
  const int need = (rowch + TPB - 1) / TPB;
  if (need <= 1) return 1;
  if (need <= 2) return 2;
  if (need <= 4) return 4;
  if (need <= 8) return 8;
  return 0;
}
// lane-group width for stage-2 rows of nchp chunks
inline void pick_group(int nchp, int& Lw, int& cplp) {
  Lw = 8;
  while (Lw < nchp && Lw < 64) Lw <<= 1;
  cplp = (nchp + Lw - 1) / Lw;
}
inline bool x_in_lds(int B, int d) { return (size_t)B * d * 4 <= (size_t)X_LDS_MAX; }

// Launch a kernel. With a timing pair (tev != nullptr) the launch goes through
// hipExtLaunchKernelGGL, which stamps tev[0] and tev[1] with the dispatch's own start and
// end times (the timestamps a kernel-trace profiler reports), not with marker packets
// queued around it.
template <typename K, typename... A>
void launch(K kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, const hipEvent_t* tev,
            A... a) {
  if (tev)
    hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, s, tev[0], tev[1], 0u, a...);
  else
    kern<<<grid, block, lds, s>>>(a...);
}

}  // namespace
}  // namespace sffn
