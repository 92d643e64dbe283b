// The decode step over a static per-device scratch array instead of the handle's
// workspace, for callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid allocation). The array is a file-scope __device__
// object: every GPU the library runs on holds its own copy, at its own address, until the
// process ends. Its address on a device is looked up once, at handle creation with that
// device current, and every call passes that address to the kernels (in host code the
// array's name is only a host-side stand-in, never a device address).
#include <mutex>

#include "sffn_device.h"

namespace sffn {

// 16 MiB: the decode workspace of the OPT-6.7B- and Llama-7B-shaped layers up to 64 tokens,
// of the OPT-175B-shaped layer up to 32 (sparse_ffn_workspace_bytes at the call's batch)
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// Writes entries [off, off + cnt) of the range table from the arguments (at most
// RS_ARG_MAX + 1 per launch) and, from the first launch, zeroes the arrival counters of the
// stream-K up projection and of the down projection's join (every call leaves them zero,
// but the array keeps whatever the last call on this device left, and nothing here may
// assume who that was).
__global__ __launch_bounds__(TPB) void k_static_prologue(const RangeArg part, int off, int cnt,
                                                         int32_t* __restrict__ rs,
                                                         int32_t* __restrict__ sk_cnt, int ncnt,
                                                         int32_t* __restrict__ dn_cnt, int ndn) {
  const int i = blockIdx.x * TPB + threadIdx.x;
  if (i < cnt) rs[off + i] = part.r[i];
  for (int j = i; j < ncnt; j += gridDim.x * TPB) sk_cnt[j] = 0;
  for (int j = i; j < ndn; j += gridDim.x * TPB) dn_cnt[j] = 0;
}

}  // namespace

bool static_scratch_setup(int dev) {
  if (dev < 0 || dev >= MAX_DEVICES) return false;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev]) return true;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return false;
  g_ptr[dev] = p;
  return true;
}

void* static_scratch_ptr(int dev) {
  if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_ptr[dev];
}

hipError_t run_decode_static(const LayerDev& H, const int32_t* rs_host, int g, void* base,
                             const float* x, int B, float* y, int32_t* idx, int32_t* count,
                             uint64_t* tokmask, float* scores, hipStream_t s) {
  LayerDev L = H;
  carve_workspace(L, base, B, H.single_pass);
  const int ncnt = (L.n + 15) / 16 + 1;
  const int ndn = L.d / 32 + 2;
  for (int off = 0; off <= g; off += RS_ARG_MAX + 1) {
    const int cnt = std::min(RS_ARG_MAX + 1, g + 1 - off);
    RangeArg part{};
    std::copy(rs_host + off, rs_host + off + cnt, part.r);
    const int items = off == 0 ? std::max(cnt, std::max(ncnt, ndn)) : cnt;
    hipLaunchKernelGGL(k_static_prologue, dim3((items + TPB - 1) / TPB), dim3(TPB), 0, s, part,
                       off, cnt, L.rs, L.sk_cnt, off == 0 ? ncnt : 0, L.dn_cnt,
                       off == 0 ? ndn : 0);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode(L, x, B, y, idx, count, tokmask, scores, s, nullptr);
}

}  // namespace sffn
