// Measurement helper (gfx950): a plain read stream over device memory, the achievable-peak
// denominator reported beside the nominal HBM bandwidth. Every kernel of the decode path
// is bound by how fast it can read weight rows, so the rate this stream reaches is the
// ceiling those kernels are measured against. It is not a step of the method.
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

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_read_probe, dim3(workgroups), dim3(TPB), 0, s,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace sffn
