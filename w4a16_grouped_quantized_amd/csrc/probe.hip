// probe.hip — the achievable HBM read rate of this part, measured the way the
// layer's kernels read their weights: 16-byte loads, whole wavefronts over
// contiguous 1 KB runs, every byte read once.  The layer's achieved GB/s is
// reported against this ceiling as well as against the nominal peak.
#include "moe_w4a16.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kProbeBlock = 256;
constexpr int kProbeUnroll = 4;

// Grid-stride read of n16 16-byte words; kProbeUnroll loads in flight per
// thread and iteration.  The xor of everything read is stored only if it
// equals a value no input makes on purpose, which keeps every load alive.
__global__ __launch_bounds__(kProbeBlock) void k_read_probe(const uint4* __restrict__ p, size_t n16,
                                                            uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeBlock;
  size_t i = (size_t)blockIdx.x * kProbeBlock + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (!buf || !sink) return MOE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (bytes & 15u)) return MOE_ERR_ALIGN;
  if (blocks < 1 || blocks > 65536) return MOE_ERR_SHAPE;
  if (bytes == 0) return MOE_OK;
  hipLaunchKernelGGL(k_read_probe, dim3(blocks), dim3(kProbeBlock), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}
