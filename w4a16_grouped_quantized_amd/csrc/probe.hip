// probe.hip — the achievable HBM read rate of this part, measured the way the
// weight-streaming kernels read: 16-byte non-temporal loads (data read once
// passes by the CU's vector cache; on this part they read ~13% faster than
// plain loads), whole wavefronts over contiguous 1 KB runs, several kilobytes
// in flight per wavefront, every byte read once.  The layer's achieved GB/s is
// reported against this ceiling as well as against the nominal peak.
#include "moe_w4a16.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kProbeBlock = 256;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kProbeTile = 10;  // 1 KB wavefront loads per tile (10 KB contiguous)

// Each wavefront reads contiguous 10 KB tiles (ten 1 KB loads), the tiles
// dealt to the grid's wavefronts in turn, and requests its next tile before
// it folds the current one (twenty loads in flight per lane), as the
// weight-streaming kernels do (of 4, 8, 10 and 16 KB tiles at 4, 8 and 16
// workgroups per CU, 10 KB tiles read fastest or within 2% of the fastest).
// The tail past the last whole tile is read one 16-byte word per lane.  The xor of everything read is stored only if it
// equals a value no input makes on purpose, which keeps every load alive.
__global__ __launch_bounds__(kProbeBlock) void k_read_probe(const uint4* __restrict__ p, size_t n16,
                                                            uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const size_t nw = (size_t)gridDim.x * (kProbeBlock / 64);
  const size_t w0 = (size_t)blockIdx.x * (kProbeBlock / 64) + (threadIdx.x >> 6);
  const size_t per_tile = (size_t)kProbeTile * 64;  // 16-byte words
  const size_t ntiles = n16 / per_tile;
  uint32_t acc = 0;
  uint4 a[kProbeTile], b[kProbeTile];
  auto load = [&](uint4 (&v)[kProbeTile], size_t t) {
#pragma unroll
    for (int u = 0; u < kProbeTile; ++u) {
      const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + t * per_tile + (size_t)u * 64 + lane));
      v[u] = make_uint4(q.x, q.y, q.z, q.w);
    }
  };
  auto fold = [&](const uint4 (&v)[kProbeTile]) {
#pragma unroll
    for (int u = 0; u < kProbeTile; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  };
  size_t t = w0;
  if (t < ntiles) load(a, t);
  for (; t < ntiles; t += 2 * nw) {
    const size_t t2 = t + nw;
    if (t2 < ntiles) load(b, t2);
    fold(a);
    if (t2 < ntiles) {
      if (t2 + nw < ntiles) load(a, t2 + nw);
      fold(b);
    }
  }
  for (size_t i = ntiles * per_tile + w0 * 64 + lane; i < n16; i += nw * 64) {
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
