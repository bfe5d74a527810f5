// pack.hip — one-time rearrangement of plain weights into the device layout
// described in layout.hpp, and the workspace zero-fill.
#include "launch.hpp"

namespace moe {

// One thread per 16-byte output chunk (tile, group, lane) of one expert;
// expert e's codes at src + e * sstride (plain) and dst + e * dstride.
// INT4 codes are reordered inside the chunk (layout.hpp); MXFP4 codes are
// copied as they are.
template <bool INT4>
__global__ void k_pack_codes(const uint8_t* __restrict__ src, size_t sstride, uint8_t* __restrict__ dst,
                             size_t dstride, int E, int N, int K, int is_gu, int I) {
  const int GK = K / kGroup, T = N / 64;
  const size_t per_e = (size_t)T * GK * kWave;
  const size_t total = per_e * E;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(i / per_e);
    const size_t r0 = i % per_e;
    const int l = (int)(r0 % kWave);
    const int g = (int)((r0 / kWave) % GK);
    const int b = (int)(r0 / ((size_t)kWave * GK));
    const int row = is_gu ? gu_row(b, l, I) : 64 * b + l;
    const uint8_t* s = src + (size_t)e * sstride + (size_t)row * (K / 2) + (size_t)g * 16;
    uint4* out = reinterpret_cast<uint4*>(dst + (size_t)e * dstride + ((size_t)(b * GK + g) * kWave + l) * 16);
    if constexpr (!INT4) {
      *out = *reinterpret_cast<const uint4*>(s);
      continue;
    }
    uint32_t d[4];
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      uint32_t v = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t byte = s[4 * dw + q];  // codes of inputs 8dw+2q (low) and 8dw+2q+1 (high)
        v |= (byte & 0xFu) << (4 * q);
        v |= (byte >> 4) << (16 + 4 * q);
      }
      d[dw] = v;
    }
    *out = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// One thread per (tile, pack of P groups, lane) of one expert; strides in
// elements, as for k_pack_codes; S is the scale's type (bf16 bits or E8M0).
template <typename S>
__global__ void k_pack_scales(const S* __restrict__ src, size_t sstride, S* __restrict__ dst,
                              size_t dstride, int E, int N, int K, int is_gu, int I, int P) {
  const int GK = K / kGroup, T = N / 64, NP = GK / P;
  const size_t per_e = (size_t)T * NP * kWave;
  const size_t total = per_e * E;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(i / per_e);
    const size_t r0 = i % per_e;
    const int l = (int)(r0 % kWave);
    const int gp = (int)((r0 / kWave) % NP);
    const int b = (int)(r0 / ((size_t)kWave * NP));
    const int row = is_gu ? gu_row(b, l, I) : 64 * b + l;
    const S* s = src + (size_t)e * sstride + (size_t)row * GK + (size_t)gp * P;
    S* d = dst + (size_t)e * dstride + ((size_t)(b * NP + gp) * kWave + l) * P;
    for (int q = 0; q < P; ++q) d[q] = s[q];
  }
}

// Shared BF16 matrix: one thread per (tile, chunk of 8 inputs, lane).
__global__ void k_pack_bf16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int N, int K,
                            int is_gu, int I) {
  const int T = N / 64, C = K / 8;
  const size_t total = (size_t)T * C * kWave;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(i % kWave);
    const int c = (int)((i / kWave) % C);
    const int b = (int)(i / ((size_t)kWave * C));
    const int row = is_gu ? gu_row(b, l, I) : 64 * b + l;
    const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)row * K + (size_t)c * 8);
    *reinterpret_cast<uint4*>(dst + ((size_t)(b * C + c) * kWave + l) * 8) = v;
  }
}

// Range data of each expert (layout.hpp): non-negative floats combined
// with an integer atomic max on their bit patterns, which orders them like
// the values and makes the result independent of the order of arrival.
__device__ __forceinline__ void max_bits(uint32_t* p, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

// One wavefront per gate row r (and its up row I + r) of one expert: the
// dequantised L2 norms of both rows (lane l takes groups l, l + 64, ...),
// their product into word 2, and the largest |scale| into word 0.
__global__ __launch_bounds__(256) void k_pack_meta_gu(const uint8_t* __restrict__ q, const uint16_t* __restrict__ sc,
                                                      uint32_t* __restrict__ meta, int H, int I) {
  const int e = blockIdx.y;
  const int r = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= I) return;
  const int GK = H / kGroup;
  float norm[2] = {0.f, 0.f}, smax = 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const size_t row = (size_t)e * 2 * I + (size_t)(half ? I + r : r);
    for (int g = lane; g < GK; g += kWave) {
      const uint4 w = *reinterpret_cast<const uint4*>(q + row * (H / 2) + (size_t)g * 16);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
      int sum = 0;  // sum of q^2 over the group (exact)
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int qv = (int)((wd[d] >> (4 * n)) & 0xFu) - 8;
          sum += qv * qv;
        }
      const float s = fabsf(bf16_to_f32(sc[row * GK + g]));
      norm[half] += s * s * (float)sum;
      smax = fmaxf(smax, s);
    }
  }
  const float prod = sqrtf(wave_sum(norm[0])) * sqrtf(wave_sum(norm[1]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) smax = fmaxf(smax, __shfl_xor(smax, off, 64));
  if (lane == 0) {
    max_bits(meta + (size_t)e * kMetaWords + 0, smax);
    max_bits(meta + (size_t)e * kMetaWords + 2, prod);
  }
}

// One wavefront per down row n of one expert (lane l takes groups l, l + 64,
// ...): the row's dequantised L1 norm into word 3 (max over rows) and the
// largest |scale| into word 1.
__global__ __launch_bounds__(256) void k_pack_meta_dn(const uint8_t* __restrict__ q, const uint16_t* __restrict__ sc,
                                                      uint32_t* __restrict__ meta, int H, int I) {
  const int e = blockIdx.y;
  const int r = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= H) return;
  const int GK = I / kGroup;
  const size_t row = (size_t)e * H + r;
  float norm = 0.f, smax = 0.f;
  for (int g = lane; g < GK; g += kWave) {
    const uint4 w = *reinterpret_cast<const uint4*>(q + row * (I / 2) + (size_t)g * 16);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    int sum = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int n = 0; n < 8; ++n) sum += abs((int)((wd[d] >> (4 * n)) & 0xFu) - 8);
    const float s = fabsf(bf16_to_f32(sc[row * GK + g]));
    norm += s * (float)sum;
    smax = fmaxf(smax, s);
  }
  norm = wave_sum(norm);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) smax = fmaxf(smax, __shfl_xor(smax, off, 64));
  if (lane == 0) {
    max_bits(meta + (size_t)e * kMetaWords + 1, smax);
    max_bits(meta + (size_t)e * kMetaWords + 3, norm);
  }
}

__global__ void k_fill_zero(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail, size_t ntail) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

static int grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

hipError_t launch_pack(const Shape& s, const uint8_t* w13_q, const uint16_t* w13_s,
                       const uint8_t* w2_q, const uint16_t* w2_s, const uint16_t* sh_w13,
                       const uint16_t* sh_w2, uint8_t* packed, const PackedLayout& P,
                       hipStream_t st) {
  const int H = s.H, I = s.I, E = s.E;
  const KSplit kg = ksplit_for(H / kGroup), kd = ksplit_for(I / kGroup);
  hipError_t err;
  size_t n = (size_t)E * (2 * I / 64) * (H / kGroup) * kWave;
  hipLaunchKernelGGL(k_pack_codes<true>, dim3(grid_for(n)), dim3(256), 0, st, w13_q, gu_codes_bytes(H, I), packed + P.gu_q,
                     P.gu_q_stride, E, 2 * I, H, 1, I);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  n = (size_t)E * (2 * I / 64) * (H / kGroup / kg.P) * kWave;
  hipLaunchKernelGGL(k_pack_scales<uint16_t>, dim3(grid_for(n)), dim3(256), 0, st, w13_s, gu_scales_bytes(H, I) / 2,
                     reinterpret_cast<uint16_t*>(packed + P.gu_s), P.gu_s_stride / 2, E, 2 * I, H, 1, I, kg.P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  n = (size_t)E * (H / 64) * (I / kGroup) * kWave;
  hipLaunchKernelGGL(k_pack_codes<true>, dim3(grid_for(n)), dim3(256), 0, st, w2_q, dn_codes_bytes(H, I), packed + P.dn_q,
                     P.dn_q_stride, E, H, I, 0, I);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  n = (size_t)E * (H / 64) * (I / kGroup / kd.P) * kWave;
  hipLaunchKernelGGL(k_pack_scales<uint16_t>, dim3(grid_for(n)), dim3(256), 0, st, w2_s, dn_scales_bytes(H, I) / 2,
                     reinterpret_cast<uint16_t*>(packed + P.dn_s), P.dn_s_stride / 2, E, H, I, 0, I, kd.P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  uint32_t* meta = reinterpret_cast<uint32_t*>(packed + P.meta);
  if ((err = launch_fill_zero(meta, (size_t)E * kMetaWords * 4, st)) != hipSuccess) return err;
  hipLaunchKernelGGL(k_pack_meta_gu, dim3((I + kWavesPerBlock - 1) / kWavesPerBlock, E), dim3(256), 0, st, w13_q,
                     w13_s, meta, H, I);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_pack_meta_dn, dim3((H + kWavesPerBlock - 1) / kWavesPerBlock, E), dim3(256), 0, st, w2_q, w2_s,
                     meta, H, I);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (s.has_shared) {
    n = (size_t)(2 * I / 64) * (H / 8) * kWave;
    hipLaunchKernelGGL(k_pack_bf16, dim3(grid_for(n)), dim3(256), 0, st, sh_w13,
                       reinterpret_cast<uint16_t*>(packed + P.sh_gu), 2 * I, H, 1, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    n = (size_t)(H / 64) * (I / 8) * kWave;
    hipLaunchKernelGGL(k_pack_bf16, dim3(grid_for(n)), dim3(256), 0, st, sh_w2,
                       reinterpret_cast<uint16_t*>(packed + P.sh_dn), H, I, 0, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16, tail = bytes % 16;
  hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(n16)), dim3(256), 0, st, reinterpret_cast<uint4*>(p), n16,
                     reinterpret_cast<uint8_t*>(p) + n16 * 16, tail);
  return hipGetLastError();
}

// MXFP4 routed experts into the same tiles (codes as stored, E8M0 scale
// bytes packed like the bf16 scales); the shared BF16 expert as for INT4.
// The range data of the many-token path is left zero: the MXFP4 layout
// serves the one-launch layer only.
hipError_t launch_pack_mxfp4(const Shape& s, const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                             const uint8_t* w2_s, const uint16_t* sh_w13, const uint16_t* sh_w2, uint8_t* packed,
                             const PackedLayout& P, hipStream_t st) {
  const int H = s.H, I = s.I, E = s.E;
  const KSplit kg = ksplit_for(H / kGroup), kd = ksplit_for(I / kGroup);
  hipError_t err;
  size_t n = (size_t)E * (2 * I / 64) * (H / kGroup) * kWave;
  hipLaunchKernelGGL(k_pack_codes<false>, dim3(grid_for(n)), dim3(256), 0, st, w13_q, gu_codes_bytes(H, I),
                     packed + P.gu_q, P.gu_q_stride, E, 2 * I, H, 1, I);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  n = (size_t)E * (2 * I / 64) * (H / kGroup / kg.P) * kWave;
  hipLaunchKernelGGL(k_pack_scales<uint8_t>, dim3(grid_for(n)), dim3(256), 0, st, w13_s, gu_scales_bytes(H, I, 1),
                     packed + P.gu_s, P.gu_s_stride, E, 2 * I, H, 1, I, kg.P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  n = (size_t)E * (H / 64) * (I / kGroup) * kWave;
  hipLaunchKernelGGL(k_pack_codes<false>, dim3(grid_for(n)), dim3(256), 0, st, w2_q, dn_codes_bytes(H, I),
                     packed + P.dn_q, P.dn_q_stride, E, H, I, 0, I);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  n = (size_t)E * (H / 64) * (I / kGroup / kd.P) * kWave;
  hipLaunchKernelGGL(k_pack_scales<uint8_t>, dim3(grid_for(n)), dim3(256), 0, st, w2_s, dn_scales_bytes(H, I, 1),
                     packed + P.dn_s, P.dn_s_stride, E, H, I, 0, I, kd.P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = launch_fill_zero(packed + P.meta, (size_t)E * kMetaWords * 4, st)) != hipSuccess) return err;
  if (s.has_shared) {
    n = (size_t)(2 * I / 64) * (H / 8) * kWave;
    hipLaunchKernelGGL(k_pack_bf16, dim3(grid_for(n)), dim3(256), 0, st, sh_w13,
                       reinterpret_cast<uint16_t*>(packed + P.sh_gu), 2 * I, H, 1, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    n = (size_t)(H / 64) * (I / 8) * kWave;
    hipLaunchKernelGGL(k_pack_bf16, dim3(grid_for(n)), dim3(256), 0, st, sh_w2,
                       reinterpret_cast<uint16_t*>(packed + P.sh_dn), H, I, 0, I);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
