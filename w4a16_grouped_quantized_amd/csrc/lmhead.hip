// lmhead.hip — the LM head as FP8: one-time quantisation of the BF16 head
// and the per-token GEMV (bpdata.com Ling-3.0-flash MoE article,
// "Optimalizáció 2": the head is converted from BF16 to FP8 when it is
// assembled, which roughly halves the bytes the layer reads per token; the
// model section gives its shape, hidden 2,560 onto a 157,184-token
// vocabulary).
//
// Format (the pages leave it open): E4M3 codes [V][H] (the OCP 8-bit float:
// bias 7, largest finite 448, no infinities) and one float32 scale per row,
// s = amax / 448; q = round-to-nearest-even(w / s), saturating at +-448.
//
// The GEMV is bound by the 402 MB (FP8) or 805 MB (BF16) of head bytes read
// per call.  A wavefront takes two rows at a time: 2 * H bytes as 16-byte
// lane loads (five per lane at H = 2560, 1 KB contiguous per load), so a
// lane's input columns are the same for every row pair it visits and the
// token's inputs stay in registers for the whole launch.  Rows are dealt to
// the grid's wavefronts in turn, and each wavefront requests the next pair
// before computing the current one.  FP8 codes are widened to exact BF16
// pairs by the part's scaled converter (scale 1) and multiplied with
// v_dot2_f32_bf16; the row scale is applied to the fp32 sum.
#include <algorithm>

#include "launch.hpp"

namespace moe {

namespace {

// Round-to-nearest-even of a finite float32 to E4M3 (the magnitude code; the
// caller adds the sign): codes are consecutive along the value axis, so the
// code of a normal value is its exponent field times 8 plus its rounded
// 3-bit mantissa, and a mantissa that rounds up to 16 carries into the next
// exponent by itself.
__device__ __forceinline__ uint32_t e4m3_magnitude_code(float a) {
  if (a != a) return 0x7F;          // NaN
  if (!(a < 448.0f)) return 0x7E;  // saturate (448 and beyond)
  if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);  // subnormal steps of 2^-9 (8 -> 2^-6)
  const int e = (int)((__float_as_uint(a) >> 23) & 255u) - 127;    // -6 .. 8
  const uint32_t mq = (uint32_t)__builtin_rintf(ldexpf(a, 3 - e));  // 8 .. 16
  return (uint32_t)((e + 7) << 3) + mq - 8u;
}

__device__ __forceinline__ uint32_t e4m3_code(float v) {
  return (__float_as_uint(v) >> 31 << 7) | e4m3_magnitude_code(fabsf(v));
}

// One wavefront per row: amax over the row, the scale, the codes.
__global__ __launch_bounds__(256) void k_lmhead_quant(const uint16_t* __restrict__ w, int V, int H,
                                                      uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= V) return;
  const uint4* wr = reinterpret_cast<const uint4*>(w + (size_t)row * H);
  const int nc = H / 8;  // 8 bf16 per 16-byte chunk
  float amax = 0.f;
  for (int c = lane; c < nc; c += kWave) {
    const uint4 v = wr[c];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(__uint_as_float(d[i] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(d[i] & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (lane == 0) scale[row] = s;
  uint2* qr = reinterpret_cast<uint2*>(q + (size_t)row * H);
  for (int c = lane; c < nc; c += kWave) {
    const uint4 v = wr[c];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint32_t code[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      code[2 * i] = e4m3_code(__fdiv_rn(__uint_as_float(d[i] << 16), s));
      code[2 * i + 1] = e4m3_code(__fdiv_rn(__uint_as_float(d[i] & 0xFFFF0000u), s));
    }
    qr[c] = make_uint2(code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24,
                       code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24);
  }
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a), __builtin_bit_cast(bf16x2_v, b), c, false);
}
// Two E4M3 codes (bytes 0,1 or, with HI, 2,3 of v) as an exact bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v, 1.0f, HI));
}

// FP8: a 16-byte chunk is 16 codes (input columns 16c .. 16c+15), its token
// inputs 8 bf16 pairs.  BF16: a chunk is 8 weights, 4 input pairs.
template <bool FP8>
struct Head {
  static constexpr int kPerChunk = FP8 ? 16 : 8;  // columns per chunk
  static constexpr int kXw = kPerChunk / 2;        // input dwords per chunk
  __device__ static __forceinline__ float dot(uint4 w, const uint32_t* x, float acc) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
    if constexpr (FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = dot2(fp8x2_bf16<false>(d[i]), x[2 * i], acc);
        acc = dot2(fp8x2_bf16<true>(d[i]), x[2 * i + 1], acc);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = dot2(d[i], x[i], acc);
    }
    return acc;
  }
};

// logits[t][v] (fp32) for M tokens, NCH chunks per lane per row pair.
template <bool FP8, int NCH, int M>
__global__ __launch_bounds__(256) void k_lmhead_gemv(const uint8_t* __restrict__ wq, const float* __restrict__ scale,
                                                     int V, int H, const uint16_t* __restrict__ x,
                                                     float* __restrict__ logits) {
  typedef Head<FP8> Hd;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nwv = gridDim.x * 4;
  const int rowbytes = FP8 ? H : 2 * H;
  const int CR = rowbytes / 16;  // chunks per row
  const int npairs = (V + 1) / 2;
  // this lane's chunks of a row pair: c = lane + 64 i, row c >= CR
  uint32_t xr[M][NCH][Hd::kXw];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + kWave * i;
    const int cc = c < CR ? c : c - CR;
#pragma unroll
    for (int t = 0; t < M; ++t) {
      const uint32_t* xs = reinterpret_cast<const uint32_t*>(x + (size_t)t * H) + cc * Hd::kXw;
#pragma unroll
      for (int j = 0; j < Hd::kXw; ++j) xr[t][i][j] = 0u;
      if (c < 2 * CR) {
#pragma unroll
        for (int j = 0; j < Hd::kXw; ++j) xr[t][i][j] = xs[j];
      }
    }
  }
  auto load = [&](uint4 (&w)[NCH], int p) {
    const uint8_t* base = wq + (size_t)p * 2 * rowbytes;
    const int nc = 2 * p + 1 < V ? 2 * CR : CR;  // the last pair of an odd V has one row
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + kWave * i;
      w[i] = c < nc ? ld_stream(base + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
    }
  };
  auto compute = [&](const uint4 (&w)[NCH], int p) {
    float acc[M][2];
#pragma unroll
    for (int t = 0; t < M; ++t) acc[t][0] = acc[t][1] = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + kWave * i;
#pragma unroll
      for (int t = 0; t < M; ++t) {
        const float d = Hd::dot(w[i], xr[t][i], 0.f);
        if (c < CR) acc[t][0] += d;
        else acc[t][1] += d;
      }
    }
#pragma unroll
    for (int t = 0; t < M; ++t)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        float v = acc[t][r];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        const int row = 2 * p + r;
        if (lane == 0 && row < V) logits[(size_t)t * V + row] = FP8 ? v * scale[row] : v;
      }
  };
  uint4 wa[NCH], wb[NCH];
  int p = gw;
  if (p < npairs) load(wa, p);
  for (; p < npairs; p += 2 * nwv) {
    const int p2 = p + nwv;
    if (p2 < npairs) load(wb, p2);
    compute(wa, p);
    if (p2 < npairs) {
      if (p2 + nwv < npairs) load(wa, p2 + nwv);
      compute(wb, p2);
    }
  }
}

// Workgroups of the GEMV: enough resident wavefronts per CU to keep the
// head streaming.
constexpr int kLmWgPerCu = 8;

int device_cus() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess)
    return 0;
  return ncu;
}

template <bool FP8, int NCH>
hipError_t gemv_m(const uint8_t* w, const float* s, int V, int H, const uint16_t* x, int M, float* out,
                  hipStream_t st) {
  const int ncu = device_cus();
  if (ncu <= 0) return hipErrorInvalidDevice;
  const int npairs = (V + 1) / 2;
  const int grid = std::max(1, std::min(ncu * kLmWgPerCu, (npairs + 3) / 4));
#define LM_M(MM)                                                                                           \
  case MM:                                                                                                 \
    hipLaunchKernelGGL((k_lmhead_gemv<FP8, NCH, MM>), dim3(grid), dim3(256), 0, st, w, s, V, H, x, out);  \
    break;
  switch (M) {
    LM_M(1)
    LM_M(2)
    LM_M(3)
    LM_M(4)
    default: return hipErrorInvalidValue;
  }
#undef LM_M
  return hipGetLastError();
}
}  // namespace

bool lmhead_supported(int H, bool fp8) {
  // a row pair in 5 (FP8) or 10 (BF16) lane loads at H = 2560, or in one
  // load per lane for small heads
  return H > 0 && H % 16 == 0 && (H == 2560 || H <= (fp8 ? 512 : 256));
}

hipError_t launch_lmhead_quant(const uint16_t* w, int V, int H, uint8_t* q, float* s, hipStream_t st) {
  if (V == 0) return hipSuccess;
  hipLaunchKernelGGL(k_lmhead_quant, dim3((V + 3) / 4), dim3(256), 0, st, w, V, H, q, s);
  return hipGetLastError();
}

hipError_t launch_lmhead_gemv(bool fp8, const uint8_t* w, const float* s, int V, int H, const uint16_t* x, int M,
                              float* out, hipStream_t st) {
  if (V == 0 || M == 0) return hipSuccess;
  const int chunks = fp8 ? H / 8 : H / 4;
  if (fp8) {
    if (chunks == 320) return gemv_m<true, 5>(w, s, V, H, x, M, out, st);
    if (chunks <= 64) return gemv_m<true, 1>(w, s, V, H, x, M, out, st);
  } else {
    if (chunks == 640) return gemv_m<false, 10>(w, s, V, H, x, M, out, st);
    if (chunks <= 64) return gemv_m<false, 1>(w, s, V, H, x, M, out, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
