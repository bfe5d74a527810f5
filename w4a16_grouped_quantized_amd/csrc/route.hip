// route.hip — router GEMV, top-k selection and softmax weights (one launch).
//
// Each wavefront owns one router row (fp32, H inputs): lane l holds inputs
// 256*i + 4*l .. +3 for i < H/256, so every wavefront load of a row is one
// contiguous KiB.  The row stays in registers while the wavefront walks the
// tokens; per token the 4*H/256 products of a lane are summed in order and
// the lanes are combined by a fixed xor butterfly (a tree, not one long
// serial sum).  The workgroup that finishes last selects, per token, the k
// largest logits (ties -> lower expert id) and writes the softmax over them.
// With MOE_F_INPUT_RMSNORM each wavefront first normalises the token
// (unit-gain RMSNorm, rounded to bf16) and workgroup 0 stores the result.
#include "launch.hpp"

namespace moe {

struct RouteArgs {
  int M, E, k, H;
  int rmsnorm;
  float eps;
  const float* __restrict__ wr;
  const uint16_t* __restrict__ x;
  uint16_t* __restrict__ x_norm;
  float* __restrict__ logits;  // [M][E]
  int32_t* __restrict__ cnt;
  int32_t* __restrict__ ids;
  float* __restrict__ w;
};

// Order-preserving map of a float to an unsigned key (larger float, larger key).
__device__ __forceinline__ uint32_t sort_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Top-k of logits[0..E) for one token, by one wavefront.  E <= 512: lane l
// holds experts l + 64*j.
__device__ void topk_token(const RouteArgs& a, int t, int lane) {
  constexpr int EPL = kMaxExperts / kWave;
  uint32_t key[EPL];
  uint32_t avail = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + kWave * j;
    key[j] = 0;
    if (e < a.E) {
      key[j] = sort_key(a.logits[(size_t)t * a.E + e]);
      avail |= 1u << j;
    }
  }
  uint32_t sel_key = 0;
  int sel_id = 0;
  for (int r = 0; r < a.k; ++r) {
    uint32_t bk = 0;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      // ascending j means ascending id inside a lane: strict > keeps the lower id
      if (((avail >> j) & 1u) && (bi == 0x7FFFFFFF || key[j] > bk)) { bk = key[j]; bi = lane + kWave * j; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t ok = __shfl_xor(bk, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ok > bk || (ok == bk && oi < bi)) { bk = ok; bi = oi; }
    }
    if ((bi & (kWave - 1)) == lane) avail &= ~(1u << (bi / kWave));
    if (lane == r) { sel_key = bk; sel_id = bi; }
  }
  const float v = lane < a.k ? key_value(sel_key) : 0.f;
  const float vmax = __shfl(v, 0, 64);
  const float ex = lane < a.k ? expf(v - vmax) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < a.k) {
    a.ids[(size_t)t * a.k + lane] = sel_id;
    a.w[(size_t)t * a.k + lane] = ex / sum;
  }
}

template <int NI>
__global__ __launch_bounds__(kBlock) void k_route(const RouteArgs a) {
  __shared__ int flag;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = blockIdx.x * kWavesPerBlock + wave;
  const bool has_row = e < a.E;
  const int er = has_row ? e : a.E - 1;  // rows past E load row E-1 and are discarded
  float4 wr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) wr[i] = *reinterpret_cast<const float4*>(a.wr + (size_t)er * a.H + 256 * i + 4 * lane);
  const bool writer = blockIdx.x == 0 && wave == 0;
  for (int t = 0; t < a.M; ++t) {
    const uint16_t* xt = a.x + (size_t)t * a.H;
    float xv[NI][4];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint2 v = *reinterpret_cast<const uint2*>(xt + 256 * i + 4 * lane);
      xv[i][0] = __uint_as_float(v.x << 16);
      xv[i][1] = __uint_as_float(v.x & 0xFFFF0000u);
      xv[i][2] = __uint_as_float(v.y << 16);
      xv[i][3] = __uint_as_float(v.y & 0xFFFF0000u);
    }
    if (a.rmsnorm) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) ss = fmaf(xv[i][q], xv[i][q], ss);
      ss = wave_sum(ss);
      const float d = sqrtf(ss / (float)a.H + a.eps);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        uint16_t bq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bq[q] = f32_to_bf16(xv[i][q] / d);
          xv[i][q] = bf16_to_f32(bq[q]);
        }
        if (writer) {
          uint2 o;
          o.x = (uint32_t)bq[0] | ((uint32_t)bq[1] << 16);
          o.y = (uint32_t)bq[2] | ((uint32_t)bq[3] << 16);
          *reinterpret_cast<uint2*>(a.x_norm + (size_t)t * a.H + 256 * i + 4 * lane) = o;
        }
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      acc = fmaf(wr[i].x, xv[i][0], acc);
      acc = fmaf(wr[i].y, xv[i][1], acc);
      acc = fmaf(wr[i].z, xv[i][2], acc);
      acc = fmaf(wr[i].w, xv[i][3], acc);
    }
    acc = wave_sum(acc);
    if (has_row && lane == 0) a.logits[(size_t)t * a.E + e] = acc;
  }
  if (!arrive_last(a.cnt, gridDim.x, &flag)) return;
  for (int t = wave; t < a.M; t += kWavesPerBlock) topk_token(a, t, lane);
}

namespace {
template <int NI>
hipError_t run_route(const RouteArgs& a, hipStream_t st) {
  const int grid = (a.E + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((k_route<NI>), dim3(grid), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}
}  // namespace

bool route_supported(const Shape& s) { return s.H == 2560 || s.H == 256; }

hipError_t launch_route(const Shape& s, const float* router_w, const uint16_t* x, int M,
                        bool rmsnorm, float eps, uint16_t* x_norm, int32_t* ids, float* w,
                        uint8_t* ws, const WsLayout& L, hipStream_t st) {
  RouteArgs a;
  a.M = M; a.E = s.E; a.k = s.k; a.H = s.H;
  a.rmsnorm = rmsnorm ? 1 : 0;
  a.eps = eps;
  a.wr = router_w; a.x = x; a.x_norm = x_norm;
  a.logits = reinterpret_cast<float*>(ws + L.logits);
  a.cnt = reinterpret_cast<int32_t*>(ws + L.route_cnt);
  a.ids = ids; a.w = w;
  if (s.H == 2560) return run_route<10>(a, st);
  if (s.H == 256) return run_route<1>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
