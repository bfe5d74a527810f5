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

// k-th largest of one 32-bit key per lane (keys of absent lanes are 0),
// found bit by bit from the top with one ballot per bit.
__device__ __forceinline__ uint32_t kth_largest_lane_key(uint32_t key, int k) {
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    if (__popcll(__ballot(key >= cand)) >= k) thr = cand;
  }
  return thr;
}

// Top-k of logits[0..E) for one token, by one wavefront (E <= 512: lane l
// holds experts l + 64*j as order-preserving keys).
//  1. Prune: the k-th largest of the 64 lane maxima is at most the k-th
//     largest logit (those k maxima are k distinct logits), so only logits
//     at or above it can win; typically about k of them survive.
//  2. If more than 64 survive (heavy ties), select exactly instead: the k-th
//     largest key bit by bit over all keys, every key above it, and the
//     lowest ids among the keys equal to it.
//  3. The survivors are gathered into lanes 0..C-1 and ranked by
//     (key desc, id asc); ranks 0..k-1 are the result, in that order.
__device__ void topk_token(const RouteArgs& a, int t, int lane, int* lds) {
  constexpr int EPL = kMaxExperts / kWave;
  uint32_t key[EPL];
  bool present[EPL];
  float val[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + kWave * j;
    present[j] = e < a.E;
    val[j] = present[j] ? ld_coherent(&a.logits[(size_t)t * a.E + e]) : 0.f;
  }
  uint32_t lmax = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    key[j] = present[j] ? sort_key(val[j]) : 0u;  // real keys of finite logits are > 0
    lmax = key[j] > lmax ? key[j] : lmax;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint32_t thr0 = kth_largest_lane_key(lmax, a.k);
  uint32_t cand = 0;
  int C = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const bool c = present[j] && key[j] >= thr0;
    cand |= (uint32_t)c << j;
    C += __popcll(__ballot(c));
  }
  if (C > kWave) {
    // exact selection of exactly k entries
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cb = thr | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) cnt += __popcll(__ballot(present[j] && key[j] >= cb));
      if (cnt >= a.k) thr = cb;
    }
    int room = a.k;
#pragma unroll
    for (int j = 0; j < EPL; ++j) room -= __popcll(__ballot(present[j] && key[j] > thr));
    cand = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {  // ascending j, then lane: ascending id
      const bool eq = present[j] && key[j] == thr;
      const uint64_t eb = __ballot(eq);
      const bool take = (present[j] && key[j] > thr) || (eq && __popcll(eb & lt) < room);
      cand |= (uint32_t)take << j;
      room -= __popcll(eb);
      if (room < 0) room = 0;
    }
    C = a.k;
  }
  // gather the C candidates into lanes 0..C-1 (through LDS)
  uint32_t* lkey = reinterpret_cast<uint32_t*>(lds);
  int* lid = lds + kWave;
  int* lorder = lds + 2 * kWave;
  int base = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const bool c = (cand >> j) & 1u;
    const uint64_t bal = __ballot(c);
    if (c) {
      const int pos = base + __popcll(bal & lt);
      lkey[pos] = key[j];
      lid[pos] = lane + kWave * j;
    }
    base += __popcll(bal);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const uint32_t mk = lane < C ? lkey[lane] : 0u;
  const int mi = lane < C ? lid[lane] : 0x7FFFFFFF;
  int rank = 0;
  for (int c = 0; c < C; ++c) {
    const uint32_t ok = (uint32_t)__builtin_amdgcn_readlane((int)mk, c);
    const int oi = __builtin_amdgcn_readlane(mi, c);
    rank += (ok > mk || (ok == mk && oi < mi)) ? 1 : 0;
  }
  if (lane < C && rank < a.k) lorder[rank] = lane;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const int src = lane < a.k ? lorder[lane] : 0;
  const uint32_t rk = __shfl(mk, src, 64);
  const int ri = __shfl(mi, src, 64);
  const float v = lane < a.k ? key_value(rk) : 0.f;
  const float vmax = __shfl(v, 0, 64);
  const float ex = lane < a.k ? expf(v - vmax) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < a.k) {
    a.ids[(size_t)t * a.k + lane] = ri;
    a.w[(size_t)t * a.k + lane] = ex / sum;
  }
}

template <int NI>
__global__ __launch_bounds__(kBlock) void k_route(const RouteArgs a) {
  __shared__ int flag;
  __shared__ int topk_lds[kWavesPerBlock][3 * kMaxTopK];
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
    if (has_row && lane == 0) st_coherent(&a.logits[(size_t)t * a.E + e], acc);
  }
  if (!arrive_last(a.cnt, gridDim.x, &flag)) return;
  for (int t = wave; t < a.M; t += kWavesPerBlock) topk_token(a, t, lane, topk_lds[wave]);
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
