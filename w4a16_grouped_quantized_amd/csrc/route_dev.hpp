// route_dev.hpp — device code shared by the small-M router kernels: the
// launch arguments and the per-token top-k selection with softmax weights.
#pragma once
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

// The largest value with zero low 16 bits that at least k lanes' keys reach
// (keys of absent lanes are 0): a lower bound of the k-th largest key, within
// its 16-bit prefix.  Two bits per step: the three candidate values of a step
// are counted with independent ballots.
__device__ __forceinline__ uint32_t kth_largest_lane_prefix(uint32_t key, int k) {
  uint32_t thr = 0;
#pragma unroll
  for (int b = 30; b >= 16; b -= 2) {
    const uint32_t c1 = thr | (1u << b), c2 = thr | (2u << b), c3 = thr | (3u << b);
    const int n1 = __popcll(__ballot(key >= c1));
    const int n2 = __popcll(__ballot(key >= c2));
    const int n3 = __popcll(__ballot(key >= c3));
    thr = n3 >= k ? c3 : n2 >= k ? c2 : n1 >= k ? c1 : thr;
  }
  return thr;
}

// Top-k of logits[0..E) for one token, by one wavefront (E <= 512: lane l
// holds experts l + 64*j as order-preserving keys).
//  1. Prune: the k-th largest of the 64 lane maxima is at most the k-th
//     largest logit (those k maxima are k distinct logits), so only logits
//     at or above it can win.  The bound used is that value with its low 16
//     bits cleared; typically about k logits survive.
//  2. If more than 64 survive (heavy ties), select exactly instead: the k-th
//     largest key bit by bit over all keys, every key above it, and the
//     lowest ids among the keys equal to it.
//  3. The survivors are gathered into LDS slots 0..C-1; lane c < C ranks
//     survivor c by (key desc, id asc) against all of them (read four at a
//     time at wavefront-uniform addresses); ranks 0..k-1 are the result, in
//     that order.
// The selection itself on keys held in registers (key[j] of expert
// lane + 64*j; absent entries are not present).  Lanes < k return the id and
// softmax weight of rank `lane` (the weight only with want_w; 0 otherwise).
constexpr int kTopkEPL = kMaxExperts / kWave;
__device__ __forceinline__ void topk_select_general(const uint32_t (&key)[kTopkEPL], const bool (&present)[kTopkEPL],
                                                    int k, int lane, int* lds, int& out_id, float& out_w,
                                                    bool want_w = true) {
  constexpr int EPL = kTopkEPL;
  uint32_t lmax = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) lmax = (present[j] && key[j] > lmax) ? key[j] : lmax;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint32_t thr0 = kth_largest_lane_prefix(lmax, k);
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
      if (cnt >= k) thr = cb;
    }
    int room = k;
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
    C = k;
  }
  // gather the C candidates into LDS slots 0..C-1
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
  for (int c0 = 0; c0 < C; c0 += 4) {
    const uint4 k4 = *reinterpret_cast<const uint4*>(lkey + c0);
    const int4 i4 = *reinterpret_cast<const int4*>(lid + c0);
    const uint32_t ok[4] = {k4.x, k4.y, k4.z, k4.w};
    const int oi[4] = {i4.x, i4.y, i4.z, i4.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      rank += (c0 + q < C && (ok[q] > mk || (ok[q] == mk && oi[q] < mi))) ? 1 : 0;
  }
  if (lane < C && rank < k) lorder[rank] = lane;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const int src = lane < k ? lorder[lane] : 0;
  const uint32_t rk = lkey[src];
  const int ri = lid[src];
  out_id = ri;
  if (!want_w) {  // the ids alone
    out_w = 0.f;
    return;
  }
  const float v = lane < k ? key_value(rk) : 0.f;
  const float vmax = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float ex = lane < k ? expf(v - vmax) : 0.f;
  float sum = ex;
  if (k <= 8) {  // lanes 0..7 hold the k terms
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) sum += __shfl_xor(sum, off, 64);
  } else {
    sum = wave_sum(ex);
  }
  out_w = ex / sum;
}

// The same selection for k <= 8, in few dependent steps (the general one
// spends most of its time in serialised ballot and LDS round trips).
//  1. Threshold: the smallest of the eight group maxima (lanes 8g .. 8g+7,
//     all their keys): every group holds a key at or above it, so at least
//     eight keys reach it (about twelve for N(0, 1) logits).  Lane maxima
//     with max3, group maxima with three DPP steps, their minimum on the
//     scalar unit.
//  2. The candidates (keys at or above it) go to LDS as 64-bit composites
//     (key << 32 | 0xFFFF - id): the larger composite is the larger key,
//     then the lower id.  All eight ballots are taken before any position,
//     and every lane writes (non-candidates to a slot of their own), so no
//     step waits on the previous one.  More than 64 candidates (heavy
//     ties): the general selection.
//  3. Candidate c's rank is the number of larger composites, read sixteen
//     at a time; ranks below k are the result, in order.
//  4. The weights' sum runs over the same pairs as in the general selection
//     (lanes 1, 2 and 4 apart), through DPP instead of LDS shuffles; the
//     sums are the same bits.
// The LDS area takes kTopkLdsInts ints per wavefront.
constexpr int kTopkLdsInts = 288;  // 128 candidate slots + 16 result slots, 8 bytes each
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
__device__ __forceinline__ void topk_select_small(const uint32_t (&key)[kTopkEPL], const bool (&present)[kTopkEPL], int k,
                                                  int lane, int* lds, int& out_id, float& out_w, bool want_w = true) {
  constexpr int EPL = kTopkEPL;
  uint32_t kv[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) kv[j] = present[j] ? key[j] : 0u;
  uint32_t m = kv[0];
#pragma unroll
  for (int j = 1; j < EPL; ++j) m = max(m, kv[j]);
  m = max(m, dpp_u32<kDppXor1>(m));
  m = max(m, dpp_u32<kDppXor2>(m));
  m = max(m, dpp_u32<kDppHalfMirror>(m));
  uint32_t gmax[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) gmax[g] = (uint32_t)__builtin_amdgcn_readlane((int)m, 8 * g);
  const uint32_t thr = min(min(min(gmax[0], gmax[1]), min(gmax[2], gmax[3])), min(min(gmax[4], gmax[5]), min(gmax[6], gmax[7])));
  bool c[EPL];
  uint64_t b[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    c[j] = present[j] && kv[j] >= thr;
    b[j] = __ballot(c[j]);
  }
  int pre[EPL + 1];
  pre[0] = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) pre[j + 1] = pre[j] + __popcll(b[j]);
  const int C = pre[EPL];
  if (C > kWave) {  // heavy ties: the general selection
    topk_select_general(key, present, k, lane, lds, out_id, out_w, want_w);
    return;
  }
  uint64_t* cand = reinterpret_cast<uint64_t*>(lds);  // [0, 64) candidates, [64, 128) discarded writes
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b[j] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b[j], 0u));
    cand[c[j] ? pre[j] + below : kWave + lane] = ((uint64_t)kv[j] << 32) | (uint32_t)(0xFFFF - (lane + kWave * j));
  }
  // zeros after the C candidates up to the next multiple of 16 (a zero is
  // below every candidate: keys are never 0), so the ranking below reads
  // whole blocks of 16 without a bound check per entry
  if (lane < 16) cand[C + lane] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const uint64_t mine = cand[lane];
  int rank = 0;
  for (int i0 = 0; i0 < C; i0 += 16) {
    ulonglong2 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = reinterpret_cast<const ulonglong2*>(cand)[i0 / 2 + q];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      rank += v[q].x > mine ? 1 : 0;
      rank += v[q].y > mine ? 1 : 0;
    }
  }
  uint64_t* res = cand + 2 * kWave;
  if (lane < C && rank < k) res[rank] = mine;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const uint64_t r = res[lane < k ? lane : 0];
  out_id = 0xFFFF - (int)(uint32_t)(r & 0xFFFFu);
  if (!want_w) {
    out_w = 0.f;
    return;
  }
  const float v = lane < k ? key_value((uint32_t)(r >> 32)) : 0.f;
  const float vmax = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float ex = lane < k ? expf(v - vmax) : 0.f;
  float sum = ex + dpp_f32<kDppXor1>(ex);
  sum = sum + dpp_f32<kDppXor2>(sum);
  sum = sum + dpp_f32<kDppHalfMirror>(sum);
  out_w = ex / sum;
}

// The top-k selection every path uses: the small-k form for k <= 8, else
// the general one.  lds: kTopkLdsInts ints of this wavefront.
__device__ __forceinline__ void topk_select(const uint32_t (&key)[kTopkEPL], const bool (&present)[kTopkEPL], int k,
                                            int lane, int* lds, int& out_id, float& out_w, bool want_w = true) {
  if (k <= 8) topk_select_small(key, present, k, lane, lds, out_id, out_w, want_w);
  else topk_select_general(key, present, k, lane, lds, out_id, out_w, want_w);
}

// Top-k of logits[t][0..E) (fp32, written by the other workgroups of the
// launch before their arrival); stores ids and weights of token t.
__device__ __forceinline__ void topk_token(const RouteArgs& a, int t, int lane, int* lds) {
  uint32_t key[kTopkEPL];
  bool present[kTopkEPL];
#pragma unroll
  for (int j = 0; j < kTopkEPL; ++j) {
    const int e = lane + kWave * j;
    present[j] = e < a.E;
    key[j] = present[j] ? sort_key(ld_fresh(&a.logits[(size_t)t * a.E + e])) : 0u;
  }
  int id;
  float w;
  topk_select(key, present, a.k, lane, lds, id, w);
  if (lane < a.k) {
    st_coherent(&a.ids[(size_t)t * a.k + lane], id);
    st_coherent(&a.w[(size_t)t * a.k + lane], w);
  }
}

// The RMSNorm divisor of a token from its sum of squares (unit gain).
__device__ __forceinline__ float rms_divisor(float ss, int H, float eps) { return sqrtf(ss / (float)H + eps); }

// Lane l's inputs 256*i + 4*l .. +3 of a token row, as bf16 pairs.
template <int NI>
__device__ __forceinline__ void fetch_token(const uint16_t* __restrict__ xt, int lane, uint2 (&packed)[NI]) {
#pragma unroll
  for (int i = 0; i < NI; ++i) packed[i] = *reinterpret_cast<const uint2*>(xt + 256 * i + 4 * lane);
}

// The second half of load_token: `packed` (as fetched) to floats, normalised
// when asked (then `packed` is rewritten with the normalised bf16 values).
template <int NI>
__device__ __forceinline__ void decode_token(int H, bool rmsnorm, float eps, float (&xv)[NI][4], uint2 (&packed)[NI]) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint2 v = packed[i];
    xv[i][0] = __uint_as_float(v.x << 16);
    xv[i][1] = __uint_as_float(v.x & 0xFFFF0000u);
    xv[i][2] = __uint_as_float(v.y << 16);
    xv[i][3] = __uint_as_float(v.y & 0xFFFF0000u);
  }
  if (!rmsnorm) return;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) ss = fmaf(xv[i][q], xv[i][q], ss);
  ss = wave_sum_dpp(ss);
  // x / d as x * (1 / d): within about one fp32 ulp of the quotient, so the
  // bf16 result is the correctly rounded one or its neighbour
  const float rd = 1.0f / rms_divisor(ss, H, eps);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t lo = f32x2_to_bf16x2(xv[i][0] * rd, xv[i][1] * rd);
    const uint32_t hi = f32x2_to_bf16x2(xv[i][2] * rd, xv[i][3] * rd);
    xv[i][0] = __uint_as_float(lo << 16);
    xv[i][1] = __uint_as_float(lo & 0xFFFF0000u);
    xv[i][2] = __uint_as_float(hi << 16);
    xv[i][3] = __uint_as_float(hi & 0xFFFF0000u);
    packed[i].x = lo;
    packed[i].y = hi;
  }
}

// One wavefront's view of token t: lane l holds inputs 256*i + 4*l .. +3 as
// float (raw, or RMS-normalised and rounded to bf16); `packed` receives the
// same values as bf16 pairs.  The sum of squares runs in a fixed order
// (i, then the 4 inputs, then wave_sum_dpp), so every wavefront that
// calls this gets the same bits.
template <int NI>
__device__ __forceinline__ void load_token(const uint16_t* __restrict__ xt, int H, int lane, bool rmsnorm, float eps,
                                           float (&xv)[NI][4], uint2 (&packed)[NI]) {
  fetch_token<NI>(xt, lane, packed);
  decode_token<NI>(H, rmsnorm, eps, xv, packed);
}

// Logits of router row e for every token (one wavefront, rows past E load
// row E-1 and store nothing).  The row stays in registers while the
// wavefront walks the tokens, whose inputs are fetched kRouteBatch at a time
// (one memory round trip per batch); `writer` also stores the normalised
// tokens.
// With keys, each logit is stored as its order-preserving key (never 0)
// instead of into a.logits.
template <int NI>
__device__ __forceinline__ void router_row(const RouteArgs& a, int e, int lane, bool writer, uint32_t* keys = nullptr) {
  const bool has_row = e < a.E;
  const int er = has_row ? e : a.E - 1;
  constexpr int kRouteBatch = 4;
  // the first batch of tokens is requested with the router row (one round
  // trip for both; inside the token loop it would follow the row)
  uint2 batch[kRouteBatch][NI];
#pragma unroll
  for (int b = 0; b < kRouteBatch; ++b)
    if (b < a.M) fetch_token<NI>(a.x + (size_t)b * a.H, lane, batch[b]);
  float4 wr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) wr[i] = ld_stream_f4(a.wr + (size_t)er * a.H + 256 * i + 4 * lane);
  for (int t0 = 0; t0 < a.M; t0 += kRouteBatch) {
    if (t0 > 0) {
#pragma unroll
      for (int b = 0; b < kRouteBatch; ++b)
        if (t0 + b < a.M) fetch_token<NI>(a.x + (size_t)(t0 + b) * a.H, lane, batch[b]);
    }
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
      const int t = t0 + b;
      if (t >= a.M) break;
      float xv[NI][4];
      uint2 (&packed)[NI] = batch[b];
      decode_token<NI>(a.H, a.rmsnorm != 0, a.eps, xv, packed);
      if (a.rmsnorm && writer) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          *reinterpret_cast<uint2*>(a.x_norm + (size_t)t * a.H + 256 * i + 4 * lane) = packed[i];
      }
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        acc = fmaf(wr[i].x, xv[i][0], acc);
        acc = fmaf(wr[i].y, xv[i][1], acc);
        acc = fmaf(wr[i].z, xv[i][2], acc);
        acc = fmaf(wr[i].w, xv[i][3], acc);
      }
      acc = wave_sum_dpp(acc);
      if (has_row && lane == 0) {
        if (keys) {
          const uint32_t key = sort_key(acc);  // 0 only for one NaN pattern: stored as the lowest key instead
          st_coherent(reinterpret_cast<int32_t*>(&keys[(size_t)t * a.E + e]), (int32_t)(key ? key : 1u));
        }
        else st_coherent(&a.logits[(size_t)t * a.E + e], acc);
      }
    }
  }
}

}  // namespace moe
