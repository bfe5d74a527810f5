// experts.hip — routed INT4 and shared BF16 expert FFNs for small token
// counts (decode M = 1 and multi-token verify), plus the weighted combine.
//
// Two launches per call:
//   k_gate_up: for every distinct routed expert of the call and every 64-row
//              tile of its gate_up matrix, h = silu(W1 x) * (W3 x) for each
//              (token, slot) routed to it; the shared expert's gate_up rows
//              are extra workgroups (K split over KS workgroups, reduced by
//              the last one to arrive).
//   k_down:    for every distinct expert and 64-row tile of its down matrix,
//              the per-slot partial rows w[t][j] * (W2 h); the shared down
//              rows likewise; the last workgroup to finish a tile sums
//              out[t][n] = sum_j partial[t,j][n] + shared[t][n]
//              in a fixed order (deterministic, no float atomics).
//
// Memory shape: one wavefront lane owns one weight row; each of the 4
// wavefronts of a workgroup streams a contiguous run of K-groups with
// coalesced 16-byte loads (1 KiB per wavefront load), all issued before any
// math.  The activations of a group are wavefront-uniform and live in scalar
// registers, so the VALU work per 16-byte chunk is 12 shifts/masks and 16
// v_dot2_f32_bf16 with no cross-lane reduction.
#include "experts_dev.hpp"

namespace moe {


// --------------------------------------------------------------- gate_up

template <int GW, int P, int CW>
__global__ __launch_bounds__(kBlock) void k_gate_up(const ExpArgs a) {
  __shared__ UnitLds L;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const uint32_t magic = bf16_pair_magic();
  const int GK = a.H / kGroup;
  const int nrouted = a.S * a.Tgu;
  const int blk = blockIdx.x;
  if (blk < nrouted) {
    const int u = blk / a.Tgu, b = blk % a.Tgu;
    const Unit U = find_unit(a.ids, a.S, a.E, u, L);
    if (U.e < 0) return;
    const int e = U.e;
    uint64_t m = U.mask;
    const bool active = wave * GW < GK;
    const int g0 = active ? wave * GW : 0;
    // the first column's group corrections are requested before the weights
    int p = member_slot(a.S, 0, m, L);
    GroupBias<false> gb;
    if (tid < GK) gb.load(a.x + (size_t)(p / a.k) * a.H, tid);
    uint4 wq[GW];
    ScalePack<P> sc[GW / P];
    const uint8_t* qb = a.gu_q + (size_t)e * a.gu_q_stride + ((size_t)(b * GK + g0) * kWave + lane) * 16;
#pragma unroll
    for (int i = 0; i < GW; ++i) wq[i] = ld_stream(qb + (size_t)i * kWave * 16);
    const uint16_t* sb = a.gu_s + (size_t)e * a.gu_s_stride + ((size_t)(b * (GK / P) + g0 / P) * kWave + lane) * P;
#pragma unroll
    for (int j = 0; j < GW / P; ++j) sc[j].load(sb + (size_t)j * kWave * P);
    // one member (slot p routed to this expert): h of tile b for its token
    auto member = [&](int p) {
      const uint16_t* act = a.x + (size_t)(p / a.k) * a.H;
      if (tid < GK) L.bias[tid] = gb.value();
      lds_sync();
      L.red[wave][lane] = active ? routed_dot<GW, P, false>(wq, sc, act, L.bias, g0, magic) : 0.f;
      lds_sync();
      if (tid < 32) {
        float g = 0.f, up = 0.f;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) { g += L.red[w][tid]; up += L.red[w][tid + 32]; }
        // tile b's 32 outputs are exactly group b of h
        store_hilo(a.h + ((size_t)p * a.I + 32 * b) * 2, tid, silu_f32(g) * up);
      }
      lds_sync();
    };
    // the first member outside the loop: its products then wait for each
    // group's codes as they reach them, not for all of them at a loop entry
    member(p);
    for (int c = 1; c < U.nmem; ++c) {
      p = member_slot(a.S, c, m, L);
      if (tid < GK) gb.load(a.x + (size_t)(p / a.k) * a.H, tid);
      member(p);
    }
    return;
  }
  if constexpr (CW == 0) {
    return;  // no shared expert compiled into this variant
  } else {
    // shared expert: tile b, K slice ks
    const int idx = blk - nrouted;
    const int b = idx / a.KSgu, ks = idx % a.KSgu;
    const int c0 = (ks * kWavesPerBlock + wave) * CW;  // first 8-input chunk of this wavefront
    uint4 wc[CW];
    const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh_gu) +
                          ((size_t)(b * (a.H / 8) + c0) * kWave + lane) * 16;
#pragma unroll
    for (int c = 0; c < CW; ++c) wc[c] = ld_stream(base + (size_t)c * kWave * 16);
    for (int t = 0; t < a.M; ++t) {
      L.red[wave][lane] = shared_dot<CW, false>(wc, a.x + (size_t)t * a.H, c0);
      lds_sync();
      if (tid < kWave) {
        float part = 0.f;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) part += L.red[w][tid];
        if (a.KSgu == 1) L.red[0][tid] = part;
        else st_coherent(&a.shgu_part[(((size_t)t * a.Tgu + b) * a.KSgu + ks) * kWave + tid], part);
      }
      lds_sync();
      if (a.KSgu == 1 && tid < 32)
        store_hilo(a.h_sh + ((size_t)t * a.I + 32 * b) * 2, tid, silu_f32(L.red[0][tid]) * L.red[0][tid + 32]);
      lds_sync();
    }
    if (a.KSgu == 1) return;
    if (!arrive_last(&a.shgu_cnt[b * kCntStride], a.KSgu, &L.flag)) return;
    for (int t = wave; t < a.M; t += kWavesPerBlock) {
      float pv[kMaxKSplit];
#pragma unroll
      for (int s2 = 0; s2 < kMaxKSplit; ++s2)
        pv[s2] = s2 < a.KSgu ? ld_fresh(&a.shgu_part[(((size_t)t * a.Tgu + b) * a.KSgu + s2) * kWave + lane]) : 0.f;
      float part = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < kMaxKSplit; ++s2) part += pv[s2];
      const float up = __shfl_down(part, 32, 64);
      if (lane < 32) store_hilo(a.h_sh + ((size_t)t * a.I + 32 * b) * 2, lane, silu_f32(part) * up);
    }
  }
}

// --------------------------------------------------------------- down + combine

// out[t][n] = sum_j w[t][j] * partial[t*k+j][n] + sum_s shared_part[t][s][n],

template <int GW, int P, int CW>
__global__ __launch_bounds__(kBlock) void k_down(const ExpArgs a) {
  __shared__ UnitLds L;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const uint32_t magic = bf16_pair_magic();
  const int GK = a.I / kGroup;
  const int nrouted = a.S * a.Tdn;
  const int expected = a.S + (a.has_shared ? a.KSdn : 0);
  const int blk = blockIdx.x;
  int b;
  if (blk < nrouted) {
    const int u = blk / a.Tdn;
    b = blk % a.Tdn;
    const Unit U = find_unit(a.ids, a.S, a.E, u, L);
    if (U.e >= 0) {
      const int e = U.e;
      uint64_t m = U.mask;
      const bool active = wave * GW < GK;
      const int g0 = active ? wave * GW : 0;
      int p = member_slot(a.S, 0, m, L);
      GroupBias<true> gb;
      if (tid < GK) gb.load(a.h + (size_t)p * a.I * 2, tid);
      uint4 wq[GW];
      ScalePack<P> sc[GW / P];
      const uint8_t* qb = a.dn_q + (size_t)e * a.dn_q_stride + ((size_t)(b * GK + g0) * kWave + lane) * 16;
#pragma unroll
      for (int i = 0; i < GW; ++i) wq[i] = ld_stream(qb + (size_t)i * kWave * 16);
      const uint16_t* sb = a.dn_s + (size_t)e * a.dn_s_stride + ((size_t)(b * (GK / P) + g0 / P) * kWave + lane) * P;
#pragma unroll
      for (int j = 0; j < GW / P; ++j) sc[j].load(sb + (size_t)j * kWave * P);
      auto member = [&](int p) {
        const uint16_t* act = a.h + (size_t)p * a.I * 2;
        if (tid < GK) L.bias[tid] = gb.value();
        lds_sync();
        L.red[wave][lane] = active ? routed_dot<GW, P, true>(wq, sc, act, L.bias, g0, magic) : 0.f;
        lds_sync();
        if (tid < kWave) {
          float part = 0.f;
#pragma unroll
          for (int w = 0; w < kWavesPerBlock; ++w) part += L.red[w][tid];
          st_coherent(&a.dpart[(size_t)p * a.H + 64 * b + tid], part * a.topk_w[p]);
        }
        lds_sync();
      };
      // the first member outside the loop, as in k_gate_up
      member(p);
      for (int c = 1; c < U.nmem; ++c) {
        p = member_slot(a.S, c, m, L);
        if (tid < GK) gb.load(a.h + (size_t)p * a.I * 2, tid);
        member(p);
      }
    }
  } else if constexpr (CW == 0) {
    return;  // no shared expert compiled into this variant (never launched)
  } else {
    const int idx = blk - nrouted;
    b = idx / a.KSdn;
    const int ks = idx % a.KSdn;
    const int c0 = (ks * kWavesPerBlock + wave) * CW;
    uint4 wc[CW];
    const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh_dn) +
                          ((size_t)(b * (a.I / 8) + c0) * kWave + lane) * 16;
#pragma unroll
    for (int c = 0; c < CW; ++c) wc[c] = ld_stream(base + (size_t)c * kWave * 16);
    for (int t = 0; t < a.M; ++t) {
      L.red[wave][lane] = shared_dot<CW, true>(wc, a.h_sh + (size_t)t * a.I * 2, c0);
      lds_sync();
      if (tid < kWave) {
        float part = 0.f;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) part += L.red[w][tid];
        st_coherent(&a.shdn_part[((size_t)t * a.KSdn + ks) * a.H + 64 * b + tid], part);
      }
      lds_sync();
    }
  }
  if (!arrive_last(&a.dn_cnt[b * kCntStride], expected, &L.flag)) return;
  combine_tile(a, b, true);
}

// --------------------------------------------------------------- dispatch

namespace {
template <int GW, int P, int CW>
hipError_t run_gate_up(const ExpArgs& a, hipStream_t st) {
  const int grid = a.S * a.Tgu + (a.has_shared ? a.Tgu * a.KSgu : 0);
  hipLaunchKernelGGL((k_gate_up<GW, P, CW>), dim3(grid), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}
template <int GW, int P, int CW>
hipError_t run_down(const ExpArgs& a, hipStream_t st) {
  const int grid = a.S * a.Tdn + (a.has_shared ? a.Tdn * a.KSdn : 0);
  hipLaunchKernelGGL((k_down<GW, P, CW>), dim3(grid), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

// Compiled (GW, P, CW) triples; CW is the shared expert's chunks per
// wavefront (0 when there is no shared expert).
//  gate_up: H=2560 -> 80 groups -> GW 20, P 4, CW 20;  H=256 -> GW 2, P 2, CW 2
//  down:    I=768  -> 24 groups -> GW 6,  P 2, CW 6;   I=64  -> GW 1, P 1, CW 1
struct Variant { int GW, P, CW; };
}  // namespace

static bool gu_variant(const Shape& s, Variant& v) {
  const KSplit k = ksplit_for(s.H / kGroup);
  const SharedSplit sh = shared_gu_split(s.H);
  v = {k.GW, k.P, s.has_shared ? sh.CW : 0};
  return (v.GW == 20 && v.P == 4 && (v.CW == 0 || v.CW == 20)) || (v.GW == 2 && v.P == 2 && (v.CW == 0 || v.CW == 2));
}
static bool dn_variant(const Shape& s, Variant& v) {
  const KSplit k = ksplit_for(s.I / kGroup);
  const SharedSplit sh = shared_dn_split(s.I);
  v = {k.GW, k.P, s.has_shared ? sh.CW : 0};
  return (v.GW == 6 && v.P == 2 && (v.CW == 0 || v.CW == 6)) || (v.GW == 1 && v.P == 1 && (v.CW == 0 || v.CW == 1));
}

bool experts_supported(const Shape& s) {
  Variant a, b;
  return gu_variant(s, a) && dn_variant(s, b);
}

hipError_t launch_gate_up(const Shape& s, const uint8_t* packed, const PackedLayout& PL, const uint16_t* x,
                          int M, const int32_t* ids, uint8_t* ws, const WsLayout& L, hipStream_t st) {
  const ExpArgs a = make_expert_args(s, packed, PL, x, M, ids, nullptr, nullptr, ws, L);
  Variant gv;
  if (!gu_variant(s, gv)) return hipErrorInvalidValue;
#define GU_CASE(GW_, P_, CW_) \
  if (gv.GW == GW_ && gv.P == P_ && gv.CW == CW_) return run_gate_up<GW_, P_, CW_>(a, st);
  GU_CASE(20, 4, 0) GU_CASE(20, 4, 20) GU_CASE(2, 2, 0) GU_CASE(2, 2, 2)
#undef GU_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_down(const Shape& s, const uint8_t* packed, const PackedLayout& PL, int M,
                       const int32_t* ids, const float* w, uint16_t* out, uint8_t* ws, const WsLayout& L,
                       hipStream_t st) {
  const ExpArgs a = make_expert_args(s, packed, PL, nullptr, M, ids, w, out, ws, L);
  Variant dv;
  if (!dn_variant(s, dv)) return hipErrorInvalidValue;
#define DN_CASE(GW_, P_, CW_) \
  if (dv.GW == GW_ && dv.P == P_ && dv.CW == CW_) return run_down<GW_, P_, CW_>(a, st);
  DN_CASE(6, 2, 0) DN_CASE(6, 2, 6) DN_CASE(1, 1, 0) DN_CASE(1, 1, 1)
#undef DN_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
