// layer.hip — the small-M MoE layer (decode, verify) in one launch.
//
// The separate kernels of the small-M path (router, gate_up, down) each pay a
// launch and a drain, and the routed expert loads cannot start before the
// router's last workgroup has chosen the experts.  Here every step is a
// workgroup role of one grid, in this order:
//
//   leader          (workgroup 0) group corrections of every token (and the
//                   normalised tokens with RMSNorm); then either the top-k of
//                   every token, once all router keys have landed, or the
//                   caller's ids; the table of distinct experts ("units");
//                   then one 64-bit routing flag per routed workgroup that
//                   carries its unit's expert, first slot and weight;
//   router rows     (only when the launch routes) 4 rows each, stored as
//                   order-preserving keys that the leader polls for;
//   shared gate_up  tile x K slice of the shared expert; the last slice of a
//                   tile sums the slices into h_sh, the last tile raises the
//                   flag of every shared down workgroup;
//   routed gate_up  (unit, tile): waits for its routing flag, then h of its
//                   32 rows (and the group correction of those 32 values)
//                   for every token routed to the unit; the last tile of a
//                   unit raises the flags of that unit's down workgroups;
//   shared down     tile x K slice: weights requested at once, then waits
//                   for h_sh;
//   routed down     (unit, tile): waits for routing, requests its weights,
//                   waits for the unit's h, writes its partial rows already
//                   multiplied by the slot weight;
//   combine         the last partial of an output tile (routed or shared)
//                   sums the tile over the token's slots in slot order plus
//                   the shared rows and rounds to bf16.
//
// Waits only ever point at workgroups with smaller ids, which the hardware
// dispatches first, so every wait ends; each poll is bounded anyway and
// records bit 1 of the error word if it gives up.  Data crossing workgroups
// is stored agent-coherently (written through to memory, past the XCD's L2,
// which is not coherent with the others); a flag is raised only after the
// producer's stores have completed, and a consumer reads the data only after
// it has seen the flag, through addresses it had not touched before in this
// launch.  Activations are read by whole wavefronts at uniform addresses,
// through scalar loads (cached per XCD): so every cache line read that way
// is complete when the flag that releases its reader is raised (no line
// mixes data of producers that finish at different times).
#include "experts_dev.hpp"
#include "route_dev.hpp"

namespace moe {

struct LayerArgs {
  ExpArgs a;
  RouteArgs r;      // router part: r.ids / r.w are a.ids / a.topk_w
  int route;        // this launch computes ids and weights
  int rmsnorm;      // tokens are RMS-normalised first (only with route)
  LayerGrid g;
  uint64_t* __restrict__ flags;  // [kFlagPlanes][grid]
  uint32_t* __restrict__ rkeys;  // [M][E] router keys
  float* __restrict__ gb;        // [M][H/32] group corrections of the tokens
  float* __restrict__ hb;        // [S][hb_stride(I)] group corrections of h
  int32_t* __restrict__ hcnt;    // gate_up tiles finished per unit (kCntStride apart)
  int32_t* __restrict__ shdone;  // shared gate_up tiles finished
};

// Routing flag: low word 1 + (expert | first slot << 10 | several members << 16),
// or kNoUnit; high word the first slot's weight.
constexpr uint32_t kNoUnit = 0x80000000u;
constexpr uint32_t kMulti = 1u << 16;

struct UnitInfo {
  int e, p;      // expert, first slot
  bool multi;    // more than one slot routed to the expert (then read the ids)
  float w;       // weight of slot p
  bool none;     // no unit with this index
};
__device__ __forceinline__ UnitInfo decode_unit(uint64_t v) {
  UnitInfo U;
  const uint32_t lo = (uint32_t)v;
  U.none = (lo & kNoUnit) != 0;
  const uint32_t c = lo - 1;
  U.e = (int)(c & 1023u);
  U.p = (int)((c >> 10) & 63u);
  U.multi = (c & kMulti) != 0;
  U.w = __uint_as_float((uint32_t)(v >> 32));
  return U;
}

// The leader: see the file comment.  LDS: dyn holds the tokens as bf16
// [M][H]; lids / lw the ids and weights of every slot.
template <int NI>
__device__ void leader(const LayerArgs& A, uint32_t* dyn, int* lids, float* lw, uint64_t* unit_flag, int* topk_lds) {
  const ExpArgs& a = A.a;
  const LayerGrid& G = A.g;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int GK = a.H / kGroup;
  // 1. tokens into LDS (normalised with RMSNorm, and then also stored for the
  //    caller and the shared gate_up), then their group corrections
  for (int t = wave; t < a.M; t += kWavesPerBlock) {
    float xv[NI][4];
    uint2 packed[NI];
    load_token<NI>(a.x + (size_t)t * a.H, a.H, lane, A.rmsnorm != 0, A.r.eps, xv, packed);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const size_t o = (size_t)t * a.H + 256 * i + 4 * lane;
      *reinterpret_cast<uint2*>(dyn + o / 2) = packed[i];
      if (A.rmsnorm)
        st_coherent(reinterpret_cast<uint64_t*>(A.r.x_norm + o), ((uint64_t)packed[i].y << 32) | packed[i].x);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (A.rmsnorm)  // normalised tokens ready for the shared gate_up
    for (int i = G.gSG + tid; i < G.gRG; i += kBlock) st_coherent(&A.flags[3 * (size_t)G.grid + i], (uint64_t)1);
  for (int j = tid; j < a.M * GK; j += kBlock)
    st_coherent(&A.gb[j], group_bias_lds<false>(dyn + (size_t)(j / GK) * a.H / 2, j % GK));
  // 2. ids and weights of every slot
  if (A.route) {
    for (int t = wave; t < a.M; t += kWavesPerBlock) {
      uint32_t key[kTopkEPL];
      bool present[kTopkEPL];
      const uint32_t* kt = A.rkeys + (size_t)t * a.E;
      int spins = 0;
      for (;;) {
        bool missing = false;
#pragma unroll
        for (int j = 0; j < kTopkEPL; ++j) {
          const int e = lane + kWave * j;
          present[j] = e < a.E;
          key[j] = present[j] ? (uint32_t)ld_coherent(reinterpret_cast<const int32_t*>(&kt[e])) : 1u;
          missing = missing || key[j] == 0;
        }
        if (__ballot(missing) == 0) break;
        if (++spins > kSpinLimit) {
          if (lane == 0) atomicOr(a.err, 2);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      int id;
      float w;
      topk_select(key, present, a.k, lane, topk_lds + wave * 3 * kMaxTopK, id, w);
      if (lane < a.k) {
        st_coherent(&A.r.ids[(size_t)t * a.k + lane], id);
        st_coherent(&A.r.w[(size_t)t * a.k + lane], w);
        lids[t * a.k + lane] = id;
        lw[t * a.k + lane] = w;
      }
      // clear the keys for the next call
#pragma unroll
      for (int j = 0; j < kTopkEPL; ++j)
        if (present[j]) st_coherent(reinterpret_cast<int32_t*>(const_cast<uint32_t*>(&kt[lane + kWave * j])), 0);
    }
  } else {
    for (int p = tid; p < a.S; p += kBlock) {
      lids[p] = a.ids[p];
      lw[p] = a.topk_w[p];
    }
  }
  __syncthreads();
  // 3. units (distinct valid experts in order of first occurrence; S <= 64)
  //    and their flags
  if (wave == 0) {
    const int id = lane < a.S ? lids[lane] : -1;
    const bool valid = id >= 0 && id < a.E;
    bool first = valid;
    int nmem = 0;
    for (int q = 0; q < a.S; ++q) {
      const int v = __builtin_amdgcn_readlane(id, q);
      first = first && !(q < lane && v == id);
      nmem += (valid && v == id) ? 1 : 0;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint64_t fb = __ballot(first);
    const int u = __popcll(fb & lt);
    if (first) {
      const uint32_t c = (uint32_t)id | ((uint32_t)lane << 10) | (nmem > 1 ? kMulti : 0u);
      unit_flag[u] = ((uint64_t)__float_as_uint(lw[lane]) << 32) | (c + 1);
    }
    const int nu = __popcll(fb);
    if (lane >= nu) unit_flag[lane] = kNoUnit;
    if (lane == 0) topk_lds[0] = __ballot(first && nmem > 1) != 0;
  }
  __syncthreads();
  // a unit of several slots reads the ids and weights from memory: make the
  // stores of the top-k complete first
  if (A.route && topk_lds[0]) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int i = G.gRG + tid; i < G.gSD; i += kBlock) st_coherent(&A.flags[i], unit_flag[(i - G.gRG) / a.Tgu]);
  for (int i = G.gRD + tid; i < G.grid; i += kBlock) st_coherent(&A.flags[i], unit_flag[(i - G.gRD) / a.Tdn]);
}

template <int NI, int GWG, int PG, int CWG, int GWD, int PD, int CWD>
__global__ __launch_bounds__(kBlock) void k_layer(const LayerArgs A) {
  extern __shared__ __align__(16) uint32_t dyn[];  // the leader's tokens
  __shared__ float red[kWavesPerBlock][kWave];
  __shared__ int flag;
  __shared__ uint64_t fval[2];  // one slot per successive wait
  __shared__ int topk_lds[kWavesPerBlock * 3 * kMaxTopK];
  __shared__ int lids[kMaxUnits];
  __shared__ float lw[kMaxUnits];
  __shared__ uint64_t unit_flag[kMaxUnits];
  __shared__ __align__(16) uint16_t hl[2 * kGroup];
  const ExpArgs& a = A.a;
  const LayerGrid& G = A.g;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int blk = blockIdx.x;
  const uint32_t magic = bf16_pair_magic();

  // ------------------------------------------------------------ leader
  if (blk == 0) {
    leader<NI>(A, dyn, lids, lw, unit_flag, topk_lds);
    return;
  }
  // ------------------------------------------------------------ router rows
  if (blk < G.gSG) {
    router_row<NI>(A.r, (blk - 1) * kWavesPerBlock + wave, lane, false, A.rkeys);
    return;
  }

  // ------------------------------------------------------------ shared gate_up
  if (blk < G.gRG) {
    if constexpr (CWG == 0) {
      return;
    } else {
      const int idx = blk - G.gSG, b = idx / a.KSgu, ks = idx % a.KSgu;
      const int c0 = (ks * kWavesPerBlock + wave) * CWG;
      uint4 wc[CWG];
      const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh_gu) + ((size_t)(b * (a.H / 8) + c0) * kWave + lane) * 16;
#pragma unroll
      for (int c = 0; c < CWG; ++c) wc[c] = *reinterpret_cast<const uint4*>(base + (size_t)c * kWave * 16);
      const uint16_t* act = a.x;
      if (A.rmsnorm) {
        wait_flag(&A.flags[3 * (size_t)G.grid + blk], a.err, &fval[0]);
        act = after_wait(static_cast<const uint16_t*>(A.r.x_norm));
      }
      for (int t = 0; t < a.M; ++t) {
        red[wave][lane] = shared_dot<CWG, false>(wc, act + (size_t)t * a.H, c0);
        lds_sync();
        if (tid < kWave) {
          float part = 0.f;
#pragma unroll
          for (int w = 0; w < kWavesPerBlock; ++w) part += red[w][tid];
          st_coherent(&a.shgu_part[(((size_t)t * a.Tgu + b) * a.KSgu + ks) * kWave + tid], part);
        }
        lds_sync();
      }
      if (!arrive_last(&a.shgu_cnt[b * kCntStride], a.KSgu, &flag)) return;
      for (int t = wave; t < a.M; t += kWavesPerBlock) {
        float pv[kMaxKSplit];
#pragma unroll
        for (int s2 = 0; s2 < kMaxKSplit; ++s2)
          pv[s2] = s2 < a.KSgu ? ld_coherent(&a.shgu_part[(((size_t)t * a.Tgu + b) * a.KSgu + s2) * kWave + lane]) : 0.f;
        float part = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < kMaxKSplit; ++s2) part += pv[s2];
        const float up = __shfl_down(part, 32, 64);
        if (lane < 32) store_hilo_coherent(a.h_sh + ((size_t)t * a.I + 32 * b) * 2, lane, silu_f32(part) * up);
      }
      if (!arrive_last(A.shdone, a.Tgu, &flag)) return;
      for (int i = G.gSD + tid; i < G.gRD; i += kBlock) st_coherent(&A.flags[2 * (size_t)G.grid + i], (uint64_t)1);
      return;
    }
  }

  // ------------------------------------------------------------ routed gate_up
  if (blk < G.gSD) {
    const int idx = blk - G.gRG, u = idx / a.Tgu, b = idx % a.Tgu;
    const int GK = a.H / kGroup;
    const UnitInfo U = decode_unit(wait_flag(&A.flags[blk], a.err, &fval[0]));
    if (U.none) return;
    const bool active = wave * GWG < GK;
    const int g0 = active ? wave * GWG : 0;
    uint4 wq[GWG];
    ScalePack<PG> sc[GWG / PG];
    const uint8_t* qb = a.gu_q + (size_t)U.e * a.gu_q_stride + ((size_t)(b * GK + g0) * kWave + lane) * 16;
#pragma unroll
    for (int i = 0; i < GWG; ++i) wq[i] = *reinterpret_cast<const uint4*>(qb + (size_t)i * kWave * 16);
    const uint16_t* sb = a.gu_s + (size_t)U.e * a.gu_s_stride + ((size_t)(b * (GK / PG) + g0 / PG) * kWave + lane) * PG;
#pragma unroll
    for (int j = 0; j < GWG / PG; ++j) sc[j].load(sb + (size_t)j * kWave * PG);
    uint64_t m = U.multi ? find_unit_wave<true>(a.ids, a.S, a.E, u, lane).mask : (1ull << U.p);
    const uint16_t* xs = after_wait(A.rmsnorm ? static_cast<const uint16_t*>(A.r.x_norm) : a.x);
    const float* gbs = after_wait(static_cast<const float*>(A.gb));
    while (m) {
      const int p = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int t = p / a.k;
      red[wave][lane] = active ? routed_dot<GWG, PG, false>(wq, sc, xs + (size_t)t * a.H,
                                                             as_scalar_ptr(gbs + (size_t)t * GK), g0, magic)
                               : 0.f;
      lds_sync();
      if (tid < 32) {
        float gt = 0.f, up = 0.f;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) { gt += red[w][tid]; up += red[w][tid + 32]; }
        const float v = silu_f32(gt) * up;
        const uint16_t hi = f32_to_bf16(v);
        const uint16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
        hl[tid] = hi;
        hl[32 + tid] = lo;
        uint16_t* hg = a.h + ((size_t)p * a.I + 32 * b) * 2;
        st_coherent(&hg[tid], hi);
        st_coherent(&hg[32 + tid], lo);
      }
      lds_sync();
      if (tid == 0)
        st_coherent(&A.hb[(size_t)p * hb_stride(a.I) + b], group_bias_lds<true>(reinterpret_cast<const uint32_t*>(hl), 0));
      lds_sync();
    }
    if (!arrive_last(&A.hcnt[u * kCntStride], a.Tgu, &flag)) return;
    for (int i = tid; i < a.Tdn; i += kBlock)
      st_coherent(&A.flags[(size_t)G.grid + G.gRD + u * a.Tdn + i], (uint64_t)1);
    return;
  }

  int b = 0;
  // ------------------------------------------------------------ shared down
  if (blk < G.gRD) {
    if constexpr (CWD == 0) {
      return;
    } else {
      const int idx = blk - G.gSD;
      b = idx / a.KSdn;
      const int ks = idx % a.KSdn;
      const int c0 = (ks * kWavesPerBlock + wave) * CWD;
      uint4 wc[CWD];
      const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh_dn) + ((size_t)(b * (a.I / 8) + c0) * kWave + lane) * 16;
#pragma unroll
      for (int c = 0; c < CWD; ++c) wc[c] = *reinterpret_cast<const uint4*>(base + (size_t)c * kWave * 16);
      wait_flag(&A.flags[2 * (size_t)G.grid + blk], a.err, &fval[0]);
      const uint16_t* hs = after_wait(static_cast<const uint16_t*>(a.h_sh));
      for (int t = 0; t < a.M; ++t) {
        red[wave][lane] = shared_dot<CWD, true>(wc, hs + (size_t)t * a.I * 2, c0);
        lds_sync();
        if (tid < kWave) {
          float part = 0.f;
#pragma unroll
          for (int w = 0; w < kWavesPerBlock; ++w) part += red[w][tid];
          st_coherent(&a.shdn_part[((size_t)t * a.KSdn + ks) * a.H + 64 * b + tid], part);
        }
        lds_sync();
      }
    }
  } else {
    // ---------------------------------------------------------- routed down
    const int idx = blk - G.gRD, u = idx / a.Tdn;
    b = idx % a.Tdn;
    const UnitInfo U = decode_unit(wait_flag(&A.flags[blk], a.err, &fval[0]));
    if (!U.none) {
      const int GK = a.I / kGroup;
      const bool active = wave * GWD < GK;
      const int g0 = active ? wave * GWD : 0;
      uint4 wq[GWD];
      ScalePack<PD> sc[GWD / PD];
      const uint8_t* qb = a.dn_q + (size_t)U.e * a.dn_q_stride + ((size_t)(b * GK + g0) * kWave + lane) * 16;
#pragma unroll
      for (int i = 0; i < GWD; ++i) wq[i] = *reinterpret_cast<const uint4*>(qb + (size_t)i * kWave * 16);
      const uint16_t* sb = a.dn_s + (size_t)U.e * a.dn_s_stride + ((size_t)(b * (GK / PD) + g0 / PD) * kWave + lane) * PD;
#pragma unroll
      for (int j = 0; j < GWD / PD; ++j) sc[j].load(sb + (size_t)j * kWave * PD);
      uint64_t m = U.multi ? find_unit_wave<true>(a.ids, a.S, a.E, u, lane).mask : (1ull << U.p);
      wait_flag(&A.flags[(size_t)G.grid + blk], a.err, &fval[1]);
      const uint16_t* hs = after_wait(static_cast<const uint16_t*>(a.h));
      const float* hbs = after_wait(static_cast<const float*>(A.hb));
      while (m) {
        const int p = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const float wp = U.multi ? ld_coherent(&a.topk_w[p]) : U.w;
        red[wave][lane] = active ? routed_dot<GWD, PD, true>(wq, sc, hs + (size_t)p * a.I * 2,
                                                              as_scalar_ptr(hbs + (size_t)p * hb_stride(a.I)), g0, magic)
                                 : 0.f;
        lds_sync();
        if (tid < kWave) {
          float part = 0.f;
#pragma unroll
          for (int w = 0; w < kWavesPerBlock; ++w) part += red[w][tid];
          st_coherent(&a.dpart[(size_t)p * a.H + 64 * b + tid], part * wp);
        }
        lds_sync();
      }
    }
  }
  // ------------------------------------------------------------ combine
  const int expected = a.S + (a.has_shared ? a.KSdn : 0);
  if (!arrive_last(&a.dn_cnt[b * kCntStride], expected, &flag)) return;
  combine_tile(a, b, A.route == 0);
}

// ------------------------------------------------------------------ dispatch

namespace {
struct LayerVariant { int NI, GWG, PG, CWG, GWD, PD, CWD; };

bool layer_variant(const Shape& s, LayerVariant& v) {
  const KSplit kg = ksplit_for(s.H / kGroup), kd = ksplit_for(s.I / kGroup);
  const SharedSplit sg = shared_gu_split(s.H), sd = shared_dn_split(s.I);
  v = {s.H / 256, kg.GW, kg.P, s.has_shared ? sg.CW : 0, kd.GW, kd.P, s.has_shared ? sd.CW : 0};
  const bool ling = v.NI == 10 && v.GWG == 20 && v.PG == 4 && (v.CWG == 0 || v.CWG == 20) && v.GWD == 6 && v.PD == 2 &&
                    (v.CWD == 0 || v.CWD == 6);
  const bool tiny = v.NI == 1 && v.GWG == 2 && v.PG == 2 && (v.CWG == 0 || v.CWG == 2) && v.GWD == 1 && v.PD == 1 &&
                    (v.CWD == 0 || v.CWD == 1);
  return ling || tiny;
}

template <int NI, int GWG, int PG, int CWG, int GWD, int PD, int CWD>
hipError_t run_layer(const LayerArgs& A, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((k_layer<NI, GWG, PG, CWG, GWD, PD, CWD>), dim3(A.g.grid), dim3(kBlock), lds, st, A);
  return hipGetLastError();
}
}  // namespace

bool layer_supported(const Shape& s, int M) {
  LayerVariant v;
  return (int64_t)M * s.k <= kMaxUnits && layer_variant(s, v);
}

hipError_t launch_layer(const Shape& s, const uint8_t* packed, const PackedLayout& PL, const float* router_w,
                        const uint16_t* x, int M, bool route, bool rmsnorm, float eps, uint16_t* x_norm,
                        int32_t* ids, float* w, uint16_t* out, uint8_t* ws, const WsLayout& L, hipStream_t st) {
  LayerVariant v;
  if (!layer_variant(s, v)) return hipErrorInvalidValue;
  LayerArgs A;
  A.a = make_expert_args(s, packed, PL, x, M, ids, w, out, ws, L);
  RouteArgs& r = A.r;
  r.M = M; r.E = s.E; r.k = s.k; r.H = s.H;
  r.rmsnorm = rmsnorm ? 1 : 0;
  r.eps = eps;
  r.wr = router_w; r.x = x; r.x_norm = x_norm;
  r.logits = reinterpret_cast<float*>(ws + L.logits);
  r.cnt = reinterpret_cast<int32_t*>(ws + L.route_cnt);
  r.ids = ids; r.w = w;
  A.route = route ? 1 : 0;
  A.rmsnorm = rmsnorm ? 1 : 0;
  A.g = layer_roles(s.H, s.E, s.I, s.has_shared, route ? 1 : 0, M * s.k);
  A.flags = reinterpret_cast<uint64_t*>(ws + L.flags);
  A.rkeys = reinterpret_cast<uint32_t*>(ws + L.rkeys);
  A.gb = reinterpret_cast<float*>(ws + L.gb);
  A.hb = reinterpret_cast<float*>(ws + L.hb);
  A.hcnt = reinterpret_cast<int32_t*>(ws + L.hcnt);
  A.shdone = reinterpret_cast<int32_t*>(ws + L.shdone);
  const size_t lds = (size_t)M * s.H * 2;  // the leader's tokens
#define LAYER_CASE(NI_, GWG_, PG_, CWG_, GWD_, PD_, CWD_)                                                   \
  if (v.NI == NI_ && v.GWG == GWG_ && v.PG == PG_ && v.CWG == CWG_ && v.GWD == GWD_ && v.PD == PD_ &&       \
      v.CWD == CWD_)                                                                                         \
    return run_layer<NI_, GWG_, PG_, CWG_, GWD_, PD_, CWD_>(A, lds, st);
  LAYER_CASE(10, 20, 4, 20, 6, 2, 6)
  LAYER_CASE(10, 20, 4, 0, 6, 2, 0)
  LAYER_CASE(1, 2, 2, 2, 1, 1, 1)
  LAYER_CASE(1, 2, 2, 0, 1, 1, 0)
#undef LAYER_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
