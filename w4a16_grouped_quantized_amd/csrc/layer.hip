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
//                   carries its unit's expert, first slot and weight, and one
//                   per combine workgroup with the number of units;
//   router rows     (only when the launch routes) 4 rows each, stored as
//                   order-preserving keys that the leader polls for;
//   shared gate_up  tile x K slice of the shared expert; the last slice of a
//                   tile sums the slices into h_sh, the last tile raises the
//                   flag of every shared down workgroup;
//   routed experts  (unit, gate_up tile): wait for the routing flag, then h
//                   of the tile's 32 rows for every token routed to the unit,
//                   and at once the matching 32 columns of the down matrix
//                   applied to it for every output row: one weighted partial
//                   row per (slot, tile).  The last tile of a unit counts the
//                   unit as done;
//   shared down     tile x K slice: weights requested at once, then waits
//                   for h_sh; counts itself as done;
//   combine         (token, quarter of an output tile): once all units and
//                   shared slices are done, the sum of the token's partial
//                   rows and the shared slices in a fixed order, rounded to
//                   bf16.
//
// Waits only ever point at workgroups with smaller ids, which the hardware
// dispatches first, so every wait ends; each poll is bounded anyway and
// records bit 1 of the error word if it gives up.  Data crossing workgroups
// is stored agent-coherently (written through to memory, past the XCD's L2,
// which is not coherent with the others); a flag or count is raised only
// after the producer's stores have completed, and a consumer reads the data
// only after it has seen it, through addresses it had not touched before in
// this launch.  Activations are read by whole wavefronts at uniform
// addresses, through scalar loads (cached per XCD): so every cache line read
// that way is complete when the flag that releases its reader is raised.
#include <algorithm>

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
  float* __restrict__ ypart;     // [H/64][S][I/32][64] down partials (weighted) per output tile, slot, group of h
  int32_t* __restrict__ hcnt;    // gate_up tiles finished per unit (kCntStride apart)
  int32_t* __restrict__ shdone;  // shared gate_up tiles finished
  int32_t* __restrict__ udone;   // units finished
  int32_t* __restrict__ sdone;   // shared down workgroups finished
  int32_t* __restrict__ cdone;   // combine workgroups finished
};

// Partial rows summed per batch of loads in the combine.
constexpr int kCombineBatch = 12;

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
// [M][H], later the router keys [M][E]; lids / lw the ids and weights of
// every slot.
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
    for (int i = G.gSG + tid; i < G.gRG; i += kBlock) st_coherent(&A.flags[2 * (size_t)G.grid + i], (uint64_t)1);
  for (int j = tid; j < a.M * GK; j += kBlock)
    st_coherent(&A.gb[j], group_bias_lds<false>(dyn + (size_t)(j / GK) * a.H / 2, j % GK));
  // 2. ids and weights of every slot
  if (A.route) {
    // every thread polls its share of the router keys (agent-coherent loads
    // are served one at a time per wavefront, so the four wavefronts split
    // them) into LDS, where the tokens no longer needed were
    uint32_t* lkeys = dyn;  // [M][E]
    const int nk = a.M * a.E;
    __syncthreads();
    int spins = 0;
    for (;;) {
      int miss = 0;
      for (int i = tid; i < nk; i += kBlock) {
        const uint32_t v = (uint32_t)ld_coherent(reinterpret_cast<const int32_t*>(&A.rkeys[i]));
        lkeys[i] = v;
        miss |= v == 0;
      }
      if (!__syncthreads_or(miss)) break;
      if (++spins > kSpinLimit) {
        if (tid == 0) atomicOr(a.err, 2);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    // clear the keys for the next call
    for (int i = tid; i < nk; i += kBlock) st_coherent(reinterpret_cast<int32_t*>(&A.rkeys[i]), 0);
    for (int t = wave; t < a.M; t += kWavesPerBlock) {
      uint32_t key[kTopkEPL];
      bool present[kTopkEPL];
#pragma unroll
      for (int j = 0; j < kTopkEPL; ++j) {
        const int e = lane + kWave * j;
        present[j] = e < a.E;
        key[j] = present[j] ? lkeys[t * a.E + e] : 0u;
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
  if (wave == 0 && A.route && a.M == 1) {
    // one routed token: its k experts are distinct, unit u is slot u
    if (lane < a.S) {
      const uint32_t c = (uint32_t)lids[lane] | ((uint32_t)lane << 10);
      unit_flag[lane] = ((uint64_t)__float_as_uint(lw[lane]) << 32) | (c + 1);
    } else {
      unit_flag[lane] = kNoUnit;
    }
    if (lane == 0) {
      topk_lds[0] = 0;
      topk_lds[1] = a.S;
    }
  } else if (wave == 0) {
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
    const bool multi = __ballot(first && nmem > 1) != 0;
    if (lane == 0) {
      topk_lds[0] = multi;
      topk_lds[1] = nu;
    }
  }
  __syncthreads();
  // a unit of several slots reads the ids and weights from memory: make the
  // stores of the top-k complete first
  if (A.route && topk_lds[0]) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // routed workgroups of unit u: gRG + u*Tgu + b
  for (int u = wave; u < a.S; u += kWavesPerBlock) {
    const uint64_t f = unit_flag[u];
    for (int b = lane; b < a.Tgu; b += kWave) st_coherent(&A.flags[G.gRG + u * a.Tgu + b], f);
  }
  // combine workgroups: the number of units, plus one
  const uint64_t nu1 = (uint64_t)(1 + topk_lds[1]);
  for (int i = G.gCB + tid; i < G.grid; i += kBlock) st_coherent(&A.flags[i], nu1);
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
  __shared__ __align__(16) uint16_t hl[kGroup];  // one tile's h (fp16)
  __shared__ float hsc[2];                        // its correction and scale exponent
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
        wait_flag(&A.flags[2 * (size_t)G.grid + blk], a.err, &fval[0]);
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
          pv[s2] = s2 < a.KSgu ? ld_fresh(&a.shgu_part[(((size_t)t * a.Tgu + b) * a.KSgu + s2) * kWave + lane]) : 0.f;
        float part = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < kMaxKSplit; ++s2) part += pv[s2];
        const float up = __shfl_down(part, 32, 64);
        if (lane < 32) store_hilo_coherent(a.h_sh + ((size_t)t * a.I + 32 * b) * 2, lane, silu_f32(part) * up);
      }
      if (!arrive_last(A.shdone, a.Tgu, &flag)) return;
      for (int i = G.gSD + tid; i < G.gCB; i += kBlock) st_coherent(&A.flags[(size_t)G.grid + i], (uint64_t)1);
      return;
    }
  }

  // ------------------------------------------------------------ routed experts
  // (unit u, gate_up tile b): h of the tile's 32 rows for every token routed
  // to the unit, then that 32-column slice of the down matrix applied to it
  // for all H output rows.
  if (blk < G.gSD) {
    const int idx = blk - G.gRG, u = idx / a.Tgu, b = idx % a.Tgu;
    const int GK = a.H / kGroup, GKD = a.I / kGroup;
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
    // down slice: row tile t = wave*NI + j (NI = H/256 tiles per wavefront), group b
    uint4 wd[NI];
    uint32_t sd[NI];
    const uint8_t* db = a.dn_q + (size_t)U.e * a.dn_q_stride;
    const uint16_t* dsb = a.dn_s + (size_t)U.e * a.dn_s_stride;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int t = wave * NI + j;
      wd[j] = *reinterpret_cast<const uint4*>(db + ((size_t)(t * GKD + b) * kWave + lane) * 16);
      sd[j] = dsb[((size_t)(t * (GKD / PD) + b / PD) * kWave + lane) * PD + b % PD];
    }
    uint64_t m = U.multi ? find_unit_wave<true>(a.ids, a.S, a.E, u, lane).mask : (1ull << U.p);
    const uint16_t* xs = after_wait(A.rmsnorm ? static_cast<const uint16_t*>(A.r.x_norm) : a.x);
    const float* gbs = after_wait(static_cast<const float*>(A.gb));
    while (m) {
      const int p = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int tok = p / a.k;
      const float wp = U.multi ? ld_coherent(&a.topk_w[p]) : U.w;
      red[wave][lane] = active ? routed_dot<GWG, PG, false>(wq, sc, xs + (size_t)tok * a.H,
                                                             as_scalar_ptr(gbs + (size_t)tok * GK), g0, magic)
                               : 0.f;
      lds_sync();
      if (tid < kWave) {
        // h of the tile as fp16 under a power-of-two scale 2^sh chosen from
        // its largest magnitude (exact rescaling, 11 significant bits)
        float v = 0.f;
        if (tid < 32) {
          float gt = 0.f, up = 0.f;
#pragma unroll
          for (int w = 0; w < kWavesPerBlock; ++w) { gt += red[w][tid]; up += red[w][tid + 32]; }
          v = silu_f32(gt) * up;
        }
        float mx = fabsf(v);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        int ex = 0;
        frexpf(mx, &ex);
        const int sh = mx > 0.f ? ex - 15 : 0;  // |h| * 2^-sh < 2^15
        const _Float16 hv = (_Float16)ldexpf(v, -sh);
        const float hs = wave_sum(tid < 32 ? (float)hv : 0.f);
        if (tid < 32) hl[tid] = __builtin_bit_cast(uint16_t, hv);
        if (tid == 0) {
          hsc[0] = -1032.0f * hs;
          hsc[1] = __int_as_float(sh);
        }
      }
      lds_sync();
      // the tile's h as 16 fp16 pairs, wavefront-uniform
      uint32_t hp[16];
      const uint4* h4 = reinterpret_cast<const uint4*>(hl);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 q = h4[i];
        hp[4 * i] = uniform(q.x); hp[4 * i + 1] = uniform(q.y); hp[4 * i + 2] = uniform(q.z); hp[4 * i + 3] = uniform(q.w);
      }
      const float bias = __uint_as_float(uniform(__float_as_uint(hsc[0])));
      const int sh = uniform(__float_as_int(hsc[1]));
      // ypart[n][p][b][64]: the rows one combine workgroup reads are contiguous
      float* yp = A.ypart + ((size_t)p * a.Tgu + b) * kWave;
      const size_t ntile_stride = (size_t)a.S * a.Tgu * kWave;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        float pr = bias;
        // opaque copy: the code pairs are extracted here, not hoisted out of
        // the member loop (160 extracted pairs would stay live in VGPRs)
        uint4 w = wd[j];
        asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
        const uint32_t wdw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t pair = ((wdw[d] >> (4 * i)) & 0x000F000Fu) | 0x64006400u;  // fp16 (1024 + u)
            pr = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pair), __builtin_bit_cast(half2_t, hp[4 * d + i]), pr, false);
          }
        const float y = ldexpf(pr * bf16_to_f32(sd[j]), sh) * wp;
        st_coherent(&yp[(size_t)(wave * NI + j) * ntile_stride + lane], y);
      }
      lds_sync();
    }
    if (!arrive_last(&A.hcnt[u * kCntStride], a.Tgu, &flag)) return;
    if (tid == 0) __hip_atomic_fetch_add(A.udone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // ------------------------------------------------------------ shared down
  if (blk < G.gCB) {
    if constexpr (CWD == 0) {
      return;
    } else {
      const int idx = blk - G.gSD;
      const int b = idx / a.KSdn, ks = idx % a.KSdn;
      const int c0 = (ks * kWavesPerBlock + wave) * CWD;
      uint4 wc[CWD];
      const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh_dn) + ((size_t)(b * (a.I / 8) + c0) * kWave + lane) * 16;
#pragma unroll
      for (int c = 0; c < CWD; ++c) wc[c] = *reinterpret_cast<const uint4*>(base + (size_t)c * kWave * 16);
      wait_flag(&A.flags[(size_t)G.grid + blk], a.err, &fval[0]);
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
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(A.sdone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }

  // ------------------------------------------------------------ combine
  // (token t, output tile n, quarter c4): once every unit and every shared
  // down slice has finished, out[t][col] for the 16 columns of the quarter =
  // the sum of the token's partial rows and the shared slices, in a fixed
  // order, rounded to bf16.
  {
    constexpr int kCols = kWave / kCombineSplit;           // 16 columns
    constexpr int kRowSlots = kBlock / kCols;              // 16 rows in flight per pass
    const int idx = blk - G.gCB;
    const int c4 = idx % kCombineSplit, tn = idx / kCombineSplit, t = tn / a.Tdn, n = tn % a.Tdn;
    const int nu = (int)(uint32_t)wait_flag(&A.flags[blk], a.err, &fval[0]) - 1;
    const int sd_total = a.has_shared ? a.Tdn * a.KSdn : 0;
    if (tid == 0) {
      int spins = 0;
      while (ld_coherent(A.udone) < nu || ld_coherent(A.sdone) < sd_total) {
        if (++spins > kSpinLimit) {
          atomicOr(a.err, 2);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    // thread (rs, c): column 64n + 16c4 + c, partial rows rs, rs + 16, ...
    // (row j*Tgu + b of the token is slot j, tile b); a slot whose id is out
    // of range (caller ids only) was never written: its rows are loaded but
    // not added
    const int c = tid % kCols, rs = tid / kCols;
    const int col = 64 * n + kCols * c4 + c;
    const int nrow = a.k * a.Tgu;
    const float* base = A.ypart + ((size_t)n * a.S + (size_t)t * a.k) * a.Tgu * kWave + kCols * c4 + c;
    uint64_t vmask = ~0ull;
    if (!A.route) {
      vmask = 0;
      for (int j = 0; j < a.k; ++j) {
        const int e = a.ids[t * a.k + j];
        vmask |= (uint64_t)(e >= 0 && e < a.E) << j;
      }
    }
    float acc = 0.f;
    for (int r0 = rs; r0 < nrow; r0 += kRowSlots * kCombineBatch) {
      const float* src = base + (size_t)r0 * kWave;
      float pv[kCombineBatch];
#pragma unroll
      for (int q = 0; q < kCombineBatch; ++q)
        pv[q] = r0 + kRowSlots * q < nrow ? ld_fresh(src + q * kRowSlots * kWave) : 0.f;
#pragma unroll
      for (int q = 0; q < kCombineBatch; ++q) {
        const int r = r0 + kRowSlots * q;
        const bool use = r < nrow && (A.route || ((vmask >> (r / a.Tgu)) & 1ull));
        acc += use ? pv[q] : 0.f;
      }
    }
    float* cred = &red[0][0];  // [kRowSlots][kCols]
    cred[rs * kCols + c] = acc;
    lds_sync();
    if (tid < kCols) {
      float y = 0.f;
#pragma unroll
      for (int r = 0; r < kRowSlots; ++r) y += cred[r * kCols + tid];
      if (a.has_shared) {
        float sv[kMaxKSplit];
#pragma unroll
        for (int s2 = 0; s2 < kMaxKSplit; ++s2)
          sv[s2] = s2 < a.KSdn ? ld_fresh(&a.shdn_part[((size_t)t * a.KSdn + s2) * a.H + col]) : 0.f;
#pragma unroll
        for (int s2 = 0; s2 < kMaxKSplit; ++s2) y += sv[s2];
      }
      a.out[(size_t)t * a.H + col] = f32_to_bf16(y);
      const bool bad = (~vmask & (a.k >= 64 ? ~0ull : ((1ull << a.k) - 1))) != 0;
      if (bad && n == 0 && c4 == 0 && tid == 0) atomicOr(a.err, 1);
    }
    // the last combine workgroup resets the completion counters
    if (arrive_last(A.cdone, a.M * a.Tdn * kCombineSplit, &flag) && tid == 0) {
      st_coherent(A.udone, 0);
      st_coherent(A.sdone, 0);
    }
  }
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
  A.g = layer_roles(s.H, s.E, s.I, s.has_shared, route ? 1 : 0, M, s.k);
  A.flags = reinterpret_cast<uint64_t*>(ws + L.flags);
  A.rkeys = reinterpret_cast<uint32_t*>(ws + L.rkeys);
  A.gb = reinterpret_cast<float*>(ws + L.gb);
  A.ypart = reinterpret_cast<float*>(ws + L.ypart);
  A.hcnt = reinterpret_cast<int32_t*>(ws + L.hcnt);
  A.shdone = reinterpret_cast<int32_t*>(ws + L.shdone);
  A.udone = reinterpret_cast<int32_t*>(ws + L.udone);
  A.sdone = reinterpret_cast<int32_t*>(ws + L.sdone);
  A.cdone = reinterpret_cast<int32_t*>(ws + L.cdone);
  // the leader's tokens, then (routing in the launch) its router keys
  const size_t lds = (size_t)M * std::max(s.H * 2, route ? s.E * 4 : 0);
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
