// layer.hip — the small-M MoE layer (decode, verify) in one launch.
//
// The separate kernels of the small-M path (router, gate_up, down) each pay a
// launch and a drain, and the routed expert loads cannot start before the
// router's last workgroup has chosen the experts.  Here every step is a
// workgroup role of one grid, in this order:
//
//   leader          (workgroup 0) the call's tag: one more than the last
//                   call's, kept in the workspace; with RMSNorm first the
//                   normalised tokens; then the tag into every other
//                   workgroup's flag;
//   router rows     (only when the launch routes) 4 rows each, stored as
//                   order-preserving keys with the tag;
//   shared gate_up  tile x K slice of the shared expert; the last slice of a
//                   tile sums the slices into h_sh (fp32, with the tag);
//   routed gate_up  (slot u, gate_up tile b): the top-k of every token from
//                   the keys (or the caller's ids), the distinct experts in
//                   order of first occurrence ("units"); workgroups u below
//                   their number take unit u's expert and compute h of the
//                   tile's 32 rows for every token routed to it, stored as
//                   fp16 pairs under a power-of-two scale, with the tag;
//   down            (16 output rows): the same routing, the down rows of
//                   every slot's expert requested at once and the shared
//                   expert's rows at the start, then waits for the h of the
//                   token's slots and the shared h, and writes
//                   out = sum_slots w * (W_down h) + W_shared_down h_sh.
//
// Every workgroup reads the tag from its flag (set only by the leader,
// cleared by its owner).  A consumer polls the words it needs until their
// high half holds the call's tag: data and its readiness travel together, so
// no counter, fence or reset sits between a producer and its readers, and
// data of earlier calls (or left by other paths) can never pass as this
// call's.  Waits only ever point at workgroups with smaller ids, which the
// hardware dispatches first, so every wait ends; each poll is bounded anyway
// and records bit 1 of the error word if it gives up.  Words crossing
// workgroups are stored agent-coherently (written through to memory, past the
// XCD's L2, which is not coherent with the others); a 64-bit word is stored
// and loaded whole, so its tag and payload always belong together.
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
  uint32_t* __restrict__ epoch;  // tag of the last call
  int32_t* __restrict__ arrive;  // [kArriveCounters] spaced: workgroups that have read the epoch
  uint64_t* __restrict__ flags;  // [grid] normalised tokens ready (RMSNorm only)
  uint64_t* __restrict__ rkeys;  // [M][E] router keys | tag
  uint64_t* __restrict__ hval;   // [S][I/32][16] fp16 pairs of h | tag
  uint64_t* __restrict__ hmeta;  // [S][I/32] exponent of the tile's scale | tag
  uint64_t* __restrict__ hsh;    // [M][I] shared h, fp32 bits | tag
};

__device__ __forceinline__ uint64_t tagged(uint32_t v, uint32_t T) { return ((uint64_t)T << 32) | v; }
__device__ __forceinline__ bool has_tag(uint64_t w, uint32_t T) { return (uint32_t)(w >> 32) == T; }

__device__ __forceinline__ uint32_t next_tag(uint32_t epoch) { return epoch + 1u ? epoch + 1u : 1u; }

// The leader: see the file comment.
template <int NI>
__device__ void leader(const LayerArgs& A) {
  const ExpArgs& a = A.a;
  const LayerGrid& G = A.g;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (A.rmsnorm) {
    for (int t = wave; t < a.M; t += kWavesPerBlock) {
      float xv[NI][4];
      uint2 packed[NI];
      load_token<NI>(a.x + (size_t)t * a.H, a.H, lane, true, A.r.eps, xv, packed);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const size_t o = (size_t)t * a.H + 256 * i + 4 * lane;
        st_coherent(reinterpret_cast<uint64_t*>(A.r.x_norm + o), ((uint64_t)packed[i].y << 32) | packed[i].x);
      }
    }
    // the normalised tokens complete before the flags of their readers
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = G.gSG + tid; i < G.gDN; i += kBlock) st_coherent(&A.flags[i], (uint64_t)1);
  }
  // the epoch advances once every other workgroup has read it
  if (tid == 0) {
    const uint32_t T = next_tag((uint32_t)ld_coherent(reinterpret_cast<const int32_t*>(A.epoch)));
    const int others = G.grid - 1;
    for (int spins = 0;; ++spins) {
      int n[kArriveCounters];
#pragma unroll
      for (int c = 0; c < kArriveCounters; ++c) n[c] = ld_coherent(&A.arrive[c * kCntStride]);
      int sum = 0;
#pragma unroll
      for (int c = 0; c < kArriveCounters; ++c) sum += n[c];
      if (sum >= others) break;
      if (spins >= kSpinLimit) {
        atomicOr(a.err, 2);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
#pragma unroll
    for (int c = 0; c < kArriveCounters; ++c) st_coherent(&A.arrive[c * kCntStride], 0);
    st_coherent(reinterpret_cast<int32_t*>(A.epoch), (int32_t)T);
  }
}

// The call's tag in a workgroup other than the leader, from the epoch that
// thread 0 read at the start (ev), and that workgroup's arrival: issued once
// the epoch load (and the value `after`, if any) has returned.  The leader
// advances the epoch only after every arrival, so all workgroups of a call
// read the same epoch.
__device__ __forceinline__ uint32_t share_tag(uint32_t ev, uint32_t* lds) {
  if (threadIdx.x == 0) *lds = next_tag(ev);
  lds_sync();
  return *lds;
}
__device__ __forceinline__ void arrive_epoch(const LayerArgs& A, uint32_t ev, int after = 0) {
  if (threadIdx.x == 0) {
    int one = 1;
    asm volatile("" : "+v"(one) : "v"(ev), "v"(after));
    __hip_atomic_fetch_add(&A.arrive[(blockIdx.x % kArriveCounters) * kCntStride], one, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}
__device__ __forceinline__ uint32_t take_tag(const LayerArgs& A, uint32_t ev, uint32_t* lds) {
  arrive_epoch(A, ev);
  return share_tag(ev, lds);
}
__device__ __forceinline__ uint32_t read_epoch(const LayerArgs& A) {
  return threadIdx.x == 0 ? (uint32_t)ld_coherent(reinterpret_cast<const int32_t*>(A.epoch)) : 0u;
}

// This call's router keys of every token into lkeys (LDS): every thread
// polls its entries (tid + m * kBlock) agent-coherently until they carry the
// tag; the workgroup follows.
constexpr int kKeyBatch = 8;  // key polls issued before their tags are checked
constexpr uint64_t kDnLoadDelay = 160;  // 1.6 us in s_memrealtime ticks (100 MHz)
__device__ void gather_keys(const LayerArgs& A, uint32_t T, uint32_t* lkeys) {
  const int tid = threadIdx.x;
  const int nk = A.a.M * A.a.E;  // <= 32 per thread
  uint32_t todo = 0;
  for (int m = 0; m < 32; ++m)
    if (tid + m * kBlock < nk) todo |= 1u << m;
  for (int spins = 0;; ++spins) {
    for (int m0 = 0; m0 < 32; m0 += kKeyBatch) {
      if (!((todo >> m0) & ((1u << kKeyBatch) - 1))) continue;
      uint64_t v[kKeyBatch];
#pragma unroll
      for (int m = 0; m < kKeyBatch; ++m)
        v[m] = ((todo >> (m0 + m)) & 1u) ? ld_coherent(&A.rkeys[tid + (m0 + m) * kBlock]) : 0ull;
#pragma unroll
      for (int m = 0; m < kKeyBatch; ++m)
        if (((todo >> (m0 + m)) & 1u) && has_tag(v[m], T)) {
          lkeys[tid + (m0 + m) * kBlock] = (uint32_t)v[m];
          todo &= ~(1u << (m0 + m));
        }
    }
    if (!__syncthreads_or(todo != 0)) break;
    if (spins >= kSpinLimit) {
      if (tid == 0) atomicOr(A.a.err, 2);
      break;
    }
    __builtin_amdgcn_s_sleep(4);
  }
}

// ids and weights of every slot into lids / lw (LDS): the top-k of the keys
// in lkeys (one wavefront per token), or the caller's.
__device__ void select_slots(const LayerArgs& A, const uint32_t* lkeys, int* topk_lds, int* lids, float* lw,
                             bool want_w = true) {
  const ExpArgs& a = A.a;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (A.route) {
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
      topk_select(key, present, a.k, lane, topk_lds + wave * 3 * kMaxTopK, id, w, want_w);
      if (lane < a.k) {
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
  lds_sync();
}

__device__ __forceinline__ bool id_ok(int e, int E) { return e >= 0 && e < E; }

// Three workgroups per CU (at most 168 VGPRs): a decode grid (under 768
// workgroups) is resident at once, so no role waits for a slot.
template <int NI, int GWG, int PG, int CWG, int PD, int NPQ, int NSC, int DG>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void k_layer(const LayerArgs A) {
  extern __shared__ __align__(16) uint32_t dyn[];  // router keys [M][E], then group corrections [M][H/32]
  __shared__ float red[kWavesPerBlock][kWave];
  __shared__ int flag;
  __shared__ uint64_t fval;
  __shared__ uint32_t tag_lds;
  __shared__ __align__(16) int topk_lds[kWavesPerBlock * 3 * kMaxTopK];
  __shared__ int lids[kMaxUnits];
  __shared__ float lw[kMaxUnits];
  __shared__ int uexp[kMaxUnits + 1];      // expert of each unit; [kMaxUnits] = number of units
  __shared__ uint64_t umask[kMaxUnits];    // its slots
  // down: one token's h records (fp16 pairs), their corrections and
  // exponents, and the shared h as bf16 (hi, lo)
  __shared__ __align__(16) uint32_t hst[kBlock / kDnRows * NPQ][16];
  __shared__ float hbias[kBlock / kDnRows * NPQ];
  __shared__ int hexp[kBlock / kDnRows * NPQ];
  __shared__ __align__(16) uint16_t shhi[NSC > 0 ? 8 * (kBlock / kDnRows) * NSC : 1];
  __shared__ __align__(16) uint16_t shlo[NSC > 0 ? 8 * (kBlock / kDnRows) * NSC : 1];
  const ExpArgs& a = A.a;
  const LayerGrid& G = A.g;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int blk = blockIdx.x;

  // ------------------------------------------------------------ leader
  if (blk == 0) {
    leader<NI>(A);
    return;
  }

  // ------------------------------------------------------------ router rows
  if (blk < G.gSG) {
    const uint32_t ev = read_epoch(A);
    const int e = (blk - 1) * kWavesPerBlock + wave;
    const bool has_row = e < a.E;
    const int er = has_row ? e : a.E - 1;
    float4 wr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) wr[i] = *reinterpret_cast<const float4*>(A.r.wr + (size_t)er * a.H + 256 * i + 4 * lane);
    // the logits of every token first (red[wave][t]), then the tag
    for (int t = 0; t < a.M; ++t) {
      float xv[NI][4];
      uint2 packed[NI];
      load_token<NI>(a.x + (size_t)t * a.H, a.H, lane, A.rmsnorm != 0, A.r.eps, xv, packed);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        acc = fmaf(wr[i].x, xv[i][0], acc);
        acc = fmaf(wr[i].y, xv[i][1], acc);
        acc = fmaf(wr[i].z, xv[i][2], acc);
        acc = fmaf(wr[i].w, xv[i][3], acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) red[wave][t] = acc;
    }
    const uint32_t T = share_tag(ev, &tag_lds);
    for (int t = lane; t < a.M; t += kWave)
      if (has_row) st_coherent(&A.rkeys[(size_t)t * a.E + e], tagged(sort_key(red[wave][t]), T));
    arrive_epoch(A, ev);
    return;
  }

  // ------------------------------------------------------------ shared gate_up
  if (blk < G.gGU) {
    if constexpr (CWG == 0) {
      return;
    } else {
      const uint32_t ev = read_epoch(A);
      const int idx = blk - G.gSG, b = idx / a.KSgu, ks = idx % a.KSgu;
      // this stream starts at once and runs under the routing (the router
      // rows, the key hand-off and the top-k), which moves few bytes
      const int c0 = (ks * kWavesPerBlock + wave) * CWG;
      uint4 wc[CWG];
      const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh_gu) + ((size_t)(b * (a.H / 8) + c0) * kWave + lane) * 16;
#pragma unroll
      for (int c = 0; c < CWG; ++c) wc[c] = *reinterpret_cast<const uint4*>(base + (size_t)c * kWave * 16);
      const uint16_t* act = a.x;
      if (A.rmsnorm) {  // the normalised tokens are ready with the flag
        wait_flag(&A.flags[blk], a.err, &fval);
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
      const uint32_t T = take_tag(A, ev, &tag_lds);
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
        if (lane < 32)
          st_coherent(&A.hsh[(size_t)t * a.I + 32 * b + lane], tagged(__float_as_uint(silu_f32(part) * up), T));
      }
      return;
    }
  }

  uint32_t* lkeys = dyn;
  float* gbias = reinterpret_cast<float*>(dyn) + (A.route ? a.M * a.E : 0);

  // ------------------------------------------------------------ routed gate_up
  // (slot u, gate_up tile b): h of the tile's 32 rows for every token routed
  // to unit u's expert.
  if (blk < G.gDN) {
    const uint32_t ev = read_epoch(A);
    const int idx = blk - G.gGU, u = idx / a.Tgu, b = idx % a.Tgu;
    const int GK = a.H / kGroup;
    // group corrections of the tokens (the caller's now; normalised ones
    // once the flag says they are stored)
    if (!A.rmsnorm)
      for (int j = tid; j < a.M * GK; j += kBlock) {
        GroupBias<false> gl;
        gl.load(a.x + (size_t)(j / GK) * a.H, j % GK);
        gbias[j] = gl.value();
      }
    if (A.rmsnorm) wait_flag(&A.flags[blk], a.err, &fval);
    const uint32_t T = take_tag(A, ev, &tag_lds);
    const uint16_t* act = A.rmsnorm ? after_wait(static_cast<const uint16_t*>(A.r.x_norm)) : a.x;
    if (A.rmsnorm)
      for (int j = tid; j < a.M * GK; j += kBlock) {
        GroupBias<false> gl;
        gl.load(act + (size_t)(j / GK) * a.H, j % GK);
        gbias[j] = gl.value();
      }
    if (A.route) gather_keys(A, T, lkeys);
    // the routed workgroups need the ids only, but the first one also hands
    // the weights to the caller
    select_slots(A, lkeys, topk_lds, lids, lw, idx == 0);
    // units: distinct valid experts in order of first occurrence (S <= 64);
    // the experts of one routed token are distinct: unit u is slot u
    if (wave == 0 && A.route && a.M == 1) {
      if (lane < a.S) {
        uexp[lane] = lids[lane];
        umask[lane] = 1ull << lane;
      }
      if (lane == 0) uexp[kMaxUnits] = a.S;
    } else if (wave == 0) {
      const int id = lane < a.S ? lids[lane] : -1;
      const bool valid = id_ok(id, a.E);
      bool first = valid;
      uint64_t mem = 0;
      for (int q = 0; q < a.S; ++q) {
        const int v = __builtin_amdgcn_readlane(id, q);
        first = first && !(q < lane && v == id);
        mem |= (uint64_t)(valid && v == id) << q;
      }
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      const uint64_t fb = __ballot(first);
      if (first) {
        const int r = __popcll(fb & lt);
        uexp[r] = id;
        umask[r] = mem;
      }
      if (lane == 0) uexp[kMaxUnits] = __popcll(fb);
    }
    lds_sync();
    if (A.route && u == 0 && b == 0)  // the routing, for the caller
      for (int p = tid; p < a.S; p += kBlock) {
        A.r.ids[p] = lids[p];
        A.r.w[p] = lw[p];
      }
    if (u >= uexp[kMaxUnits]) return;
    const int e = uexp[u];
    uint64_t m = umask[u];
    const bool active = wave * GWG < GK;
    const int g0 = active ? wave * GWG : 0;
    uint4 wq[GWG];
    ScalePack<PG> sc[GWG / PG];
    const uint8_t* qb = a.gu_q + (size_t)e * a.gu_q_stride + ((size_t)(b * GK + g0) * kWave + lane) * 16;
#pragma unroll
    for (int i = 0; i < GWG; ++i) wq[i] = *reinterpret_cast<const uint4*>(qb + (size_t)i * kWave * 16);
    const uint16_t* sb = a.gu_s + (size_t)e * a.gu_s_stride + ((size_t)(b * (GK / PG) + g0 / PG) * kWave + lane) * PG;
#pragma unroll
    for (int j = 0; j < GWG / PG; ++j) sc[j].load(sb + (size_t)j * kWave * PG);
    const uint32_t magic = bf16_pair_magic();
    while (m) {
      const int p = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int tok = p / a.k;
      red[wave][lane] = active ? routed_dot<GWG, PG, false>(wq, sc, act + (size_t)tok * a.H, gbias + tok * GK, g0, magic)
                               : 0.f;
      lds_sync();
      if (wave == 0) {
        // h of the tile as fp16 under a power-of-two scale 2^sh chosen from
        // its largest magnitude (exact rescaling, 11 significant bits)
        float v = 0.f;
        if (lane < 32) {
          float gt = 0.f, up = 0.f;
#pragma unroll
          for (int w = 0; w < kWavesPerBlock; ++w) { gt += red[w][lane]; up += red[w][lane + 32]; }
          v = silu_f32(gt) * up;
        }
        float mx = fabsf(v);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        int ex = 0;
        frexpf(mx, &ex);
        const int sh = mx > 0.f ? ex - 15 : 0;  // |h| * 2^-sh < 2^15
        const uint32_t hb = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(v, -sh));
        const uint32_t nb = (uint32_t)__shfl_down((int)hb, 1, 64);
        const size_t rec = (size_t)p * a.Tgu + b;
        if (lane < 32 && !(lane & 1)) st_coherent(&A.hval[rec * 16 + lane / 2], tagged(hb | (nb << 16), T));
        if (lane == 0) st_coherent(&A.hmeta[rec], tagged((uint32_t)sh, T));
      }
      lds_sync();
    }
    return;
  }

  // ------------------------------------------------------------ down
  // rows row0 .. row0+7: thread (row, q) takes the (slot, group) pairs
  // j = q + 32 i of a token and the shared chunks q + 32 c, and the 32
  // partial sums of a row are added in q order.
  {
    constexpr int Q = kBlock / kDnRows;
    const uint32_t ev = read_epoch(A);
    const int r = blk - G.gDN;
    const int row = tid % kDnRows, q = tid / kDnRows;
    const int row0 = r * kDnRows, tile = row0 >> 6, lrow = (row0 & 63) + row;
    constexpr int GKD = DG;  // I / 32
    // the shared expert's rows, requested at once
    uint4 wsh[NSC > 0 ? NSC : 1];
    if constexpr (NSC > 0) {
#pragma unroll
      for (int c = 0; c < NSC; ++c) {
        const int cc = q + Q * c;
        wsh[c] = cc < a.I / 8 ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.sh_dn) +
                                                                  ((size_t)(tile * (a.I / 8) + cc) * kWave + lrow) * 16)
                              : make_uint4(0, 0, 0, 0);
      }
    }
    const uint32_t T = take_tag(A, ev, &tag_lds);
    if (A.route) gather_keys(A, T, lkeys);
    select_slots(A, lkeys, topk_lds, lids, lw);
    if (!A.route && r == 0 && tid < a.S && !id_ok(lids[tid], a.E)) atomicOr(a.err, 1);
    // The routed gate_up stream, which the h records wait for, goes first:
    // the down rows are needed only once those records land, several
    // microseconds later, so they are requested kDnLoadDelay after the
    // routing (realtime ticks of 10 ns; measured: 22.5 us per layer without
    // the delay, 21.5 with 1.4 to 1.8 us, worse again from 2.5 us).
    {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__builtin_amdgcn_s_memrealtime() - t0 < kDnLoadDelay) __builtin_amdgcn_s_sleep(1);
    }
    const int nrec = a.k * GKD;  // (slot, group) records of one token, <= Q * NPQ
    for (int t = 0; t < a.M; ++t) {
      // this token's down rows of every slot's expert
      uint4 wd[NPQ];
      uint32_t sdv[NPQ];
#pragma unroll
      for (int i = 0; i < NPQ; ++i) {
        const int j = q + Q * i, jj = j / GKD, g = j - jj * GKD;
        const int e = j < nrec ? lids[t * a.k + jj] : -1;
        if (id_ok(e, a.E)) {
          wd[i] = *reinterpret_cast<const uint4*>(a.dn_q + (size_t)e * a.dn_q_stride +
                                                  ((size_t)(tile * GKD + g) * kWave + lrow) * 16);
          sdv[i] = a.dn_s[(size_t)e * a.dn_s_stride + ((size_t)(tile * (GKD / PD) + g / PD) * kWave + lrow) * PD + g % PD];
        } else {
          wd[i] = make_uint4(0, 0, 0, 0);
          sdv[i] = 0;
        }
      }
      // the token's shared h (columns tid + 256 c), which lands long before
      // the routed h: polled first, on its own
      if constexpr (NSC > 0) {
        uint32_t shtodo = 0;
        for (int c = 0; c * kBlock < a.I; ++c)
          if (tid + c * kBlock < a.I) shtodo |= 1u << c;
        for (int spins = 0;; ++spins) {
          for (uint32_t rem = shtodo; rem; rem &= rem - 1) {
            const int c = __ffs(rem) - 1;
            const int col = tid + c * kBlock;
            const uint64_t v = ld_coherent(&A.hsh[(size_t)t * a.I + col]);
            if (has_tag(v, T)) {
              const float f = __uint_as_float((uint32_t)v);
              const uint16_t hi = f32_to_bf16(f);
              shhi[col] = hi;
              shlo[col] = f32_to_bf16(f - bf16_to_f32(hi));
              shtodo &= ~(1u << c);
            }
          }
          if (!__syncthreads_or(shtodo != 0)) break;
          if (spins >= kSpinLimit) {
            if (tid == 0) atomicOr(a.err, 2);
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
      }
      // the token's h records (thread tid < nrec takes record tid): its
      // exponent word is polled (one word per record and round, so the
      // polls stay light next to the weight stream), then the pairs read
      int rst = 2;  // 0: poll the exponent, 1: read the pairs, 2: staged
      size_t rec = 0;
      if (tid < nrec) {
        const int p = t * a.k + tid / DG;
        if (id_ok(lids[p], a.E)) {
          rst = 0;
          rec = (size_t)p * a.Tgu + tid % DG;
        }
      }
      int sh = 0;
      bool first = true;
      for (int spins = 0;; ++spins) {
        if (rst == 0) {
          const uint64_t mv = ld_coherent(&A.hmeta[rec]);
          if (has_tag(mv, T)) {
            sh = (int)(uint32_t)mv;
            rst = 1;
          }
        }
        if (rst == 1) {
          uint32_t hw[16];
          bool ok = true;
          if (first) {  // plain loads: the pairs are almost always there with the exponent
            const uint4* p4 = reinterpret_cast<const uint4*>(A.hval + rec * 16);
#pragma unroll
            for (int w = 0; w < 8; ++w) {
              const uint4 v = ld_fresh(p4 + w);
              hw[2 * w] = v.x;
              hw[2 * w + 1] = v.z;
              ok = ok && v.y == T && v.w == T;
            }
            first = false;
          } else {  // a pair lagged (or a stale copy was cached): agent-coherent loads
#pragma unroll
            for (int w = 0; w < 16; ++w) {
              const uint64_t v = ld_coherent(&A.hval[rec * 16 + w]);
              hw[w] = (uint32_t)v;
              ok = ok && has_tag(v, T);
            }
          }
          if (ok) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < 16; ++w) {
              const half2_t h2 = __builtin_bit_cast(half2_t, hw[w]);
              s += (float)h2[0];
              s += (float)h2[1];
            }
            uint4* dst = reinterpret_cast<uint4*>(hst[tid]);
#pragma unroll
            for (int w = 0; w < 4; ++w) dst[w] = make_uint4(hw[4 * w], hw[4 * w + 1], hw[4 * w + 2], hw[4 * w + 3]);
            hbias[tid] = -1032.0f * s;  // turns sum (1024 + u) h into sum (u - 8) h
            hexp[tid] = sh;
            rst = 2;
          }
        }
        if (!__syncthreads_or(rst != 2)) break;
        if (spins >= kSpinLimit) {
          if (tid == 0) atomicOr(a.err, 2);
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      float acc = 0.f;
      const uint32_t magic = fp16_pair_magic();
#pragma unroll
      for (int i = 0; i < NPQ; ++i) {
        const int j = q + Q * i;
        if (j < nrec) {
          const int p = t * a.k + j / GKD;
          if (id_ok(lids[p], a.E)) {
            const uint4* h4 = reinterpret_cast<const uint4*>(hst[j]);
            uint32_t hp[16];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint4 v = h4[w];
              hp[4 * w] = v.x; hp[4 * w + 1] = v.y; hp[4 * w + 2] = v.z; hp[4 * w + 3] = v.w;
            }
            // two accumulation chains (dwords 0-1 and 2-3), added at the end
            float pr[2] = {hbias[j], 0.f};
            const uint32_t wdw[4] = {wd[i].x, wd[i].y, wd[i].z, wd[i].w};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const uint32_t pair = ((wdw[d] >> (4 * k4)) & 0x000F000Fu) | magic;  // fp16 (1024 + u)
                pr[d >> 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pair),
                                                    __builtin_bit_cast(half2_t, hp[4 * d + k4]), pr[d >> 1], false);
              }
            acc += ldexpf((pr[0] + pr[1]) * bf16_to_f32(sdv[i]), hexp[j]) * lw[p];
          }
        }
      }
      if constexpr (NSC > 0) {
        const uint32_t* hi32 = reinterpret_cast<const uint32_t*>(shhi);
        const uint32_t* lo32 = reinterpret_cast<const uint32_t*>(shlo);
#pragma unroll
        for (int c = 0; c < NSC; ++c) {
          const int cc = q + Q * c;
          if (cc < a.I / 8) {
            const uint4 xh = *reinterpret_cast<const uint4*>(hi32 + 4 * cc);
            const uint4 xl = *reinterpret_cast<const uint4*>(lo32 + 4 * cc);
            const uint32_t xhv[4] = {xh.x, xh.y, xh.z, xh.w};
            const uint32_t xlv[4] = {xl.x, xl.y, xl.z, xl.w};
            acc = dot_chunk_bf16(wsh[c], xhv, acc);
            acc = dot_chunk_bf16(wsh[c], xlv, acc);
          }
        }
      }
      float* cred = &red[0][0];  // [Q][kDnRows]
      cred[tid] = acc;
      lds_sync();
      if (tid < kDnRows) {
        float y = 0.f;
#pragma unroll
        for (int qq = 0; qq < Q; ++qq) y += cred[qq * kDnRows + tid];
        a.out[(size_t)t * a.H + row0 + tid] = f32_to_bf16(y);
      }
      lds_sync();
    }
  }
}

// ------------------------------------------------------------------ dispatch

namespace {
struct LayerVariant { int NI, GWG, PG, CWG, PD, NPQ, NSC, DG; };

bool layer_variant(const Shape& s, LayerVariant& v) {
  const KSplit kg = ksplit_for(s.H / kGroup), kd = ksplit_for(s.I / kGroup);
  const SharedSplit sg = shared_gu_split(s.H);
  constexpr int Q = kBlock / kDnRows;
  const int npq = (s.k * (s.I / kGroup) + Q - 1) / Q;
  const int nsc = s.has_shared ? (s.I / 8 + Q - 1) / Q : 0;
  v = {s.H / 256, kg.GW, kg.P, s.has_shared ? sg.CW : 0, kd.P, npq, nsc, s.I / kGroup};
  const bool ling = v.NI == 10 && v.GWG == 20 && v.PG == 4 && (v.CWG == 0 || v.CWG == 20) && v.PD == 2 &&
                    v.NPQ == 6 && (v.NSC == 0 || v.NSC == 3) && v.DG == 24;
  const bool tiny = v.NI == 1 && v.GWG == 2 && v.PG == 2 && (v.CWG == 0 || v.CWG == 2) && v.PD == 1 && v.NPQ == 1 &&
                    (v.NSC == 0 || v.NSC == 1) && v.DG == 2;
  // every record of a token is staged by one thread
  return (ling || tiny) && (v.CWG == 0) == (v.NSC == 0) && s.k * (s.I / kGroup) <= kBlock;
}

template <int NI, int GWG, int PG, int CWG, int PD, int NPQ, int NSC, int DG>
hipError_t run_layer(const LayerArgs& A, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((k_layer<NI, GWG, PG, CWG, PD, NPQ, NSC, DG>), dim3(A.g.grid), dim3(kBlock), lds, st, A);
  return hipGetLastError();
}
}  // namespace

bool layer_supported(const Shape& s, int M) {
  LayerVariant v;
  return (int64_t)M * s.k <= kMaxUnits && (int64_t)M * s.E <= kMaxLayerKeys && layer_variant(s, v);
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
  r.logits = nullptr;
  r.cnt = nullptr;
  r.ids = ids; r.w = w;
  A.route = route ? 1 : 0;
  A.rmsnorm = rmsnorm ? 1 : 0;
  A.g = layer_roles(s.H, s.E, s.I, s.has_shared, route ? 1 : 0, M, s.k);
  A.epoch = reinterpret_cast<uint32_t*>(ws + L.epoch);
  A.arrive = reinterpret_cast<int32_t*>(ws + L.arrive);
  A.flags = reinterpret_cast<uint64_t*>(ws + L.flags);
  A.rkeys = reinterpret_cast<uint64_t*>(ws + L.rkeys);
  A.hval = reinterpret_cast<uint64_t*>(ws + L.hval);
  A.hmeta = reinterpret_cast<uint64_t*>(ws + L.hmeta);
  A.hsh = reinterpret_cast<uint64_t*>(ws + L.hsh);
  // router keys (routing in the launch), then the group corrections
  const size_t lds = (size_t)M * ((route ? s.E : 0) + s.H / kGroup) * 4;
#define LAYER_CASE(NI_, GWG_, PG_, CWG_, PD_, NPQ_, NSC_, DG_)                                              \
  if (v.NI == NI_ && v.GWG == GWG_ && v.PG == PG_ && v.CWG == CWG_ && v.PD == PD_ && v.NPQ == NPQ_ &&       \
      v.NSC == NSC_ && v.DG == DG_)                                                                          \
    return run_layer<NI_, GWG_, PG_, CWG_, PD_, NPQ_, NSC_, DG_>(A, lds, st);
  LAYER_CASE(10, 20, 4, 20, 2, 6, 3, 24)
  LAYER_CASE(10, 20, 4, 0, 2, 6, 0, 24)
  LAYER_CASE(1, 2, 2, 2, 1, 1, 1, 2)
  LAYER_CASE(1, 2, 2, 0, 1, 1, 0, 2)
#undef LAYER_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
