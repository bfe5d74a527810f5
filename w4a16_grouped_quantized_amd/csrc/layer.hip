// layer.hip — the small-M MoE layer (decode, verify) in one launch.
//
// The separate kernels of the small-M path (router, gate_up, down) each pay a
// launch and a drain, and the routed expert loads cannot start before the
// router's last workgroup has chosen the experts.  Here every step is a
// workgroup role of one grid, in this order:
//
//   leader          (workgroup 0) the call's tag: one more than the last
//                   call's, kept in the workspace; with RMSNorm also the
//                   normalised tokens for the caller;
//   router rows     (only when the launch routes) 4 rows each, stored as
//                   order-preserving keys with the tag;
//   selectors       (kSelectors, only when the launch routes) each gathers
//                   every key, runs the top-k and softmax once per token and
//                   publishes the ids and weights of every slot, tagged, in
//                   its own copy of the routing record (the first one also
//                   hands them to the caller);
//   shared gate_up  tile x K slice of the shared expert; the last slice of a
//                   tile sums the slices into h_sh (fp32, with the tag);
//   routed gate_up  (unit u, gate_up tile b): reads a routing record, finds
//                   the distinct experts in order of first occurrence
//                   ("units"); workgroups u below their number take unit
//                   u's expert and compute h of the tile's 32 rows for every
//                   token routed to it, stored as fp16 pairs under a
//                   power-of-two scale, with the tag;
//   down            (8 output rows, of every token, or of one when M >= 2):
//                   reads a routing record, requests the
//                   down rows of every slot's expert (the shared expert's at
//                   the start), then polls the shared h and the h records and
//                   writes out = sum_slots w * (W_down h) + W_shared_down h_sh.
//
// Every workgroup reads the call's tag from the epoch word.  A consumer polls
// the words it needs until their high half holds the call's tag: data and its
// readiness travel together, so no counter, fence or reset sits between a
// producer and its readers, and data of earlier calls (or left by other
// paths) can never pass as this call's.  Every wait but one points at
// workgroups with smaller ids, which the hardware dispatches first.  The
// exception is the leader (workgroup 0), which waits for every other
// workgroup's arrival before it advances the epoch; no workgroup waits for
// the leader.  So the grid makes progress as long as one workgroup slot
// besides the leader's is free and each XCD takes its workgroups in id
// order: the unfinished workgroup with the smallest id (the leader aside)
// waits only for finished ones, and if it is not resident yet, every
// workgroup ahead of it on its XCD has finished and left a slot.  A decode
// grid (M = 1) fits on the device at once; at M >= 2 the later down
// workgroups take the slots that the router rows, the selectors and the
// routed gate_up workgroups leave.  Each poll is bounded and records bit 1
// of the error word if it gives up.  Words crossing workgroups are stored agent-coherently (written
// through past the XCD's L2, which is not coherent with the others) and
// polled with agent-coherent loads; a 64-bit word is stored and loaded whole,
// so its tag and payload always belong together.  Vector loads return in
// issue order, and a CU serves its wavefronts' requests roughly in order
// too, so a poll issued behind bulk weight loads on the same CU waits for
// them; and a product waits for every load issued before its operands, so
// each role requests its scales before its codes.
#include <algorithm>
#include <type_traits>

#include "experts_dev.hpp"
#include "route_dev.hpp"

namespace moe {

// Optional timeline of the launch (a build with -DMOE_LAYER_TRACE only):
// thread 0 of each workgroup records the realtime clock (10 ns ticks) at
// numbered points of its role; moe_layer_trace_read copies the records out.
#ifdef MOE_LAYER_TRACE
constexpr int kTraceWgs = 2048, kTracePoints = 16;
__device__ uint64_t g_layer_trace[kTraceWgs * kTracePoints];
#define LTRACE_AT(p, who)                                                                         \
  do {                                                                                            \
    if ((who) && blockIdx.x < kTraceWgs)                                                          \
      g_layer_trace[blockIdx.x * kTracePoints + (p)] = __builtin_amdgcn_s_memrealtime();          \
  } while (0)
#define LTRACE(p) LTRACE_AT(p, threadIdx.x == 0)
#define LTRACE_WAIT() __builtin_amdgcn_s_waitcnt(0)
#define LTRACE_ID()                                                                               \
  do {                                                                                            \
    if (threadIdx.x == 0 && blockIdx.x < kTraceWgs) {                                             \
      uint32_t hw, xcc;                                                                           \
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));                            \
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));                          \
      g_layer_trace[blockIdx.x * kTracePoints + kTracePoints - 1] = ((uint64_t)xcc << 32) | hw;   \
    }                                                                                             \
  } while (0)
#else
#define LTRACE_AT(p, who) do {} while (0)
#define LTRACE(p) do {} while (0)
#define LTRACE_ID() do {} while (0)
#define LTRACE_WAIT() do {} while (0)
#endif

struct LayerArgs {
  ExpArgs a;
  RouteArgs r;      // router part: r.ids / r.w are a.ids / a.topk_w
  int route;        // this launch computes ids and weights
  int rmsnorm;      // tokens are RMS-normalised first (only with route)
  LayerGrid g;
  uint32_t* __restrict__ epoch;  // tag of the last call
  int32_t* __restrict__ arrive;  // [kArriveCounters] spaced: workgroups that have read the epoch
  uint64_t* __restrict__ rkeys;  // [M][E] router keys | tag
  uint64_t* __restrict__ rrec;   // [kSelectors][2][kMaxUnits] routing records: ids | tag, weight bits | tag
  uint64_t* __restrict__ hval;   // [S][I/32][16] fp16 pairs of h | tag
  uint64_t* __restrict__ hmeta;  // [S][I/32] exponent of the tile's scale | tag
  uint64_t* __restrict__ hsh;    // [M][I] shared h, fp32 bits | tag
};

__device__ __forceinline__ uint64_t tagged(uint32_t v, uint32_t T) { return ((uint64_t)T << 32) | v; }
__device__ __forceinline__ bool has_tag(uint64_t w, uint32_t T) { return (uint32_t)(w >> 32) == T; }

__device__ __forceinline__ uint32_t next_tag(uint32_t epoch) { return epoch + 1u ? epoch + 1u : 1u; }

// The leader: see the file comment.
template <int NI>
__device__ __forceinline__ void leader(const LayerArgs& A) {
  const ExpArgs& a = A.a;
  const LayerGrid& G = A.g;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (A.rmsnorm) {
    for (int t = wave; t < a.M; t += kWavesPerBlock) {
      float xv[NI][4];
      uint2 packed[NI];
      load_token<NI>(a.x + (size_t)t * a.H, a.H, lane, true, A.r.eps, xv, packed);
#pragma unroll
      for (int i = 0; i < NI; ++i)
        *reinterpret_cast<uint2*>(A.r.x_norm + (size_t)t * a.H + 256 * i + 4 * lane) = packed[i];
    }
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
  LTRACE(1);
}

// The call's tag in a workgroup other than the leader, from the epoch that
// thread 0 read at the start (ev), and that workgroup's arrival: issued once
// the epoch load has returned.  The leader advances the epoch only after
// every arrival, so all workgroups of a call read the same epoch.
__device__ __forceinline__ uint32_t share_tag(uint32_t ev, uint32_t* lds) {
  if (threadIdx.x == 0) *lds = next_tag(ev);
  lds_sync();
  return *lds;
}
__device__ __forceinline__ void arrive_epoch(const LayerArgs& A, uint32_t ev) {
  if (threadIdx.x == 0) {
    int one = 1;
    asm volatile("" : "+v"(one) : "v"(ev));
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
__device__ __forceinline__ void gather_keys(const LayerArgs& A, uint32_t T, uint32_t* lkeys) {
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
    __builtin_amdgcn_s_sleep(1);
  }
}

// ids and weights of every slot of every token into lids / lw (LDS): the
// top-k of the keys in lkeys, one wavefront per token.
__device__ __forceinline__ void select_slots(const LayerArgs& A, const uint32_t* lkeys, int* topk_lds, int* lids,
                                             float* lw) {
  const ExpArgs& a = A.a;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
    topk_select(key, present, a.k, lane, topk_lds + wave * kTopkLdsInts, id, w, true);
    if (lane < a.k) {
      lids[t * a.k + lane] = id;
      lw[t * a.k + lane] = w;
    }
  }
  lds_sync();
}

// The ids (and with want_w the weights) of every slot into lids / lw (LDS),
// by one wavefront: polled from routing record copy c until every word
// carries the call's tag, or the caller's when the launch does not route.
__device__ __forceinline__ void routing_wave(const LayerArgs& A, uint32_t T, int c, int lane, int* lids, float* lw,
                                             bool want_w) {
  const ExpArgs& a = A.a;
  if (!A.route) {
    for (int p = lane; p < a.S; p += kWave) {
      lids[p] = a.ids[p];
      if (want_w) lw[p] = a.topk_w[p];
    }
    return;
  }
  const uint64_t* rec = A.rrec + (size_t)c * 2 * kMaxUnits;
  bool need = lane < a.S;  // S <= 64: one slot per lane
  for (int spins = 0;; ++spins) {
    if (need) {
      const uint64_t vi = ld_coherent(&rec[lane]);
      const uint64_t vw = want_w ? ld_coherent(&rec[kMaxUnits + lane]) : tagged(0u, T);
      if (has_tag(vi, T) && has_tag(vw, T)) {
        lids[lane] = (int)(uint32_t)vi;
        if (want_w) lw[lane] = __uint_as_float((uint32_t)vw);
        need = false;
      }
    }
    if (!__ballot(need)) break;
    if (spins >= kSpinLimit) {
      if (lane == 0) atomicOr(a.err, 2);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ bool id_ok(int e, int E) { return e >= 0 && e < E; }

// Tokens a launch takes (all of them are staged in LDS by the workgroups
// that read them).
constexpr int kLayerMaxTokens = 4;

// Tokens t0 .. t0+nt-1 into LDS: xl[t * H/2 + d] holds inputs 2d, 2d+1 of
// token t0+t as bf16 (RMS-normalised when the launch asks, by the same
// function and in the same order as every other wavefront that normalises,
// so every copy has the same bits), then gb[t * H/32 + g] the group
// corrections of each.  Whole-workgroup call.
template <int NI, bool GB = true>
__device__ __forceinline__ void stage_tokens(const LayerArgs& A, int t0, int nt, uint32_t* xl, float* gb) {
  const ExpArgs& a = A.a;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int HD = a.H / 2;
  if (A.rmsnorm) {
    for (int t = wave; t < nt; t += kWavesPerBlock) {
      float xv[NI][4];
      uint2 packed[NI];
      load_token<NI>(a.x + (size_t)(t0 + t) * a.H, a.H, lane, true, A.r.eps, xv, packed);
#pragma unroll
      for (int i = 0; i < NI; ++i) *reinterpret_cast<uint2*>(xl + (size_t)t * HD + 128 * i + 2 * lane) = packed[i];
    }
  } else {
    const int nc = nt * (a.H / 8);  // 16-byte chunks
    for (int c = tid; c < nc; c += kBlock)
      reinterpret_cast<uint4*>(xl)[c] = reinterpret_cast<const uint4*>(a.x + (size_t)t0 * a.H)[c];
  }
  lds_sync();
  if constexpr (GB) {
    const int GK = a.H / kGroup;
    for (int j = tid; j < nt * GK; j += kBlock) gb[j] = group_bias_lds<false>(xl + (size_t)(j / GK) * HD, j % GK);
    lds_sync();
  }
}

// The routed role's tokens as fp16, in place of the staged bf16 pairs: token
// t's inputs times 2^-r_t (r_t puts the largest magnitude below 2^15; bf16's
// 8 significant bits fit fp16's 11, so the copy is exact down to fp16's
// normal range, 2^-29 of the largest input), the pairs of odd dwords divided
// by 16 more (see routed_dot_lds_h), and in gb the group corrections
// -1032 (sum of the even dwords' values) - 1152 (sum of the odd dwords'),
// which turn the products with 1024 + u and 1024 + 16 u into products with
// the codes u - 8.  xexp[t] = r_t.  Whole-workgroup call.
__device__ __forceinline__ void to_fp16_tokens(int nt, int H, uint32_t* xl, float* gb, int* xexp,
                                               float (*red)[kWave]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int HD = H / 2, GK = H / kGroup;
  for (int t = 0; t < nt; ++t) {
    uint32_t* x = xl + (size_t)t * HD;
    float m = 0.f;
    for (int c = tid; c < HD; c += kBlock)
      m = fmaxf(m, fmaxf(fabsf(bf16_to_f32(x[c] & 0xFFFFu)), fabsf(bf16_to_f32(x[c] >> 16))));
    m = wave_max_dpp(m);
    if (lane == 0) red[wave][0] = m;
    lds_sync();
    m = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
    int e = 0;
    frexpf(m, &e);  // m < 2^e
    const int r = e - 15;
    for (int c = tid; c < HD; c += kBlock) {
      const int sh = (c & 1) ? -r - 4 : -r;
      const _Float16 lo = (_Float16)ldexpf(bf16_to_f32(x[c] & 0xFFFFu), sh);
      const _Float16 hi = (_Float16)ldexpf(bf16_to_f32(x[c] >> 16), sh);
      x[c] = __builtin_bit_cast(uint32_t, (half2_t){lo, hi});
    }
    if (tid == 0) xexp[t] = r;
    lds_sync();
    for (int g = tid; g < GK; g += kBlock) {
      float se = 0.f, so = 0.f;
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const half2_t ve = __builtin_bit_cast(half2_t, x[16 * g + j]);
        const half2_t vo = __builtin_bit_cast(half2_t, x[16 * g + j + 1]);
        se += (float)ve[0] + (float)ve[1];
        so += (float)vo[0] + (float)vo[1];
      }
      gb[t * GK + g] = -1032.0f * se - 1152.0f * so;
    }
    lds_sync();
  }
}

// Three workgroups per CU (at most 168 VGPRs, LDS within a third of the CU):
// a decode grid fits on the device at once.
// F: the routed experts' format, 0 INT4 (bf16 scales), 1 MXFP4 (E8M0 scales).
// PT: one down workgroup per (row block, token) (M >= 2); otherwise each
// down workgroup walks the tokens of its rows.
template <int F, int NI, int GWG, int PG, int CWG, int PD, int NPQ, int NSC, int DG, bool PT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void k_layer(const LayerArgs A) {
  extern __shared__ __align__(16) uint32_t dyn[];  // router keys [M][E], then the staged tokens
  __shared__ float red[kWavesPerBlock][kWave];
  __shared__ int flag;
  __shared__ uint32_t tag_lds;
  __shared__ int xexp[kLayerMaxTokens];  // routed role: exponents of the fp16 tokens
  __shared__ __align__(16) int topk_lds[kWavesPerBlock * kTopkLdsInts];
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
  LTRACE(0);
  LTRACE_ID();

  // ------------------------------------------------------------ leader
  if (blk == 0) {
    leader<NI>(A);
    return;
  }

  // ------------------------------------------------------------ router rows
  if (blk < G.gSL) {
    const uint32_t ev = read_epoch(A);
    const int e = (blk - 1) * kWavesPerBlock + wave;
    const bool has_row = e < a.E;
    const int er = has_row ? e : a.E - 1;
    float4 wr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) wr[i] = ld_stream_f4(A.r.wr + (size_t)er * a.H + 256 * i + 4 * lane);
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
      acc = wave_sum_dpp(acc);
      if (lane == 0) red[wave][t] = acc;
    }
    const uint32_t T = share_tag(ev, &tag_lds);
    for (int t = lane; t < a.M; t += kWave)
      if (has_row) st_coherent(&A.rkeys[(size_t)t * a.E + e], tagged(sort_key(red[wave][t]), T));
    LTRACE_WAIT();
    LTRACE(1);
    arrive_epoch(A, ev);
    return;
  }

  // LDS: router keys [M][E] (routing in the launch), then the staged tokens
  // and their group corrections
  uint32_t* lkeys = dyn;
  uint32_t* xl = dyn + (A.route ? a.M * a.E : 0);
  float* gbias = reinterpret_cast<float*>(xl + (size_t)a.M * (a.H / 2));

  // ------------------------------------------------------------ selectors
  if (blk < G.gSG) {
    const uint32_t ev = read_epoch(A);
    const uint32_t T = take_tag(A, ev, &tag_lds);
    const int c = blk - G.gSL;
    // The top-k runs twice, the same instructions both times: first on
    // stand-in keys (distinct, so it takes its usual path) while the router
    // rows are still being computed, which brings its code into the
    // instruction cache, then on the call's keys.
    for (int i = tid; i < a.M * a.E; i += kBlock) lkeys[i] = (uint32_t)(i + 1);
    lds_sync();
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == 1) {
        gather_keys(A, T, lkeys);
        LTRACE(1);
      }
      select_slots(A, lkeys, topk_lds, lids, lw);
    }
    LTRACE(3);
    uint64_t* rec = A.rrec + (size_t)c * 2 * kMaxUnits;
    for (int p = tid; p < a.S; p += kBlock) {
      st_coherent(&rec[p], tagged((uint32_t)lids[p], T));
      st_coherent(&rec[kMaxUnits + p], tagged(__float_as_uint(lw[p]), T));
      if (c == 0) {  // the routing, for the caller
        A.r.ids[p] = lids[p];
        A.r.w[p] = lw[p];
      }
    }
    LTRACE_WAIT();
    LTRACE(2);
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
      for (int c = 0; c < CWG; ++c) wc[c] = ld_stream(base + (size_t)c * kWave * 16);
      stage_tokens<NI>(A, 0, a.M, xl, gbias);
      for (int t = 0; t < a.M; ++t) {
        red[wave][lane] = shared_dot_lds<CWG>(wc, xl + (size_t)t * (a.H / 2), c0);
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
      LTRACE_WAIT();
      LTRACE(2);
      return;
    }
  }

  // ------------------------------------------------------------ routed gate_up
  // (unit u, gate_up tile b): h of the tile's 32 rows for every token routed
  // to unit u's expert.
  if (blk < G.gDN) {
    const uint32_t ev = read_epoch(A);
    const int idx = blk - G.gGU, u = idx / a.Tgu, b = idx % a.Tgu;
    const int GK = a.H / kGroup;
    stage_tokens<NI, false>(A, 0, a.M, xl, gbias);
    if constexpr (F == 0) to_fp16_tokens(a.M, a.H, xl, gbias, xexp, red);
    const uint32_t T = take_tag(A, ev, &tag_lds);
    LTRACE(1);
    // units: distinct valid experts in order of first occurrence (S <= 64);
    // the experts of one routed token are distinct: unit u is slot u
    if (wave == 0) {
      routing_wave(A, T, idx % kSelectors, lane, lids, lw, false);
      if (A.route && a.M == 1) {
        if (lane < a.S) {
          uexp[lane] = lids[lane];
          umask[lane] = 1ull << lane;
        }
        if (lane == 0) uexp[kMaxUnits] = a.S;
      } else {
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
    }
    lds_sync();
    LTRACE(2);
    if (u >= uexp[kMaxUnits]) return;
    const int e = uexp[u];
    uint64_t m = umask[u];
    LTRACE(3);
    const bool active = wave * GWG < GK;
    const int g0 = active ? wave * GWG : 0;
    // the scales first, so that each group's product waits for its own
    // codes only (loads return in issue order)
    uint4 wq[GWG];
    // scale element size 2 (bf16) or 1 (E8M0); the strides count bf16 elements
    const size_t sidx = ((size_t)(b * (GK / PG) + g0 / PG) * kWave + lane) * PG;
    ScalePack<PG> sc[F == 0 ? GWG / PG : 1];
    ScaleBytes<PG> scb[F == 1 ? GWG / PG : 1];
    if constexpr (F == 0) {
      const uint16_t* sb = a.gu_s + (size_t)e * a.gu_s_stride + sidx;
#pragma unroll
      for (int j = 0; j < GWG / PG; ++j) sc[j].load(sb + (size_t)j * kWave * PG);
    } else {
      const uint8_t* sb = reinterpret_cast<const uint8_t*>(a.gu_s) + (size_t)e * a.gu_s_stride * 2 + sidx;
#pragma unroll
      for (int j = 0; j < GWG / PG; ++j) scb[j].load(sb + (size_t)j * kWave * PG);
    }
    __builtin_amdgcn_sched_barrier(0);
    LTRACE(4);
    const uint8_t* qb = a.gu_q + (size_t)e * a.gu_q_stride + ((size_t)(b * GK + g0) * kWave + lane) * 16;
#pragma unroll
    for (int i = 0; i < GWG; ++i) wq[i] = ld_stream(qb + (size_t)i * kWave * 16);
    const uint32_t magic16 = fp16_pair_magic();
    LTRACE(5);
    auto dot_member = [&](int tok, auto first) -> float {
      if constexpr (F == 0)
        return active ? ldexpf(routed_dot_lds_h<GWG, PG, !decltype(first)::value>(
                                   wq, sc, xl + (size_t)tok * (a.H / 2), gbias + tok * GK, g0, magic16),
                               xexp[tok])
                      : 0.f;
      else
        return active ? routed_dot_lds_fp4<GWG, PG>(wq, scb, xl + (size_t)tok * (a.H / 2), g0) : 0.f;
    };
    // The first member's products come right after the requests, outside
    // the loop over members: the compiler then waits for each group's codes
    // as the products reach them, where a loop entry would make it wait for
    // all of them first.  A decode unit has one member, so the loop body
    // never computes.
    int p = __ffsll((unsigned long long)m) - 1;
    m &= m - 1;
    float dv = dot_member(p / a.k, std::true_type{});
    for (;;) {
      red[wave][lane] = dv;
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
        const float mx = wave_max_dpp(fabsf(v));
        int ex = 0;
        frexpf(mx, &ex);
        const int sh = mx > 0.f ? ex - 15 : 0;  // |h| * 2^-sh < 2^15
        // INT4: the values of odd dwords (lanes 2-3 mod 4) divided by 16 more,
        // for the down role's shift-free pairs (see routed_dot_lds_h)
        const int odd = F == 0 ? ((lane >> 1) & 1) : 0;
        const uint32_t hb = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(v, -sh - 4 * odd));
        // the odd neighbour's half (quad_perm [1,1,3,3])
        const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hb, 0xF5, 0xF, 0xF, false);
        const size_t rec = (size_t)p * a.Tgu + b;
        if (lane < 32 && !(lane & 1)) st_coherent(&A.hval[rec * 16 + lane / 2], tagged(hb | (nb << 16), T));
        if (lane == 0) st_coherent(&A.hmeta[rec], tagged((uint32_t)sh, T));
      }
      lds_sync();
      if (!m) break;
      p = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      dv = dot_member(p / a.k, std::false_type{});
    }
    LTRACE_WAIT();
    LTRACE(6);
    return;
  }

  // ------------------------------------------------------------ down
  // rows row0 .. row0+7: thread (row, q) takes the (slot, group) pairs
  // j = q + 32 i of a token and the shared chunks q + 32 c, and the 32
  // partial sums of a row are added in q order.  With PT each workgroup
  // takes one token of its rows, and the M workgroups of a row block have
  // ids 8 apart, so they run on one XCD (ids are dealt to the XCDs in
  // turn), whose L2 then serves the shared expert's down rows to all but
  // the first.
  {
    constexpr int Q = kBlock / kDnRows;
    const uint32_t ev = read_epoch(A);
    const int idx = blk - G.gDN;
    const int r = PT ? ((idx >> 3) / a.M) * 8 + (idx & 7) : idx;
    const int t_first = PT ? (idx >> 3) % a.M : 0, t_end = PT ? t_first + 1 : a.M;
    const int row = tid % kDnRows, q = tid / kDnRows;
    const int row0 = r * kDnRows, tile = row0 >> 6, lrow = (row0 & 63) + row;
    constexpr int GKD = DG;  // I / 32
    // the shared expert's rows, requested at once
    uint4 wsh[NSC > 0 ? NSC : 1];
    if constexpr (NSC > 0) {
#pragma unroll
      for (int c = 0; c < NSC; ++c) {
        const int cc = q + Q * c;
        wsh[c] = cc < a.I / 8 ? ld_stream(reinterpret_cast<const uint8_t*>(a.sh_dn) +
                                          ((size_t)(tile * (a.I / 8) + cc) * kWave + lrow) * 16)
                              : make_uint4(0, 0, 0, 0);
      }
    }
    const uint32_t T = take_tag(A, ev, &tag_lds);
    if (wave == 0) routing_wave(A, T, r % kSelectors, lane, lids, lw, true);
    lds_sync();
    LTRACE(3);
    if (!A.route && idx == 0 && tid < a.S && !id_ok(lids[tid], a.E)) atomicOr(a.err, 1);
    const int nrec = a.k * GKD;  // (slot, group) records of one token, <= Q * NPQ
    for (int t = t_first; t < t_end; ++t) {
      // this token's down rows of every slot's expert: the scales first,
      // so that the first record's product waits for its own codes only
      // (loads return in issue order)
      uint4 wd[NPQ];
      uint32_t sdv[NPQ];
#pragma unroll
      for (int i = 0; i < NPQ; ++i) {
        const int j = q + Q * i, jj = j / GKD, g = j - jj * GKD;
        const int e = j < nrec ? lids[t * a.k + jj] : -1;
        const size_t si = ((size_t)(tile * (GKD / PD) + g / PD) * kWave + lrow) * PD + g % PD;
        if constexpr (F == 0)
          sdv[i] = id_ok(e, a.E) ? a.dn_s[(size_t)e * a.dn_s_stride + si] : 0u;
        else
          sdv[i] = id_ok(e, a.E) ? reinterpret_cast<const uint8_t*>(a.dn_s)[(size_t)e * a.dn_s_stride * 2 + si] : 0u;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NPQ; ++i) {
        const int j = q + Q * i, jj = j / GKD, g = j - jj * GKD;
        const int e = j < nrec ? lids[t * a.k + jj] : -1;
        wd[i] = id_ok(e, a.E) ? ld_stream(a.dn_q + (size_t)e * a.dn_q_stride +
                                          ((size_t)(tile * GKD + g) * kWave + lrow) * 16)
                              : make_uint4(0, 0, 0, 0);
      }
      LTRACE(5);
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
      LTRACE(6);
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
            float se = 0.f, so = 0.f;
#pragma unroll
            for (int w = 0; w < 16; w += 2) {
              const half2_t he = __builtin_bit_cast(half2_t, hw[w]);
              const half2_t ho = __builtin_bit_cast(half2_t, hw[w + 1]);
              se += (float)he[0];
              se += (float)he[1];
              so += (float)ho[0];
              so += (float)ho[1];
            }
            uint4* dst = reinterpret_cast<uint4*>(hst[tid]);
#pragma unroll
            for (int w = 0; w < 4; ++w) dst[w] = make_uint4(hw[4 * w], hw[4 * w + 1], hw[4 * w + 2], hw[4 * w + 3]);
            // turns the products with 1024 + u (even dwords) and 1024 + 16 u
            // (odd dwords, whose h is stored divided by 16) into products
            // with u - 8
            hbias[tid] = F == 0 ? -1032.0f * se - 1152.0f * so : 0.f;
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
      LTRACE(7);
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
            if constexpr (F == 0) {
              // nibbles 0, 4 and 1, 5 of each code dword straight from it,
              // 2, 6 and 3, 7 from it shifted by 8: fp16 (1024 + u) and
              // (1024 + 16 u) pairs, as in routed_dot_lds_h
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const uint32_t t8 = wdw[d] >> 8;
                const uint32_t pairs[4] = {(wdw[d] & 0x000F000Fu) | magic, (wdw[d] & 0x00F000F0u) | magic,
                                           (t8 & 0x000F000Fu) | magic, (t8 & 0x00F000F0u) | magic};
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4)
                  pr[d >> 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pairs[k4]),
                                                      __builtin_bit_cast(half2_t, hp[4 * d + k4]), pr[d >> 1], false);
              }
              acc += ldexpf((pr[0] + pr[1]) * bf16_to_f32(sdv[i]), hexp[j]) * lw[p];
            } else {
              // byte k4 of dword d: the E2M1 pair of inputs 8d+2k4, +1 as exact fp16
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const auto f = [&](uint32_t pair, int k4) {
                  pr[d >> 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pair),
                                                      __builtin_bit_cast(half2_t, hp[4 * d + k4]), pr[d >> 1], false);
                };
                f(fp4x2_f16<0>(wdw[d]), 0);
                f(fp4x2_f16<1>(wdw[d]), 1);
                f(fp4x2_f16<2>(wdw[d]), 2);
                f(fp4x2_f16<3>(wdw[d]), 3);
              }
              acc += e8m0_scaled(pr[0] + pr[1], sdv[i], hexp[j]) * lw[p];
            }
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
      LTRACE_WAIT();
      LTRACE(8);
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
  // every record of a token is staged by one thread; the down workgroups
  // of one row block sit 8 ids apart
  return (ling || tiny) && (v.CWG == 0) == (v.NSC == 0) && s.k * (s.I / kGroup) <= kBlock &&
         (s.H / kDnRows) % 8 == 0;
}

// The workgroups of a launch wait for one another; a grid larger than the
// device holds at once still completes (see the file comment), but the
// launch is refused (and the caller takes the separate kernels) unless the
// device holds the leader and one more workgroup.
template <int F, int NI, int GWG, int PG, int CWG, int PD, int NPQ, int NSC, int DG, bool PT>
hipError_t run_layer(const LayerArgs& A, size_t lds, hipStream_t st) {
  auto kern = k_layer<F, NI, GWG, PG, CWG, PD, NPQ, NSC, DG, PT>;
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), kBlock, lds) !=
          hipSuccess)
    return hipErrorInvalidValue;
  if ((int64_t)per_cu * ncu < 2) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kern, dim3(A.g.grid), dim3(kBlock), lds, st, A);
  return hipGetLastError();
}
}  // namespace

#ifdef MOE_LAYER_TRACE
extern "C" int moe_layer_trace_read(void* dst, size_t bytes) {
  if (bytes > sizeof(g_layer_trace)) bytes = sizeof(g_layer_trace);
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_layer_trace), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess ? 0 : -6;
}
#endif

bool layer_supported(const Shape& s, int M) {
  LayerVariant v;
  return M <= kLayerMaxTokens && (int64_t)M * s.k <= kMaxUnits && (int64_t)M * s.E <= kMaxLayerKeys &&
         layer_variant(s, v);
}

hipError_t launch_layer(const Shape& s, const uint8_t* packed, const PackedLayout& PL, const float* router_w,
                        const uint16_t* x, int M, bool route, bool rmsnorm, float eps, uint16_t* x_norm,
                        int32_t* ids, float* w, uint16_t* out, uint8_t* ws, const WsLayout& L, hipStream_t st,
                        bool mxfp4) {
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
  const bool pt = M > 1;
  A.g = layer_roles(s.H, s.E, s.I, s.has_shared, route ? 1 : 0, M, s.k, pt ? 1 : 0);
  A.epoch = reinterpret_cast<uint32_t*>(ws + L.epoch);
  A.arrive = reinterpret_cast<int32_t*>(ws + L.arrive);
  A.rkeys = reinterpret_cast<uint64_t*>(ws + L.rkeys);
  A.rrec = reinterpret_cast<uint64_t*>(ws + L.rrec);
  A.hval = reinterpret_cast<uint64_t*>(ws + L.hval);
  A.hmeta = reinterpret_cast<uint64_t*>(ws + L.hmeta);
  A.hsh = reinterpret_cast<uint64_t*>(ws + L.hsh);
  // router keys (routing in the launch), then the staged tokens and their
  // group corrections
  const size_t lds = ((size_t)M * (route ? s.E : 0) + (size_t)M * (s.H / 2 + s.H / kGroup)) * 4;
#define LAYER_CASE(NI_, GWG_, PG_, CWG_, PD_, NPQ_, NSC_, DG_)                                              \
  if (v.NI == NI_ && v.GWG == GWG_ && v.PG == PG_ && v.CWG == CWG_ && v.PD == PD_ && v.NPQ == NPQ_ &&       \
      v.NSC == NSC_ && v.DG == DG_)                                                                          \
    return mxfp4 ? (pt ? run_layer<1, NI_, GWG_, PG_, CWG_, PD_, NPQ_, NSC_, DG_, true>(A, lds, st)           \
                       : run_layer<1, NI_, GWG_, PG_, CWG_, PD_, NPQ_, NSC_, DG_, false>(A, lds, st))         \
                 : (pt ? run_layer<0, NI_, GWG_, PG_, CWG_, PD_, NPQ_, NSC_, DG_, true>(A, lds, st)           \
                       : run_layer<0, NI_, GWG_, PG_, CWG_, PD_, NPQ_, NSC_, DG_, false>(A, lds, st));
  LAYER_CASE(10, 20, 4, 20, 2, 6, 3, 24)
  LAYER_CASE(10, 20, 4, 0, 2, 6, 0, 24)
  LAYER_CASE(1, 2, 2, 2, 1, 1, 1, 2)
  LAYER_CASE(1, 2, 2, 0, 1, 1, 0, 2)
#undef LAYER_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
