// common.hpp — device helpers and the workspace layout shared by the kernels
// and the host entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace moe {

// The shared expert's K split targets the same bytes per wavefront as the
// routed matrix of the same phase (its K-groups per wavefront).
inline SharedSplit shared_gu_split(int H) { return shared_split_for(H, ksplit_for(H / kGroup).GW); }
inline SharedSplit shared_dn_split(int I) { return shared_split_for(I, ksplit_for(I / kGroup).GW); }

// Stable grouping of the (token, slot) pairs by expert runs in workgroups of
// kPermSeg pairs; per-workgroup expert histograms live in the workspace.
constexpr int kPermSeg = 2048;
inline int perm_groups(long long S) { return (int)((S + kPermSeg - 1) / kPermSeg); }

// Arrival counters are kCntStride ints apart (256 bytes): atomics on one
// line are serialised, so counters that fill at the same time never share one.
constexpr int kCntStride = 64;
// Last-arriver trees: groups of kArriveFan workgroups count on their own
// counter, the last of each group on a top counter.
constexpr int kArriveFan = 16;
// (token, slot) pairs of the one-launch small-M layer (M*k <= this).
constexpr int kMaxUnits = 64;
// Router keys one launch of that layer can hold (M*E <= this).
constexpr int kMaxLayerKeys = 8192;
// Counters its workgroups arrive on (workgroup b on b % this), so that the
// arrivals of one call spread over several lines.
constexpr int kArriveCounters = 8;
// Router workgroups (4 rows each) of up to 512 experts: one top counter and
// one per group of kArriveFan.
constexpr int kRouteCounters = 1 + (512 / 4 + kArriveFan - 1) / kArriveFan;

// Workgroup roles of the one-launch small-M layer, in launch order: the
// leader (workgroup 0: the call's tag, the normalised tokens), router rows
// (4 per workgroup) and selectors (the top-k, published in kSelectors
// copies), both only when the launch routes, shared gate_up (tile x K
// slice), routed gate_up (slot x gate_up tile; slots past the number of
// distinct experts have nothing to do), down (kDnRows output rows each, of
// every token or of one: every routed and the shared down projection of
// those rows, and the output).  S = M*k (token, slot) pairs bound the distinct-expert units.
struct LayerGrid {
  int gSL, gSG, gGU, gDN, grid;  // router rows: workgroups 1 .. gSL-1; selectors gSL .. gSG-1
};
constexpr int kDnRows = 8;
constexpr int kSelectors = 8;
// per_token: one down workgroup per (row block, token) instead of one per
// row block walking the tokens.
inline LayerGrid layer_roles(int H, int E, int I, int has_shared, int route, int M, int k, int per_token) {
  const SharedSplit sg = shared_gu_split(H);
  LayerGrid g;
  g.gSL = 1 + (route ? (E + 3) / 4 : 0);
  g.gSG = g.gSL + (route ? kSelectors : 0);
  g.gGU = g.gSG + (has_shared ? (I / 32) * sg.KS : 0);
  g.gDN = g.gGU + M * k * (I / 32);
  g.grid = g.gDN + (H / kDnRows) * (per_token ? M : 1);
  return g;
}

// Both paths share one header: the error word at offset 0, the small-M
// path's arrival counters, which must stay zero between calls whichever
// path ran last (each counter is reset by the workgroup that completes it),
// and the hand-off words of the one-launch layer.  Those carry the call's
// tag (a 32-bit count of one-launch calls on this workspace, never 0) in
// their high word, so a reader tells this call's data from anything older
// without the words ever being cleared.  Per-call arrays follow the header.
struct WsHeader {
  size_t err;        // int32 sticky error word
  size_t route_cnt;  // int32 [kRouteCounters] spaced: top counter, then one per group
  size_t shgu_cnt;   // int32 [I/32] spaced: K slices finished per shared gate_up tile
  size_t dn_cnt;     // int32 [H/64] spaced: partial rows finished per down tile
  size_t epoch;      // uint32: tag of the last one-launch call
  size_t arrive;     // int32 [kArriveCounters] spaced: workgroups that have read the epoch this call
  size_t rkeys;      // uint64 [kMaxLayerKeys]: router logits [M][E] as order-preserving keys | tag
  size_t rrec;       // uint64 [kSelectors][2][kMaxUnits]: the routing (ids | tag, weight bits | tag) per selector
  size_t hval;       // uint64 [kMaxUnits][I/32][16]: h per (slot, tile) as fp16 pairs | tag
  size_t hmeta;      // uint64 [kMaxUnits][I/32]: the power-of-two exponent of that h | tag
  size_t hsh;        // uint64 [kMaxUnits][I]: shared-expert h per token, fp32 bits | tag
};

// The header is the same for every token count (a call of any M finds the
// counters and hand-off words where the previous call left them).
inline size_t ws_header(int H, int E, int I, int has_shared, WsHeader* w) {
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  const size_t cs = (size_t)4 * kCntStride;
  (void)E;
  w->err = take(4);
  w->route_cnt = take(cs * kRouteCounters);
  w->shgu_cnt = take(cs * (I / 32));
  w->dn_cnt = take(cs * (H / 64));
  w->epoch = take(4);
  w->arrive = take(cs * kArriveCounters);
  w->rkeys = take((size_t)kMaxLayerKeys * 8);
  w->rrec = take((size_t)kSelectors * 2 * kMaxUnits * 8);
  w->hval = take((size_t)kMaxUnits * (I / 32) * 16 * 8);
  w->hmeta = take((size_t)kMaxUnits * (I / 32) * 8);
  w->hsh = take(has_shared ? (size_t)kMaxUnits * I * 8 : 0);
  return off;
}

// Workspace: counters and the sticky error word first, then the per-call
// scratch arrays, each 256-byte aligned.
struct WsLayout : WsHeader {
  size_t logits;                             // fp32 [Mmax][E]
  size_t h;                                  // bf16 [Mmax*k][I]
  size_t h_sh;                               // bf16 [Mmax][I]
  size_t shgu_part;                          // fp32 [Mmax][Tgu][KSgu][64]
  size_t dpart;                              // fp32 [Mmax*k][H]
  size_t shdn_part;                          // fp32 [Mmax][KSdn][H]
  size_t ghist;                              // int32 [perm_groups(Mmax*k)][E] (moe_permute)
  size_t total;
  int Tgu, Tdn, KSgu, KSdn, CWgu, CWdn;
};

inline WsLayout ws_layout(int H, int E, int k, int I, int has_shared, int Mmax) {
  WsLayout w;
  w.Tgu = I / 32;
  w.Tdn = H / 64;
  SharedSplit sg = shared_gu_split(H);
  SharedSplit sd = shared_dn_split(I);
  w.KSgu = sg.KS; w.CWgu = sg.CW;
  w.KSdn = sd.KS; w.CWdn = sd.CW;
  size_t off = ws_header(H, E, I, has_shared, &w);
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  size_t M = (size_t)Mmax;
  w.logits = take(M * E * 4);
  w.h = take(M * k * I * 2 * 2);                  // (hi, lo) per value
  w.h_sh = take(has_shared ? M * I * 2 * 2 : 0);
  w.shgu_part = take(has_shared ? M * w.Tgu * w.KSgu * 64 * 4 : 0);
  w.dpart = take(M * k * H * 4);
  w.shdn_part = take(has_shared ? M * w.KSdn * H * 4 : 0);
  w.ghist = take((size_t)perm_groups((long long)M * k) * E * 4);  // moe_permute
  w.total = off;
  return w;
}

// Rows of one work item of the grouped GEMMs (an expert's sorted rows are cut
// into items of at most this many: three 32-row MFMA blocks).
constexpr int kItemRows = 96;

// Workspace of the many-token (prefill) path.
struct PfLayout : WsHeader {
  size_t logits;                    // fp32 [M][E]
  size_t rt_planes;                 // bf16 [3][E][H] router weights split in three exact parts
  size_t counts, offsets;           // int32 [E], [E+1]
  size_t perm, inv;                 // int32 [S]: pair at each sorted position, sorted position of each pair
  size_t ghist;                     // int32 [perm_groups(S)][E]
  size_t tile_e, tile_j, ntile;     // int32 [items], [items], [1]: work items (expert, row block)
  size_t xh, rexp;                  // fp16 [M][H] scaled rows of x; int32 [M][2]: the exponent r of each
                                    // row's scaling and the exponent bound tx of its squared L2 norm
  size_t hbuf;                      // fp16 [S][I] scaled h per sorted position
  size_t hsh;                       // bf16 [2][M][I] shared-expert h as (hi, lo) planes
  size_t y, ysh;                    // fp16 [S][H] per sorted position (scaled), fp32 [M][H]
  size_t total;
  int items;                        // bound on the routed work items
};

inline PfLayout pf_layout(int H, int E, int k, int I, int has_shared, int M) {
  PfLayout w;
  size_t off = ws_header(H, E, I, has_shared, &w);
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  const size_t S = (size_t)M * k;
  // sum over experts of ceil(count / kItemRows) <= E + S / kItemRows
  w.items = E + (int)((S + kItemRows - 1) / kItemRows);
  w.logits = take((size_t)M * E * 4);
  w.rt_planes = take((size_t)3 * E * H * 2);
  w.counts = take((size_t)E * 4);
  w.offsets = take((size_t)(E + 1) * 4);
  w.perm = take(S * 4);
  w.inv = take(S * 4);
  w.ghist = take((size_t)perm_groups((long long)S) * E * 4);
  w.tile_e = take((size_t)w.items * 4);
  w.tile_j = take((size_t)w.items * 4);
  w.ntile = take(4);
  w.xh = take((size_t)M * H * 2);
  w.rexp = take((size_t)M * 8);
  w.hbuf = take(S * I * 2);
  w.hsh = take(has_shared ? (size_t)2 * M * I * 2 : 0);
  w.y = take(S * H * 2);
  w.ysh = take(has_shared ? (size_t)M * H * 4 : 0);
  w.total = off;
  return w;
}

// ---------------------------------------------------------------- device helpers

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Activations read by whole wavefronts at uniform addresses go through the
// constant address space, so they are fetched with scalar loads into SGPRs
// (they are never written while a kernel reads them).
typedef __attribute__((address_space(4))) const uint32_t* cptr32;
__device__ __forceinline__ cptr32 as_scalar_ptr(const void* p) { return (cptr32)(p); }

// bf16 (128, 128) in both halves, kept in a VGPR the compiler cannot fold, so
// that (w & 0x000F000F) | magic becomes a single v_and_or_b32.
__device__ __forceinline__ uint32_t bf16_pair_magic() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(m));
  return m;
}
// fp16 (1024, 1024) likewise: (w & 0x000F000F) | magic is the fp16 pair
// (1024 + u0, 1024 + u1), exact.
__device__ __forceinline__ uint32_t fp16_pair_magic() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// One 32-input group of a routed row against 16 dwords of bf16 activations:
// returns init + sum_k (128 + u_k) * x_k.  With init = -136 * sum_k x_k this
// is sum_k (u_k - 8) * x_k = sum_k q_k * x_k: every code is turned into the
// exact bf16 value 128 + u by OR-ing it under the exponent of 128.
__device__ __forceinline__ float dot_group_q4(uint4 w, const uint32_t* xg, float init, uint32_t magic) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float p = init;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t pair = ((wd[d] >> (4 * i)) & 0x000F000Fu) | magic;
      p = dot2_bf16(pair, xg[4 * d + i], p);
    }
  }
  return p;
}

// The same against an activation kept as a bf16 (hi, lo) pair, hi + lo
// carrying ~16 significant bits: dwords 0..15 of xg hold hi, 16..31 lo.
__device__ __forceinline__ float dot_group_q4_hilo(uint4 w, const uint32_t* xg, float init, uint32_t magic) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float p = init;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t pair = ((wd[d] >> (4 * i)) & 0x000F000Fu) | magic;
      p = dot2_bf16(pair, xg[4 * d + i], p);
      p = dot2_bf16(pair, xg[16 + 4 * d + i], p);
    }
  }
  return p;
}

// An fp32 value as two bf16 whose sum carries ~16 significant bits; stored
// as one group of 32 hi values followed by the group's 32 lo values.
__device__ __forceinline__ void store_hilo(uint16_t* __restrict__ group_base, int i, float v) {
  const uint16_t hi = f32_to_bf16(v);
  const uint16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
  group_base[i] = hi;
  group_base[32 + i] = lo;
}

// store_hilo through agent-coherent stores (read by other workgroups of the
// same launch).
__device__ __forceinline__ void store_hilo_coherent(uint16_t* __restrict__ group_base, int i, float v);

// Eight bf16 weights (natural order) against 4 dwords of bf16 activations.
__device__ __forceinline__ float dot_chunk_bf16(uint4 w, const uint32_t* xc, float acc) {
  acc = dot2_bf16(w.x, xc[0], acc);
  acc = dot2_bf16(w.y, xc[1], acc);
  acc = dot2_bf16(w.z, xc[2], acc);
  acc = dot2_bf16(w.w, xc[3], acc);
  return acc;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The same sum through the ALU's lane moves instead of the LDS crossbar:
// lane pairs, quads, 8-lane and 16-lane groups by DPP, the two rows of each
// half by a swizzle, the two halves by scalar reads; every lane gets the
// same bits.  A mirror move pairs each lane with a lane of the other group,
// whose value at that point is that group's sum, so each step adds the same
// two partial sums as a butterfly would (addition commutes).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_move<0x141>(v);  // row_half_mirror: the other quad of 8 lanes
  v += dpp_move<0x140>(v);  // row_mirror: the other 8 lanes of a row
  v += __uint_as_float((uint32_t)__builtin_amdgcn_ds_swizzle((int)__float_as_uint(v), 0x401F));  // lane ^ 16
  const float h0 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
  const float h1 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 32));
  return h0 + h1;
}

// 16 bytes of a weight stream, read once per launch: a non-temporal load, so
// the bytes pass the CU's vector cache without being kept there.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld_stream_f4(const float* p) {
  const uint4 v = ld_stream(p);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// The largest v of the wavefront, in every lane, by the same row moves as
// wave_sum_dpp (no LDS round trip per step).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));
  v = fmaxf(v, dpp_move<0x4E>(v));
  v = fmaxf(v, dpp_move<0x141>(v));
  v = fmaxf(v, dpp_move<0x140>(v));
  v = fmaxf(v, __uint_as_float((uint32_t)__builtin_amdgcn_ds_swizzle((int)__float_as_uint(v), 0x401F)));
  const float h0 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
  const float h1 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 32));
  return fmaxf(h0, h1);
}

// Two floats to a bf16 pair (round to nearest even), in one instruction.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Data handed between workgroups of one launch.  They may sit on different
// XCDs, whose L2 caches are not coherent with each other, and an agent-scope
// release fence (a full L2 write-back) per workgroup costs several
// microseconds per launch on this part.  So the data itself travels with
// agent-coherent stores (written through to the coherent level), and the
// only ordering needed is that a producer's stores have completed before its
// arrival or flag is seen.  Agent-coherent loads are served one at a time
// per wavefront (about 0.1 us each even on an idle part), so they are kept
// for polls; data is read with ld_fresh (below).
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A plain load of data stored agent-coherently by other workgroups of this
// launch, issued after the hand-off that publishes it (behind a barrier with
// an acquire fence).  Correct because the reader's caches cannot hold an
// older copy: they start each launch invalidated, the reader touches the
// line for the first time here, and every byte of a line read this way was
// written before its hand-off.  Unlike ld_coherent it pipelines.
template <typename T>
__device__ __forceinline__ T ld_fresh(const T* p) { return *p; }

__device__ __forceinline__ void st_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_coherent(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Last-arriver protocol: each thread waits for its own coherent stores to
// complete (s_waitcnt 0), the barrier gathers the workgroup, thread 0 counts
// the arrival.  The workgroup that arrives last sees every other
// workgroup's coherent stores, resets the counter for the next call and gets
// true in all its threads.  Loads that follow read the others' data with
// ld_fresh.
__device__ __forceinline__ bool arrive_last(int* counter, int expected, int* lds_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == expected - 1);
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// arrive_last over n workgroups numbered i < n in groups of kArriveFan: each
// group counts on cnt[(i / kArriveFan + 1) * kCntStride], the last of each
// group on cnt[0].  A store completed before a workgroup's arrival is seen by
// the last of all (each level's last arriver saw the arrivals below it).
__device__ __forceinline__ bool arrive_last_tree(int* cnt, int i, int n, int* lds_flag) {
  const int g = i / kArriveFan;
  const int in_g = (n - g * kArriveFan) < kArriveFan ? (n - g * kArriveFan) : kArriveFan;
  if (!arrive_last(&cnt[(g + 1) * kCntStride], in_g, lds_flag)) return false;
  return arrive_last(cnt, (n + kArriveFan - 1) / kArriveFan, lds_flag);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses,
// not for its in-flight global loads (a plain __syncthreads also waits for
// outstanding global memory operations, which would stall every wavefront
// until most of its weight stream had landed).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void store_hilo_coherent(uint16_t* __restrict__ group_base, int i, float v) {
  const uint16_t hi = f32_to_bf16(v);
  const uint16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
  st_coherent(&group_base[i], hi);
  st_coherent(&group_base[32 + i], lo);
}

// Polls that give up after this many rounds set bit 1 of the error word.
constexpr int kSpinLimit = 1 << 22;

// A pointer passed through an empty asm after a wait: loads through it
// (scalar loads from the constant address space in particular, which the
// compiler may otherwise hoist) are issued after the wait.
template <typename T>
__device__ __forceinline__ T* after_wait(T* p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  uint32_t lo = (uint32_t)uniform((int)(uint32_t)v), hi = (uint32_t)uniform((int)(v >> 32));
  asm volatile("" : "+s"(lo), "+s"(hi));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

}  // namespace moe
