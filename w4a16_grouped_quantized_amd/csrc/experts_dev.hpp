// experts_dev.hpp — device code shared by the small-M expert kernels: the
// launch arguments, the distinct-expert units of a call, the INT4 and BF16
// dot products of one wavefront's K-run, and the weighted combine.
#pragma once
#include "launch.hpp"

namespace moe {

struct ExpArgs {
  int M, E, k, H, I, S, has_shared;
  int Tgu, Tdn, KSgu, KSdn;
  const int32_t* __restrict__ ids;
  const float* __restrict__ topk_w;
  const uint16_t* __restrict__ x;
  // packed weights
  const uint8_t* __restrict__ gu_q;
  const uint16_t* __restrict__ gu_s;
  const uint8_t* __restrict__ dn_q;
  const uint16_t* __restrict__ dn_s;
  const uint16_t* __restrict__ sh_gu;
  const uint16_t* __restrict__ sh_dn;
  size_t gu_q_stride, gu_s_stride, dn_q_stride, dn_s_stride;  // bytes / elements (scales)
  // workspace
  int32_t* __restrict__ err;
  int32_t* __restrict__ shgu_cnt;
  int32_t* __restrict__ dn_cnt;
  uint16_t* __restrict__ h;       // [S][I/32][hi 32 | lo 32]
  uint16_t* __restrict__ h_sh;    // [M][I/32][hi 32 | lo 32]
  float* __restrict__ shgu_part;  // [M][Tgu][KSgu][64]
  float* __restrict__ dpart;      // [S][H]
  float* __restrict__ shdn_part;  // [M][KSdn][H]
  uint16_t* __restrict__ out;     // [M][H]
};

struct UnitLds {
  int first[kMaxExperts];
  int mem[kMaxSlots];
  int wcnt[kWavesPerBlock];
  int e, nmem, flag;
  float red[kWavesPerBlock][kWave];
  float bias[kMaxGroups];
};

// The distinct valid experts of ids[0..S) are numbered in order of first
// occurrence; a workgroup serving unit u needs that expert and the slots
// routed to it (ascending).
struct Unit {
  int e;          // -1 when the call has fewer than u + 1 distinct experts
  int nmem;
  uint64_t mask;  // member slots as bits (S <= 64)
};

// S <= 64: every wavefront finds the unit on its own with cross-lane reads
// (no LDS, no barrier).  Lane p holds slot p.
// COH: ids were written by another workgroup of the same launch.
template <bool COH = false>
__device__ __forceinline__ Unit find_unit_wave(const int32_t* __restrict__ ids, int S, int E, int u, int lane) {
  const int id = lane < S ? (COH ? ld_coherent(&ids[lane]) : ids[lane]) : -1;
  const bool valid = id >= 0 && id < E;
  bool first = valid;
  for (int q = 0; q < S; ++q) {
    const int v = __builtin_amdgcn_readlane(id, q);
    first = first && !(q < lane && v == id);
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint64_t fb = __ballot(first);
  const int rank = __popcll(fb & lt);
  const uint64_t sel = __ballot(first && rank == u);
  Unit U;
  if (sel == 0) {
    U.e = -1; U.nmem = 0; U.mask = 0;
    return U;
  }
  U.e = __builtin_amdgcn_readlane(id, __ffsll((unsigned long long)sel) - 1);
  U.mask = __ballot(valid && id == U.e);
  U.nmem = __popcll(U.mask);
  return U;
}

// Any S (<= kMaxSlots): the workgroup builds a first-occurrence table and the
// member list in LDS.  Whole-workgroup call.
__device__ void find_unit_lds(const int32_t* __restrict__ ids, int S, int E, int u, UnitLds& L) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < E; e += kBlock) L.first[e] = 0x7FFFFFFF;
  if (tid == 0) { L.e = -1; L.nmem = 0; }
  lds_sync();
  for (int p = tid; p < S; p += kBlock) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicMin(&L.first[e], p);
  }
  lds_sync();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int running = 0;
  for (int base = 0; base < S; base += kBlock) {
    const int p = base + tid;
    const int e = p < S ? ids[p] : -1;
    const bool f = (e >= 0 && e < E) && L.first[e] == p;
    const uint64_t bal = __ballot(f);
    if (lane == 0) L.wcnt[wave] = __popcll(bal);
    lds_sync();
    int before = running, total = running;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      if (w < wave) before += L.wcnt[w];
      total += L.wcnt[w];
    }
    if (f && before + __popcll(bal & lt) == u) L.e = e;
    running = total;
    lds_sync();
    if (running > u) break;
  }
  const int eu = L.e;
  if (eu < 0) return;
  int count = 0;
  for (int base = 0; base < S; base += kBlock) {
    const int p = base + tid;
    const bool m = p < S && ids[p] == eu;
    const uint64_t bal = __ballot(m);
    if (lane == 0) L.wcnt[wave] = __popcll(bal);
    lds_sync();
    int before = count, total = count;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      if (w < wave) before += L.wcnt[w];
      total += L.wcnt[w];
    }
    if (m) L.mem[before + __popcll(bal & lt)] = p;
    count = total;
    lds_sync();
  }
  if (tid == 0) L.nmem = count;
  lds_sync();
}

__device__ __forceinline__ Unit find_unit(const int32_t* __restrict__ ids, int S, int E, int u, UnitLds& L) {
  if (S <= kWave) return find_unit_wave(ids, S, E, u, threadIdx.x & 63);
  find_unit_lds(ids, S, E, u, L);
  Unit U;
  U.e = L.e; U.nmem = L.nmem; U.mask = 0;
  return U;
}

// Slot of member c (called with c = 0, 1, ... in order; `m` carries the
// remaining mask between calls when S <= 64).
__device__ __forceinline__ int member_slot(int S, int c, uint64_t& m, const UnitLds& L) {
  if (S <= kWave) {
    const int p = __ffsll((unsigned long long)m) - 1;
    m &= m - 1;
    return p;
  }
  return uniform(L.mem[c]);
}

// P bf16 scales of one lane-load, as float.
template <int P>
struct ScalePack {
  uint32_t w[(P + 1) / 2];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ p) {
    if constexpr (P == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x; w[1] = v.y;
    } else if constexpr (P == 2) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      w[0] = *p;
    }
  }
  __device__ __forceinline__ float get(int q) const {
    const uint32_t v = w[q >> 1];
    return (q & 1) ? __uint_as_float(v & 0xFFFF0000u) : __uint_as_float(v << 16);
  }
};

// -136 * (sum of the 32 values of group g of act): the correction that turns
// sum (128 + u) * x into sum q * x.  Loaded by one lane per group.  With HILO
// the group holds 32 hi then 32 lo bf16 values whose pairwise sums are the
// activation, and the sum runs over all 64.
template <bool HILO>
struct GroupBias {
  static constexpr int NV = HILO ? 8 : 4;
  uint4 v[NV];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ act, int g) {
    const uint4* p = reinterpret_cast<const uint4*>(act + g * kGroup * (HILO ? 2 : 1));
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = p[i];
  }
  __device__ __forceinline__ float value() const {
    const uint32_t one2 = 0x3F803F80u;  // bf16 (1.0, 1.0)
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      s = dot2_bf16(v[i].x, one2, s);
      s = dot2_bf16(v[i].y, one2, s);
      s = dot2_bf16(v[i].z, one2, s);
      s = dot2_bf16(v[i].w, one2, s);
    }
    return -136.0f * s;
  }
};

// Group corrections read by routed_dot: from LDS, or from global memory
// through scalar loads (wavefront-uniform values).
__device__ __forceinline__ float bias_at(const float* b, int i) { return b[i]; }
__device__ __forceinline__ float bias_at(cptr32 b, int i) { return __uint_as_float(b[i]); }

// One wavefront's K-run of a routed tile against one activation vector;
// bias[g] holds the group corrections of that vector (LDS).  HILO: the
// activation is stored as (hi, lo) bf16 groups (see store_hilo).  The
// activation dwords of B groups are fetched with one batch of scalar loads
// (scalar loads return out of order, so each batch costs one full wait).
template <int GW, int P, bool HILO, typename BiasPtr = const float*>
__device__ __forceinline__ float routed_dot(const uint4 (&wq)[GW], const ScalePack<P> (&sc)[GW / P],
                                            const uint16_t* __restrict__ act, BiasPtr bias, int g0,
                                            uint32_t magic) {
  constexpr int DW = HILO ? 32 : 16;  // activation dwords per group
  constexpr int B = HILO ? 1 : 2;     // groups per scalar-load batch
  float acc = 0.f, lag1 = 0.f, lag2 = 0.f;
#pragma unroll
  for (int g = 0; g < GW; g += B) {
    // The batch address passes through an empty asm that also consumes the
    // accumulator as it stood two batches earlier: the loads of batch i can
    // start once batch i-2 is done, i.e. one batch of scalar prefetch, and
    // the compiler cannot hoist all of them (they would not fit in SGPRs).
    uint64_t addr = reinterpret_cast<uint64_t>(act) + (uint64_t)(g0 + g) * DW * 4;
    addr = ((uint64_t)(uint32_t)uniform((int)(addr >> 32)) << 32) | (uint32_t)uniform((int)(uint32_t)addr);
    asm volatile("" : "+s"(addr) : "v"(lag2));
    const cptr32 xb = as_scalar_ptr(reinterpret_cast<const void*>(addr));
    uint32_t xs[B][DW];
#pragma unroll
    for (int bb = 0; bb < B; ++bb)
#pragma unroll
      for (int i = 0; i < DW; ++i) xs[bb][i] = (g + bb < GW) ? xb[bb * DW + i] : 0u;
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
      const int gi = g + bb;
      if (gi < GW) {
        // Opaque copy: keeps the code-pair extraction next to its dot
        // products instead of letting it be hoisted out of the caller's
        // token loop (16 extracted pairs per group would stay in VGPRs).
        uint4 w = wq[gi];
        asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
        float pr;
        if constexpr (HILO) pr = dot_group_q4_hilo(w, xs[bb], bias_at(bias, g0 + gi), magic);
        else pr = dot_group_q4(w, xs[bb], bias_at(bias, g0 + gi), magic);
        acc = fmaf(sc[gi / P].get(gi % P), pr, acc);
      }
    }
    lag2 = lag1;
    lag1 = acc;
  }
  return acc;
}

// routed_dot against an activation staged in LDS (xl: the token's inputs as
// bf16 pairs in natural order, 16 dwords per group; bias: its group
// corrections).  Every lane of a wavefront reads the same addresses, so the
// reads are broadcasts.
template <int GW, int P>
__device__ __forceinline__ float routed_dot_lds(const uint4 (&wq)[GW], const ScalePack<P> (&sc)[GW / P],
                                                const uint32_t* xl, const float* bias, int g0, uint32_t magic) {
  float acc = 0.f;
#pragma unroll
  for (int gi = 0; gi < GW; ++gi) {
    const uint4* xp = reinterpret_cast<const uint4*>(xl + (g0 + gi) * 16);
    uint32_t xs[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = xp[q];
      xs[4 * q] = v.x; xs[4 * q + 1] = v.y; xs[4 * q + 2] = v.z; xs[4 * q + 3] = v.w;
    }
    // opaque copies, as in routed_dot: the code-pair extraction and the
    // scale's conversion stay next to their use instead of being hoisted
    // out of the caller's token loop (which would hold 16 pairs and a float
    // per group in registers)
    uint4 w = wq[gi];
    asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
    uint32_t sw = sc[gi / P].w[(gi % P) >> 1];
    asm volatile("" : "+v"(sw));
    const float scale = ((gi % P) & 1) ? __uint_as_float(sw & 0xFFFF0000u) : __uint_as_float(sw << 16);
    const float pr = dot_group_q4(w, xs, bias[g0 + gi], magic);
    acc = fmaf(scale, pr, acc);
    // one group's activation reads in flight at a time: hoisting them all
    // would take 16 registers per group
    __builtin_amdgcn_sched_barrier(0);
  }
  return acc;
}

// routed_dot_lds against the fp16 copy of a staged token (to_fp16_tokens):
// xh holds the inputs times 2^-r as fp16 pairs in natural order, the pairs
// of odd dwords divided by 16 once more; bias the matching group
// corrections.  Under the fp16 exponent of 1024 a code at bits 0-3 of a
// half is the exact value 1024 + u, and one at bits 4-7 the exact value
// 1024 + 16 u (fp16 keeps 10 mantissa bits), so of a code dword's four pairs
// (inputs 2i, 2i+1 at nibbles i and 4 + i) pairs 0 and 1 come straight from
// the dword and pairs 2 and 3 from it shifted by 8: five instructions per
// dword where bf16 (7 mantissa bits) needs seven.  The odd pairs' extra
// factor 16 is the one their inputs were divided by.  Returns the sum
// times 2^-r.
// OPQ: the opaque copies of routed_dot_lds, for calls inside a loop over
// tokens (a call outside any loop has nothing to be hoisted out of).
template <int GW, int P, bool OPQ = true>
__device__ __forceinline__ float routed_dot_lds_h(const uint4 (&wq)[GW], const ScalePack<P> (&sc)[GW / P],
                                                  const uint32_t* xh, const float* bias, int g0, uint32_t magic16) {
  float acc = 0.f;
#pragma unroll
  for (int gi = 0; gi < GW; ++gi) {
    const uint4* xp = reinterpret_cast<const uint4*>(xh + (g0 + gi) * 16);
    uint32_t xs[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = xp[q];
      xs[4 * q] = v.x; xs[4 * q + 1] = v.y; xs[4 * q + 2] = v.z; xs[4 * q + 3] = v.w;
    }
    uint4 w = wq[gi];
    uint32_t sw = sc[gi / P].w[(gi % P) >> 1];
    if constexpr (OPQ) {  // opaque copies, as in routed_dot_lds
      asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
      asm volatile("" : "+v"(sw));
    }
    const float scale = ((gi % P) & 1) ? __uint_as_float(sw & 0xFFFF0000u) : __uint_as_float(sw << 16);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    float pr = bias[g0 + gi];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t t = wd[d] >> 8;
      const auto f = [&](uint32_t pair, uint32_t x) {
        pr = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pair), __builtin_bit_cast(half2_t, x), pr, false);
      };
      f((wd[d] & 0x000F000Fu) | magic16, xs[4 * d]);
      f((wd[d] & 0x00F000F0u) | magic16, xs[4 * d + 1]);
      f((t & 0x000F000Fu) | magic16, xs[4 * d + 2]);
      f((t & 0x00F000F0u) | magic16, xs[4 * d + 3]);
    }
    acc = fmaf(scale, pr, acc);
    // one group's activation reads in flight at a time
    __builtin_amdgcn_sched_barrier(0);
  }
  return acc;
}

// ---- MXFP4 routed experts (tiled layout, codes as the checkpoint stores
// them, E8M0 scale bytes packed P per lane-load)

// P E8M0 scale bytes of consecutive groups.
template <int P>
struct ScaleBytes {
  uint32_t w;
  __device__ __forceinline__ void load(const uint8_t* __restrict__ p) {
    if constexpr (P == 4) w = *reinterpret_cast<const uint32_t*>(p);
    else if constexpr (P == 2) w = *reinterpret_cast<const uint16_t*>(p);
    else w = *p;
  }
  __device__ __forceinline__ uint32_t get(int q) const { return (w >> (8 * q)) & 0xFFu; }
};

// v * 2^(c - 127), exact (the E8M0 scale c; c = 255 is NaN).
__device__ __forceinline__ float e8m0_scaled(float v, uint32_t c, int extra = 0) {
  return c == 255u ? __builtin_nanf("") : ldexpf(v, (int)c - 127 + extra);
}

// Byte BYTE of v (two E2M1 codes, the low nibble first) as an exact bf16 or
// fp16 pair, by the part's scaled converters with scale 1.
template <int BYTE>
__device__ __forceinline__ uint32_t fp4x2_bf16(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((int)v, 1.0f, BYTE));
}
template <int BYTE>
__device__ __forceinline__ uint32_t fp4x2_f16(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, BYTE));
}

// One 32-input MXFP4 group (byte b of dword d: inputs 8d+2b, 8d+2b+1)
// against 16 dwords of bf16 activations in natural pairs, unscaled.
__device__ __forceinline__ float dot_group_fp4(uint4 w, const uint32_t* xg) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float p = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    p = dot2_bf16(fp4x2_bf16<0>(wd[d]), xg[4 * d], p);
    p = dot2_bf16(fp4x2_bf16<1>(wd[d]), xg[4 * d + 1], p);
    p = dot2_bf16(fp4x2_bf16<2>(wd[d]), xg[4 * d + 2], p);
    p = dot2_bf16(fp4x2_bf16<3>(wd[d]), xg[4 * d + 3], p);
  }
  return p;
}

// routed_dot_lds for MXFP4 rows: each group's sum scaled by its E8M0 scale.
template <int GW, int P>
__device__ __forceinline__ float routed_dot_lds_fp4(const uint4 (&wq)[GW], const ScaleBytes<P> (&sc)[GW / P],
                                                    const uint32_t* xl, int g0) {
  float acc = 0.f;
#pragma unroll
  for (int gi = 0; gi < GW; ++gi) {
    const uint4* xp = reinterpret_cast<const uint4*>(xl + (g0 + gi) * 16);
    uint32_t xs[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = xp[q];
      xs[4 * q] = v.x; xs[4 * q + 1] = v.y; xs[4 * q + 2] = v.z; xs[4 * q + 3] = v.w;
    }
    uint4 w = wq[gi];
    asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
    uint32_t sw = sc[gi / P].w;
    asm volatile("" : "+v"(sw));
    acc += e8m0_scaled(dot_group_fp4(w, xs), (sw >> (8 * (gi % P))) & 0xFFu);
    __builtin_amdgcn_sched_barrier(0);
  }
  return acc;
}

// Shared BF16 rows (CW chunks of 8 inputs from chunk c0 on) against an
// activation staged in LDS as bf16 pairs (4 dwords per chunk).
template <int CW>
__device__ __forceinline__ float shared_dot_lds(const uint4 (&wc)[CW], const uint32_t* xl, int c0) {
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    const uint4 v = *reinterpret_cast<const uint4*>(xl + (c0 + c) * 4);
    const uint32_t xs[4] = {v.x, v.y, v.z, v.w};
    acc = dot_chunk_bf16(wc[c], xs, acc);
  }
  return acc;
}

// Shared BF16 rows: CW chunks of 8 inputs from chunk c0 on.
template <int CW, bool HILO>
__device__ __forceinline__ float shared_dot(const uint4 (&wc)[CW], const uint16_t* __restrict__ act, int c0) {
  const cptr32 a32 = as_scalar_ptr(act);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    uint32_t xs[HILO ? 8 : 4];
    if constexpr (HILO) {
      const int cc = c0 + c;  // group cc / 4, quarter cc % 4
      const cptr32 hi = a32 + (cc >> 2) * 32 + (cc & 3) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) { xs[i] = hi[i]; xs[4 + i] = hi[16 + i]; }
      acc = dot_chunk_bf16(wc[c], xs, acc);
      acc = dot_chunk_bf16(wc[c], xs + 4, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[i] = a32[(c0 + c) * 4 + i];
      acc = dot_chunk_bf16(wc[c], xs, acc);
    }
  }
  return acc;
}

// -136 * (sum of group g of an activation staged in LDS): 16 dwords, or 32
// with HILO (hi then lo), summed as bf16 pairs in a fixed order.
template <bool HILO>
__device__ __forceinline__ float group_bias_lds(const uint32_t* act, int g) {
  constexpr int DW = HILO ? 32 : 16;
  const uint32_t one2 = 0x3F803F80u;
  const uint4* p = reinterpret_cast<const uint4*>(act + g * DW);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < DW / 4; ++i) {
    const uint4 v = p[i];
    s = dot2_bf16(v.x, one2, s);
    s = dot2_bf16(v.y, one2, s);
    s = dot2_bf16(v.z, one2, s);
    s = dot2_bf16(v.w, one2, s);
  }
  return -136.0f * s;
}

// out[t][n] = sum_j partial[t*k+j][n] + sum_s shared_part[t][s][n] for the 64
// rows n of tile b, in slot order then slice order, rounded to bf16.  The
// routed partials arrive already multiplied by their slot's weight.  With
// check_ids, slots whose id is out of range add nothing (their partial was
// never written) and are recorded in the error word.  All loads of a block
// of 8 slots are issued before any of them is used.
__device__ void combine_tile(const ExpArgs& a, int b, bool check_ids) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = 64 * b + lane;
  bool bad = false;
  for (int t = wave; t < a.M; t += kWavesPerBlock) {
    float y = 0.f;
    for (int j0 = 0; j0 < a.k; j0 += 8) {
      int ev[8];
      float pv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int p = t * a.k + j0 + jj;
        const bool in = j0 + jj < a.k;
        ev[jj] = (in && check_ids) ? a.ids[p] : 0;
        pv[jj] = in ? ld_fresh(&a.dpart[(size_t)p * a.H + n]) : 0.f;
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const bool ok = j0 + jj < a.k && ev[jj] >= 0 && ev[jj] < a.E;
        bad = bad || (j0 + jj < a.k && !ok);
        y = ok ? y + pv[jj] : y;
      }
    }
    if (a.has_shared) {
      float sv[kMaxKSplit];
#pragma unroll
      for (int s2 = 0; s2 < kMaxKSplit; ++s2)
        sv[s2] = s2 < a.KSdn ? ld_fresh(&a.shdn_part[((size_t)t * a.KSdn + s2) * a.H + n]) : 0.f;
#pragma unroll
      for (int s2 = 0; s2 < kMaxKSplit; ++s2) y += sv[s2];
    }
    a.out[(size_t)t * a.H + n] = f32_to_bf16(y);
  }
  if (bad && b == 0 && lane == 0) atomicOr(a.err, 1);
}

// Launch arguments of the expert kernels (host side).
inline ExpArgs make_expert_args(const Shape& s, const uint8_t* packed, const PackedLayout& PL, const uint16_t* x,
                         int M, const int32_t* ids, const float* w, uint16_t* out, uint8_t* ws,
                         const WsLayout& L) {
  ExpArgs a;
  a.M = M; a.E = s.E; a.k = s.k; a.H = s.H; a.I = s.I; a.S = M * s.k; a.has_shared = s.has_shared;
  a.Tgu = L.Tgu; a.Tdn = L.Tdn; a.KSgu = L.KSgu; a.KSdn = L.KSdn;
  a.ids = ids; a.topk_w = w; a.x = x;
  a.gu_q = packed + PL.gu_q;
  a.gu_s = reinterpret_cast<const uint16_t*>(packed + PL.gu_s);
  a.dn_q = packed + PL.dn_q;
  a.dn_s = reinterpret_cast<const uint16_t*>(packed + PL.dn_s);
  a.sh_gu = reinterpret_cast<const uint16_t*>(packed + PL.sh_gu);
  a.sh_dn = reinterpret_cast<const uint16_t*>(packed + PL.sh_dn);
  a.gu_q_stride = PL.gu_q_stride; a.gu_s_stride = PL.gu_s_stride / 2;
  a.dn_q_stride = PL.dn_q_stride; a.dn_s_stride = PL.dn_s_stride / 2;
  a.err = reinterpret_cast<int32_t*>(ws + L.err);
  a.shgu_cnt = reinterpret_cast<int32_t*>(ws + L.shgu_cnt);
  a.dn_cnt = reinterpret_cast<int32_t*>(ws + L.dn_cnt);
  a.h = reinterpret_cast<uint16_t*>(ws + L.h);
  a.h_sh = reinterpret_cast<uint16_t*>(ws + L.h_sh);
  a.shgu_part = reinterpret_cast<float*>(ws + L.shgu_part);
  a.dpart = reinterpret_cast<float*>(ws + L.dpart);
  a.shdn_part = reinterpret_cast<float*>(ws + L.shdn_part);
  a.out = out;
  return a;
}

}  // namespace moe
