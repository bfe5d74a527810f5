// experts_fmt.hip — the routed experts in the two other formats the pages
// serve, for decode and verify (M <= 8 tokens): MXFP4 (bpdata.com
// Ling-3.0-flash MoE article, model section and "Optimalizáció 1": the FP4
// checkpoint run with MXFP4 MoE kernels; E2M1 codes with one E8M0 scale per
// 32 inputs) and block FP8 (vLLM recipe page "inclusionAI/Ling-3.0-flash",
// Overview and Prerequisites: the serialized block-FP8 checkpoint with BF16
// compute; E4M3 codes with one float32 scale per 128 x 128 block).  The
// shared expert stays BF16, as in the W4A16 layer.
//
// Weights are read in their plain row-major layout: every row is contiguous,
// so 16-byte lane loads of consecutive chunks are contiguous too.  A chunk is
// one scale group for MXFP4 (32 codes), 16 codes inside one 128-column block
// for FP8, 8 values for BF16.  The part's scaled converters widen FP4 and FP8
// codes to exact BF16 pairs (scale 1), v_dot2_f32_bf16 multiplies them with
// the inputs, and each chunk's sum is scaled once (an exact power of two for
// MXFP4).
//
// Two launches:
//   k_fmt_gate_up  one workgroup per (distinct expert, block of rows) of W1/W3
//                  and per block of the shared expert's rows, each block
//                  holding matching gate and up rows: every chunk's product
//                  per token into LDS, each row summed in chunk order, then
//                  h = silu(gate) * up of the block's rows into the workspace
//                  as a bf16 (hi, lo) pair per value;
//   k_fmt_down     one workgroup per block of output rows: the h of every
//                  slot of a token and of the shared expert staged in LDS,
//                  the down rows' chunk products, and per row
//                  sum_j w_j * (W2_j h_j) + W2_sh h_sh in slot order.
#include <algorithm>

#include "experts_dev.hpp"

namespace moe {

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_f;

// Most rows of one gate_up item (half gate rows, half the matching up rows).
constexpr int kFmtMaxItemRows = 256;
// 16-byte loads per thread that stage the tokens (gate_up) or h (down).
constexpr int kFmtStage = 8;

__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_f, a), __builtin_bit_cast(bf16x2_f, b), c, false);
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v, 1.0f, HI));
}

// A matrix of one format: codes (row-major, rows of `rowbytes`), scales, K.
struct FmtMat {
  const uint8_t* q;
  const void* s;
  int K;
};

// The chunk's codes against x (bf16 pairs of the chunk's columns), unscaled.
template <int F>
__device__ __forceinline__ float chunk_dot(uint4 w, const uint32_t* x) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  float acc = 0.f;
  if constexpr (F == kFmtMxfp4) {  // 32 E2M1 codes, byte b of dword i = columns 8i + 2b, +1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fdot2(fp4x2_bf16<0>(d[i]), x[4 * i], acc);
      acc = fdot2(fp4x2_bf16<1>(d[i]), x[4 * i + 1], acc);
      acc = fdot2(fp4x2_bf16<2>(d[i]), x[4 * i + 2], acc);
      acc = fdot2(fp4x2_bf16<3>(d[i]), x[4 * i + 3], acc);
    }
  } else if constexpr (F == kFmtFp8Block) {  // 16 E4M3 codes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fdot2(fp8x2_bf16<false>(d[i]), x[2 * i], acc);
      acc = fdot2(fp8x2_bf16<true>(d[i]), x[2 * i + 1], acc);
    }
  } else {  // 8 bf16
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fdot2(d[i], x[i], acc);
  }
  return acc;
}

template <int F>
constexpr int chunk_cols() { return F == kFmtMxfp4 ? 32 : (F == kFmtFp8Block ? 16 : 8); }

// Scale of chunk c of row n (what its chunk_dot is multiplied by), as raw
// bits: the E8M0 byte for MXFP4, the fp32 bits for FP8.  Requested with the
// codes and decoded only where it is used, so that no instruction needs the
// loaded value (and waits for it) before the next chunk's requests.
template <int F>
__device__ __forceinline__ uint32_t chunk_scale(const FmtMat& m, int n, int c) {
  if constexpr (F == kFmtMxfp4) {
    return reinterpret_cast<const uint8_t*>(m.s)[(size_t)n * (m.K / 32) + c];
  } else if constexpr (F == kFmtFp8Block) {
    const int kb = (m.K + 127) / 128;
    return reinterpret_cast<const uint32_t*>(m.s)[(size_t)(n / 128) * kb + (c * 16) / 128];
  } else {
    return 0u;
  }
}
template <int F>
__device__ __forceinline__ float scaled(float dot, uint32_t sc) {
  if constexpr (F == kFmtMxfp4) {
    const int e = (int)sc;
    return e == 255 ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(dot, e - 127);
  } else {
    return dot * __uint_as_float(sc);
  }
}
template <int F>
__device__ __forceinline__ uint4 chunk_load(const FmtMat& m, int n, int c) {
  const size_t rowbytes = F == kFmtMxfp4 ? (size_t)m.K / 2 : (F == kFmtFp8Block ? (size_t)m.K : (size_t)m.K * 2);
  return ld_stream(m.q + (size_t)n * rowbytes + (size_t)c * 16);
}

// Sum of values[r * stride + c] over c < n for rows r < rows, into fn(r, sum):
// tpr (a power of two, <= 64) neighbouring threads per row, thread `part`
// adding the values c = part, part + tpr, ... in order, then the parts
// combined by an xor butterfly (the same order every call).
template <typename Fn>
__device__ __forceinline__ void row_sums(const float* values, int rows, int stride, int n, Fn fn) {
  int tpr = 64;
  while (tpr > 1 && tpr * rows > 256) tpr >>= 1;
  const int tid = threadIdx.x, part = tid & (tpr - 1);
  for (int r0 = 0; r0 < rows; r0 += 256 / tpr) {
    const int r = r0 + tid / tpr;
    float s = 0.f;
    if (r < rows)
      for (int c = part; c < n; c += tpr) s += values[r * stride + c];
    for (int off = 1; off < tpr; off <<= 1) s += __shfl_xor(s, off, 64);
    if (r < rows && part == 0) fn(r, s);
  }
}

struct FmtArgs {
  int M, E, k, H, I, has_shared;
  const int32_t* ids;
  const float* topk_w;
  const uint16_t* x;
  // routed experts: plain layout, per-expert strides in bytes
  const uint8_t* w13_q; const uint8_t* w13_s; const uint8_t* w2_q; const uint8_t* w2_s;
  size_t w13_q_stride, w13_s_stride, w2_q_stride, w2_s_stride;
  const uint16_t* sh_w13; const uint16_t* sh_w2;
  uint16_t* hb;     // [M*k + M][2][I] h as bf16 hi, lo: routed slots, then the shared expert per token
  int32_t* err;
  uint16_t* out;    // [M][H] bf16
  int ra, rsh;      // rows per gate_up item (routed format, shared BF16)
  int rb;           // output rows per down workgroup
};

// ------------------------------------------------------------------ gate_up
// Item of a workgroup: (unit u, row block b) of the routed experts for
// blockIdx.x < U_max * (2I / ra), else a block of the shared expert's rows.
template <int F, int NC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_fmt_gate_up(const FmtArgs A) {
  extern __shared__ __align__(16) uint32_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int H = A.H, I = A.I, M = A.M, S = M * A.k;
  // LDS: the tokens, chunk by chunk with one padding dword after each chunk
  // (lanes read neighbouring chunks: the padding spreads them over the
  // banks), then the chunk products
  uint32_t* xl = lds;
  __shared__ float rsum[kFmtMaxItemRows];

  const int ublocks = (2 * I) / A.ra;
  const int umax = std::min(S, A.E);
  const bool shared = (int)blockIdx.x >= umax * ublocks;
  int u = 0, b, rows;
  uint64_t mask;
  FmtMat m;
  if (!shared) {
    u = blockIdx.x / ublocks;
    b = blockIdx.x % ublocks;
    const Unit U = find_unit_wave(A.ids, S, A.E, u, lane);
    if (U.e < 0) return;  // fewer distinct experts than unit u
    mask = U.mask;
    m.q = A.w13_q + (size_t)U.e * A.w13_q_stride;
    m.s = A.w13_s + (size_t)U.e * A.w13_s_stride;
    rows = A.ra;
  } else {
    b = blockIdx.x - umax * ublocks;
    mask = (M >= 64) ? ~0ull : ((1ull << M) - 1);  // one entry per token
    m.q = reinterpret_cast<const uint8_t*>(A.sh_w13);
    m.s = nullptr;
    rows = A.rsh;
  }
  m.K = H;
  // the item's rows: gate rows g0 .. g0 + rows/2 - 1 and the matching up rows
  const int half = rows / 2, g0 = b * half;
  constexpr int FB = F;  // routed format; the shared rows are BF16
  const int cpr = shared ? H / chunk_cols<kFmtBf16>() : H / chunk_cols<FB>();
  const int nch = rows * cpr;
  uint4 w[NC];
  uint32_t sc[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int j = tid + 256 * i;
    sc[i] = 0u;
    w[i] = make_uint4(0, 0, 0, 0);
    if (j < nch) {
      const int rl = j / cpr, c = j % cpr;
      const int n = rl < half ? g0 + rl : I + g0 + (rl - half);
      if (shared) {
        w[i] = chunk_load<kFmtBf16>(m, n, c);
      } else {
        sc[i] = chunk_scale<FB>(m, n, c);
        w[i] = chunk_load<FB>(m, n, c);
      }
    }
  }
  // the tokens (after the weight requests) in the layout of this item's chunks
  const int hw = (shared ? chunk_cols<kFmtBf16>() : chunk_cols<FB>()) / 2, pdx = hw + 1, nck = H / (2 * hw);
  float* contrib = reinterpret_cast<float*>(lds + (size_t)M * nck * pdx);  // [rows * cpr]
  {
    // 16-byte loads, all requested before the first is stored (M * H / 8 <=
    // 256 * kFmtStage), then written dword by dword into the padded layout
    const uint4* x4 = reinterpret_cast<const uint4*>(A.x);
    const int n4 = M * (H / 8);
    uint4 v[kFmtStage];
#pragma unroll
    for (int m2 = 0; m2 < kFmtStage; ++m2) {
      const int i4 = tid + 256 * m2;
      v[m2] = i4 < n4 ? x4[i4] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m2 = 0; m2 < kFmtStage; ++m2) {
      const int i4 = tid + 256 * m2;
      if (i4 < n4) {
        const uint32_t dv[4] = {v[m2].x, v[m2].y, v[m2].z, v[m2].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = 4 * i4 + e, t = idx / (H / 2), d = idx - t * (H / 2), c = d / hw, q = d - c * hw;
          xl[(t * nck + c) * pdx + q] = dv[e];
        }
      }
    }
  }
  __syncthreads();
  while (mask) {
    const int p = __ffsll((unsigned long long)mask) - 1;
    mask &= mask - 1;
    const int t = shared ? p : p / A.k;
    const uint32_t* xt = xl + (size_t)t * nck * pdx;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int j = tid + 256 * i;
      if (j < nch) {
        const uint32_t* xp = xt + (j % cpr) * pdx;
        if (shared) {
          uint32_t xs[chunk_cols<kFmtBf16>() / 2];
#pragma unroll
          for (int q = 0; q < chunk_cols<kFmtBf16>() / 2; ++q) xs[q] = xp[q];
          contrib[j] = chunk_dot<kFmtBf16>(w[i], xs);
        } else {
          uint32_t xs[chunk_cols<FB>() / 2];
#pragma unroll
          for (int q = 0; q < chunk_cols<FB>() / 2; ++q) xs[q] = xp[q];
          contrib[j] = scaled<FB>(chunk_dot<FB>(w[i], xs), sc[i]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one chunk's inputs in registers at a time
    }
    __syncthreads();
    // each row's chunk products, then h = silu(gate) * up of the item's rows,
    // stored as bf16 (hi, lo): hb[slot][0][r] and hb[slot][1][r]
    const int slot = shared ? S + p : p;
    row_sums(contrib, rows, cpr, cpr, [&](int r, float v) { rsum[r] = v; });
    __syncthreads();
    for (int r = tid; r < half; r += 256) {
      const float h = silu_f32(rsum[r]) * rsum[half + r];
      const uint16_t hi = f32_to_bf16(h);
      A.hb[(size_t)slot * 2 * I + g0 + r] = hi;
      A.hb[(size_t)slot * 2 * I + I + g0 + r] = f32_to_bf16(h - bf16_to_f32(hi));
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ down
template <int F, int NC>
__global__ __launch_bounds__(256) void k_fmt_down(const FmtArgs A) {
  extern __shared__ __align__(16) uint32_t lds[];
  const int tid = threadIdx.x;
  const int H = A.H, I = A.I, M = A.M, k = A.k, S = M * k;
  const int RB = A.rb, n0 = blockIdx.x * RB;
  const int nseg = k + (A.has_shared ? 1 : 0);
  // LDS: h of every segment as bf16 hi and lo [nseg][I] each, then the
  // chunk products
  // h of each segment in chunks of its format, one padding dword after each
  // chunk (bank spread): routed segment seg at seg * segf, the shared one at
  // k * segf; the lo halves after all hi halves
  constexpr int hwf = chunk_cols<F>() / 2, pdf = hwf + 1;
  const int segf = (I / chunk_cols<F>()) * pdf;
  const int hiw = k * segf + (A.has_shared ? (I / 8) * 5 : 0);
  uint32_t* hhi = lds;
  uint32_t* hlo = lds + hiw;
  float* contrib = reinterpret_cast<float*>(lds + 2 * hiw);
  __shared__ float lw[kMaxTopK];
  const int cprf = I / chunk_cols<F>(), cprs = I / chunk_cols<kFmtBf16>();
  const int nrouted = k * RB * cprf, nch = nrouted + (A.has_shared ? RB * cprs : 0);
  const int rowlen = k * cprf + (A.has_shared ? cprs : 0);  // products of one output row
  // every slot's expert id into LDS first: the weight requests then depend on
  // no global load (a load's wait also waits for every load issued before it)
  __shared__ int sid[kMaxUnits];
  if (tid < S) {
    const int e = A.ids[tid];
    sid[tid] = e;
    if (blockIdx.x == 0 && (e < 0 || e >= A.E)) atomicOr(A.err, 1);
  }
  __syncthreads();
  // chunk i of this thread: a routed chunk (reloaded for every token) or a
  // shared one (loaded once: the shared rows serve every token), decoded once
  // into c | r << 10 | seg << 17 (seg = k: shared; -1: none)
  int cinfo[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int j = tid + 256 * i;
    int seg = -1, r = 0, c = 0;
    if (j < nrouted) {
      seg = j / (RB * cprf);
      const int rem = j - seg * RB * cprf;
      r = rem / cprf;
      c = rem - r * cprf;
    } else if (j < nch) {
      seg = k;
      r = (j - nrouted) / cprs;
      c = (j - nrouted) - r * cprs;
    }
    cinfo[i] = seg < 0 ? -1 : (c | r << 10 | seg << 17);
  }
  constexpr int lgf = hwf == 16 ? 4 : (hwf == 8 ? 3 : 2);  // log2 of a chunk's dwords
  uint4 w[NC];
  uint32_t sc[NC];
  const size_t rowbytes = F == kFmtMxfp4 ? (size_t)I / 2 : (size_t)I;
  const uint8_t* shq = reinterpret_cast<const uint8_t*>(A.sh_w2);
  const int q4 = I / 4, n4 = nseg * q4;  // h: I dwords per segment (I/2 hi, I/2 lo)
  for (int t = 0; t < M; ++t) {
    // h (hi, lo) of the token's slots and of the shared expert, and the slot
    // weights, requested first and without a branch (an index past the end
    // reads entry 0 and is not stored): they come from the workspace, and a
    // wait for them then does not also wait for the weight stream requested
    // after them (nseg * I / 4 <= 256 * kFmtStage)
    uint4 hv[kFmtStage];
#pragma unroll
    for (int m2 = 0; m2 < kFmtStage; ++m2) {
      const int i4 = tid + 256 * m2 < n4 ? tid + 256 * m2 : 0;
      const int seg = i4 / q4, d4 = i4 - seg * q4;
      const int slot = seg < k ? t * k + seg : S + t;
      hv[m2] = reinterpret_cast<const uint4*>(A.hb + (size_t)slot * 2 * I)[d4];
    }
    const float lwv = A.topk_w[t * k + tid % k];
    // every chunk's two requests with no branch around them: a chunk that
    // adds nothing (none, or an id out of range) reads a valid address of
    // expert 0 and is dropped when the products are formed.  A load under a
    // branch whose result merges with another value makes the wave wait for
    // it before the next request; here all of them are in flight at once.
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int ci = cinfo[i];
      const int cv = ci < 0 ? 0 : ci;
      const int seg = cv >> 17, n = n0 + ((cv >> 10) & 127), c = cv & 1023;
      const bool routed = seg < k;
      const int e0 = sid[t * k + (routed ? seg : 0)];
      const int e = (e0 >= 0 && e0 < A.E) ? e0 : 0;
      // 32-bit byte offsets (fmt_plan checks that every matrix fits): a
      // 64-bit multiply-add here ends up reading the register pair of a
      // load still in flight, which makes the wave wait for it
      const uint32_t qoff = routed ? (uint32_t)e * (uint32_t)A.w2_q_stride + (uint32_t)n * (uint32_t)rowbytes
                                   : (uint32_t)n * (uint32_t)(I * 2);
      w[i] = ld_stream((routed ? A.w2_q : shq) + qoff + (uint32_t)c * 16u);
      const int cs = routed ? c : 0;
      if constexpr (F == kFmtMxfp4) {
        sc[i] = A.w2_s[(uint32_t)e * (uint32_t)A.w2_s_stride + (uint32_t)n * (uint32_t)(I / 32) + (uint32_t)cs];
      } else {
        const int kb = (I + 127) / 128;
        sc[i] = *reinterpret_cast<const uint32_t*>(A.w2_s + (uint32_t)e * (uint32_t)A.w2_s_stride +
                                                   (uint32_t)((n / 128) * kb + (cs * 16) / 128) * 4u);
      }
    }
    // the slot weights (0 for an id out of range) and h into LDS
    if (tid < k) {
      const int e = sid[t * k + tid];
      lw[tid] = (e >= 0 && e < A.E) ? lwv : 0.f;
    }
#pragma unroll
    for (int m2 = 0; m2 < kFmtStage; ++m2) {
      const int i4 = tid + 256 * m2;
      if (i4 < n4) {
        const int seg = i4 / q4, d4 = i4 - seg * q4;
        const bool lo = 4 * d4 >= I / 2;
        const int dd0 = 4 * d4 - (lo ? I / 2 : 0);
        const int lg = seg < k ? lgf : 2;  // 4 dwords per BF16 chunk
        uint32_t* dst = (lo ? hlo : hhi) + seg * segf;
        const uint32_t dv[4] = {hv[m2].x, hv[m2].y, hv[m2].z, hv[m2].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dd = dd0 + e;  // 4 consecutive dwords stay in one chunk
          dst[(dd >> lg) * ((1 << lg) + 1) + (dd & ((1 << lg) - 1))] = dv[e];
        }
      }
    }
    __syncthreads();
    // products: a routed chunk goes to row r, position seg * cprf + c of the
    // row, weighted by its slot (0 for an id out of range); a shared chunk to
    // position k * cprf + c
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      // opaque: the chunk's operand reads cannot be hoisted above this point
      // (every chunk's inputs would otherwise be held at once)
      int ci = cinfo[i];
      uint4 wi = w[i];
      asm volatile("" : "+v"(ci), "+v"(wi.x), "+v"(wi.y), "+v"(wi.z), "+v"(wi.w));
      if (ci >= 0) {
        const int seg = ci >> 17, r = (ci >> 10) & 127, c = ci & 1023;
        float v;
        if (seg < k && (unsigned)sid[t * k + seg] >= (unsigned)A.E) {
          v = 0.f;  // an id out of range adds nothing
        } else if (seg < k) {
          // the hi half, then the lo half (one set of inputs in registers)
          const uint32_t* hp = hhi + seg * segf + c * pdf;
          uint32_t xs[hwf];
#pragma unroll
          for (int q = 0; q < hwf; ++q) xs[q] = hp[q];
          const float dh = chunk_dot<F>(wi, xs);
          __builtin_amdgcn_sched_barrier(0);
          const uint32_t* lp = hlo + seg * segf + c * pdf;
#pragma unroll
          for (int q = 0; q < hwf; ++q) xs[q] = lp[q];
          v = lw[seg] * scaled<F>(dh + chunk_dot<F>(wi, xs), sc[i]);
        } else {
          const uint32_t* hp = hhi + k * segf + c * 5;
          const uint32_t* lp = hlo + k * segf + c * 5;
          uint32_t xs[4], ys[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            xs[q] = hp[q];
            ys[q] = lp[q];
          }
          v = chunk_dot<kFmtBf16>(wi, xs) + chunk_dot<kFmtBf16>(wi, ys);
        }
        contrib[r * rowlen + seg * cprf + c] = v;
      }
      __builtin_amdgcn_sched_barrier(0);  // one chunk's inputs in registers at a time
    }
    __syncthreads();
    // every row: its weighted routed products, then the shared ones
    row_sums(contrib, RB, rowlen, rowlen, [&](int r, float y) { A.out[(size_t)t * H + n0 + r] = f32_to_bf16(y); });
    __syncthreads();
  }
}

constexpr int kFmtNcGu = 10, kFmtNcDn = 12;

template <int F>
hipError_t run_fmt(const FmtArgs& A, hipStream_t st) {
  const int ublocks = (2 * A.I) / A.ra;
  const int umax = std::min(A.M * A.k, A.E);
  const int gsh = A.has_shared ? (2 * A.I) / A.rsh : 0;
  const int cmax = std::max(A.ra * (A.H / chunk_cols<F>()), A.has_shared ? A.rsh * (A.H / 8) : 0);
  const int xw = std::max((A.H / chunk_cols<F>()) * (chunk_cols<F>() / 2 + 1), A.has_shared ? (A.H / 8) * 5 : 0);
  const size_t lds_gu = ((size_t)A.M * xw + (size_t)cmax) * 4;
  hipLaunchKernelGGL((k_fmt_gate_up<F, kFmtNcGu>), dim3(umax * ublocks + gsh), dim3(256), lds_gu, st, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t nch = (size_t)A.k * A.rb * (A.I / chunk_cols<F>()) + (A.has_shared ? (size_t)A.rb * (A.I / 8) : 0);
  const size_t hiw = (size_t)A.k * (A.I / chunk_cols<F>()) * (chunk_cols<F>() / 2 + 1) + (A.has_shared ? (A.I / 8) * 5 : 0);
  const size_t lds_dn = (2 * hiw + nch) * 4;
  hipLaunchKernelGGL((k_fmt_down<F, kFmtNcDn>), dim3(A.H / A.rb), dim3(256), lds_dn, st, A);
  return hipGetLastError();
}

}  // namespace

// Work split of the format path for a shape: rows per gate_up item for the
// routed format and the shared expert, output rows per down workgroup.  Each
// item's chunks fit the workgroup's registers (kFmtNcGu / kFmtNcDn chunks per
// thread) and its LDS products.
bool fmt_plan(const Shape& s, int fmt, int M, int* ra, int* rsh, int* rb) {
  if (fmt != kFmtMxfp4 && fmt != kFmtFp8Block) return false;
  const int cols = fmt == kFmtMxfp4 ? 32 : 16;
  // the down kernel addresses a matrix with 32-bit byte offsets
  if ((uint64_t)s.E * s.H * s.I >= ((uint64_t)1 << 32)) return false;
  if (s.H % 32 || s.I % 32 || M < 1 || M * s.k > kMaxUnits) return false;
  if ((int64_t)(s.k + 1) * 2 * s.I * 2 > (int64_t)s.k * s.H * 4) return false;  // h fits the down-partials buffer
  const int cpa = s.H / cols, cps = s.H / 8;
  // item rows: half gate, half up (the halves divide I)
  int a = std::min(2 * s.I, kFmtMaxItemRows);
  while (a > 2 && ((int64_t)a * cpa > 256 * kFmtNcGu || s.I % (a / 2))) a -= 2;
  int sh = std::min(2 * s.I, kFmtMaxItemRows);
  while (sh > 2 && ((int64_t)sh * cps > 256 * kFmtNcGu || s.I % (sh / 2))) sh -= 2;
  const int64_t per_row = (int64_t)s.k * (s.I / cols) + (s.has_shared ? s.I / 8 : 0);
  // output rows per down workgroup (<= 64, a divisor of H): the most that fit
  // the registers, so that the grid needs as few rounds of the device as it can
  int b = 64;
  while (b > 1 && (b * per_row > 256 * kFmtNcDn || s.H % b)) --b;
  // LDS of the two kernels (padded operand chunks, chunk products)
  const int64_t xw = std::max<int64_t>((int64_t)cpa * (cols / 2 + 1), s.has_shared ? (int64_t)cps * 5 : 0);
  const int64_t lds_gu = ((int64_t)M * xw + std::max<int64_t>((int64_t)a * cpa, (int64_t)sh * cps)) * 4;
  const int64_t hiw = (int64_t)s.k * (s.I / cols) * (cols / 2 + 1) + (s.has_shared ? (s.I / 8) * 5 : 0);
  const int64_t lds_dn = (2 * hiw + b * per_row) * 4;
  if ((int64_t)M * (s.H / 8) > 256 * kFmtStage || (int64_t)(s.k + 1) * (s.I / 4) > 256 * kFmtStage) return false;
  if (a < 2 || sh < 2 || (int64_t)a * cpa > 256 * kFmtNcGu || (int64_t)sh * cps > 256 * kFmtNcGu || b < 1 || b * per_row > 256 * kFmtNcDn || lds_gu > 65536 || lds_dn > 65536) return false;
  *ra = a; *rsh = sh; *rb = b;
  return true;
}

hipError_t launch_forward_fmt(const Shape& s, int fmt, const uint8_t* w13_q, const void* w13_s, const uint8_t* w2_q,
                              const void* w2_s, const uint16_t* sh_w13, const uint16_t* sh_w2, const uint16_t* x,
                              int M, const int32_t* ids, const float* w, uint16_t* out, uint8_t* ws,
                              const WsLayout& L, hipStream_t st) {
  FmtArgs A;
  if (!fmt_plan(s, fmt, M, &A.ra, &A.rsh, &A.rb)) return hipErrorInvalidValue;
  A.M = M; A.E = s.E; A.k = s.k; A.H = s.H; A.I = s.I; A.has_shared = s.has_shared;
  A.ids = ids; A.topk_w = w; A.x = x;
  A.w13_q = w13_q; A.w13_s = static_cast<const uint8_t*>(w13_s);
  A.w2_q = w2_q; A.w2_s = static_cast<const uint8_t*>(w2_s);
  const size_t gu_rows = 2 * (size_t)s.I, dn_rows = s.H;
  if (fmt == kFmtMxfp4) {
    A.w13_q_stride = gu_rows * s.H / 2; A.w13_s_stride = gu_rows * (s.H / 32);
    A.w2_q_stride = dn_rows * s.I / 2; A.w2_s_stride = dn_rows * (s.I / 32);
  } else {
    A.w13_q_stride = gu_rows * s.H; A.w13_s_stride = ((gu_rows + 127) / 128) * ((s.H + 127) / 128) * 4;
    A.w2_q_stride = dn_rows * s.I; A.w2_s_stride = ((dn_rows + 127) / 128) * ((s.I + 127) / 128) * 4;
  }
  A.sh_w13 = sh_w13; A.sh_w2 = sh_w2;
  A.hb = reinterpret_cast<uint16_t*>(ws + L.dpart);
  A.err = reinterpret_cast<int32_t*>(ws + L.err);
  A.out = out;
  return fmt == kFmtMxfp4 ? run_fmt<kFmtMxfp4>(A, st) : run_fmt<kFmtFp8Block>(A, st);
}

}  // namespace moe
