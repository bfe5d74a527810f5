// prefill.hip — the many-token path (chunked prefill).  Every expert's
// (token, slot) pairs form a dense block of rows, so the expert FFNs run as
// grouped GEMMs on the matrix cores, fp32 accumulate throughout.
//
//   router:  logits[M][E] = x[M][H] * Wr^T   (Wr fp32 split once per call into
//            three exact bf16 parts hi + mid + lo, one bf16 MFMA each; x is bf16)
//   top-k:   one wavefront per token over its logits row
//   permute: pairs grouped by expert (permute.hip), cut into work items of at
//            most 128 rows
//   x prep:  each token row of x scaled by a power of two 2^-r_t into fp16,
//            largest magnitude below 2^15 (exact: bf16 has 8 significant bits,
//            fp16 11)
//   gate_up: per item, rows x[token] times the INT4 gate/up rows dequantised
//            to fp16 as q * s * 2^p; h = silu(gate) * up, stored as fp16
//            scaled by 2^-sigma with sigma from a bound on |h| (below)
//   down:    h times the INT4 down rows, one fp16 row per sorted pair under a
//            per-expert power-of-two scale (|y| <= ||down row||_1 max|h|)
//   shared:  the same two GEMMs on all tokens with the BF16 shared weights in
//            bf16 MFMAs (x as is, h as an exact-to-16-bits hi + lo pair)
//   combine: out[t] = sum_j w[t][j] * y[pair (t, j)] + y_shared[t], slot order
//
// Exactness of the routed operands.  A code u (0..15, q = u - 8) becomes fp16
// through the fp8 converter (a byte 0..15 read as e4m3 is u * 2^-9; the
// converter's exponent scale 2^9 makes it u), then fma(u, s', -8 s') with
// s' = s * 2^p in fp16: q * s' needs at most 3 + 8 significant bits, so the
// fused result is exact in fp16's 11, and 2^p (per expert, from the largest
// |scale|) keeps |q s'| <= 2^15.  The products of fp16 operands are exact in
// the fp32 accumulators; the powers of two are taken out in the epilogues.
// Bound on h: |g| <= ||x_t||_2 ||gate_r||_2 and |u| <= ||x_t||_2 ||up_r||_2
// (Cauchy-Schwarz) and |silu(g)| <= |g|, so |h| <= ||x_t||_2^2 L_e with
// L_e = max_r ||gate_r||_2 ||up_r||_2 (computed when the weights are packed).
// With ||x_t||_2^2 < 2^tx_t and L_e < 2^le_e, sigma = tx_t + le_e - 13 puts
// |h| 2^-sigma below 2^13; h keeps fp16's 11 significant bits wherever
// |h| 2^-sigma >= 2^-14.
// The L2 bound sits within a factor of about sqrt(K) of typical values for
// dense and for one-hot rows alike (an L1 bound with max |x| would not).
#include <type_traits>

#include "launch.hpp"
#include "route_dev.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// e with |v| < 2^e for finite v (0 and subnormals give -126).
__device__ __forceinline__ int exp_above(float v) {
  const int ex = (int)((__float_as_uint(v) >> 23) & 0xFFu);
  return ex == 0 ? -126 : ex - 126;
}

// e with v < 2^e for a non-negative v computed by fp32 sums of at most a few
// thousand exact terms: the factor 1 + 2^-10 covers their rounding.
__device__ __forceinline__ int exp_bound(float v) { return exp_above(v * 1.0009765625f); }

// C[m][n] of a 32x32 MFMA block lives in lane n + 32*((m/4)%2), slot (m%4) + 4*(m/8).
__device__ __forceinline__ int c_row(int lane, int slot) { return 8 * (slot >> 2) + 4 * (lane >> 5) + (slot & 3); }

// Order of 8 consecutive K inputs inside a 16-byte fp16 operand of the INT4
// GEMMs: position j holds input (j >> 1) + 4 (j & 1), the order in which the
// converter produces the codes of one packed dword.  Input i sits at
// position 2 (i & 3) + (i >> 2).
__device__ __forceinline__ int k8_pos(int i) { return 2 * (i & 3) + (i >> 2); }

// ------------------------------------------------------------------ x prep

__global__ __launch_bounds__(kBlock) void k_pf_xprep(const uint16_t* __restrict__ x, int H,
                                                     _Float16* __restrict__ xh, int32_t* __restrict__ rexp) {
  __shared__ float red[2][kWavesPerBlock];
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  const int nch = H / 8;
  float m = 0.f, ss = 0.f;
  for (int c = tid; c < nch; c += kBlock) {
    const uint4 v = row[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float lo = bf16_to_f32(w[d] & 0xFFFFu), hi = bf16_to_f32(w[d] >> 16);
      m = fmaxf(m, fmaxf(fabsf(lo), fabsf(hi)));
      ss = fmaf(lo, lo, fmaf(hi, hi, ss));
    }
  }
  m = wave_max(m);
  ss = wave_sum(ss);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = m;
    red[1][tid >> 6] = ss;
  }
  __syncthreads();
  m = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  ss = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  const int r = exp_above(m) - 15;  // max |x| * 2^-r < 2^15
  for (int c = tid; c < nch; c += kBlock) {
    const uint4 v = row[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      f[2 * d] = ldexpf(bf16_to_f32(w[d] & 0xFFFFu), -r);
      f[2 * d + 1] = ldexpf(bf16_to_f32(w[d] >> 16), -r);
    }
    f16x8_t o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (_Float16)f[(j >> 1) + 4 * (j & 1)];
    *reinterpret_cast<f16x8_t*>(xh + (size_t)t * H + 8 * c) = o;
  }
  if (tid == 0) {
    rexp[2 * t] = r;
    rexp[2 * t + 1] = exp_bound(ss);  // ||x_t||_2^2 < 2^tx
  }
}

// ------------------------------------------------------------------ grouped GEMMs

enum GgKind { GG_RGU = 0, GG_RDN = 1, GG_SGU = 2, GG_SDN = 3 };

constexpr int kGgKc = 128;             // K per LDS chunk (two 64-K steps)
constexpr int kGgStride = kGgKc + 8;   // 16-bit elements per LDS row (16-byte pad: conflict-free MFMA reads)
constexpr int kGgLdsRows = 128;

struct GgArgs {
  int M, E, k, H, I;
  int K;        // reduction length
  int ntiles;   // 64-row weight tiles (gate_up: I/32, down: H/64)
  int ng;       // workgroups per item: ceil(ntiles / 4)
  // routed work items (permute.hip)
  const int32_t* __restrict__ counts;
  const int32_t* __restrict__ offsets;
  const int32_t* __restrict__ perm;
  const int32_t* __restrict__ tile_e;
  const int32_t* __restrict__ tile_j;
  const int32_t* __restrict__ ntile;
  // activations
  const _Float16* __restrict__ xh;    // [M][H] scaled x, K order of k8_pos
  const int32_t* __restrict__ rexp;   // [M][2]: r (x scaling) and tx (bound of ||x||^2) per token
  const _Float16* __restrict__ hbuf;  // [S][I] scaled h per sorted position, K order of k8_pos
  const uint16_t* __restrict__ x;     // [M][H] bf16
  const uint16_t* __restrict__ hsh;   // [2][M][I] bf16 (hi, lo)
  // weights of this phase
  const uint8_t* __restrict__ q;      // routed packed codes
  const uint16_t* __restrict__ s;     // routed packed scales
  size_t q_stride, s_stride;          // per expert: bytes, elements
  int P, pshift;                      // scales per lane-load of the packed layout (1, 2 or 4), log2 P
  const uint16_t* __restrict__ shw;   // shared packed bf16
  const uint32_t* __restrict__ meta;  // per-expert range data
  int meta_word;                      // 0: gate_up scales, 1: down scales
  // outputs
  _Float16* __restrict__ hout;        // [S][I]
  uint16_t* __restrict__ hsh_out;     // [2][M][I]
  _Float16* __restrict__ y;           // [S][H] y * 2^-(sigma + e2 - 1), e2 from the down-row norm bound
  float* __restrict__ ysh;            // [M][H]
};

template <int KIND>
struct GgCfg {
  static constexpr bool ROUTED = KIND == GG_RGU || KIND == GG_RDN;
  static constexpr bool HILO = KIND == GG_SDN;  // A is the shared h as hi + lo
  static constexpr int MAXMB = ROUTED ? kItemRows / 32 : 2;  // 32-row MFMA blocks per item
  static constexpr int ROWS = 32 * MAXMB;
  static constexpr int DEPTH = ROUTED ? 4 : 2;  // 64-K steps of weights in flight
};

struct RawQ {  // one 64-K step of a routed weight tile: one 32-code group per lane half
  uint4 c[2];
  uint32_t s[2];
};
struct RawS {  // one 64-K step of a shared weight tile: four 8-input chunks per lane half
  uint4 c[2][4];
};

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Everything a workgroup knows about its item once the row tables are built.
struct GgItem {
  int e, base, nrow, p;
  int ey;  // down: exponent that takes the accumulators to the stored fp16 y
  int yb;  // group of 4 weight tiles of this workgroup
};

// Main loop and epilogue for items of NMB 32-row blocks.  The loop body has
// no branches around memory operations (padding rows load row 0, prefetches
// past the end reload the last step, the chunk store and barrier run
// unconditionally), so the compiler can count the loads in flight and wait
// only for the one each step consumes.
template <int KIND, int NMB>
__device__ __forceinline__ void gg_run(const GgArgs& a, const GgItem& it, uint16_t (*sA)[kGgLdsRows * kGgStride],
                                       const int* sSrc, const int* sExp, const int* sSig) {
  using C = GgCfg<KIND>;
  using Raw = typename std::conditional<C::ROUTED, RawQ, RawS>::type;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  // ---- A chunks: thread covers 16-byte segment tid & 15 of rows (tid >> 4) + 16 jj
  constexpr int NJ = C::HILO ? 8 : 2 * NMB;  // row groups of 16 that hold data
  const int seg = tid & 15;
  // byte offsets (all operands are far below 4 GiB) from a uniform base, so
  // loads take the SGPR-base + 32-bit VGPR-offset form
  const uint8_t* abase8;
  if constexpr (C::HILO) abase8 = reinterpret_cast<const uint8_t*>(a.hsh);
  else if constexpr (KIND == GG_RGU) abase8 = reinterpret_cast<const uint8_t*>(a.xh);
  else if constexpr (KIND == GG_RDN) abase8 = reinterpret_cast<const uint8_t*>(a.hbuf);
  else abase8 = reinterpret_cast<const uint8_t*>(a.x);
  const uint32_t rowbytes = 2u * (KIND == GG_RGU || KIND == GG_SGU ? a.H : a.I);
  uint32_t aoff[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int R = (tid >> 4) + 16 * jj;
    if constexpr (C::HILO)
      aoff[jj] = (uint32_t)(R >> 6) * (uint32_t)a.M * rowbytes + (uint32_t)sSrc[R & 63] * rowbytes;
    else
      aoff[jj] = (uint32_t)sSrc[R] * rowbytes;
    aoff[jj] += seg * 16;
  }
  // staging registers: two sets (chunks of alternate parity) of one named
  // value per row group (an indexed array here ends up in scratch memory)
  uint4 st_0, st_1, st_2, st_3, st_4, st_5, st_6, st_7;
  uint4 su_0, su_1, su_2, su_3, su_4, su_5, su_6, su_7;
  auto slot = [&](auto S, auto J) -> uint4& {
    constexpr int j = decltype(J)::value;
    if constexpr (decltype(S)::value == 0) {
      if constexpr (j == 0) return st_0;
      else if constexpr (j == 1) return st_1;
      else if constexpr (j == 2) return st_2;
      else if constexpr (j == 3) return st_3;
      else if constexpr (j == 4) return st_4;
      else if constexpr (j == 5) return st_5;
      else if constexpr (j == 6) return st_6;
      else return st_7;
    } else {
      if constexpr (j == 0) return su_0;
      else if constexpr (j == 1) return su_1;
      else if constexpr (j == 2) return su_2;
      else if constexpr (j == 3) return su_3;
      else if constexpr (j == 4) return su_4;
      else if constexpr (j == 5) return su_5;
      else if constexpr (j == 6) return su_6;
      else return su_7;
    }
  };
  auto for_each_jj = [&](auto f) {
    auto one = [&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (j < NJ && (!C::HILO || (j & 3) < 2 * NMB)) f(J);
    };
    one(std::integral_constant<int, 0>{}); one(std::integral_constant<int, 1>{});
    one(std::integral_constant<int, 2>{}); one(std::integral_constant<int, 3>{});
    one(std::integral_constant<int, 4>{}); one(std::integral_constant<int, 5>{});
    one(std::integral_constant<int, 6>{}); one(std::integral_constant<int, 7>{});
  };
  auto load_A = [&](auto S, int kc0) {
    const uint8_t* ab = abase8 + 2 * kc0;
    for_each_jj([&](auto J) { slot(S, J) = *reinterpret_cast<const uint4*>(ab + aoff[decltype(J)::value]); });
  };
  auto store_A = [&](auto S, int buf) {
    for_each_jj([&](auto J) {
      constexpr int j = decltype(J)::value;
      *reinterpret_cast<uint4*>(&sA[buf][((tid >> 4) + 16 * j) * kGgStride + seg * 8]) = slot(S, J);
    });
  };
  // ---- this wavefront's weight tile (tiles past the last read tile 0 and are dropped)
  const int t = it.yb * kWavesPerBlock + wave;
  const bool tile_ok = t < a.ntiles;
  const int tt = tile_ok ? t : 0;
  const int GK = a.K / kGroup;
  const uint8_t* qe = a.q + (size_t)it.e * a.q_stride;
  const uint16_t* se = a.s + (size_t)it.e * a.s_stride;
  const uint8_t* sw = reinterpret_cast<const uint8_t*>(a.shw);
  // per-lane parts of the weight offsets; the per-step parts are uniform
  uint32_t boff[2], soff[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int row = 32 * nb + n;
    if constexpr (C::ROUTED) {
      boff[nb] = ((uint32_t)(tt * GK + h) * kWave + row) * 16;
      // group g = 2 st + h: with P >= 2 the pack index g / P and slot g % P
      // get h only in the slot; with P = 1 h is a whole pack (64 lanes) on
      soff[nb] = ((uint32_t)tt * (GK >> a.pshift) * kWave + row) * a.P + (a.P >= 2 ? h : kWave * h);
    } else {
      boff[nb] = ((uint32_t)(tt * (a.K / 8) + h) * kWave + row) * 16;
      soff[nb] = 0;
    }
  }
  auto load_B = [&](int st, Raw& r) {
    if constexpr (C::ROUTED) {
      const uint8_t* qs = qe + (size_t)st * (2 * kWave * 16);
      const int g0 = 2 * st;
      const uint16_t* ss = se + (size_t)((g0 >> a.pshift) * kWave * a.P + (g0 & (a.P - 1)));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        r.c[nb] = *reinterpret_cast<const uint4*>(qs + boff[nb]);
        r.s[nb] = ss[soff[nb]];
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // 8-input chunk 8st + 2i + h
          const uint8_t* ws = sw + (size_t)(8 * st + 2 * i) * (kWave * 16);
          r.c[nb][i] = *reinterpret_cast<const uint4*>(ws + boff[nb]);
        }
    }
  };
  f32x16_t acc[NMB][2];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
  const float pscale = ldexpf(1.0f, it.p);
  auto compute = [&](const Raw& r, int buf, int kk) {
    if constexpr (C::ROUTED) {
      f16x2_t s2[2], m2[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const _Float16 sh = (_Float16)(bf16_to_f32(r.s[nb]) * pscale);
        s2[nb] = (f16x2_t){sh, sh};
        m2[nb] = s2[nb] * (f16x2_t){(_Float16)-8.0f, (_Float16)-8.0f};
      }
      // sub-step i: lane half h takes dword i (inputs 8i..8i+7) of group 2st + h
      const uint16_t* abase = &sA[buf][n * kGgStride + kk + 32 * h];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x8_t B[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const uint32_t w = dword_of(r.c[nb], i);
          const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
          f16x2_t c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);  // inputs 0, 4
          f16x2_t c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);   // inputs 1, 5
          f16x2_t c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);  // inputs 2, 6
          f16x2_t c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);   // inputs 3, 7
          c0 = __builtin_elementwise_fma(c0, s2[nb], m2[nb]);
          c1 = __builtin_elementwise_fma(c1, s2[nb], m2[nb]);
          c2 = __builtin_elementwise_fma(c2, s2[nb], m2[nb]);
          c3 = __builtin_elementwise_fma(c3, s2[nb], m2[nb]);
          B[nb] = (f16x8_t){c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
        }
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const f16x8_t A = *reinterpret_cast<const f16x8_t*>(abase + 32 * mb * kGgStride + 8 * i);
          acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B[0], acc[mb][0], 0, 0, 0);
          acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B[1], acc[mb][1], 0, 0, 0);
        }
      }
    } else {
      // sub-step i: lane half h takes inputs 16i + 8h .. +7 (natural order)
      const uint16_t* abase = &sA[buf][n * kGgStride + kk + 8 * h];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t B0 = __builtin_bit_cast(bf16x8_t, r.c[0][i]);
        const bf16x8_t B1 = __builtin_bit_cast(bf16x8_t, r.c[1][i]);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(abase + 32 * mb * kGgStride + 16 * i);
          acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B0, acc[mb][0], 0, 0, 0);
          acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B1, acc[mb][1], 0, 0, 0);
          if constexpr (C::HILO) {
            const bf16x8_t A2 = *reinterpret_cast<const bf16x8_t*>(abase + (64 + 32 * mb) * kGgStride + 16 * i);
            acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A2, B0, acc[mb][0], 0, 0, 0);
            acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A2, B1, acc[mb][1], 0, 0, 0);
          }
        }
      }
    }
  };
  // ---- main loop: 64-K steps, weights DEPTH - 1 steps ahead in registers,
  // activations two 128-K chunks ahead in registers, double-buffered in LDS
  const int nsteps = a.K / 64;  // a multiple of 4
  const int nch = nsteps / 2;
  Raw ring[C::DEPTH];
#pragma unroll
  for (int d = 0; d < C::DEPTH - 1; ++d) load_B(d, ring[d]);
  // chunks 1, 3, 5, ... stage in the first register set, 2, 4, ... in the
  // second, so each chunk's rows are requested two chunks before they go to LDS
  constexpr std::integral_constant<int, 0> odd{};
  constexpr std::integral_constant<int, 1> even{};
  load_A(odd, 0);
  store_A(odd, 0);
  lds_sync();
  load_A(odd, kGgKc);
  load_A(even, min(2, nch - 1) * kGgKc);
  for (int st0 = 0; st0 < nsteps; st0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int st = st0 + u;
      load_B(min(st + C::DEPTH - 1, nsteps - 1), ring[(u + C::DEPTH - 1) % C::DEPTH]);
      compute(ring[u % C::DEPTH], (u >> 1) & 1, 64 * (u & 1));
      if (u & 1) {
        // end of chunk ch = st / 2 (even at u = 1, odd at u = 3): chunk ch + 1
        // into the other buffer (its last readers, chunk ch - 1, all passed
        // the previous barrier), then chunk ch + 3 into the freed registers
        const int ch = st >> 1;
        if (u == 1) {
          store_A(odd, 1);
          lds_sync();
          load_A(odd, min(ch + 3, nch - 1) * kGgKc);
        } else {
          store_A(even, 0);
          lds_sync();
          load_A(even, min(ch + 3, nch - 1) * kGgKc);
        }
      }
    }
  }
  if (!tile_ok) return;
  // ---- epilogue
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int sl = 0; sl < 16; ++sl) {
      const int r = 32 * mb + c_row(lane, sl);
      if (r >= it.nrow) continue;
      if constexpr (KIND == GG_RGU) {
        const int ex = sExp[r] - it.p;
        const float g = ldexpf(acc[mb][0][sl], ex), u = ldexpf(acc[mb][1][sl], ex);
        const float hv = ldexpf(silu_f32(g) * u, -sSig[r]);
        const int col = 32 * t + n;
        a.hout[(size_t)(it.base + r) * a.I + (col & ~7) + k8_pos(col & 7)] = (_Float16)hv;
      } else if constexpr (KIND == GG_RDN) {
        // acc = y 2^(p - sigma) and |y| < 2^(sigma + 13 + e2): the stored
        // y 2^-(sigma + e2 - 1) = acc 2^(1 - p - e2) stays below 2^14
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          a.y[(size_t)(it.base + r) * a.H + 64 * t + 32 * nb + n] = (_Float16)ldexpf(acc[mb][nb][sl], it.ey);
      } else if constexpr (KIND == GG_SGU) {
        const float hv = silu_f32(acc[mb][0][sl]) * acc[mb][1][sl];
        const uint16_t hi = f32_to_bf16(hv), lo = f32_to_bf16(hv - bf16_to_f32(hi));
        const size_t o = (size_t)(it.base + r) * a.I + 32 * t + n;
        a.hsh_out[o] = hi;
        a.hsh_out[(size_t)a.M * a.I + o] = lo;
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          a.ysh[(size_t)(it.base + r) * a.H + 64 * t + 32 * nb + n] = acc[mb][nb][sl];
      }
    }
  }
}

// One workgroup = one work item (up to 96 sorted rows of one expert, or a
// block of tokens for the shared expert) x 4 weight tiles of 64 rows, one per
// wavefront.  Workgroup ids are laid out so that the ng workgroups of one item
// run back to back on one XCD (ids are dealt to the 8 XCDs round-robin), so
// the item's activation rows are read from that XCD's L2 after the first.
template <int KIND>
__device__ __forceinline__ void gg_item(const GgArgs& a, int b, uint16_t (*sA)[kGgLdsRows * kGgStride], int* sSrc,
                                        int* sExp, int* sSig) {
  using C = GgCfg<KIND>;
  const int tid = threadIdx.x;
  // ---- work item (b: this launch part's workgroup index)
  const int xcd = b & 7, slot = b >> 3;
  const int item = (slot / a.ng) * 8 + xcd;
  GgItem it{0, 0, 0, 0, 0, slot % a.ng};
  if constexpr (C::ROUTED) {
    if (item >= uniform(a.ntile[0])) return;
    it.e = uniform(a.tile_e[item]);
    const int j = uniform(a.tile_j[item]);
    it.base = uniform(a.offsets[it.e]) + kItemRows * j;
    it.nrow = min(kItemRows, uniform(a.counts[it.e]) - kItemRows * j);
  } else {
    it.base = C::ROWS * item;
    if (it.base >= a.M) return;
    it.nrow = min(C::ROWS, a.M - it.base);
  }
  int le = 0;
  if constexpr (C::ROUTED) {
    const uint32_t* mt = a.meta + (size_t)it.e * kMetaWords;
    it.p = min(12 - exp_above(__uint_as_float(mt[a.meta_word])), 126);
    le = exp_bound(__uint_as_float(mt[2]));
    it.ey = 1 - it.p - exp_above(__uint_as_float(mt[3]));
  }
  // ---- row tables: A source row of each row, and for gate_up the row
  // exponents its epilogue needs (the down epilogue needs only it.ey)
  if (tid < C::ROWS) {
    const int rr = tid < it.nrow ? tid : 0;  // padding rows repeat row 0; their results are dropped
    if constexpr (KIND == GG_RGU) {
      const int tok = a.perm[it.base + rr] / a.k;
      sSrc[tid] = tok;
      sExp[tid] = a.rexp[2 * tok];
      sSig[tid] = a.rexp[2 * tok + 1] + le - 13;
    } else {
      sSrc[tid] = it.base + rr;
    }
  }
  lds_sync();
  const int nmb = (it.nrow + 31) >> 5;
  static_assert(C::MAXMB == 2 || C::MAXMB == 3, "item sizes handled below");
  if constexpr (C::MAXMB == 3) {
    if (nmb == 1) gg_run<KIND, 1>(a, it, sA, sSrc, sExp, sSig);
    else if (nmb == 2) gg_run<KIND, 2>(a, it, sA, sSrc, sExp, sSig);
    else gg_run<KIND, 3>(a, it, sA, sSrc, sExp, sSig);
  } else {
    if (nmb == 1) gg_run<KIND, 1>(a, it, sA, sSrc, sExp, sSig);
    else gg_run<KIND, 2>(a, it, sA, sSrc, sExp, sSig);
  }
}

template <int KIND>
__global__ __launch_bounds__(kBlock, 2) void k_gg(const GgArgs a) {
  __shared__ __align__(16) uint16_t sA[2][kGgLdsRows * kGgStride];
  __shared__ int sSrc[kGgLdsRows], sExp[kGgLdsRows], sSig[kGgLdsRows];
  gg_item<KIND>(a, blockIdx.x, sA, sSrc, sExp, sSig);
}

// The routed and the shared GEMM of one phase in one launch: the shared work
// items take the workgroup ids after the routed ones (whose count is a
// multiple of 8, so the XCD mapping of each part is kept) and fill the tail
// of the routed part.
template <int KR, int KS>
__global__ __launch_bounds__(kBlock, 2) void k_gg2(const GgArgs a, int routed_blocks) {
  __shared__ __align__(16) uint16_t sA[2][kGgLdsRows * kGgStride];
  __shared__ int sSrc[kGgLdsRows], sExp[kGgLdsRows], sSig[kGgLdsRows];
  if ((int)blockIdx.x < routed_blocks) gg_item<KR>(a, blockIdx.x, sA, sSrc, sExp, sSig);
  else gg_item<KS>(a, blockIdx.x - routed_blocks, sA, sSrc, sExp, sSig);
}

// ------------------------------------------------------------------ router GEMM

// fp32 -> (hi, mid, lo) bf16 with hi + mid + lo == v exactly (each part
// takes the next 8 significant bits; the rounding is to nearest even).
__device__ __forceinline__ void split3_one(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f32_to_bf16(v);
  const float r = v - bf16_to_f32(hi);
  mid = f32_to_bf16(r);
  lo = f32_to_bf16(r - bf16_to_f32(mid));
}

// The router weights [E][H] fp32 as three bf16 planes [3][E][H], once per call
// (one thread per 8 weights).
__global__ __launch_bounds__(kBlock) void k_rt_split(const float* __restrict__ wr, size_t n8,
                                                     uint16_t* __restrict__ planes, size_t plane_elems) {
  const size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n8) return;
  const float4 v0 = reinterpret_cast<const float4*>(wr)[2 * i];
  const float4 v1 = reinterpret_cast<const float4*>(wr)[2 * i + 1];
  const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint16_t hh[8], mm[8], ll[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) split3_one(v[j], hh[j], mm[j], ll[j]);
  auto pack = [](const uint16_t (&q)[8]) {
    return make_uint4(q[0] | ((uint32_t)q[1] << 16), q[2] | ((uint32_t)q[3] << 16), q[4] | ((uint32_t)q[5] << 16),
                      q[6] | ((uint32_t)q[7] << 16));
  };
  reinterpret_cast<uint4*>(planes)[i] = pack(hh);
  reinterpret_cast<uint4*>(planes + plane_elems)[i] = pack(mm);
  reinterpret_cast<uint4*>(planes + 2 * plane_elems)[i] = pack(ll);
}

constexpr int kRtE = 64;              // experts (MFMA rows) per workgroup
constexpr int kRtT = 128;             // tokens per workgroup: 4 wavefronts x 32
constexpr int kRtKc = 64;             // K per LDS chunk (one step)
constexpr int kRtStride = kRtKc + 8;  // bf16 per LDS row (conflict-free 16-byte reads)

struct RtArgs {
  int M, E, H;
  const uint16_t* __restrict__ x;       // [M][H] bf16
  const uint16_t* __restrict__ planes;  // [3][E][H] bf16
  float* __restrict__ logits;           // [M][E]
};

// logits^T block = W (64 experts x H, three bf16 parts, staged in LDS) times
// x^T (H x 32 tokens per wavefront, loaded into registers).  The loop body
// has no branches around memory operations: tokens past M load token M-1
// and are not stored.
__global__ __launch_bounds__(kBlock, 2) void k_rt_gemm(const RtArgs a) {
  __shared__ __align__(16) uint16_t sW[2][3][kRtE * kRtStride];
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int ntE = a.E / kRtE;
  const int et = blockIdx.x % ntE, tt = blockIdx.x / ntE;
  const int tok = min(kRtT * tt + 32 * wave + n, a.M - 1);
  const uint16_t* xrow = a.x + (size_t)tok * a.H + 8 * h;
  // weight staging: 3 planes x 64 rows x 8 segments of 16 bytes = 1536 per chunk, 6 per thread
  uint32_t soff[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int q = tid + kBlock * j;
    const int pl = q >> 9, r = (q >> 3) & 63, sg = q & 7;
    soff[j] = (uint32_t)(((size_t)pl * a.E + kRtE * et + r) * a.H + 8 * sg);
  }
  // two sets of staging registers: chunk c is fetched two steps before it is
  // stored to LDS (set c & 1)
  uint4 wa0, wa1, wa2, wa3, wa4, wa5, wb0, wb1, wb2, wb3, wb4, wb5;
  auto load_W = [&](int set, int kc0) {
    const uint16_t* base = a.planes + kc0;
    if (set == 0) {
      wa0 = *reinterpret_cast<const uint4*>(base + soff[0]);
      wa1 = *reinterpret_cast<const uint4*>(base + soff[1]);
      wa2 = *reinterpret_cast<const uint4*>(base + soff[2]);
      wa3 = *reinterpret_cast<const uint4*>(base + soff[3]);
      wa4 = *reinterpret_cast<const uint4*>(base + soff[4]);
      wa5 = *reinterpret_cast<const uint4*>(base + soff[5]);
    } else {
      wb0 = *reinterpret_cast<const uint4*>(base + soff[0]);
      wb1 = *reinterpret_cast<const uint4*>(base + soff[1]);
      wb2 = *reinterpret_cast<const uint4*>(base + soff[2]);
      wb3 = *reinterpret_cast<const uint4*>(base + soff[3]);
      wb4 = *reinterpret_cast<const uint4*>(base + soff[4]);
      wb5 = *reinterpret_cast<const uint4*>(base + soff[5]);
    }
  };
  auto store_W = [&](int set, int buf) {
    const uint4 v[6] = {set == 0 ? wa0 : wb0, set == 0 ? wa1 : wb1, set == 0 ? wa2 : wb2,
                        set == 0 ? wa3 : wb3, set == 0 ? wa4 : wb4, set == 0 ? wa5 : wb5};
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int q = tid + kBlock * j;
      const int pl = q >> 9, r = (q >> 3) & 63, sg = q & 7;
      *reinterpret_cast<uint4*>(&sW[buf][pl][r * kRtStride + 8 * sg]) = v[j];
    }
  };
  // x of one step: sub-step i, lane half h -> inputs 16i + 8h .. +7
  struct XStep {
    uint4 v[4];
  };
  auto load_X = [&](int kg, XStep& r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = *reinterpret_cast<const uint4*>(xrow + kg + 16 * i);
  };
  f32x16_t acc[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  const int nsteps = a.H / kRtKc;  // H % 256 == 0, so a multiple of 4
  XStep xr[4];  // x three steps ahead
  load_X(0, xr[0]);
  load_X(min(1, nsteps - 1) * kRtKc, xr[1]);
  load_X(min(2, nsteps - 1) * kRtKc, xr[2]);
  load_W(0, 0);
  load_W(1, min(1, nsteps - 1) * kRtKc);
  store_W(0, 0);
  lds_sync();
  load_W(0, min(2, nsteps - 1) * kRtKc);
  for (int st0 = 0; st0 < nsteps; st0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int st = st0 + u;
      load_X(min(st + 3, nsteps - 1) * kRtKc, xr[(u + 3) & 3]);
      const XStep& cur = xr[u];
      const int buf = u & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, cur.v[i]);
        // planes outer, row blocks inner: consecutive MFMAs use different accumulators
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const bf16x8_t A =
                *reinterpret_cast<const bf16x8_t*>(&sW[buf][pl][(32 * mb + n) * kRtStride + 16 * i + 8 * h]);
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[mb], 0, 0, 0);
          }
        }
      }
      // chunk st + 1 (in set (st + 1) & 1) into the other LDS buffer (its readers,
      // step st - 1, all passed the previous barrier); then fetch chunk st + 3
      // into the freed set
      store_W((u + 1) & 1, buf ^ 1);
      lds_sync();
      load_W((u + 1) & 1, min(st + 3, nsteps - 1) * kRtKc);
    }
  }
  const int tok_out = kRtT * tt + 32 * wave + n;
  if (tok_out >= a.M) return;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int sl = 0; sl < 16; ++sl)
      a.logits[(size_t)tok_out * a.E + kRtE * et + 32 * mb + c_row(lane, sl)] = acc[mb][sl];
}

// ------------------------------------------------------------------ top-k rows

struct TopkArgs {
  int M, E, k;
  const float* __restrict__ logits;
  int32_t* __restrict__ ids;
  float* __restrict__ w;
};

// One wavefront per token: the selection of the small-M router (route_dev.hpp:
// k largest logits, ties to the lower id, softmax over them) on logits that a
// previous launch produced.
__global__ __launch_bounds__(kBlock) void k_topk_rows(const TopkArgs a) {
  __shared__ __align__(16) int lds_all[kWavesPerBlock][kTopkLdsInts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWavesPerBlock + wave;
  if (t >= a.M) return;
  uint32_t key[kTopkEPL];
  bool present[kTopkEPL];
#pragma unroll
  for (int j = 0; j < kTopkEPL; ++j) {
    const int e = lane + kWave * j;
    present[j] = e < a.E;
    key[j] = present[j] ? sort_key(a.logits[(size_t)t * a.E + e]) : 0u;
  }
  int id;
  float w;
  topk_select(key, present, a.k, lane, lds_all[wave], id, w);
  if (lane < a.k) {
    a.ids[(size_t)t * a.k + lane] = id;
    a.w[(size_t)t * a.k + lane] = w;
  }
}

// ------------------------------------------------------------------ combine

struct CombineArgs {
  int M, E, k, H, has_shared;
  const int32_t* __restrict__ ids;
  const float* __restrict__ topk_w;
  const int32_t* __restrict__ inv;     // sorted position of each pair
  const _Float16* __restrict__ y;      // [S][H] per sorted position, scaled (see GgArgs::y)
  const int32_t* __restrict__ rexp;    // [M][2] per token: r, tx (the h exponent sigma = tx + le - 13)
  const uint32_t* __restrict__ meta;   // per-expert range data
  const float* __restrict__ ysh;    // [M][H]
  uint16_t* __restrict__ out;
  int32_t* __restrict__ err;
};

// One workgroup per token: the first k threads look up each slot's sorted
// row and the factor that takes its y back to the true scale 2^(sigma + e2 -
// 1) and weights it; then each thread sums 8 outputs over the slots in slot
// order (16-byte loads of every slot's row issued together), adds the shared
// expert's row and rounds to bf16.
__global__ __launch_bounds__(kBlock) void k_pf_combine(const CombineArgs a) {
  __shared__ int srow[kMaxTopK];
  __shared__ float swv[kMaxTopK];
  __shared__ int sbad;
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) sbad = 0;
  __syncthreads();
  if (tid < a.k) {
    const int p = t * a.k + tid;
    const int e = a.ids[p];
    if (e < 0 || e >= a.E) {
      srow[tid] = -1;
      swv[tid] = 0.f;
      sbad = 1;
    } else {
      const uint32_t* mt = a.meta + (size_t)e * kMetaWords;
      const int sigma = a.rexp[2 * t + 1] + exp_bound(__uint_as_float(mt[2])) - 13;
      srow[tid] = a.inv[p];
      swv[tid] = ldexpf(a.topk_w[p], sigma + exp_above(__uint_as_float(mt[3])) - 1);
    }
  }
  __syncthreads();
  for (int c = tid; c < a.H / 8; c += kBlock) {
    const int n0 = 8 * c;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < a.k; j0 += 8) {  // slots in batches of 8, loads first
      uint4 raw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = j0 + j < a.k ? srow[j0 + j] : -1;
        raw[j] = r >= 0 ? *reinterpret_cast<const uint4*>(a.y + (size_t)r * a.H + n0) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j0 + j >= a.k || srow[j0 + j] < 0) continue;
        const float wv = swv[j0 + j];
        const uint32_t d[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16x2_t v = __builtin_bit_cast(f16x2_t, d[q]);
          acc[2 * q] = fmaf(wv, (float)v[0], acc[2 * q]);
          acc[2 * q + 1] = fmaf(wv, (float)v[1], acc[2 * q + 1]);
        }
      }
    }
    if (a.has_shared) {
      const float4 v0 = *reinterpret_cast<const float4*>(a.ysh + (size_t)t * a.H + n0);
      const float4 v1 = *reinterpret_cast<const float4*>(a.ysh + (size_t)t * a.H + n0 + 4);
      acc[0] += v0.x; acc[1] += v0.y; acc[2] += v0.z; acc[3] += v0.w;
      acc[4] += v1.x; acc[5] += v1.y; acc[6] += v1.z; acc[7] += v1.w;
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
    *reinterpret_cast<uint4*>(a.out + (size_t)t * a.H + n0) = o;
  }
  if (tid == 0 && sbad) atomicOr(a.err, 1);
}

// ------------------------------------------------------------------ host side

bool prefill_supported(const Shape& s) {
  // K of both GEMMs a whole number of 256-input blocks (four 64-K steps);
  // weight tiles of 64 rows; router tiles of 64 experts; at most 8192 terms
  // in the fp32 norm sums that the h exponent bounds (exp_bound's slack)
  return s.H % 256 == 0 && s.I % 256 == 0 && s.E % 64 == 0 && s.H <= 8192 && s.I <= 8192;
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

hipError_t launch_prefill_route(const Shape& s, const float* router_w, const uint16_t* x, int M, int32_t* ids,
                                float* w, uint8_t* ws, const PfLayout& P, hipStream_t st) {
  uint16_t* planes = reinterpret_cast<uint16_t*>(ws + P.rt_planes);
  const size_t plane = (size_t)s.E * s.H, n8 = plane / 8;
  hipLaunchKernelGGL(k_rt_split, dim3((unsigned)((n8 + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, router_w, n8,
                     planes, plane);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RtArgs a{M, s.E, s.H, x, planes, reinterpret_cast<float*>(ws + P.logits)};
  hipLaunchKernelGGL(k_rt_gemm, dim3((unsigned)((s.E / kRtE) * ceil_div(M, kRtT))), dim3(kBlock), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  TopkArgs t{M, s.E, s.k, a.logits, ids, w};
  hipLaunchKernelGGL(k_topk_rows, dim3(ceil_div(M, kWavesPerBlock)), dim3(kBlock), 0, st, t);
  return hipGetLastError();
}

// Grid of a grouped GEMM: items rounded up to a multiple of the 8 XCDs, times
// the workgroups per item.
static dim3 gg_grid(int items, int ng) { return dim3((unsigned)(8 * ceil_div(items, 8) * ng)); }

hipError_t launch_prefill_forward(const Shape& s, const uint8_t* packed, const PackedLayout& PL, const uint16_t* x,
                                  int M, const int32_t* ids, const float* w, uint16_t* out, uint8_t* ws,
                                  const PfLayout& P, hipStream_t st) {
  auto i32 = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
  int32_t* err = i32(P.err);
  hipError_t e = launch_permute_items(s, ids, M, i32(P.counts), i32(P.offsets), i32(P.perm), i32(P.inv),
                                      i32(P.tile_e), i32(P.tile_j), i32(P.ntile), i32(P.ghist), err, st);
  if (e != hipSuccess) return e;
  _Float16* xh = reinterpret_cast<_Float16*>(ws + P.xh);
  hipLaunchKernelGGL(k_pf_xprep, dim3(M), dim3(kBlock), 0, st, x, s.H, xh, i32(P.rexp));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const KSplit kg = ksplit_for(s.H / kGroup), kd = ksplit_for(s.I / kGroup);
  GgArgs a{};
  a.M = M; a.E = s.E; a.k = s.k; a.H = s.H; a.I = s.I;
  a.counts = i32(P.counts); a.offsets = i32(P.offsets); a.perm = i32(P.perm);
  a.tile_e = i32(P.tile_e); a.tile_j = i32(P.tile_j); a.ntile = i32(P.ntile);
  a.xh = xh; a.rexp = i32(P.rexp);
  a.hbuf = reinterpret_cast<const _Float16*>(ws + P.hbuf);
  a.x = x;
  a.hsh = reinterpret_cast<const uint16_t*>(ws + P.hsh);
  a.meta = reinterpret_cast<const uint32_t*>(packed + PL.meta);
  a.hout = reinterpret_cast<_Float16*>(ws + P.hbuf);
  a.hsh_out = reinterpret_cast<uint16_t*>(ws + P.hsh);
  a.y = reinterpret_cast<_Float16*>(ws + P.y);
  a.ysh = reinterpret_cast<float*>(ws + P.ysh);
  // gate_up
  a.K = s.H;
  a.ntiles = s.I / 32;
  a.ng = ceil_div(a.ntiles, kWavesPerBlock);
  a.q = packed + PL.gu_q; a.s = reinterpret_cast<const uint16_t*>(packed + PL.gu_s);
  a.q_stride = PL.gu_q_stride; a.s_stride = PL.gu_s_stride / 2; a.P = kg.P; a.pshift = kg.P == 4 ? 2 : kg.P - 1;
  a.shw = reinterpret_cast<const uint16_t*>(packed + PL.sh_gu);
  a.meta_word = 0;
  if (s.has_shared) {
    const int rb = (int)gg_grid(P.items, a.ng).x;
    const int sb = (int)gg_grid(ceil_div(M, GgCfg<GG_SGU>::ROWS), a.ng).x;
    hipLaunchKernelGGL((k_gg2<GG_RGU, GG_SGU>), dim3(rb + sb), dim3(kBlock), 0, st, a, rb);
  } else {
    hipLaunchKernelGGL(k_gg<GG_RGU>, gg_grid(P.items, a.ng), dim3(kBlock), 0, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // down
  a.K = s.I;
  a.ntiles = s.H / 64;
  a.ng = ceil_div(a.ntiles, kWavesPerBlock);
  a.q = packed + PL.dn_q; a.s = reinterpret_cast<const uint16_t*>(packed + PL.dn_s);
  a.q_stride = PL.dn_q_stride; a.s_stride = PL.dn_s_stride / 2; a.P = kd.P; a.pshift = kd.P == 4 ? 2 : kd.P - 1;
  a.shw = reinterpret_cast<const uint16_t*>(packed + PL.sh_dn);
  a.meta_word = 1;
  if (s.has_shared) {
    const int rb = (int)gg_grid(P.items, a.ng).x;
    const int sb = (int)gg_grid(ceil_div(M, GgCfg<GG_SDN>::ROWS), a.ng).x;
    hipLaunchKernelGGL((k_gg2<GG_RDN, GG_SDN>), dim3(rb + sb), dim3(kBlock), 0, st, a, rb);
  } else {
    hipLaunchKernelGGL(k_gg<GG_RDN>, gg_grid(P.items, a.ng), dim3(kBlock), 0, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  CombineArgs c{M, s.E, s.k, s.H, s.has_shared, ids, w, i32(P.inv), a.y, i32(P.rexp), a.meta, a.ysh, out, err};
  hipLaunchKernelGGL(k_pf_combine, dim3((unsigned)M), dim3(kBlock), 0, st, c);
  return hipGetLastError();
}

}  // namespace moe
