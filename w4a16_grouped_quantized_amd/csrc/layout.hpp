// layout.hpp — the library's device layout of the expert weights, and the
// work split every kernel and the packer agree on.  Host and device code.
//
// Routed INT4 matrices (per expert, W is N rows x K inputs, groups of 32):
//   rows are taken in tiles of 64; one wavefront lane owns one row of a tile.
//   gate_up (N = 2I): tile b holds gate rows 32b..32b+31 in lanes 0..31 and
//     the matching up rows I+32b..I+32b+31 in lanes 32..63, so the SiLU*up
//     product of a row pair never leaves the tile.
//   down (N = H): tile b holds rows 64b..64b+63.
//   codes: 16 bytes per (tile, group, lane) = the 32 codes of one row-group,
//     at ((tile * K/32 + group) * 64 + lane) * 16.  Inside those 16 bytes,
//     dword d covers inputs 8d..8d+7 of the group; nibble i (bits 4i..4i+3)
//     holds input 8d+2i and nibble 4+i (bits 16+4i..) holds input 8d+2i+1,
//     so (dword >> 4i) & 0x000F000F isolates the code pair of inputs
//     (8d+2i, 8d+2i+1) in the two 16-bit halves.
//   scales: bf16, P consecutive groups per lane and load:
//     at ((tile * (K/32)/P + group/P) * 64 + lane) * P + group % P  (elements).
// Experts are stored one after another, each as one block of its gate_up
// codes, gate_up scales, down codes and down scales (every part 256-byte
// aligned): the bytes a step reads for one expert then span 2-3 pages of
// the GPU's address translation instead of one page per part (measured on
// reads of 8 random experts over 48 GB of layer copies: 8.3 against 9.2 us).
// Shared BF16 matrices: tile b, chunk c of 8 inputs, lane l:
//   16 bytes at ((tile * K/8 + c) * 64 + lane) * 16, inputs in natural order;
//   same row-to-lane mapping as the routed matrices.
// Per-expert range data (kMetaWords uint32 per expert, float bit patterns of
// non-negative values, used by the many-token kernels to scale fp16 operands
// by powers of two):
//   [0] max |scale| of gate_up, [1] max |scale| of down,
//   [2] max over r < I of ||gate row r||_2 * ||up row r||_2 (dequantised),
//   [3] max over the down rows of ||down row||_1 (dequantised).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kBlock = 256;   // 4 wavefronts per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kGroup = 32;

// How a workgroup's 4 wavefronts split the K/32 groups of one tile row-set:
// W active wavefronts take GW consecutive groups each; scales are packed P
// groups per lane-load with P dividing GW.
struct KSplit {
  int W, GW, P;
};

__host__ __device__
inline KSplit ksplit_for(int groups) {
  KSplit s;
  s.W = (groups % 4 == 0) ? 4 : (groups % 2 == 0 ? 2 : 1);
  s.GW = groups / s.W;
  s.P = (s.GW % 4 == 0) ? 4 : (s.GW % 2 == 0 ? 2 : 1);
  return s;
}

// Shared-expert K split: the K inputs of one tile are cut into KS slices
// across workgroups, each slice into 4 wavefront ranges of CW chunks of 8.
struct SharedSplit {
  int KS, CW;
};

__host__ __device__
inline SharedSplit shared_split_for(int K, int target_chunks_per_wave) {
  SharedSplit s{1, K / 8 / kWavesPerBlock};
  // largest KS with K/8/4 divisible by KS and chunks per wave >= target
  for (int ks = 1; ks <= 8; ++ks) {
    int chunks = K / 8 / kWavesPerBlock;
    if (chunks % ks) continue;
    if (chunks / ks < target_chunks_per_wave) break;
    s.KS = ks;
    s.CW = chunks / ks;
  }
  return s;
}

constexpr int kMetaWords = 4;

struct PackedLayout {
  // byte offsets inside the packed buffer: of each part of expert 0, then of
  // the shared matrices, the range data and the end
  size_t gu_q, gu_s, dn_q, dn_s, sh_gu, sh_dn, meta, total;
  // per-expert strides in bytes (all equal: the size of one expert's block)
  size_t gu_q_stride, gu_s_stride, dn_q_stride, dn_s_stride;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Bytes of one expert's parts as stored (also their per-expert strides in
// the plain checkpoint layout); SB is the bytes of one scale (2 for the
// bf16 scales of INT4, 1 for the E8M0 scales of MXFP4).
__host__ __device__ inline size_t gu_codes_bytes(int H, int I) { return (size_t)2 * I * H / 2; }
__host__ __device__ inline size_t gu_scales_bytes(int H, int I, int SB = 2) { return (size_t)2 * I * (H / kGroup) * SB; }
__host__ __device__ inline size_t dn_codes_bytes(int H, int I) { return (size_t)H * I / 2; }
__host__ __device__ inline size_t dn_scales_bytes(int H, int I, int SB = 2) { return (size_t)H * (I / kGroup) * SB; }

// The routed experts in MXFP4 use the same tiles: a (tile, group, lane)
// chunk holds the row-group's 16 bytes as the checkpoint stores them (byte
// b of dword d: inputs 8d+2b in the low nibble, 8d+2b+1 in the high one),
// and the E8M0 scales are packed like the bf16 ones, one byte each.
__host__ __device__
inline PackedLayout packed_layout(int H, int E, int I, int has_shared, int SB = 2) {
  PackedLayout L;
  auto a256 = [](size_t v) { return (v + 255) / 256 * 256; };
  L.gu_q = 0;
  L.gu_s = L.gu_q + a256(gu_codes_bytes(H, I));
  L.dn_q = L.gu_s + a256(gu_scales_bytes(H, I, SB));
  L.dn_s = L.dn_q + a256(dn_codes_bytes(H, I));
  const size_t block = L.dn_s + a256(dn_scales_bytes(H, I, SB));
  L.gu_q_stride = L.gu_s_stride = L.dn_q_stride = L.dn_s_stride = block;
  size_t off = block * E;
  L.sh_gu = off; if (has_shared) off = (off + (size_t)2 * I * H * 2 + 255) / 256 * 256;
  L.sh_dn = off; if (has_shared) off = (off + (size_t)H * I * 2 + 255) / 256 * 256;
  L.meta = off; off = (off + (size_t)E * kMetaWords * 4 + 255) / 256 * 256;
  L.total = off;
  return L;
}

// Row of matrix tile b served by lane l.
__host__ __device__
inline int gu_row(int b, int l, int I) { return l < 32 ? 32 * b + l : I + 32 * b + (l - 32); }

}  // namespace moe
