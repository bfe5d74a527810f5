// launch.hpp — host-side launchers of the kernels (one per .hip file).
// Every launcher assumes its arguments were validated by the C-ABI layer and
// returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

constexpr int kMaxExperts = 512;   // LDS tables are sized for this
constexpr int kMaxSlots = 4096;    // M * k handled by the decode (GEMV) kernels
constexpr int kMaxTopK = 64;
constexpr int kMaxGroups = 128;    // K/32 of the largest K (LDS group table)
constexpr int kMaxKSplit = 8;      // K slices of a shared-expert tile across workgroups

struct Shape {
  int H, E, k, I, has_shared;
};

// routed/shared GEMV kernels: true if a kernel is compiled for this shape
bool experts_supported(const Shape& s);
bool route_supported(const Shape& s);

hipError_t launch_route(const Shape& s, const float* router_w, const uint16_t* x, int M,
                        bool rmsnorm, float eps, uint16_t* x_norm, int32_t* ids, float* w,
                        uint8_t* ws, const WsLayout& L, hipStream_t st);

// gate_up stage: h (routed, per slot) and h_sh (shared) into the workspace
hipError_t launch_gate_up(const Shape& s, const uint8_t* packed, const PackedLayout& P, const uint16_t* x,
                          int M, const int32_t* ids, uint8_t* ws, const WsLayout& L, hipStream_t st);
// down stage + weighted combine: reads h / h_sh from the workspace
hipError_t launch_down(const Shape& s, const uint8_t* packed, const PackedLayout& P, int M,
                       const int32_t* ids, const float* w, uint16_t* out, uint8_t* ws, const WsLayout& L,
                       hipStream_t st);

// The whole small-M layer in one launch (M*k <= kMaxUnits): with route, the
// router, top-k and softmax too (ids and w are written); without, ids and w
// are read.  rmsnorm only with route.  mxfp4: the routed experts are MXFP4
// in the tiled layout (launch_pack_mxfp4) instead of INT4.
bool layer_supported(const Shape& s, int M);
hipError_t launch_layer(const Shape& s, const uint8_t* packed, const PackedLayout& PL, const float* router_w,
                        const uint16_t* x, int M, bool route, bool rmsnorm, float eps, uint16_t* x_norm,
                        int32_t* ids, float* w, uint16_t* out, uint8_t* ws, const WsLayout& L, hipStream_t st,
                        bool mxfp4 = false);

hipError_t launch_permute(const Shape& s, const int32_t* ids, int M, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* ghist, int32_t* err, hipStream_t st);

// The permutation plus its inverse (sorted position of each pair) and the
// work items of the grouped GEMMs: item i < *ntile covers rows
// [kItemRows * tile_j[i], ...) of expert tile_e[i]'s sorted run.
hipError_t launch_permute_items(const Shape& s, const int32_t* ids, int M, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, int32_t* tile_e, int32_t* tile_j, int32_t* ntile,
                                int32_t* ghist, int32_t* err, hipStream_t st);

// Many-token path (prefill): router GEMM + per-token top-k, and the grouped
// expert GEMMs on the matrix cores.
bool prefill_supported(const Shape& s);
hipError_t launch_prefill_route(const Shape& s, const float* router_w, const uint16_t* x, int M, int32_t* ids,
                                float* w, uint8_t* ws, const PfLayout& P, hipStream_t st);
hipError_t launch_prefill_forward(const Shape& s, const uint8_t* packed, const PackedLayout& PL, const uint16_t* x,
                                  int M, const int32_t* ids, const float* w, uint16_t* out, uint8_t* ws,
                                  const PfLayout& P, hipStream_t st);

hipError_t launch_pack(const Shape& s, const uint8_t* w13_q, const uint16_t* w13_s,
                       const uint8_t* w2_q, const uint16_t* w2_s, const uint16_t* sh_w13,
                       const uint16_t* sh_w2, uint8_t* packed, const PackedLayout& P,
                       hipStream_t st);

hipError_t launch_pack_mxfp4(const Shape& s, const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                             const uint8_t* w2_s, const uint16_t* sh_w13, const uint16_t* sh_w2, uint8_t* packed,
                             const PackedLayout& P, hipStream_t st);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// FP8 LM head: per-row E4M3 quantisation of a BF16 head, and the GEMV with an
// FP8 or the BF16 head (M <= 4 tokens).
bool lmhead_supported(int H, bool fp8);
hipError_t launch_lmhead_quant(const uint16_t* w, int V, int H, uint8_t* q, float* s, hipStream_t st);
hipError_t launch_lmhead_gemv(bool fp8, const uint8_t* w, const float* s, int V, int H, const uint16_t* x, int M,
                              float* out, hipStream_t st);

// Routed experts in MXFP4 or block FP8 (plain layout), M <= 8: gate_up then
// down + combine, with the shared expert in BF16.
constexpr int kFmtMxfp4 = 1, kFmtFp8Block = 2, kFmtBf16 = 3;
bool fmt_plan(const Shape& s, int fmt, int M, int* ra, int* rsh, int* rb);
hipError_t launch_forward_fmt(const Shape& s, int fmt, const uint8_t* w13_q, const void* w13_s, const uint8_t* w2_q,
                              const void* w2_s, const uint16_t* sh_w13, const uint16_t* sh_w2, const uint16_t* x,
                              int M, const int32_t* ids, const float* w, uint16_t* out, uint8_t* ws,
                              const WsLayout& L, hipStream_t st);

}  // namespace moe
