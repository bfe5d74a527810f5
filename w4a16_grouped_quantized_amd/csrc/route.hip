// route.hip — router GEMV, top-k selection and softmax weights (one launch).
//
// Each wavefront owns one router row (fp32, H inputs): lane l holds inputs
// 256*i + 4*l .. +3 for i < H/256, so every wavefront load of a row is one
// contiguous KiB.  The row stays in registers while the wavefront walks the
// tokens; per token the 4*H/256 products of a lane are summed in order and
// the lanes are combined by a fixed xor butterfly (a tree, not one long
// serial sum).  The workgroup that finishes last (counted through a
// two-level tree of arrival counters) selects, per token, the k
// largest logits (ties -> lower expert id) and writes the softmax over them.
// With MOE_F_INPUT_RMSNORM each wavefront first normalises the token
// (unit-gain RMSNorm, rounded to bf16) and workgroup 0 stores the result.
#include "route_dev.hpp"

namespace moe {


template <int NI>
__global__ __launch_bounds__(kBlock) void k_route(const RouteArgs a) {
  __shared__ int flag;
  __shared__ __align__(16) int topk_lds[kWavesPerBlock][kTopkLdsInts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  router_row<NI>(a, blockIdx.x * kWavesPerBlock + wave, lane, blockIdx.x == 0 && wave == 0);
  if (!arrive_last_tree(a.cnt, blockIdx.x, gridDim.x, &flag)) return;
  for (int t = wave; t < a.M; t += kWavesPerBlock) topk_token(a, t, lane, topk_lds[wave]);
}

namespace {
template <int NI>
hipError_t run_route(const RouteArgs& a, hipStream_t st) {
  const int grid = (a.E + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((k_route<NI>), dim3(grid), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}
}  // namespace

bool route_supported(const Shape& s) { return s.H == 2560 || s.H == 256; }

hipError_t launch_route(const Shape& s, const float* router_w, const uint16_t* x, int M,
                        bool rmsnorm, float eps, uint16_t* x_norm, int32_t* ids, float* w,
                        uint8_t* ws, const WsLayout& L, hipStream_t st) {
  RouteArgs a;
  a.M = M; a.E = s.E; a.k = s.k; a.H = s.H;
  a.rmsnorm = rmsnorm ? 1 : 0;
  a.eps = eps;
  a.wr = router_w; a.x = x; a.x_norm = x_norm;
  a.logits = reinterpret_cast<float*>(ws + L.logits);
  a.cnt = reinterpret_cast<int32_t*>(ws + L.route_cnt);
  a.ids = ids; a.w = w;
  if (s.H == 2560) return run_route<10>(a, st);
  if (s.H == 256) return run_route<1>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace moe
