// api.hip — the C ABI (include/moe_w4a16.h): argument checks, workspace and
// packed-layout bookkeeping, and the launches.  Nothing here allocates device
// memory or synchronises except moe_get_device_error.
#include "moe_w4a16.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "launch.hpp"

using namespace moe;

namespace {

constexpr float kRmsEps = 1e-6f;
// Token counts at which the many-token path takes over (when a kernel is
// compiled for the shape): the router as an MFMA GEMM beyond 32 tokens, the
// experts as grouped MFMA GEMMs beyond 512 (token, slot) pairs.
constexpr int kRouteGemmMinTokens = 33;
constexpr int64_t kPrefillMinSlots = 513;

bool route_gemm(const Shape& s, int M) { return M >= kRouteGemmMinTokens && prefill_supported(s); }
bool experts_gemm(const Shape& s, int M) { return (int64_t)M * s.k >= kPrefillMinSlots && prefill_supported(s); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// True if the byte ranges [a, a + n) and [b, b + n) share a byte.
bool overlap(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + n && y < x + n;
}

// Shape checks shared by every entry point.
int check_cfg(const moe_config* c, Shape* s) {
  if (!c) return MOE_ERR_NULL;
  if (c->group_size != kGroup) return MOE_ERR_UNSUPPORTED;
  if (c->hidden <= 0 || c->hidden % 256) return MOE_ERR_SHAPE;
  if (c->inter <= 0 || c->inter % 32) return MOE_ERR_SHAPE;
  if (c->n_experts < 1 || c->top_k < 1 || c->top_k > c->n_experts) return MOE_ERR_SHAPE;
  if (c->has_shared != 0 && c->has_shared != 1) return MOE_ERR_SHAPE;
  if (c->n_experts > kMaxExperts || c->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (c->hidden / kGroup > kMaxGroups || c->inter / kGroup > kMaxGroups) return MOE_ERR_UNSUPPORTED;
  s->H = c->hidden; s->E = c->n_experts; s->k = c->top_k; s->I = c->inter; s->has_shared = c->has_shared;
  return MOE_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// The library's own workspace for moe_layer_w4a16_noalloc: one copy per GPU,
// zero at load like every static, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it names a stand-in,
// not device memory); it uses the address hipGetSymbolAddress gives on each
// device.
constexpr size_t kScratchBytes = MOE_NOALLOC_WS_BYTES;
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's copy of scratch (nullptr if its address cannot be had).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t moe_packed_size(const moe_config* cfg) {
  Shape s;
  if (check_cfg(cfg, &s) != MOE_OK) return 0;
  return packed_layout(s.H, s.E, s.I, s.has_shared).total;
}

int moe_pack_weights(const moe_config* cfg, const moe_weights_plain* src, void* packed, size_t packed_bytes,
                     void* stream) {
  Shape s;
  int rc = check_cfg(cfg, &s);
  if (rc != MOE_OK) return rc;
  if (!src || !packed || !src->w13_q || !src->w13_s || !src->w2_q || !src->w2_s) return MOE_ERR_NULL;
  if (s.has_shared ? (!src->sh_w13 || !src->sh_w2) : (src->sh_w13 || src->sh_w2)) return MOE_ERR_NULL;
  if (!aligned16(packed) || !aligned16(src->w13_q) || !aligned16(src->w2_q) || !aligned4(src->w13_s) ||
      !aligned4(src->w2_s) || (s.has_shared && (!aligned16(src->sh_w13) || !aligned16(src->sh_w2))))
    return MOE_ERR_ALIGN;
  const PackedLayout P = packed_layout(s.H, s.E, s.I, s.has_shared);
  if (packed_bytes < P.total) return MOE_ERR_WORKSPACE;
  return launched(launch_pack(s, src->w13_q, src->w13_s, src->w2_q, src->w2_s, src->sh_w13, src->sh_w2,
                              static_cast<uint8_t*>(packed), P, static_cast<hipStream_t>(stream)));
}

size_t moe_workspace_size(const moe_config* cfg, int32_t max_tokens) {
  Shape s;
  if (check_cfg(cfg, &s) != MOE_OK || max_tokens < 0) return 0;
  const int M = max_tokens < 1 ? 1 : max_tokens;
  size_t n = ws_layout(s.H, s.E, s.k, s.I, s.has_shared, M).total;
  if (prefill_supported(s)) {
    const size_t p = pf_layout(s.H, s.E, s.k, s.I, s.has_shared, M).total;
    n = p > n ? p : n;
  }
  return n;
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return MOE_ERR_NULL;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  return launched(launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

int moe_route(const moe_config* cfg, const float* router_w, const uint16_t* x, int32_t M, uint32_t flags,
              uint16_t* x_norm, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_cfg(cfg, &s);
  if (rc != MOE_OK) return rc;
  if (M < 0 || (flags & ~MOE_F_INPUT_RMSNORM)) return MOE_ERR_SHAPE;
  if (M == 0) return MOE_OK;
  const bool rms = (flags & MOE_F_INPUT_RMSNORM) != 0;
  if (!router_w || !x || !topk_ids || !topk_w || !ws || (rms && !x_norm)) return MOE_ERR_NULL;
  if (!aligned16(router_w) || !aligned16(x) || !aligned16(ws) || !aligned4(topk_ids) || !aligned4(topk_w) ||
      (rms && !aligned16(x_norm)))
    return MOE_ERR_ALIGN;
  // the normalised tokens are written while other workgroups still read x
  if (rms && overlap(x, x_norm, (size_t)M * s.H * 2)) return MOE_ERR_SHAPE;
  if (route_gemm(s, M) && !rms) {
    const PfLayout P = pf_layout(s.H, s.E, s.k, s.I, s.has_shared, M);
    if (ws_bytes < P.total) return MOE_ERR_WORKSPACE;
    return launched(launch_prefill_route(s, router_w, x, M, topk_ids, topk_w, static_cast<uint8_t*>(ws), P,
                                         static_cast<hipStream_t>(stream)));
  }
  if (!route_supported(s)) return MOE_ERR_UNSUPPORTED;
  const WsLayout L = ws_layout(s.H, s.E, s.k, s.I, s.has_shared, M);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return launched(launch_route(s, router_w, x, M, rms, kRmsEps, x_norm, topk_ids, topk_w,
                               static_cast<uint8_t*>(ws), L, static_cast<hipStream_t>(stream)));
}

namespace {
// Checks shared by the expert stages; x / topk_w / out are checked only when
// the stage uses them (need_* flags).
int check_experts(const moe_config* cfg, Shape* s, const void* packed, const uint16_t* x, int32_t M,
                  const int32_t* topk_ids, const float* topk_w, const uint16_t* out, const void* ws,
                  size_t ws_bytes, bool need_x, bool need_out, WsLayout* L) {
  int rc = check_cfg(cfg, s);
  if (rc != MOE_OK) return rc;
  if (M < 0) return MOE_ERR_SHAPE;
  if (M == 0) return MOE_OK;
  if (!packed || !topk_ids || !ws || (need_x && !x) || (need_out && (!topk_w || !out))) return MOE_ERR_NULL;
  if (!aligned16(packed) || !aligned16(ws) || !aligned4(topk_ids) || (need_x && !aligned16(x)) ||
      (need_out && (!aligned16(out) || !aligned4(topk_w))))
    return MOE_ERR_ALIGN;
  if (!experts_supported(*s)) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)M * s->k > kMaxSlots) return MOE_ERR_UNSUPPORTED;
  *L = ws_layout(s->H, s->E, s->k, s->I, s->has_shared, M);
  if (ws_bytes < L->total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}
}  // namespace

int moe_gate_up_w4a16(const moe_config* cfg, const void* packed, const uint16_t* x, int32_t M,
                      const int32_t* topk_ids, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  WsLayout L;
  int rc = check_experts(cfg, &s, packed, x, M, topk_ids, nullptr, nullptr, ws, ws_bytes, true, false, &L);
  if (rc != MOE_OK || M == 0) return rc;
  const PackedLayout P = packed_layout(s.H, s.E, s.I, s.has_shared);
  return launched(launch_gate_up(s, static_cast<const uint8_t*>(packed), P, x, M, topk_ids,
                                 static_cast<uint8_t*>(ws), L, static_cast<hipStream_t>(stream)));
}

int moe_down_w4a16(const moe_config* cfg, const void* packed, int32_t M, const int32_t* topk_ids,
                   const float* topk_w, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  WsLayout L;
  int rc = check_experts(cfg, &s, packed, nullptr, M, topk_ids, topk_w, out, ws, ws_bytes, false, true, &L);
  if (rc != MOE_OK || M == 0) return rc;
  const PackedLayout P = packed_layout(s.H, s.E, s.I, s.has_shared);
  return launched(launch_down(s, static_cast<const uint8_t*>(packed), P, M, topk_ids, topk_w, out,
                              static_cast<uint8_t*>(ws), L, static_cast<hipStream_t>(stream)));
}

int moe_forward_w4a16(const moe_config* cfg, const void* packed, const uint16_t* x, int32_t M,
                      const int32_t* topk_ids, const float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                      void* stream) {
  Shape s;
  WsLayout L;
  {
    int rc0 = check_cfg(cfg, &s);
    if (rc0 == MOE_OK && M > 0 && experts_gemm(s, M)) {
      if (!packed || !x || !topk_ids || !topk_w || !out || !ws) return MOE_ERR_NULL;
      if (!aligned16(packed) || !aligned16(x) || !aligned16(out) || !aligned16(ws) || !aligned4(topk_ids) ||
          !aligned4(topk_w))
        return MOE_ERR_ALIGN;
      const PfLayout P = pf_layout(s.H, s.E, s.k, s.I, s.has_shared, M);
      if (ws_bytes < P.total) return MOE_ERR_WORKSPACE;
      const PackedLayout PL = packed_layout(s.H, s.E, s.I, s.has_shared);
      return launched(launch_prefill_forward(s, static_cast<const uint8_t*>(packed), PL, x, M, topk_ids, topk_w, out,
                                             static_cast<uint8_t*>(ws), P, static_cast<hipStream_t>(stream)));
    }
  }
  int rc = check_experts(cfg, &s, packed, x, M, topk_ids, topk_w, out, ws, ws_bytes, true, true, &L);
  if (rc != MOE_OK || M == 0) return rc;
  const PackedLayout P = packed_layout(s.H, s.E, s.I, s.has_shared);
  const uint8_t* pk = static_cast<const uint8_t*>(packed);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = launched(launch_gate_up(s, pk, P, x, M, topk_ids, w8, L, st));
  if (rc != MOE_OK) return rc;
  return launched(launch_down(s, pk, P, M, topk_ids, topk_w, out, w8, L, st));
}

int moe_layer_w4a16(const moe_config* cfg, const float* router_w, const void* packed, const uint16_t* x, int32_t M,
                    uint32_t flags, uint16_t* x_norm, int32_t* topk_ids, float* topk_w, uint16_t* out, void* ws,
                    size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_cfg(cfg, &s);
  if (rc != MOE_OK) return rc;
  if (M < 0 || (flags & ~(MOE_F_INPUT_RMSNORM | MOE_F_ONE_LAUNCH))) return MOE_ERR_SHAPE;
  if (M == 0) return MOE_OK;
  const bool rms = (flags & MOE_F_INPUT_RMSNORM) != 0;
  const bool one = M <= 2 || (flags & MOE_F_ONE_LAUNCH) != 0;
  if (!router_w || !packed || !x || !topk_ids || !topk_w || !out || !ws || (rms && !x_norm)) return MOE_ERR_NULL;
  if (!aligned16(router_w) || !aligned16(packed) || !aligned16(x) || !aligned16(out) || !aligned16(ws) ||
      !aligned4(topk_ids) || !aligned4(topk_w) || (rms && !aligned16(x_norm)))
    return MOE_ERR_ALIGN;
  if (rms && overlap(x, x_norm, (size_t)M * s.H * 2)) return MOE_ERR_SHAPE;
  if (one && layer_supported(s, M) && route_supported(s)) {
    WsLayout L;
    rc = check_experts(cfg, &s, packed, x, M, topk_ids, topk_w, out, ws, ws_bytes, true, true, &L);
    if (rc != MOE_OK) return rc;
    const PackedLayout P = packed_layout(s.H, s.E, s.I, s.has_shared);
    const hipError_t e = launch_layer(s, static_cast<const uint8_t*>(packed), P, router_w, x, M, true, rms, kRmsEps,
                                      x_norm, topk_ids, topk_w, out, static_cast<uint8_t*>(ws), L,
                                      static_cast<hipStream_t>(stream));
    // a device that cannot hold the whole grid at once takes the two calls
    if (e != hipErrorInvalidConfiguration) return launched(e);
  }
  rc = moe_route(cfg, router_w, x, M, flags & MOE_F_INPUT_RMSNORM, x_norm, topk_ids, topk_w, ws, ws_bytes, stream);
  if (rc != MOE_OK) return rc;
  return moe_forward_w4a16(cfg, packed, rms ? x_norm : x, M, topk_ids, topk_w, out, ws, ws_bytes, stream);
}

int moe_layer_w4a16_noalloc(const moe_config* cfg, const float* router_w, const void* packed, const uint16_t* x,
                            int32_t M, uint32_t flags, uint16_t* x_norm, int32_t* topk_ids, float* topk_w,
                            uint16_t* out, void* stream) {
  if (M == 0) return MOE_OK;
  // the sizes are checked before the set-up (and again by moe_layer_w4a16)
  Shape s;
  const int rc = check_cfg(cfg, &s);
  if (rc != MOE_OK) return rc;
  if (M < 0) return MOE_ERR_SHAPE;
  if (moe_workspace_size(cfg, M) > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_LAUNCH;
  return moe_layer_w4a16(cfg, router_w, packed, x, M, flags, x_norm, topk_ids, topk_w, out, ws, kScratchBytes,
                         stream);
}

int moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t M, int32_t* counts, int32_t* offsets,
                int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_cfg(cfg, &s);
  if (rc != MOE_OK) return rc;
  if (M < 0) return MOE_ERR_SHAPE;
  if (!counts || !offsets || !ws || (M > 0 && (!topk_ids || !perm))) return MOE_ERR_NULL;
  if (!aligned4(counts) || !aligned4(offsets) || !aligned4(perm) || !aligned4(topk_ids) || !aligned16(ws))
    return MOE_ERR_ALIGN;
  const WsLayout L = ws_layout(s.H, s.E, s.k, s.I, s.has_shared, M < 1 ? 1 : M);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  return launched(launch_permute(s, topk_ids, M, counts, offsets, perm, reinterpret_cast<int32_t*>(w8 + L.ghist),
                                 reinterpret_cast<int32_t*>(w8 + L.err), static_cast<hipStream_t>(stream)));
}

int moe_forward_fmt(const moe_config* cfg, int32_t fmt, const moe_weights_fmt* w, const uint16_t* x, int32_t M,
                    const int32_t* topk_ids, const float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                    void* stream) {
  Shape s;
  int rc = check_cfg(cfg, &s);
  if (rc != MOE_OK) return rc;
  if (fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_FP8_BLOCK) return MOE_ERR_UNSUPPORTED;
  if (M < 0) return MOE_ERR_SHAPE;
  if (M == 0) return MOE_OK;
  if (!w || !x || !topk_ids || !topk_w || !out || !ws || !w->w13_q || !w->w13_s || !w->w2_q || !w->w2_s)
    return MOE_ERR_NULL;
  if (s.has_shared ? (!w->sh_w13 || !w->sh_w2) : (w->sh_w13 || w->sh_w2)) return MOE_ERR_NULL;
  if (!aligned16(w->w13_q) || !aligned16(w->w2_q) || !aligned16(x) || !aligned16(out) || !aligned16(ws) ||
      !aligned4(topk_ids) || !aligned4(topk_w) ||
      (fmt == MOE_FMT_FP8_BLOCK && (!aligned4(w->w13_s) || !aligned4(w->w2_s))) ||
      (s.has_shared && (!aligned16(w->sh_w13) || !aligned16(w->sh_w2))))
    return MOE_ERR_ALIGN;
  int ra, rsh, rb;
  if (!fmt_plan(s, fmt, M, &ra, &rsh, &rb)) return MOE_ERR_UNSUPPORTED;
  const WsLayout L = ws_layout(s.H, s.E, s.k, s.I, s.has_shared, M);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  return launched(launch_forward_fmt(s, fmt, w->w13_q, w->w13_s, w->w2_q, w->w2_s, w->sh_w13, w->sh_w2, x, M,
                                     topk_ids, topk_w, out, static_cast<uint8_t*>(ws), L,
                                     static_cast<hipStream_t>(stream)));
}

size_t moe_packed_size_mxfp4(const moe_config* cfg) {
  Shape s;
  if (check_cfg(cfg, &s) != MOE_OK) return 0;
  return packed_layout(s.H, s.E, s.I, s.has_shared, 1).total;
}

int moe_pack_weights_mxfp4(const moe_config* cfg, const moe_weights_fmt* src, void* packed, size_t packed_bytes,
                           void* stream) {
  Shape s;
  int rc = check_cfg(cfg, &s);
  if (rc != MOE_OK) return rc;
  if (!src || !packed || !src->w13_q || !src->w13_s || !src->w2_q || !src->w2_s) return MOE_ERR_NULL;
  if (s.has_shared ? (!src->sh_w13 || !src->sh_w2) : (src->sh_w13 || src->sh_w2)) return MOE_ERR_NULL;
  if (!aligned16(packed) || !aligned16(src->w13_q) || !aligned16(src->w2_q) ||
      (s.has_shared && (!aligned16(src->sh_w13) || !aligned16(src->sh_w2))))
    return MOE_ERR_ALIGN;
  const PackedLayout P = packed_layout(s.H, s.E, s.I, s.has_shared, 1);
  if (packed_bytes < P.total) return MOE_ERR_WORKSPACE;
  return launched(launch_pack_mxfp4(s, static_cast<const uint8_t*>(src->w13_q), static_cast<const uint8_t*>(src->w13_s),
                                    static_cast<const uint8_t*>(src->w2_q), static_cast<const uint8_t*>(src->w2_s),
                                    src->sh_w13, src->sh_w2, static_cast<uint8_t*>(packed), P,
                                    static_cast<hipStream_t>(stream)));
}

int moe_layer_mxfp4(const moe_config* cfg, const float* router_w, const void* packed, const uint16_t* x, int32_t M,
                    uint32_t flags, uint16_t* x_norm, int32_t* topk_ids, float* topk_w, uint16_t* out, void* ws,
                    size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_cfg(cfg, &s);
  if (rc != MOE_OK) return rc;
  if (M < 0 || (flags & ~MOE_F_INPUT_RMSNORM)) return MOE_ERR_SHAPE;
  if (M == 0) return MOE_OK;
  const bool rms = (flags & MOE_F_INPUT_RMSNORM) != 0;
  if (!router_w || !packed || !x || !topk_ids || !topk_w || !out || !ws || (rms && !x_norm)) return MOE_ERR_NULL;
  if (!aligned16(router_w) || !aligned16(packed) || !aligned16(x) || !aligned16(out) || !aligned16(ws) ||
      !aligned4(topk_ids) || !aligned4(topk_w) || (rms && !aligned16(x_norm)))
    return MOE_ERR_ALIGN;
  if (rms && overlap(x, x_norm, (size_t)M * s.H * 2)) return MOE_ERR_SHAPE;
  if (!layer_supported(s, M) || !route_supported(s)) return MOE_ERR_UNSUPPORTED;
  WsLayout L;
  rc = check_experts(cfg, &s, packed, x, M, topk_ids, topk_w, out, ws, ws_bytes, true, true, &L);
  if (rc != MOE_OK) return rc;
  const PackedLayout P = packed_layout(s.H, s.E, s.I, s.has_shared, 1);
  const hipError_t e = launch_layer(s, static_cast<const uint8_t*>(packed), P, router_w, x, M, true, rms, kRmsEps,
                                    x_norm, topk_ids, topk_w, out, static_cast<uint8_t*>(ws), L,
                                    static_cast<hipStream_t>(stream), true);
  // no second path for this layout: a grid the device cannot hold at once is unsupported
  return e == hipErrorInvalidConfiguration ? MOE_ERR_UNSUPPORTED : launched(e);
}

int moe_lmhead_quantize_fp8(const uint16_t* w, int32_t V, int32_t H, uint8_t* q, float* scale, void* stream) {
  if (V < 0 || H <= 0 || H % 16) return MOE_ERR_SHAPE;
  if (V == 0) return MOE_OK;
  if (!w || !q || !scale) return MOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned4(scale)) return MOE_ERR_ALIGN;
  if (overlap(w, q, (size_t)V * H)) return MOE_ERR_SHAPE;
  return launched(launch_lmhead_quant(w, V, H, q, scale, static_cast<hipStream_t>(stream)));
}

namespace {
int lmhead_call(bool fp8, const void* w, const float* scale, int32_t V, int32_t H, const uint16_t* x, int32_t M,
                float* logits, void* stream) {
  if (V < 0 || H <= 0 || H % 16 || M < 0) return MOE_ERR_SHAPE;
  if (V == 0 || M == 0) return MOE_OK;
  if (!w || !x || !logits || (fp8 && !scale)) return MOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(x) || !aligned4(logits) || (fp8 && !aligned4(scale))) return MOE_ERR_ALIGN;
  if (M > 4 || !lmhead_supported(H, fp8)) return MOE_ERR_UNSUPPORTED;
  return launched(launch_lmhead_gemv(fp8, static_cast<const uint8_t*>(w), scale, V, H, x, M, logits,
                                     static_cast<hipStream_t>(stream)));
}
}  // namespace

int moe_lmhead_fp8(const uint8_t* q, const float* scale, int32_t V, int32_t H, const uint16_t* x, int32_t M,
                   float* logits, void* stream) {
  return lmhead_call(true, q, scale, V, H, x, M, logits, stream);
}

int moe_lmhead_bf16(const uint16_t* w, int32_t V, int32_t H, const uint16_t* x, int32_t M, float* logits,
                    void* stream) {
  return lmhead_call(false, w, nullptr, V, H, x, M, logits, stream);
}

int moe_get_device_error(void* ws, void* stream, int32_t* code_host) {
  if (!ws || !code_host) return MOE_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  // the error word is the first word of every workspace layout
  if (hipMemcpyAsync(&v, ws, sizeof v, hipMemcpyDeviceToHost, st) != hipSuccess) return MOE_ERR_LAUNCH;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_LAUNCH;
  *code_host = v;
  if (v != 0) {
    if (launch_fill_zero(ws, sizeof v, st) != hipSuccess) return MOE_ERR_LAUNCH;
    if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_LAUNCH;
    return MOE_ERR_DEVICE;
  }
  return MOE_OK;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_ALIGN: return "a pointer is not aligned (16 bytes for arrays, 4 for ids/weights)";
    case MOE_ERR_WORKSPACE: return "workspace or packed buffer too small";
    case MOE_ERR_UNSUPPORTED: return "no kernel is compiled for this shape";
    case MOE_ERR_LAUNCH: return "the HIP runtime rejected a launch or copy";
    case MOE_ERR_DEVICE: return "a device-side data error was recorded (expert id out of range)";
    default: return "unknown status";
  }
}

const char* moe_build_info(void) {
  return "arch=gfx950 layout=tile64-lanerow-expert-major-v3 "
         "route=wave-per-row-fp32+lastwg-topk|mfma-bf16x3(M>=33) "
         "gate_up=int4-dot2bf16-sgpr-act(GW20P4|GW2P2)+shared-bf16(KS-split,lastwg) "
         "down=int4-dot2bf16(GW6P2|GW1P1)+lastwg-combine "
         "layer(M=1, or M*k<=64 on request)=one-launch(router, shared, routed gate_up, down+combine; tagged hand-offs) "
         "prefill(M*k>=513)=grouped-mfma-f16-exact-int4(96-row items,xcd-aware)+shared-mfma-bf16 "
         "permute=multi-wg-stable-counting-sort "
         "max_experts=512 max_decode_slots=4096";
}

}  // extern "C"
