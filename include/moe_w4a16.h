/*
 * moe_w4a16.h — C ABI of the MI355X (gfx950) W4A16 grouped-quantized
 * routed-MoE layer.
 *
 * The layer (vLLM recipe page "inclusionAI/Ling-3.0-flash", Overview and
 * "Single-GPU int4"; bpdata.com Ling-3.0-flash MoE article, model section):
 * each token is routed to top_k of n_experts routed experts and also passes
 * through one shared expert.  Routed experts are SwiGLU FFNs whose weights are
 * symmetric INT4 with one BF16 scale per group of 32 consecutive inputs; the
 * shared expert and the router stay unquantized; activations are BF16.
 *
 *   logits[t][e] = sum_h x[t][h] * router_w[e][h]                  (fp32)
 *   ids[t]       = the top_k largest logits, largest first, ties -> lower id
 *   w[t][j]      = softmax over the top_k chosen logits
 *   expert_e(x)  = W2_e ( silu(W1_e x) * (W3_e x) )
 *   out[t]       = sum_j w[t][j] * expert_{ids[t][j]}(x[t]) + shared(x[t])
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers unless marked "host".  bf16
 *    values travel as uint16_t bit patterns.  Arrays are row-major and
 *    contiguous.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t, NULL for
 *    the default stream).  They allocate nothing, never synchronise (except
 *    moe_get_device_error) and launch fixed-size grids, so they may be
 *    captured into a HIP graph.
 *  - The caller owns every buffer.  The library keeps no mutable global
 *    state other than the static workspace of moe_layer_w4a16_noalloc; calls
 *    that share one workspace must be stream-ordered (calls on different
 *    workspaces may run concurrently).
 *  - Arguments are checked before anything is launched; a failed check
 *    returns a negative moe_status and launches nothing.  There is no
 *    fallback path: an unsupported shape is an error.
 *  - Data errors seen on the device (an expert id outside [0, n_experts))
 *    set a sticky error word in the workspace and the affected slot
 *    contributes zero; moe_get_device_error reports it.
 *  - The one-launch small-M path hands data between workgroups of one grid
 *    through flags and counters in the workspace; a hand-off that does not
 *    complete within its bounded wait sets bit 1 of the error word (the
 *    result of that call is then undefined, and the workspace must be
 *    re-initialised with moe_workspace_init).
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL                         */
  MOE_ERR_SHAPE = -2,       /* a size is out of range or inconsistent             */
  MOE_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned                   */
  MOE_ERR_WORKSPACE = -4,   /* workspace or packed buffer too small               */
  MOE_ERR_UNSUPPORTED = -5, /* shape valid but no kernel is compiled for it       */
  MOE_ERR_LAUNCH = -6,      /* the HIP runtime rejected a launch or copy          */
  MOE_ERR_DEVICE = -7       /* a device-side data error was recorded              */
} moe_status;

/* Layer shape.  group_size must be 32. */
typedef struct {
  int32_t hidden;      /* H: multiple of 256, at most 4096                    */
  int32_t n_experts;   /* E: 1 .. 512                                         */
  int32_t top_k;       /* k: 1 .. min(E, 64)                                  */
  int32_t inter;       /* I: moe_intermediate_size, multiple of 32, <= 4096   */
  int32_t group_size;  /* G: 32                                               */
  int32_t has_shared;  /* 1: one BF16 shared expert of the routed shape       */
} moe_config;

/* Weights in the plain ("checkpoint") layout, as device pointers.
 * Routed codes: u = q + 8 for q in [-8, 7], two per byte, the low nibble
 * holding the even input index; each row holds its inputs contiguously.
 * Scales: one bf16 per (row, group of 32 inputs).
 * Gate/up: rows [0, I) are the gate projection W1, rows [I, 2I) the up
 * projection W3.  The shared pointers must be NULL iff has_shared == 0. */
typedef struct {
  const uint8_t*  w13_q;   /* [E][2I][H/2]  */
  const uint16_t* w13_s;   /* [E][2I][H/32] */
  const uint8_t*  w2_q;    /* [E][H][I/2]   */
  const uint16_t* w2_s;    /* [E][H][I/32]  */
  const uint16_t* sh_w13;  /* [2I][H] bf16  */
  const uint16_t* sh_w2;   /* [H][I]  bf16  */
} moe_weights_plain;

/* Bytes of the device layout produced by moe_pack_weights (routed + shared
 * experts; the router is not part of it).  0 on an invalid config.
 * The routed experts are the symmetric 4-bit, group-32 part of the int4
 * checkpoint and the shared expert its BF16 part (vLLM recipe page
 * "inclusionAI/Ling-3.0-flash", "Single-GPU int4"). */
size_t moe_packed_size(const moe_config* cfg /* host */);

/* Rearrange plain weights into the library's device layout (same bytes,
 * tiled so that every 16-byte load of a wavefront is contiguous and one
 * lane owns one weight row).  One-time, load-time work, in the role of the
 * checkpoint loading step of the vLLM recipe page ("Single-GPU int4": a
 * pack-quantized checkpoint, symmetric W4, group_size 32, routed experts
 * only).  src: host struct of DEVICE pointers in the moe_weights_plain
 * layout; packed: device buffer of packed_bytes, owned by the caller, which
 * must not overlap the sources.  Returns MOE_ERR_NULL for a missing pointer
 * (the shared pointers must be NULL iff has_shared == 0), MOE_ERR_ALIGN for
 * a misaligned one, MOE_ERR_WORKSPACE if packed_bytes is smaller than
 * moe_packed_size(cfg). */
int moe_pack_weights(const moe_config* cfg /* host */, const moe_weights_plain* src /* host struct */,
                     void* packed, size_t packed_bytes, void* stream);

/* Workspace bytes needed for calls with up to max_tokens tokens (the
 * hand-off words, per-call scratch and the sticky error word of every call
 * below; the caller allocates it on the device).  0 on an invalid config or
 * max_tokens < 0. */
size_t moe_workspace_size(const moe_config* cfg /* host */, int32_t max_tokens);

/* Zero-fill a workspace (a kernel, not hipMemset, so it may be captured).
 * Required once before the first use of a workspace; the library keeps its
 * counters at zero between calls after that. */
int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* flags for moe_route */
#define MOE_F_INPUT_RMSNORM 0x1u  /* x is the previous layer's output y: route
                                     rmsnorm(y) = bf16(y / sqrt(mean(y^2) + 1e-6))
                                     (unit gain) and write it to x_norm [M][H].
                                     x_norm must not overlap x: the call reads x
                                     while it writes x_norm (MOE_ERR_SHAPE).    */

/* The router: every token goes to top_k of the n_experts routed experts
 * (bpdata.com Ling-3.0-flash MoE article, "Modell és kiinduló konfiguráció":
 * eight of 512 per token in every MoE layer; vLLM recipe page, Overview).
 *   router_w [E][H] fp32 row-major (one row per expert), x [M][H] bf16
 *   -> topk_ids [M][k] int32 (largest logit first, ties -> lower id),
 *      topk_w [M][k] fp32 (softmax over the chosen logits; sums to 1).
 * All arrays are device memory owned by the caller; ws is the caller's
 * workspace of ws_bytes (moe_workspace_size for at least M tokens).
 * M = 0 is a no-op.  x_norm is required iff MOE_F_INPUT_RMSNORM is set and
 * must not overlap x.  Errors: MOE_ERR_NULL, MOE_ERR_ALIGN (16 bytes for
 * router_w, x, x_norm and ws; 4 for ids and weights), MOE_ERR_SHAPE (M < 0,
 * unknown flags, x_norm overlapping x), MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED,
 * MOE_ERR_LAUNCH; nothing is launched on an error. */
int moe_route(const moe_config* cfg /* host */, const float* router_w, const uint16_t* x,
              int32_t M, uint32_t flags, uint16_t* x_norm, int32_t* topk_ids, float* topk_w,
              void* ws, size_t ws_bytes, void* stream);

/* The expert FFNs and their weighted sum: for every token, the k routed
 * experts named by topk_ids (used as given: not renormalised; duplicates are
 * summed slot by slot) weighted by topk_w, plus the one shared expert with
 * weight 1 (bpdata.com article, "Modell és kiinduló konfiguráció": eight
 * routed experts and a shared one per token; vLLM recipe page, "Single-GPU
 * int4": the routed experts symmetric W4 with groups of 32, the shared
 * expert BF16).  Each distinct expert of the call is read once and applied
 * to all of its tokens, as a multi-token verify step needs (bpdata.com,
 * "Optimalizáció 3": a 4-token verify touches up to 32 experts).
 *   packed: the output of moe_pack_weights for the same cfg; x [M][H] bf16;
 *   topk_ids [M][k] int32, topk_w [M][k] fp32 -> out [M][H] bf16 (round to
 *   nearest even).  All device memory owned by the caller; ws as for
 *   moe_route.  An id outside [0, E) sets bit 0 of the device error word
 *   and its slot adds nothing.  M = 0 is a no-op.  Errors as for moe_route
 *   (alignment: 16 bytes for packed, x, out and ws). */
int moe_forward_w4a16(const moe_config* cfg /* host */, const void* packed, const uint16_t* x,
                      int32_t M, const int32_t* topk_ids, const float* topk_w, uint16_t* out,
                      void* ws, size_t ws_bytes, void* stream);

/* flag for moe_layer_w4a16 */
#define MOE_F_ONE_LAUNCH 0x2u  /* use the one-launch kernel for every M it supports
                                  (M <= 4 and M*top_k <= 64), not only for M <= 2 */

/* One whole MoE layer for a step of M tokens (a Ling-3.0-flash MoE layer's
 * routed experts and shared expert, as moe_route and moe_forward_w4a16
 * define them): moe_route followed by
 * moe_forward_w4a16 on the ids and weights it produced (topk_ids, topk_w,
 * x_norm and out are all written; ids, weights and x_norm are those of
 * moe_route bit for bit).  For one or two tokens (decode, a verify step of
 * one draft) the router, the top-k and the expert FFNs run as one launch
 * whose routed weight loads start as soon as the experts are chosen; its
 * output agrees with the two calls' within their rounding (the expert h is
 * kept as scaled fp16 instead of a bf16 pair).  Otherwise it is the two
 * calls, unless MOE_F_ONE_LAUNCH asks for the one launch.  flags: MOE_F_INPUT_RMSNORM as for moe_route (the experts then
 * see x_norm, which must not overlap x), MOE_F_ONE_LAUNCH.  Concurrent calls
 * on one workspace race.  The single launch stands in for the pages' CUDA
 * graphs, which cut the per-kernel launch cost that dominates when few
 * experts are active (ainews.surl.tw item on Ling-3.0-flash INT4 at 38.7
 * tok/s, body; ai-radar.it article on the two flags, body).  Errors as for
 * moe_route and moe_forward_w4a16.  M = 0 is a no-op. */
int moe_layer_w4a16(const moe_config* cfg /* host */, const float* router_w, const void* packed,
                    const uint16_t* x, int32_t M, uint32_t flags, uint16_t* x_norm,
                    int32_t* topk_ids, float* topk_w, uint16_t* out,
                    void* ws, size_t ws_bytes, void* stream);

/* Bytes of the library's own workspace used by moe_layer_w4a16_noalloc. */
#define MOE_NOALLOC_WS_BYTES ((size_t)16 << 20)

/* moe_layer_w4a16 for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and errors as
 * moe_layer_w4a16 minus ws / ws_bytes: the workspace is a static device array
 * of MOE_NOALLOC_WS_BYTES inside the library, one per GPU, zero at load and
 * held until the process ends; its address on the current device is looked
 * up once (no allocation, here or later).  A call whose workspace need
 * (moe_workspace_size of its M) exceeds that size returns MOE_ERR_WORKSPACE
 * and launches nothing; for the Ling-3.0-flash shape that is M > 90.  Every
 * call on one GPU shares that GPU's array and finds the last call's contents
 * (the layer's hand-off words carry a per-call tag and its counters return
 * to zero at the end of each call, so nothing needs clearing between calls):
 * calls that overlap on one GPU (different streams, or another thread) race
 * and must be serialised by the caller.  The routing is computed inside the
 * call, so the expert ids are always in range; the device error word of this
 * workspace is not exposed.  The caller still owns every input and output. */
int moe_layer_w4a16_noalloc(const moe_config* cfg /* host */, const float* router_w, const void* packed,
                            const uint16_t* x, int32_t M, uint32_t flags, uint16_t* x_norm,
                            int32_t* topk_ids, float* topk_w, uint16_t* out, void* stream);

/* The two stages of moe_forward_w4a16 (the gate_up/SiLU half and the
 * down/combine half of the expert FFNs moe_forward_w4a16 cites), for callers
 * that schedule them
 * separately (moe_forward_w4a16 = moe_gate_up_w4a16 then moe_down_w4a16 on
 * the same workspace, stream, M and topk_ids).
 * moe_gate_up_w4a16: h = silu(W1 x) * (W3 x) for every (token, slot) and the
 *   shared expert, kept in the workspace.
 * moe_down_w4a16: the down projections of those h and the weighted combine
 *   into out [M][H] bf16.  It reads the workspace written by
 *   the preceding moe_gate_up_w4a16 of the same M and topk_ids. */
int moe_gate_up_w4a16(const moe_config* cfg /* host */, const void* packed, const uint16_t* x,
                      int32_t M, const int32_t* topk_ids, void* ws, size_t ws_bytes, void* stream);
int moe_down_w4a16(const moe_config* cfg /* host */, const void* packed, int32_t M,
                   const int32_t* topk_ids, const float* topk_w, uint16_t* out,
                   void* ws, size_t ws_bytes, void* stream);

/* Token -> expert grouping of the M*k (token, slot) pairs, the step that
 * lets each expert's weights be read once for all of its tokens in a verify
 * or prefill batch (bpdata.com article, "Optimalizáció 3"; vLLM recipe page,
 * chunked prefill):
 * counts [E] int32, offsets [E+1] int32 (exclusive prefix sum), perm [M*k]
 * int32 = flat pair index t*k + j, grouped by expert, ascending inside each
 * expert.  Pairs with an out-of-range id are left out and recorded in the
 * device error word; perm entries past offsets[E] are set to -1. */
int moe_permute(const moe_config* cfg /* host */, const int32_t* topk_ids, int32_t M,
                int32_t* counts, int32_t* offsets, int32_t* perm,
                void* ws, size_t ws_bytes, void* stream);

/* Synchronise `stream`, read the sticky device error word into *code_host
 * (0 = none; bit 0 = an expert id outside [0, E) was seen; bit 1 = a
 * hand-off inside a one-launch layer timed out) and clear it.
 * Returns MOE_OK, or MOE_ERR_DEVICE when the word was non-zero. */
int moe_get_device_error(void* ws, void* stream, int32_t* code_host /* host */);

/* ---- routed experts in the other two formats the pages serve ---------------
 * MXFP4: bpdata.com Ling-3.0-flash MoE article, model section and
 *   "Optimalizáció 1" (the FP4 checkpoint served with MXFP4 MoE kernels): E2M1
 *   codes (the OCP 4-bit float: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) with
 *   one E8M0 scale 2^(c-127) per 32 consecutive inputs.
 *     w13_q [E][2I][H/2], w2_q [E][H][I/2]: two codes per byte, the low nibble
 *     the even input; w13_s [E][2I][H/32], w2_s [E][H][I/32]: uint8 E8M0.
 * FP8_BLOCK: vLLM recipe page "inclusionAI/Ling-3.0-flash", Overview and
 *   Prerequisites (the serialized block-FP8 checkpoint, BF16 compute); the
 *   block shape is this library's reading: E4M3 codes (bias 7, largest 448)
 *   with one float32 scale per 128 x 128 block.
 *     w13_q [E][2I][H], w2_q [E][H][I]: one code per byte; w13_s
 *     [E][ceil(2I/128)][ceil(H/128)], w2_s [E][ceil(H/128)][ceil(I/128)] fp32.
 * Gate rows [0, I), up rows [I, 2I) as in moe_weights_plain; the shared expert
 * stays BF16 (sh_w13 [2I][H], sh_w2 [H][I], NULL iff has_shared == 0).  All
 * row-major, device memory owned by the caller. */
#define MOE_FMT_MXFP4 1
#define MOE_FMT_FP8_BLOCK 2
typedef struct {
  const uint8_t* w13_q;
  const void* w13_s;
  const uint8_t* w2_q;
  const void* w2_s;
  const uint16_t* sh_w13;
  const uint16_t* sh_w2;
} moe_weights_fmt;

/* moe_forward_w4a16 with the routed experts in format fmt (weights in the
 * layout above, read as they are: no packing step): out [M][H] bf16 =
 * sum_j w[t][j] * expert_{ids[t][j]}(x[t]) + shared(x[t]), h = silu(W1 x) *
 * (W3 x), fp32 accumulation, slots added in order.  Two launches (gate_up,
 * then down + combine) that allocate nothing.  M <= 8 and M*top_k <= 64
 * (MOE_ERR_UNSUPPORTED beyond, or for a shape the kernels do not cover);
 * codes and x, out, the shared weights and ws 16-byte aligned, ids and
 * weights 4, FP8 scales 4 (MOE_ERR_ALIGN); ws as for moe_forward_w4a16 with
 * M tokens.  Ids out of range are recorded in the device error word and add
 * nothing.  M = 0 is a no-op. */
int moe_forward_fmt(const moe_config* cfg /* host */, int32_t fmt, const moe_weights_fmt* w /* host struct */,
                    const uint16_t* x, int32_t M, const int32_t* topk_ids, const float* topk_w, uint16_t* out,
                    void* ws, size_t ws_bytes, void* stream);

/* The MXFP4 layer in one launch, as moe_layer_w4a16 is for INT4: the
 * routed experts in MXFP4 (the FP4 checkpoint the bpdata.com article's model
 * section and "Optimalizáció 1" serve with MXFP4 MoE kernels), packed once
 * by moe_pack_weights_mxfp4 into the library's tiled layout (each 16-byte
 * row-group as the checkpoint stores it, the E8M0 scale bytes packed like
 * the INT4 layout's bf16 scales, the shared BF16 expert as for INT4, each
 * expert's parts contiguous).
 * moe_packed_size_mxfp4: bytes of that layout (0 on an invalid config).
 * moe_pack_weights_mxfp4: src holds DEVICE pointers in the moe_weights_fmt
 *   MXFP4 layout; packed (device, caller-owned, not overlapping the sources)
 *   of packed_bytes; MOE_ERR_NULL / MOE_ERR_ALIGN (16 bytes for the codes,
 *   the shared weights and packed) / MOE_ERR_WORKSPACE as moe_pack_weights.
 * moe_layer_mxfp4: arguments, results and errors as moe_layer_w4a16 (flags:
 *   MOE_F_INPUT_RMSNORM); ids and weights equal moe_route's bit for bit and
 *   out agrees with moe_route + moe_forward_fmt on the plain weights within
 *   their rounding (h kept as scaled fp16).  Only the shapes and token counts
 *   the one-launch layer covers (M <= 4, M * top_k <= 64, a device that holds
 *   at least two of its workgroups at once): MOE_ERR_UNSUPPORTED otherwise,
 *   with nothing launched; use moe_route + moe_forward_fmt there. */
size_t moe_packed_size_mxfp4(const moe_config* cfg /* host */);
int moe_pack_weights_mxfp4(const moe_config* cfg /* host */, const moe_weights_fmt* src /* host struct */,
                           void* packed, size_t packed_bytes, void* stream);
int moe_layer_mxfp4(const moe_config* cfg /* host */, const float* router_w, const void* packed,
                    const uint16_t* x, int32_t M, uint32_t flags, uint16_t* x_norm,
                    int32_t* topk_ids, float* topk_w, uint16_t* out,
                    void* ws, size_t ws_bytes, void* stream);

/* ---- LM head as FP8 (the step after the last MoE layer) -------------------
 * bpdata.com Ling-3.0-flash MoE article, "Optimalizáció 2": the BF16 LM head
 * (model section: hidden 2,560 onto 157,184 tokens) is converted to FP8 when
 * the head is assembled, which roughly halves the bytes it reads per token.
 * The pages fix neither the FP8 flavour nor the scale; this library uses E4M3
 * (the OCP 8-bit float: bias 7, largest finite 448, no infinities) with one
 * float32 scale per row.
 *
 * moe_lmhead_quantize_fp8: one-time.  w [V][H] bf16 -> q [V][H] E4M3 codes
 *   and scale [V] fp32: scale[v] = amax_v / 448 (1 for an all-zero row) and
 *   q[v][h] = the E4M3 code nearest to w[v][h] / scale[v] (ties to the even
 *   code, saturating at +-448), both divisions in float32.
 * moe_lmhead_fp8: logits [M][V] fp32 = scale[v] * sum_h e4m3(q[v][h]) * x[t][h]
 *   for x [M][H] bf16, accumulated in fp32.
 * moe_lmhead_bf16: logits [M][V] fp32 = sum_h w[v][h] * x[t][h] with the BF16
 *   head itself (the unquantised product, for comparison).
 * Device pointers owned by the caller; w, q and x 16-byte aligned, scale and
 * logits 4 (MOE_ERR_ALIGN).  H a positive multiple of 16 and V >= 0
 * (MOE_ERR_SHAPE; q must not overlap w); the products take M <= 4 and
 * H = 2560 or H <= 512 (FP8) / 256 (BF16), else MOE_ERR_UNSUPPORTED.  V = 0 or
 * M = 0 is a no-op.  Asynchronous on `stream`, no allocation. */
int moe_lmhead_quantize_fp8(const uint16_t* w, int32_t V, int32_t H, uint8_t* q, float* scale, void* stream);
int moe_lmhead_fp8(const uint8_t* q, const float* scale, int32_t V, int32_t H, const uint16_t* x, int32_t M,
                   float* logits, void* stream);
int moe_lmhead_bf16(const uint16_t* w, int32_t V, int32_t H, const uint16_t* x, int32_t M, float* logits,
                    void* stream);

const char* moe_status_string(int status);

/* Measurement aid, not part of the layer: reads `bytes` of device memory at
 * `buf` once (each wavefront of `blocks` workgroups of 256 threads takes
 * contiguous 10 KB tiles in turn, 16-byte non-temporal loads, the next tile requested before
 * the current one is folded) and writes nothing unless the xor of the data
 * equals a fixed value (then one word per workgroup into sink[blocks], device
 * memory).  The pages find decode bound by weight reads (bpdata.com article,
 * intro), so the kernels' bandwidth is reported against the rate this plain
 * read reaches on the same part as well as against the nominal peak.  buf
 * 16-byte aligned, bytes a multiple of 16 (MOE_ERR_ALIGN), 1 <= blocks <=
 * 65536 (MOE_ERR_SHAPE). */
int moe_probe_read(const void* buf, size_t bytes, uint32_t* sink /* [blocks] */, int32_t blocks, void* stream);

/* Static description of the compiled library: target arch, kernel variants and the
 * packed-layout tag, for logging next to every measurement. */
const char* moe_build_info(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W4A16_H */
