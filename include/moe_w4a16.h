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
 *    state; calls that share one workspace must be stream-ordered (calls on
 *    different workspaces may run concurrently).
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
 * experts; the router is not part of it).  0 on an invalid config. */
size_t moe_packed_size(const moe_config* cfg /* host */);

/* Rearrange plain weights into the library's device layout (same bytes,
 * tiled so that every 16-byte load of a wavefront is contiguous and one
 * lane owns one weight row).  One-time, load-time work; `packed` must not
 * overlap the sources.  Returns MOE_ERR_WORKSPACE if packed_bytes is smaller
 * than moe_packed_size(cfg). */
int moe_pack_weights(const moe_config* cfg /* host */, const moe_weights_plain* src /* host struct */,
                     void* packed, size_t packed_bytes, void* stream);

/* Workspace bytes needed for calls with up to max_tokens tokens. */
size_t moe_workspace_size(const moe_config* cfg /* host */, int32_t max_tokens);

/* Zero-fill a workspace (a kernel, not hipMemset, so it may be captured).
 * Required once before the first use of a workspace; the library keeps its
 * counters at zero between calls after that. */
int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* flags for moe_route */
#define MOE_F_INPUT_RMSNORM 0x1u  /* x is the previous layer's output y: route
                                     rmsnorm(y) = bf16(y / sqrt(mean(y^2) + 1e-6))
                                     (unit gain) and write it to x_norm [M][H]   */

/* Router GEMV + top-k + softmax weights (steps a1, a2).
 *   router_w [E][H] fp32, x [M][H] bf16 -> topk_ids [M][k] int32 (largest
 *   logit first, ties -> lower id), topk_w [M][k] fp32 (softmax over the
 *   chosen logits; sums to 1).
 * M = 0 is a no-op.  x_norm is required iff MOE_F_INPUT_RMSNORM is set. */
int moe_route(const moe_config* cfg /* host */, const float* router_w, const uint16_t* x,
              int32_t M, uint32_t flags, uint16_t* x_norm, int32_t* topk_ids, float* topk_w,
              void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs + weighted combine (steps a3-a7): for every token, the k
 * routed experts named by topk_ids (used as given: not renormalised;
 * duplicates are summed slot by slot) weighted by topk_w, plus the shared
 * expert with weight 1.  Each distinct expert of the call is read once and
 * applied to all of its tokens.  out [M][H] bf16 (round to nearest even).
 * `packed` is the output of moe_pack_weights for the same cfg.
 * M = 0 is a no-op. */
int moe_forward_w4a16(const moe_config* cfg /* host */, const void* packed, const uint16_t* x,
                      int32_t M, const int32_t* topk_ids, const float* topk_w, uint16_t* out,
                      void* ws, size_t ws_bytes, void* stream);

/* flag for moe_layer_w4a16 */
#define MOE_F_ONE_LAUNCH 0x2u  /* use the one-launch kernel for every M it supports
                                  (M*top_k <= 64), not only for M = 1 */

/* One whole layer for a step of M tokens: moe_route followed by
 * moe_forward_w4a16 on the ids and weights it produced (topk_ids, topk_w,
 * x_norm and out are all written; ids, weights and x_norm are those of
 * moe_route bit for bit).  For one token (decode) the router, the top-k and
 * the expert FFNs run as one launch whose routed weight loads start as soon
 * as the experts are chosen; its output agrees with the two calls' within
 * their rounding (the expert h is kept as scaled fp16 instead of a bf16
 * pair).  Otherwise it is the two calls, unless MOE_F_ONE_LAUNCH asks for the
 * one launch.  flags: MOE_F_INPUT_RMSNORM as for moe_route (the experts then
 * see x_norm), MOE_F_ONE_LAUNCH.  Concurrent calls on one workspace race.
 * M = 0 is a no-op. */
int moe_layer_w4a16(const moe_config* cfg /* host */, const float* router_w, const void* packed,
                    const uint16_t* x, int32_t M, uint32_t flags, uint16_t* x_norm,
                    int32_t* topk_ids, float* topk_w, uint16_t* out,
                    void* ws, size_t ws_bytes, void* stream);

/* The two stages of moe_forward_w4a16, for callers that schedule them
 * separately (moe_forward_w4a16 = moe_gate_up_w4a16 then moe_down_w4a16 on
 * the same workspace, stream, M and topk_ids).
 * moe_gate_up_w4a16: h = silu(W1 x) * (W3 x) for every (token, slot) and the
 *   shared expert, kept in the workspace (steps a3, a4, a6).
 * moe_down_w4a16: the down projections of those h and the weighted combine
 *   into out [M][H] bf16 (steps a5, a6).  It reads the workspace written by
 *   the preceding moe_gate_up_w4a16 of the same M and topk_ids. */
int moe_gate_up_w4a16(const moe_config* cfg /* host */, const void* packed, const uint16_t* x,
                      int32_t M, const int32_t* topk_ids, void* ws, size_t ws_bytes, void* stream);
int moe_down_w4a16(const moe_config* cfg /* host */, const void* packed, int32_t M,
                   const int32_t* topk_ids, const float* topk_w, uint16_t* out,
                   void* ws, size_t ws_bytes, void* stream);

/* Token -> expert grouping of the M*k (token, slot) pairs (step a3):
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

const char* moe_status_string(int status);

/* Static description of the compiled library: target arch, kernel variants and the
 * packed-layout tag, for logging next to every measurement. */
const char* moe_build_info(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W4A16_H */
