/*
 * moe_oracle.h — CPU oracle for the W4A16 grouped-quantized routed-MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, fp64 reference of what
 * the layer computes.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no code with the HIP library.
 *
 * What it follows (the pages it is written from):
 *  - vLLM recipe page "inclusionAI/Ling-3.0-flash", Overview: 512 routed
 *    experts, 8 active per token, plus one shared expert.
 *  - same page, "Single-GPU int4": symmetric W4, group_size 32, applied to the
 *    routed experts only; the shared expert stays unquantized (BF16).
 *  - same page, launch commands: BF16 activations/compute (--dtype bfloat16).
 *  - bpdata.com article on Ling-3.0-flash MoE inference, model section: each
 *    MoE layer sends every token to 8 of 512 routed experts and also uses one
 *    shared expert; hidden size 2,560; Humming section: moe_intermediate 768.
 * Where the pages say nothing, the readings are: router = softmax over the
 * top-k logits (equivalently the full softmax renormalised over the chosen
 * set), ties broken toward the lower expert id, SwiGLU experts with gate rows
 * [0,I) and up rows [I,2I), offset-binary nibbles (u = q + 8) with the low
 * nibble holding the even k, groups of 32 along K, the shared expert added
 * with weight 1, and an RMSNorm with unit gain between stacked layers.
 *
 * The further formats follow:
 *  - bpdata.com article, model section and "Optimalizáció 1": the FP4
 *    checkpoint served with MXFP4 MoE kernels (E2M1 codes with one E8M0
 *    scale per block of 32, the OCP MX format);
 *  - same article, "Optimalizáció 2": the BF16 LM head (2,560 -> 157,184)
 *    turned into FP8 when the head is assembled, halving its read volume;
 *    reading: E4M3 with one float32 scale per row, amax / 448;
 *  - vLLM recipe page, Overview and Prerequisites: the serialized block-FP8
 *    checkpoint with BF16 compute; reading: E4M3 codes with one float32
 *    scale per 128 x 128 block.
 *
 * All pointers are host pointers.  Arrays are row-major and contiguous.
 * bf16 values travel as uint16_t bit patterns.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t hidden;      /* H */
  int32_t n_experts;   /* E */
  int32_t top_k;       /* k */
  int32_t inter;       /* I */
  int32_t group_size;  /* G */
  int32_t has_shared;  /* 0 or 1 */
} oracle_cfg;

/* Routed experts are passed as one pointer per expert so that a caller can
 * hold only the experts it needs; a NULL entry that gets selected is an
 * error. */
typedef struct {
  const uint8_t*  const* w13_q;   /* E x [2I][H/2] */
  const uint16_t* const* w13_s;   /* E x [2I][H/G] */
  const uint8_t*  const* w2_q;    /* E x [H][I/2]  */
  const uint16_t* const* w2_s;    /* E x [H][I/G]  */
  const uint16_t* sh_w13;         /* [2I][H] bf16, or NULL when has_shared == 0 */
  const uint16_t* sh_w2;          /* [H][I]  bf16 */
} oracle_experts;

/* bf16 -> double (exact). */
double oracle_bf16_to_f64(uint16_t b);
/* double -> bf16, round to nearest even (subnormals and overflow handled). */
uint16_t oracle_f64_to_bf16(double v);
void oracle_f64_to_bf16_array(const double* v, uint16_t* out, int64_t n);

/* W[n][k] = (code(n,k) - 8) * scale[n][k/G], code read from q[n][k/2]. */
int oracle_dequant(const uint8_t* q, const uint16_t* s, int32_t N, int32_t K,
                   int32_t G, double* W);

/* Router: logits[t][e] = sum_h x[t][h] * Wr[e][h] (fp64); ids = the k largest
 * (ties: lower id), sorted by logit descending; w = softmax over the chosen
 * logits; gap[t] = logit(k-th) - logit((k+1)-th) (+inf when k == E).
 * logits and gap may be NULL. */
int oracle_route(const oracle_cfg* cfg, const float* router_w, const uint16_t* x,
                 int32_t M, int32_t* ids, double* w, double* gap, double* logits);

/* One quantized SwiGLU expert on one token: y = W2 (silu(W1 x) * (W3 x)). */
int oracle_expert_q(const oracle_cfg* cfg, const uint8_t* w13_q, const uint16_t* w13_s,
                    const uint8_t* w2_q, const uint16_t* w2_s, const double* x,
                    double* h /* [I] or NULL */, double* y /* [H] */);

/* The BF16 shared expert on one token. */
int oracle_expert_dense(const oracle_cfg* cfg, const uint16_t* sh_w13,
                        const uint16_t* sh_w2, const double* x,
                        double* h /* [I] or NULL */, double* y /* [H] */);

/* out[t] = sum_j w[t][j] * expert(ids[t][j], x[t]) + shared(x[t]).
 * Slots whose id is outside [0, E) contribute 0; the return value is the
 * number of such slots (negative on argument errors). */
int oracle_forward(const oracle_cfg* cfg, const oracle_experts* ex,
                   const uint16_t* x, int32_t M, const int32_t* ids,
                   const double* w, double* out);

/* Counting sort of the M*k (token, slot) pairs by expert id.
 * counts[E]; offsets[E+1] (exclusive prefix sum); perm[M*k] lists the flat
 * pair index t*k + j, grouped by expert, ascending pair index inside each
 * expert.  Pairs with out-of-range ids are left out (their count returned). */
int oracle_permute(const int32_t* ids, int32_t M, int32_t k, int32_t E,
                   int32_t* counts, int32_t* offsets, int32_t* perm);

/* Between stacked layers: out = bf16( y / sqrt(mean(y^2) + eps) ), unit gain. */
int oracle_rmsnorm(const uint16_t* y, int32_t M, int32_t H, double eps, uint16_t* out);

/* Number of OpenMP threads the oracle uses (1 without OpenMP). */
int oracle_num_threads(void);


/* ---- further weight formats ------------------------------------------- */
/* FP8 E4M3 (OCP): bias 7, no infinities, S.1111.111 NaN, largest 448. */
double oracle_e4m3_to_f64(uint8_t c);
/* Nearest finite E4M3 code (ties to the even mantissa, saturating at 448). */
uint8_t oracle_f32_to_e4m3(float v);
/* Online FP8 LM head: per-row scale amax/448 and E4M3 codes of w/scale
 * (float32 arithmetic); w [V][H] bf16 -> q [V][H], s [V]. */
int oracle_lmhead_quantize(const uint16_t* w, int32_t V, int32_t H, uint8_t* q, float* s);
/* out [M][V] = s[v] * sum_h e4m3(q[v][h]) * x[t][h], in double. */
int oracle_lmhead_gemv_fp8(const uint8_t* q, const float* s, int32_t V, int32_t H, const uint16_t* x,
                           int32_t M, double* out);
/* out [M][V] = sum_h w[v][h] * x[t][h] for a BF16 head, in double. */
int oracle_lmhead_gemv_bf16(const uint16_t* w, int32_t V, int32_t H, const uint16_t* x, int32_t M,
                            double* out);
/* E2M1 (OCP 4-bit float) code -> value; E8M0 scale code -> 2^(c-127). */
double oracle_e2m1_to_f64(uint8_t c);
double oracle_e8m0_to_f64(uint8_t c);

/* Routed-expert weight formats. */
enum { ORACLE_FMT_INT4_G32 = 0, ORACLE_FMT_MXFP4 = 1, ORACLE_FMT_FP8_BLOCK = 2 };
/* Routed experts in format fmt (per expert, as in oracle_experts):
 *   INT4_G32   q [N][K/2] nibbles, s bf16 [N][K/32]
 *   MXFP4      q [N][K/2] E2M1 nibbles, s uint8 E8M0 [N][K/32]
 *   FP8_BLOCK  q [N][K] E4M3 codes, s float32 [ceil(N/128)][ceil(K/128)] */
typedef struct {
  int32_t fmt;
  const uint8_t* const* w13_q;
  const void* const* w13_s;
  const uint8_t* const* w2_q;
  const void* const* w2_s;
  const uint16_t* sh_w13;
  const uint16_t* sh_w2;
} oracle_experts_fmt;
/* Dequantise an N x K matrix of format fmt into W [N][K]. */
int oracle_dequant_fmt(int32_t fmt, const uint8_t* q, const void* s, int32_t N, int32_t K, double* W);
/* oracle_forward with routed experts in format ex->fmt (shared expert BF16). */
int oracle_forward_fmt(const oracle_cfg* cfg, const oracle_experts_fmt* ex, const uint16_t* x, int32_t M,
                       const int32_t* ids, const double* w, double* out);

#ifdef __cplusplus
}
#endif
#endif
