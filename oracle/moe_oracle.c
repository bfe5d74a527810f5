/*
 * moe_oracle.c — fp64 CPU oracle for the W4A16 grouped-quantized MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h for what it follows).  Every
 * quantity is computed in double precision with explicit loops in the order
 * the definition states; there is no blocking, fusion or reordering.  OpenMP,
 * when present, only splits independent output rows across threads.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* bf16 is the upper half of an IEEE float32. */
double oracle_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bf16 (ties to even) directly, without going
 * through float32 first.  bf16 keeps 8 significant bits; its smallest
 * subnormal step is 2^-133 and its largest finite value (2 - 2^-7) * 2^127. */
uint16_t oracle_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  double r;
  if (a == 0.0) {
    r = 0.0;
  } else {
    int e;
    frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
    int qexp = e - 8;             /* step between neighbouring bf16 values */
    if (qexp < -133) qexp = -133; /* subnormal range: fixed step */
    r = nearbyint(ldexp(a, -qexp)); /* default rounding mode: ties to even */
    r = ldexp(r, qexp);
  }
  const double maxf = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
  uint16_t bits;
  if (r > maxf) {
    bits = 0x7F80; /* overflow -> inf */
  } else {
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    bits = (uint16_t)(u >> 16);
  }
  return (uint16_t)(bits | (neg ? 0x8000 : 0));
}

void oracle_f64_to_bf16_array(const double* v, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(v[i]);
}

/* The stored 4-bit code of element (n, k) of an N x K matrix whose rows hold
 * K/2 bytes: the low nibble carries the even k, the high nibble the odd k. */
static int code_at(const uint8_t* q, int32_t K, int32_t n, int32_t k) {
  uint8_t byte = q[(int64_t)n * (K / 2) + k / 2];
  return (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
}

/* Symmetric INT4 with one bf16 scale per group of G consecutive k. */
static double wq_at(const uint8_t* q, const uint16_t* s, int32_t K, int32_t G,
                    int32_t n, int32_t k) {
  int code = code_at(q, K, n, k);
  double scale = oracle_bf16_to_f64(s[(int64_t)n * (K / G) + k / G]);
  return (double)(code - 8) * scale;
}

int oracle_dequant(const uint8_t* q, const uint16_t* s, int32_t N, int32_t K,
                   int32_t G, double* W) {
  if (!q || !s || !W || N < 0 || K <= 0 || G <= 0 || K % G || K % 2) return -1;
  for (int32_t n = 0; n < N; ++n)
    for (int32_t k = 0; k < K; ++k)
      W[(int64_t)n * K + k] = wq_at(q, s, K, G, n, k);
  return 0;
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

int oracle_route(const oracle_cfg* cfg, const float* router_w, const uint16_t* x,
                 int32_t M, int32_t* ids, double* w, double* gap, double* logits) {
  if (!cfg || !router_w || (!x && M > 0) || !ids || !w || M < 0) return -1;
  const int32_t H = cfg->hidden, E = cfg->n_experts, k = cfg->top_k;
  if (H <= 0 || E <= 0 || k < 1 || k > E) return -1;
  double* l = (double*)malloc(sizeof(double) * (size_t)E);
  char* taken = (char*)malloc((size_t)E);
  if (!l || !taken) { free(l); free(taken); return -2; }
  for (int32_t t = 0; t < M; ++t) {
    const uint16_t* xt = x + (int64_t)t * H;
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h)
        acc += oracle_bf16_to_f64(xt[h]) * (double)router_w[(int64_t)e * H + h];
      l[e] = acc;
      if (logits) logits[(int64_t)t * E + e] = acc;
    }
    /* Selection: k passes, each taking the largest logit not yet taken; a
     * strict comparison keeps the lower id on ties. */
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
      taken[best] = 1;
      ids[(int64_t)t * k + j] = best;
    }
    if (gap) {
      if (k == E) {
        gap[t] = INFINITY;
      } else {
        int32_t next = -1;
        for (int32_t e = 0; e < E; ++e)
          if (!taken[e] && (next < 0 || l[e] > l[next])) next = e;
        gap[t] = l[ids[(int64_t)t * k + k - 1]] - l[next];
      }
    }
    /* Softmax over the chosen logits, shifted by the largest for range. */
    const double l0 = l[ids[(int64_t)t * k]];
    double denom = 0.0;
    for (int32_t j = 0; j < k; ++j) denom += exp(l[ids[(int64_t)t * k + j]] - l0);
    for (int32_t j = 0; j < k; ++j)
      w[(int64_t)t * k + j] = exp(l[ids[(int64_t)t * k + j]] - l0) / denom;
  }
  free(l);
  free(taken);
  return 0;
}

int oracle_expert_q(const oracle_cfg* cfg, const uint8_t* w13_q, const uint16_t* w13_s,
                    const uint8_t* w2_q, const uint16_t* w2_s, const double* x,
                    double* h_out, double* y) {
  if (!cfg || !w13_q || !w13_s || !w2_q || !w2_s || !x || !y) return -1;
  const int32_t H = cfg->hidden, I = cfg->inter, G = cfg->group_size;
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  if (!h) return -2;
#pragma omp parallel for schedule(static)
  for (int32_t r = 0; r < I; ++r) {
    double g = 0.0, u = 0.0;
    for (int32_t k = 0; k < H; ++k) {
      g += wq_at(w13_q, w13_s, H, G, r, k) * x[k];       /* gate row r     */
      u += wq_at(w13_q, w13_s, H, G, I + r, k) * x[k];   /* up row I + r   */
    }
    h[r] = silu(g) * u;
  }
#pragma omp parallel for schedule(static)
  for (int32_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int32_t r = 0; r < I; ++r) acc += wq_at(w2_q, w2_s, I, G, n, r) * h[r];
    y[n] = acc;
  }
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
  free(h);
  return 0;
}

int oracle_expert_dense(const oracle_cfg* cfg, const uint16_t* sh_w13,
                        const uint16_t* sh_w2, const double* x, double* h_out,
                        double* y) {
  if (!cfg || !sh_w13 || !sh_w2 || !x || !y) return -1;
  const int32_t H = cfg->hidden, I = cfg->inter;
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  if (!h) return -2;
#pragma omp parallel for schedule(static)
  for (int32_t r = 0; r < I; ++r) {
    double g = 0.0, u = 0.0;
    for (int32_t k = 0; k < H; ++k) {
      g += oracle_bf16_to_f64(sh_w13[(int64_t)r * H + k]) * x[k];
      u += oracle_bf16_to_f64(sh_w13[(int64_t)(I + r) * H + k]) * x[k];
    }
    h[r] = silu(g) * u;
  }
#pragma omp parallel for schedule(static)
  for (int32_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int32_t r = 0; r < I; ++r) acc += oracle_bf16_to_f64(sh_w2[(int64_t)n * I + r]) * h[r];
    y[n] = acc;
  }
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
  free(h);
  return 0;
}

int oracle_forward(const oracle_cfg* cfg, const oracle_experts* ex,
                   const uint16_t* x, int32_t M, const int32_t* ids,
                   const double* w, double* out) {
  if (!cfg || !ex || M < 0 || (M > 0 && (!x || !ids || !w || !out))) return -1;
  const int32_t H = cfg->hidden, E = cfg->n_experts, k = cfg->top_k;
  if (cfg->has_shared && (!ex->sh_w13 || !ex->sh_w2)) return -1;
  double* xt = (double*)malloc(sizeof(double) * (size_t)H);
  double* y = (double*)malloc(sizeof(double) * (size_t)H);
  if (!xt || !y) { free(xt); free(y); return -2; }
  int bad = 0;
  for (int32_t t = 0; t < M; ++t) {
    for (int32_t h = 0; h < H; ++h) xt[h] = oracle_bf16_to_f64(x[(int64_t)t * H + h]);
    double* ot = out + (int64_t)t * H;
    for (int32_t n = 0; n < H; ++n) ot[n] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = ids[(int64_t)t * k + j];
      if (e < 0 || e >= E) { ++bad; continue; }
      if (!ex->w13_q[e] || !ex->w13_s[e] || !ex->w2_q[e] || !ex->w2_s[e]) {
        free(xt); free(y);
        return -3; /* selected expert not supplied */
      }
      oracle_expert_q(cfg, ex->w13_q[e], ex->w13_s[e], ex->w2_q[e], ex->w2_s[e], xt, NULL, y);
      const double wj = w[(int64_t)t * k + j];
      for (int32_t n = 0; n < H; ++n) ot[n] += wj * y[n];
    }
    if (cfg->has_shared) {
      oracle_expert_dense(cfg, ex->sh_w13, ex->sh_w2, xt, NULL, y);
      for (int32_t n = 0; n < H; ++n) ot[n] += y[n];
    }
  }
  free(xt);
  free(y);
  return bad;
}

int oracle_permute(const int32_t* ids, int32_t M, int32_t k, int32_t E,
                   int32_t* counts, int32_t* offsets, int32_t* perm) {
  if (M < 0 || k < 1 || E < 1 || !counts || !offsets || (M > 0 && (!ids || !perm))) return -1;
  int bad = 0;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < (int64_t)M * k; ++p) {
    int32_t e = ids[p];
    if (e < 0 || e >= E) { ++bad; continue; }
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  /* Fill by scanning pairs in ascending order: stable inside each expert. */
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!cursor) return -2;
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t p = 0; p < (int64_t)M * k; ++p) {
    int32_t e = ids[p];
    if (e < 0 || e >= E) continue;
    perm[cursor[e]++] = (int32_t)p;
  }
  free(cursor);
  return bad;
}

int oracle_rmsnorm(const uint16_t* y, int32_t M, int32_t H, double eps, uint16_t* out) {
  if (M < 0 || H <= 0 || (M > 0 && (!y || !out))) return -1;
  for (int32_t t = 0; t < M; ++t) {
    double ss = 0.0;
    for (int32_t h = 0; h < H; ++h) {
      double v = oracle_bf16_to_f64(y[(int64_t)t * H + h]);
      ss += v * v;
    }
    const double d = sqrt(ss / (double)H + eps);
    for (int32_t h = 0; h < H; ++h)
      out[(int64_t)t * H + h] = oracle_f64_to_bf16(oracle_bf16_to_f64(y[(int64_t)t * H + h]) / d);
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Further weight formats: FP8 E4M3, MXFP4 (E2M1 codes with an E8M0 scale per
 * 32), block-FP8 experts, and the FP8 LM head.
 * ------------------------------------------------------------------------ */

/* E4M3 (the OCP 8-bit float with 4 exponent and 3 mantissa bits): sign bit
 * 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.  Exponent 0 holds
 * the subnormals m * 2^-9; otherwise the value is (1 + m/8) * 2^(e-7).  There
 * are no infinities: S.1111.111 is NaN, so the largest finite value is
 * S.1111.110 = 1.75 * 2^8 = 448. */
double oracle_e4m3_to_f64(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* The E4M3 code nearest to v among the finite codes of v's sign (so values
 * beyond 448 saturate to 448), a tie going to the code with the even
 * mantissa.  Written as a search over every finite magnitude code, the
 * plainest statement of round-to-nearest-even; NaN maps to 0x7F. */
uint8_t oracle_f32_to_e4m3(float v) {
  if (isnan(v)) return 0x7F;
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs((double)v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);  /* the largest finite code, infinity included */
  int best = 0;
  double best_d = a;  /* distance to code 0 */
  for (int c = 1; c <= 0x7E; ++c) {
    const double d = fabs(oracle_e4m3_to_f64((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* Online FP8 quantisation of a BF16 LM head [V][H] (bpdata.com Ling-3.0-flash
 * article, "Optimalizáció 2": the BF16 head is turned into FP8 when the LM
 * head is assembled, which halves the bytes the layer reads).  The pages fix
 * neither the FP8 flavour nor the scale granularity; the reading here: E4M3,
 * one float32 scale per row, s = amax / 448 with amax the largest |w| of the
 * row (s = 1 for an all-zero row), q = the E4M3 code of w / s, both
 * divisions in float32. */
int oracle_lmhead_quantize(const uint16_t* w, int32_t V, int32_t H, uint8_t* q, float* s) {
  if (!w || !q || !s || V < 0 || H <= 0) return -1;
#pragma omp parallel for schedule(static)
  for (int32_t v = 0; v < V; ++v) {
    float amax = 0.0f;
    for (int32_t h = 0; h < H; ++h) {
      const float a = fabsf((float)oracle_bf16_to_f64(w[(int64_t)v * H + h]));
      if (a > amax) amax = a;
    }
    const float sv = amax > 0.0f ? amax / 448.0f : 1.0f;
    s[v] = sv;
    for (int32_t h = 0; h < H; ++h)
      q[(int64_t)v * H + h] = oracle_f32_to_e4m3((float)oracle_bf16_to_f64(w[(int64_t)v * H + h]) / sv);
  }
  return 0;
}

/* logits[t][v] = s[v] * sum_h e4m3(q[v][h]) * x[t][h] (x bf16), in double. */
int oracle_lmhead_gemv_fp8(const uint8_t* q, const float* s, int32_t V, int32_t H, const uint16_t* x,
                           int32_t M, double* out) {
  if (!q || !s || !x || !out || V < 0 || H <= 0 || M < 0) return -1;
  for (int32_t t = 0; t < M; ++t) {
#pragma omp parallel for schedule(static)
    for (int32_t v = 0; v < V; ++v) {
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h)
        acc += oracle_e4m3_to_f64(q[(int64_t)v * H + h]) * oracle_bf16_to_f64(x[(int64_t)t * H + h]);
      out[(int64_t)t * V + v] = (double)s[v] * acc;
    }
  }
  return 0;
}

/* The same product with the BF16 head itself. */
int oracle_lmhead_gemv_bf16(const uint16_t* w, int32_t V, int32_t H, const uint16_t* x, int32_t M,
                            double* out) {
  if (!w || !x || !out || V < 0 || H <= 0 || M < 0) return -1;
  for (int32_t t = 0; t < M; ++t) {
#pragma omp parallel for schedule(static)
    for (int32_t v = 0; v < V; ++v) {
      double acc = 0.0;
      for (int32_t h = 0; h < H; ++h)
        acc += oracle_bf16_to_f64(w[(int64_t)v * H + h]) * oracle_bf16_to_f64(x[(int64_t)t * H + h]);
      out[(int64_t)t * V + v] = acc;
    }
  }
  return 0;
}

/* E2M1 (the OCP 4-bit float): sign bit 3, exponent bits 2..1 with bias 1,
 * mantissa bit 0.  Exponent 0 holds 0 and the subnormal 0.5; otherwise
 * (1 + m/2) * 2^(e-1): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_to_f64(uint8_t c) {
  const int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + m / 2.0, e - 1);
  return s ? -mag : mag;
}

/* E8M0 scale: 2^(c - 127); 255 is NaN. */
double oracle_e8m0_to_f64(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

/* Element (n, k) of an N x K expert matrix in format fmt:
 *  INT4_G32   4-bit codes (low nibble = even k), value (u - 8) * bf16 scale of
 *             the group of 32 consecutive k;
 *  MXFP4      4-bit E2M1 codes (same packing), value e2m1(u) * 2^(c - 127)
 *             with c the E8M0 scale of the group of 32 (OCP MX: one shared
 *             scale per block of 32 elements);
 *  FP8_BLOCK  one E4M3 code per byte, value e4m3(c) * the float32 scale of
 *             the 128 x 128 block (n / 128, k / 128); the pages name the
 *             serialized block-FP8 checkpoint only, the block shape is the
 *             reading. */
static double w_fmt_at(int32_t fmt, const uint8_t* q, const void* s, int32_t N, int32_t K, int32_t n,
                       int32_t k) {
  (void)N;
  if (fmt == ORACLE_FMT_FP8_BLOCK) {
    const int32_t kb = (K + 127) / 128;
    const float* sf = (const float*)s;
    return oracle_e4m3_to_f64(q[(int64_t)n * K + k]) * (double)sf[(int64_t)(n / 128) * kb + k / 128];
  }
  const int code = code_at(q, K, n, k);
  if (fmt == ORACLE_FMT_MXFP4)
    return oracle_e2m1_to_f64((uint8_t)code) * oracle_e8m0_to_f64(((const uint8_t*)s)[(int64_t)n * (K / 32) + k / 32]);
  return (double)(code - 8) * oracle_bf16_to_f64(((const uint16_t*)s)[(int64_t)n * (K / 32) + k / 32]);
}

int oracle_dequant_fmt(int32_t fmt, const uint8_t* q, const void* s, int32_t N, int32_t K, double* W) {
  if (!q || !s || !W || N < 0 || K <= 0 || K % 32) return -1;
  if (fmt != ORACLE_FMT_INT4_G32 && fmt != ORACLE_FMT_MXFP4 && fmt != ORACLE_FMT_FP8_BLOCK) return -1;
  for (int32_t n = 0; n < N; ++n)
    for (int32_t k = 0; k < K; ++k) W[(int64_t)n * K + k] = w_fmt_at(fmt, q, s, N, K, n, k);
  return 0;
}

/* One routed expert in format fmt: h = silu(W1 x) * (W3 x), y = W2 h. */
static int expert_fmt(const oracle_cfg* cfg, int32_t fmt, const uint8_t* w13_q, const void* w13_s,
                      const uint8_t* w2_q, const void* w2_s, const double* x, double* y) {
  const int32_t H = cfg->hidden, I = cfg->inter;
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  if (!h) return -2;
#pragma omp parallel for schedule(static)
  for (int32_t r = 0; r < I; ++r) {
    double g = 0.0, u = 0.0;
    for (int32_t k = 0; k < H; ++k) {
      g += w_fmt_at(fmt, w13_q, w13_s, 2 * I, H, r, k) * x[k];
      u += w_fmt_at(fmt, w13_q, w13_s, 2 * I, H, I + r, k) * x[k];
    }
    h[r] = silu(g) * u;
  }
#pragma omp parallel for schedule(static)
  for (int32_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int32_t r = 0; r < I; ++r) acc += w_fmt_at(fmt, w2_q, w2_s, H, I, n, r) * h[r];
    y[n] = acc;
  }
  free(h);
  return 0;
}

/* oracle_forward with the routed experts in format ex->fmt (the shared
 * expert stays BF16). */
int oracle_forward_fmt(const oracle_cfg* cfg, const oracle_experts_fmt* ex, const uint16_t* x, int32_t M,
                       const int32_t* ids, const double* w, double* out) {
  if (!cfg || !ex || M < 0 || (M > 0 && (!x || !ids || !w || !out))) return -1;
  if (ex->fmt != ORACLE_FMT_INT4_G32 && ex->fmt != ORACLE_FMT_MXFP4 && ex->fmt != ORACLE_FMT_FP8_BLOCK) return -1;
  const int32_t H = cfg->hidden, E = cfg->n_experts, k = cfg->top_k;
  if (cfg->has_shared && (!ex->sh_w13 || !ex->sh_w2)) return -1;
  double* xt = (double*)malloc(sizeof(double) * (size_t)H);
  double* y = (double*)malloc(sizeof(double) * (size_t)H);
  if (!xt || !y) { free(xt); free(y); return -2; }
  int bad = 0;
  for (int32_t t = 0; t < M; ++t) {
    for (int32_t h = 0; h < H; ++h) xt[h] = oracle_bf16_to_f64(x[(int64_t)t * H + h]);
    double* ot = out + (int64_t)t * H;
    for (int32_t n = 0; n < H; ++n) ot[n] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = ids[(int64_t)t * k + j];
      if (e < 0 || e >= E) { ++bad; continue; }
      if (!ex->w13_q[e] || !ex->w13_s[e] || !ex->w2_q[e] || !ex->w2_s[e]) {
        free(xt); free(y);
        return -3;
      }
      expert_fmt(cfg, ex->fmt, ex->w13_q[e], ex->w13_s[e], ex->w2_q[e], ex->w2_s[e], xt, y);
      const double wj = w[(int64_t)t * k + j];
      for (int32_t n = 0; n < H; ++n) ot[n] += y[n] * wj;
    }
    if (cfg->has_shared) {
      oracle_expert_dense(cfg, ex->sh_w13, ex->sh_w2, xt, NULL, y);
      for (int32_t n = 0; n < H; ++n) ot[n] = ot[n] + y[n];
    }
  }
  free(xt);
  free(y);
  return bad;
}
