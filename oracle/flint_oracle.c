/*
 * CPU oracle of the Flint routed-expert MoE block (NVFP4 W4A16 and BF16
 * experts).  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library; the product path never
 * does, and this file shares no code, header or table with the HIP library.
 *
 * Plain, slow and written for reading.  Every floating-point step follows the
 * numerics rule stated in the module docstring of the vLLM page
 * "vllm.models.flint.ops.moe" (the "Numerics" paragraph):
 *   - router logits are bf16;
 *   - top-k selection and the sigmoid / renormalisation are fp32 with an exact
 *     exp and exact (round-to-nearest) division; routing weights are rounded
 *     to bf16;
 *   - expert weights are dequantised exactly (E2M1 value times E4M3 scale),
 *     products are accumulated in fp32 and the per-expert fp32 global scale
 *     multiplies the fp32 accumulator;
 *   - act = bf16(silu(g) * u) from fp32 g and u;
 *   - y_e = bf16(acc_e * global_scale_e);
 *   - routed = bf16(sum_e tw_e * y_e) accumulated in fp32;
 *   - out = bf16(routed + shared).
 *
 * Notation: RN32(v) rounds a real to binary32 (C's (float) cast of a double,
 * round to nearest even); RNb rounds binary32 to bfloat16 (nearest even).
 * An "fp32 accumulation" is evaluated here as the real sum, accumulated in
 * double (each product of a bf16 value and a dequantised weight is exact in
 * double), and rounded once with RN32: the correctly rounded fp32 result,
 * which any fp32 summation order approximates.
 *
 * Readings of points the pages leave open are listed where they are used.
 * Parity-unpinned parts: the SiLU sigmoid (the pages use hardware
 * approximations; here it is the exact sigmoid, rounded once).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FMT_NVFP4 0
#define ORC_FMT_BF16 1

/* ---------------------------------------------------------------- formats */

/* bfloat16 bits -> value.  bf16 is the top half of a binary32. */
float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* RNb: binary32 -> bfloat16, round to nearest, ties to even.  NaN stays NaN
 * (quietened, sign kept); overflow past the largest bf16 gives infinity. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t low = u & 0xffffu;        /* the 16 bits that are dropped */
  uint32_t hi = u >> 16;
  if (low > 0x8000u || (low == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

/* E2M1 (OCP Microscaling Formats v1.0, FP4 E2M1): 1 sign bit, 2 exponent
 * bits with bias 1, 1 mantissa bit; exponent 0 is subnormal (m * 0.5).
 * Values: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.  No inf or NaN. */
double orc_e2m1(unsigned code) {
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
  return s ? -mag : mag;
}

/* E4M3 "fn" (OCP 8-bit floating point spec, E4M3; torch.float8_e4m3fn):
 * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
 * subnormal (m/8 * 2^-6); no infinities; S.1111.111 is NaN. */
double orc_e4m3fn(unsigned b) {
  unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  double mag;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u)
    mag = ldexp(m / 8.0, -6);
  else
    mag = ldexp(1.0 + m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* Packed codes: byte c of a row holds K elements 2c (low nibble) and 2c+1
 * (high nibble).  The pages unpack each int32 word into its eight codes in
 * ascending K order (page "vllm.models.flint.ops.moe", _dequant_rows); with
 * little-endian words that is this nibble order (reading S2). */
static unsigned nibble(const uint8_t *row, long k) {
  uint8_t b = row[k >> 1];
  return (k & 1) ? (unsigned)(b >> 4) : (unsigned)(b & 15u);
}

static double g_e2m1[16];
static double g_e4m3[256];
static int g_tables_ready = 0;

static void tables(void) {
  if (g_tables_ready) return;
  for (unsigned c = 0; c < 16; ++c) g_e2m1[c] = orc_e2m1(c);
  for (unsigned b = 0; b < 256; ++b) g_e4m3[b] = orc_e4m3fn(b);
  g_tables_ready = 1;
}

/* One NVFP4 weight: E2M1 value times its block's E4M3 scale (one scale per
 * 16 consecutive K elements).  The product has at most 6 significant bits,
 * so it is exact in double, fp32 and bf16. */
static double nvfp4_weight(const uint8_t *codes_row, const uint8_t *scale_row,
                           long k) {
  return g_e2m1[nibble(codes_row, k)] * g_e4m3[scale_row[k / 16]];
}

/* Dequantise a [rows, K] NVFP4 matrix into bf16 bits (the product is exact in
 * bf16; NaN scales give NaN). */
void orc_nvfp4_dequant(const uint8_t *w, const uint8_t *s, long rows, long K,
                       uint16_t *out) {
  tables();
  for (long r = 0; r < rows; ++r)
    for (long k = 0; k < K; ++k)
      out[r * K + k] =
          orc_f32_to_bf16((float)nvfp4_weight(w + r * (K / 2), s + r * (K / 16), k));
}

/* ---------------------------------------------------------------- routing */

/* logits[t, e] = RNb(RN32(sum_h x[t, h] * router[e, h])): bf16 router logits
 * (page "vllm.models.flint.ops.moe", numerics rule and the router kernel's
 * description: a GEMV whose fp32 result is stored as bf16). */
void orc_logits(const uint16_t *x, const uint16_t *router, long M, long H,
                long E, uint16_t *logits) {
#pragma omp parallel for schedule(static)
  for (long t = 0; t < M; ++t)
    for (long e = 0; e < E; ++e) {
      double acc = 0.0;
      for (long h = 0; h < H; ++h)
        acc += (double)orc_bf16_to_f32(x[t * H + h]) *
               (double)orc_bf16_to_f32(router[e * H + h]);
      logits[t * E + e] = orc_f32_to_bf16((float)acc);
    }
}

/* The fp32 sigmoid score of one bf16 logit l: s = RN32(1 / RN32(1 + a)) with
 * a = RN32(exp(-l)) correctly rounded (the pages ask for an exact exp and a
 * round-to-nearest division).  exp is glibc's double exp, then rounded once;
 * the tests check a against a 50-digit decimal exp for every bf16 input. */
float orc_router_score(uint16_t logit_bits) {
  float l = orc_bf16_to_f32(logit_bits);
  float a = (float)exp(-(double)l);
  float d = 1.0f + a;
  return 1.0f / d;
}

/* Whether logit a (bf16 bits) of expert ia ranks above logit b of expert ib
 * in the routing selection.  The rule (page "vllm.models.flint.ops.moe",
 * "Numerics" paragraph and the top-k routine _topk_row of the router): the
 * larger logit comes first and equal logits go to the smaller expert index.
 * Points the rule leaves to the bit patterns (reading S12):
 *   - +0 ranks above -0;
 *   - a NaN whose sign bit is clear ranks above +inf, one whose sign bit is
 *     set below -inf; among NaNs of one sign the larger payload lies further
 *     from zero (above for the positive sign, below for the negative).
 * Written here as comparisons of values and classes, not as an integer key. */
static int ranks_above(uint16_t a, long ia, uint16_t b, long ib) {
  const float fa = orc_bf16_to_f32(a), fb = orc_bf16_to_f32(b);
  const int na = isnan(fa), nb = isnan(fb);
  /* class: 2 = positive NaN, 1 = a number (finite or infinite), 0 = negative NaN */
  const int ca = na ? (signbit(fa) ? 0 : 2) : 1;
  const int cb = nb ? (signbit(fb) ? 0 : 2) : 1;
  if (ca != cb) return ca > cb;
  if (ca == 1) {
    if (fa != fb) return fa > fb;
    if (!signbit(fa) != !signbit(fb)) return signbit(fb) != 0; /* +0 above -0 */
    return ia < ib;
  }
  /* two NaNs of one sign: by payload, away from zero */
  const int pa = a & 0x7f, pb = b & 0x7f;
  if (pa != pb) return ca == 2 ? pa > pb : pa < pb;
  return ia < ib;
}

/* Top-k of one row of bf16 logits with renormalised sigmoid weights (page
 * "vllm.models.flint.ops.moe", the "Numerics" paragraph and _topk_row).
 * Each expert's place in the descending order is the number of experts that
 * rank above it (ranks_above); those at places 0 .. k-1 are selected, and
 * place j is ids[t, j].
 *
 * Scores s_j (fp32) of the selected logits are renormalised:
 *   S = s_0 + s_1 + ... + s_{k-1}   (fp32, left to right in selection order;
 *                                    the pages sum with an unordered
 *                                    reduction, this order is our reading)
 *   D = RN32(S + 1e-20)            (1e-20 as its nearest fp32)
 *   tw_j = RNb(RN32(s_j / D)), stored as fp32.
 * scores (may be NULL) receives s_j. */
void orc_topk(const uint16_t *logits, long M, long E, long k, int32_t *ids,
              float *tw, float *scores) {
#pragma omp parallel for schedule(static)
  for (long t = 0; t < M; ++t) {
    const uint16_t *row = logits + t * E;
    float s[256];
    for (long e = 0; e < E; ++e) {
      long place = 0;
      for (long f = 0; f < E; ++f)
        if (f != e && ranks_above(row[f], f, row[e], e)) ++place;
      if (place < k) {
        ids[t * k + place] = (int32_t)e;
        s[place] = orc_router_score(row[e]);
      }
    }
    float S = 0.0f;
    for (long j = 0; j < k; ++j) S = S + s[j];
    float D = S + 1e-20f;
    for (long j = 0; j < k; ++j) {
      tw[t * k + j] = orc_bf16_to_f32(orc_f32_to_bf16(s[j] / D));
      if (scores) scores[t * k + j] = s[j];
    }
  }
}

/* ---------------------------------------------------------- expert stages */

/* Weight element (row r, column c) of expert e of a [E, R, C] matrix. */
typedef struct {
  int fmt;                /* ORC_FMT_NVFP4 or ORC_FMT_BF16 */
  const uint8_t *codes;   /* NVFP4: [E, R, C/2] */
  const uint8_t *scales;  /* NVFP4: [E, R, C/16] E4M3 */
  const float *alpha;     /* NVFP4: [E] global scale; unused for BF16 */
  const uint16_t *bf16;   /* BF16:  [E, R, C] */
  long R, C;
} weights_view;

static double weight_at(const weights_view *w, long e, long r, long c) {
  if (w->fmt == ORC_FMT_NVFP4)
    return nvfp4_weight(w->codes + (e * w->R + r) * (w->C / 2),
                        w->scales + (e * w->R + r) * (w->C / 16), c);
  return (double)orc_bf16_to_f32(w->bf16[(e * w->R + r) * w->C + c]);
}

/* RN32(RN32(sum_c a[c] * W[e, r, c]) * alpha_e): fp32 accumulation, then the
 * per-expert global scale applied to the fp32 accumulator (NVFP4 only; the
 * BF16 experts have none).  *abs_sum receives sum |a[c] W[e, r, c]| (times
 * alpha), the scale of the accumulation's rounding error. */
static float project(const weights_view *w, long e, long r, const float *a,
                     double *abs_sum) {
  double acc = 0.0, mag = 0.0;
  for (long c = 0; c < w->C; ++c) {
    double p = (double)a[c] * weight_at(w, e, r, c);
    acc += p;
    mag += fabs(p);
  }
  float v = (float)acc;
  if (w->fmt == ORC_FMT_NVFP4) {
    v = (float)((double)v * (double)w->alpha[e]);
    mag *= (double)w->alpha[e];
  }
  if (abs_sum) *abs_sum = mag;
  return v;
}

/* silu(g) in fp32: the exact g * sigmoid(g), rounded once.  The pages compute
 * the sigmoid with hardware reciprocal/exp2 approximations; this oracle uses
 * the exact function (parity unpinned: covered by the tolerance). */
float orc_silu(float g) {
  double gd = (double)g;
  return (float)(gd / (1.0 + exp(-gd)));
}

/* Gate/up + SwiGLU for every pair p = t*k + j (expert e = ids[p]):
 *   G = RN32(RN32(sum_h x[t,h] W13[e, n, h]) * alpha_e)       gate rows 0..I-1
 *   U = RN32(RN32(sum_h x[t,h] W13[e, I+n, h]) * alpha_e)     up rows I..2I-1
 *   act[p, n] = RNb(RN32(silu(G) * U)).
 * w13 is [E, 2I, H] ([gate; up], ModelOpt layout).  g, u, gabs, uabs may be
 * NULL; otherwise they receive G, U and their accumulation magnitudes.
 * npairs = M*k; ids holds the expert of every pair; token of pair p is
 * p / k. */
void orc_gate_up(const uint16_t *x, long M, long H, long I, long k,
                 const int32_t *ids, int fmt, const uint8_t *codes,
                 const uint8_t *scales, const float *alpha,
                 const uint16_t *bf16w, long E, uint16_t *act, float *g,
                 float *u, double *gabs, double *uabs) {
  tables();
  weights_view w = {fmt, codes, scales, alpha, bf16w, 2 * I, H};
  (void)E;
#pragma omp parallel for schedule(dynamic)
  for (long p = 0; p < M * k; ++p) {
    long t = p / k, e = ids[p];
    float *xr = (float *)malloc(sizeof(float) * (size_t)H);
    for (long h = 0; h < H; ++h) xr[h] = orc_bf16_to_f32(x[t * H + h]);
    for (long n = 0; n < I; ++n) {
      double ga, ua;
      float G = project(&w, e, n, xr, &ga);
      float U = project(&w, e, I + n, xr, &ua);
      float v = (float)((double)orc_silu(G) * (double)U);
      act[p * I + n] = orc_f32_to_bf16(v);
      if (g) g[p * I + n] = G;
      if (u) u[p * I + n] = U;
      if (gabs) gabs[p * I + n] = ga;
      if (uabs) uabs[p * I + n] = ua;
    }
    free(xr);
  }
}

/* Down projection of every pair: y[p, h] = RNb(RN32(RN32(sum_i act[p,i]
 * W2[e, h, i]) * alpha_e)), w2 is [E, H, I].  yabs may be NULL. */
void orc_down(const uint16_t *act, long npairs, long H, long I,
              const int32_t *ids, int fmt, const uint8_t *codes,
              const uint8_t *scales, const float *alpha, const uint16_t *bf16w,
              long E, uint16_t *y, float *yacc, double *yabs) {
  tables();
  weights_view w = {fmt, codes, scales, alpha, bf16w, H, I};
  (void)E;
#pragma omp parallel for schedule(dynamic)
  for (long p = 0; p < npairs; ++p) {
    float *ar = (float *)malloc(sizeof(float) * (size_t)I);
    for (long i = 0; i < I; ++i) ar[i] = orc_bf16_to_f32(act[p * I + i]);
    for (long h = 0; h < H; ++h) {
      double mag;
      float v = project(&w, ids[p], h, ar, &mag);
      y[p * H + h] = orc_f32_to_bf16(v);
      if (yacc) yacc[p * H + h] = v;
      if (yabs) yabs[p * H + h] = mag;
    }
    free(ar);
  }
}

/* Weighted combine and shared add for every token t and column h:
 *   R = RN32(sum_j tw[t, j] * y[t*k + j, h])        (fp32 accumulation)
 *   routed = RNb(R),  out = RNb(RN32(routed + sh[t, h])).
 * sh may be NULL (no shared expert: sh = 0).  routed may be NULL. */
void orc_combine(const uint16_t *y, const float *tw, const uint16_t *sh, long M,
                 long H, long k, uint16_t *out, uint16_t *routed) {
#pragma omp parallel for schedule(static)
  for (long t = 0; t < M; ++t)
    for (long h = 0; h < H; ++h) {
      double acc = 0.0;
      for (long j = 0; j < k; ++j)
        acc += (double)tw[t * k + j] * (double)orc_bf16_to_f32(y[(t * k + j) * H + h]);
      uint16_t r = orc_f32_to_bf16((float)acc);
      float s = sh ? orc_bf16_to_f32(sh[t * H + h]) : 0.0f;
      out[t * H + h] = orc_f32_to_bf16(orc_bf16_to_f32(r) + s);
      if (routed) routed[t * H + h] = r;
    }
}

/* Number of OpenMP threads the stage functions use (rows are independent and
 * each row's arithmetic is sequential, so results do not depend on it). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_get_threads(void) { return omp_get_max_threads(); }
