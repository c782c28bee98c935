/*
 * oracle.c -- plain, slow CPU definition of the fused FP8 FFN block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (libfrt) never links, loads or calls it, and the two share no source,
 * header, table or helper.
 *
 * What is computed follows the FlashRT pages:
 *   - FlashRT project page (agentlenshq), "main ideas": weights and
 *     activations in FP8 with per-tensor calibrated scales;
 *   - itsolotime article, section 7.1 (FP8 path, E4M3) and 7.2 (the encoder
 *     FFN loop: fp16/bf16 residual stream, RMSNorm, gate and up GEMMs,
 *     gated activation fused with re-quantisation, down GEMM, residual add);
 *   - FlashRT architecture doc, component "Calibration": amax per FP8 GEMM
 *     input in a measurement pass, then alpha = act_scale * weight_scale
 *     baked as host scalars;
 *   - itsolotime article, section 7.2 (the NVFP4 encoder FFN: bf16/fp16
 *     residual kept at high precision, AWQ pre-scale of the normalised
 *     activations, 4-bit gate/up and down GEMMs, a gated combine that
 *     re-quantises to 4 bits), here in the OCP microscaling FP4 format;
 *   - FlashRT architecture doc, component "Kernel library": the fused
 *     residual + norm + quant kernel, and the "qkv split + RoPE" fusion that
 *     follows the fused QKV projection on the attention side (the FusedQKV
 *     weight of the Pi0/Pi0.5 specs, itsolotime article section 5.2).
 * Every rounding point the pages leave open is fixed here: OCP E4M3FN with
 * saturation at +-448, round-to-nearest-even everywhere, the RMSNorm mean
 * square summed in fp64 with 1/rms rounded once to fp32, FP8 products summed
 * exactly and rounded once to fp32, activations evaluated in fp64 and rounded
 * once to fp32, bf16 outputs by round-to-nearest-even.
 *
 * Style: scalar loops, no SIMD intrinsics, no blocking.  The only
 * parallelism is pthreads over independent output elements.
 *
 * Parity status: every function here is pinned by the CPU tests
 * (codec vs the OCP table and torch, bf16 vs torch, GEMM vs fp64 matmul,
 * RMSNorm closed form, activations vs torch fp64, block vs an independent
 * transcription, calibration brute force).  Nothing is "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_ACT_GEGLU_TANH 0 /* gelu_tanh(gate) * up              */
#define ORC_ACT_SWIGLU 1     /* silu(gate) * up                   */
#define ORC_ACT_GELU_TANH 2  /* gelu_tanh(up), no gate projection */

/* ------------------------------------------------------------------------ */
/* bf16: the top 16 bits of an fp32 after round-to-nearest-even.            */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t f32_to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

float orc_bf16_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

uint16_t orc_bf16_round(float v) {
  uint32_t u = f32_to_bits(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN stays a quiet NaN */
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lower = u & 0xffffu;
  uint32_t upper = u >> 16;
  /* round half to even on the dropped 16 bits */
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits.           */
/* Exponent field 0 is subnormal (m * 2^-9).  S.1111.111 is NaN; there is   */
/* no infinity; the largest finite value is S.1111.110 = 448.              */
/* ------------------------------------------------------------------------ */

double orc_e4m3_decode(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 0xf;
  int m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Round to nearest integer, ties to even.  x >= 0 and small. */
static long rne_nonneg(double x) {
  double f = floor(x);
  double r = x - f;
  long n = (long)f;
  if (r > 0.5) return n + 1;
  if (r < 0.5) return n;
  return (n & 1) ? n + 1 : n;
}

uint8_t orc_e4m3_encode(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  if (isnan(v)) return (uint8_t)(sign | 0x7f);
  double a = fabs((double)v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7e); /* saturate, incl. inf */
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: value = m * 2^-9, m in 0..8 (8 is the min normal) */
    long m = rne_nonneg(a * 512.0);
    return (uint8_t)(sign | (uint8_t)m); /* m == 8 encodes 0x08 = 2^-6 */
  }
  int e2;
  double fr = frexp(a, &e2); /* a = fr * 2^e2, fr in [0.5, 1) */
  int e = e2 - 1;            /* a = (2*fr) * 2^e, 2*fr in [1, 2) */
  long mant = rne_nonneg((2.0 * fr - 1.0) * 8.0);
  if (mant == 8) { /* carry into the next binade */
    mant = 0;
    e += 1;
  }
  /* a < 448 and RNE at step 32 in [256,512) keeps e+7 <= 15 and the code
     at most 0x7e: 448 <= a < 464 was excluded above only for a >= 448,
     and 432 < a < 448 rounds to 448 (mant 6) at most. */
  return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | (int)mant));
}

/* e4m3 codes as integers in units of 2^-9 (exact): the value of code c is
   k(c) * 2^-9 with |k| <= 448 * 512.  NaN codes never reach a GEMM. */
static int32_t code_units(uint8_t c) {
  double v = orc_e4m3_decode(c);
  return (int32_t)(v * 512.0);
}

void orc_e4m3_encode_array(const float *in, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(in[i]);
}
void orc_e4m3_decode_array(const uint8_t *in, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(in[i]);
}
void orc_bf16_round_array(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_round(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Activations, evaluated in fp64 with host libm and rounded once to fp32.  */
/* gelu_tanh is Hendrycks & Gimpel's tanh approximation of GELU.            */
/* ------------------------------------------------------------------------ */

double orc_gelu_tanh(double z) {
  const double pi = 3.14159265358979323846;
  const double c = sqrt(2.0 / pi);
  return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

float orc_act_f32(int act_kind_is_silu, float z) {
  return act_kind_is_silu ? (float)orc_silu((double)z) : (float)orc_gelu_tanh((double)z);
}

/* ------------------------------------------------------------------------ */
/* A tiny parallel-for over [0, n).                                         */
/* ------------------------------------------------------------------------ */

typedef void (*range_fn)(void *ctx, int64_t begin, int64_t end);
typedef struct {
  range_fn fn;
  void *ctx;
  int64_t begin, end;
} range_job;

static void *run_range(void *p) {
  range_job *j = (range_job *)p;
  j->fn(j->ctx, j->begin, j->end);
  return NULL;
}

static void parallel_for(int64_t n, int nthreads, range_fn fn, void *ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t th[256];
  int started[256];
  range_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].begin = n * t / nthreads;
    jobs[t].end = n * (t + 1) / nthreads;
    started[t] = pthread_create(&th[t], NULL, run_range, &jobs[t]) == 0;
    if (!started[t]) run_range(&jobs[t]); /* no thread: do it inline */
  }
  for (int t = 0; t < nthreads; ++t)
    if (started[t]) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Exact FP8 GEMM: out[m][n] = f32( sum_k dec(a[m][k]) * dec(b[n][k]) ).    */
/* a is [M,K] row-major codes, b is [N,K] (nn.Linear [out,in]) codes.       */
/* Each product is an integer in units of 2^-18 below 2^36; for K < 2^15   */
/* the int64 sum is exact, so the only rounding is the final one to fp32.   */
/* ------------------------------------------------------------------------ */

typedef struct {
  int M, N, K;
  const uint8_t *a, *b;
  float *out;
  int32_t units[256];
} gemm_ctx;

static void gemm_range(void *p, int64_t begin, int64_t end) {
  gemm_ctx *g = (gemm_ctx *)p;
  for (int64_t idx = begin; idx < end; ++idx) {
    int m = (int)(idx / g->N);
    int n = (int)(idx % g->N);
    const uint8_t *ar = g->a + (int64_t)m * g->K;
    const uint8_t *br = g->b + (int64_t)n * g->K;
    int64_t acc = 0;
    for (int k = 0; k < g->K; ++k)
      acc += (int64_t)g->units[ar[k]] * (int64_t)g->units[br[k]];
    g->out[idx] = (float)ldexp((double)acc, -18);
  }
}

int orc_gemm_e4m3(int M, int N, int K, const uint8_t *a, const uint8_t *b, float *out,
                  int nthreads) {
  if (K >= (1 << 15)) return -1; /* exactness bound of the int64 sum */
  gemm_ctx g;
  g.M = M;
  g.N = N;
  g.K = K;
  g.a = a;
  g.b = b;
  g.out = out;
  for (int c = 0; c < 256; ++c) g.units[c] = ((c & 0x7f) == 0x7f) ? 0 : code_units((uint8_t)c);
  parallel_for((int64_t)M * N, nthreads, gemm_range, &g);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-tensor weight quantisation (architecture doc, "Weights": transpose + */
/* Quant() transforms with a per-tensor scale collected into a table).      */
/*   s = amax > 0 ? f32(amax / 448) : 1;  inv = f32(1/s);                   */
/*   code = e4m3( f32(w * inv) )                                            */
/* ------------------------------------------------------------------------ */

float orc_scale_from_amax(float amax) { return amax > 0.0f ? amax / 448.0f : 1.0f; }

typedef struct {
  const uint16_t *w;
  uint8_t *codes;
  float inv;
  float part_max[256];
  int64_t n;
  int nthreads;
  const uint16_t *colw; /* optional per-column factor (norm fusion), NULL = none */
  int64_t cols;
} quant_ctx;

/* element i of the tensor being quantised: bf16 w[i], or with norm fusion
   f32(w[i] * colw[i % cols]) -- a product of two bf16 values, exact in fp32 */
static float quant_value(const quant_ctx *q, int64_t i) {
  float v = orc_bf16_to_f32(q->w[i]);
  if (q->colw) v = v * orc_bf16_to_f32(q->colw[i % q->cols]);
  return v;
}

static void amax_range(void *p, int64_t begin, int64_t end) {
  /* one range per thread: begin..end covers thread t's slice */
  quant_ctx *q = (quant_ctx *)p;
  int64_t t = begin; /* ranges are thread indices here */
  for (; t < end; ++t) {
    int64_t lo = q->n * t / q->nthreads, hi = q->n * (t + 1) / q->nthreads;
    float m = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      float a = fabsf(quant_value(q, i));
      if (a > m) m = a;
    }
    q->part_max[t] = m;
  }
}

static void encode_range(void *p, int64_t begin, int64_t end) {
  quant_ctx *q = (quant_ctx *)p;
  for (int64_t i = begin; i < end; ++i) q->codes[i] = orc_e4m3_encode(quant_value(q, i) * q->inv);
}

/* amax is an exact max (order does not matter); the threads only split the
   elements. */
/* Pi0-style norm fusion (FlashRT itsolotime article, section 5.2: the
   decoder spec folds the RMSNorm weight into the gate/up matrices before
   Quant()): tensor [rows][cols] times colw[col] per input column, then the
   same per-tensor quantisation. */
float orc_quant_tensor_fold(const uint16_t *w, int64_t rows, int64_t cols, const uint16_t *colw,
                            uint8_t *codes, int nthreads) {
  quant_ctx q;
  int64_t n = rows * cols;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  q.w = w;
  q.codes = codes;
  q.n = n;
  q.nthreads = nthreads;
  q.colw = colw;
  q.cols = cols;
  parallel_for(nthreads, nthreads, amax_range, &q);
  float amax = 0.0f;
  for (int t = 0; t < nthreads; ++t)
    if (q.part_max[t] > amax) amax = q.part_max[t];
  float s = orc_scale_from_amax(amax);
  q.inv = 1.0f / s;
  parallel_for(n, nthreads, encode_range, &q);
  return s;
}

float orc_quant_tensor_mt(const uint16_t *w, int64_t n, uint8_t *codes, int nthreads) {
  quant_ctx q;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  q.colw = NULL;
  q.cols = 1;
  q.w = w;
  q.codes = codes;
  q.n = n;
  q.nthreads = nthreads;
  parallel_for(nthreads, nthreads, amax_range, &q);
  float amax = 0.0f;
  for (int t = 0; t < nthreads; ++t)
    if (q.part_max[t] > amax) amax = q.part_max[t];
  float s = orc_scale_from_amax(amax);
  q.inv = 1.0f / s;
  parallel_for(n, nthreads, encode_range, &q);
  return s;
}

float orc_quant_tensor(const uint16_t *w, int64_t n, uint8_t *codes) {
  return orc_quant_tensor_mt(w, n, codes, 1);
}

/* ------------------------------------------------------------------------ */
/* Step 1: fused residual add + RMSNorm + E4M3 quantise, one row at a time. */
/*   r'  = bf16( r + y )                          (new residual, stored)     */
/*   S   = sum r'^2 in fp64;  inv_rms = f32( 1/sqrt(S/H + eps) ), fp64 math */
/*   t   = f32( r' * inv_rms )                                              */
/*   x   = f32( t * w )                       (RMSNorm weight w), or with   */
/*         AdaRMSNorm modulation (itsolotime article, section 5.2: Pi0.5    */
/*         modulates through AdaRMSNorm Dense layers instead of a folded    */
/*         weight): x = f32( f32( t * f32(1 + scale) ) + shift )            */
/*   xq  = e4m3( f32(x * inv_x) )                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
  int H;
  const uint16_t *r_prev, *y_prev, *w_norm;
  const uint16_t *mod_scale, *mod_shift; /* both NULL, or both [H] bf16 */
  float eps, inv_x;
  uint16_t *r_out;
  float *x_out; /* optional: the unquantised normalised row */
  uint8_t *xq_out;
} norm_ctx;

static void norm_range(void *p, int64_t begin, int64_t end) {
  norm_ctx *c = (norm_ctx *)p;
  int H = c->H;
  for (int64_t m = begin; m < end; ++m) {
    const uint16_t *r = c->r_prev + m * H;
    const uint16_t *y = c->y_prev ? c->y_prev + m * H : NULL;
    uint16_t *ro = c->r_out + m * H;
    double S = 0.0;
    for (int j = 0; j < H; ++j) {
      float sum = orc_bf16_to_f32(r[j]) + (y ? orc_bf16_to_f32(y[j]) : 0.0f);
      ro[j] = orc_bf16_round(sum);
      double rv = (double)orc_bf16_to_f32(ro[j]);
      S += rv * rv;
    }
    float inv_rms = (float)(1.0 / sqrt(S / (double)H + (double)c->eps));
    for (int j = 0; j < H; ++j) {
      float t = orc_bf16_to_f32(ro[j]) * inv_rms;
      float x;
      if (c->mod_scale) {
        float one_plus = 1.0f + orc_bf16_to_f32(c->mod_scale[j]);
        float ts = t * one_plus;
        x = ts + orc_bf16_to_f32(c->mod_shift[j]);
      } else {
        x = t * orc_bf16_to_f32(c->w_norm[j]);
      }
      if (c->x_out) c->x_out[m * H + j] = x;
      if (c->xq_out) c->xq_out[m * H + j] = orc_e4m3_encode(x * c->inv_x);
    }
  }
}

void orc_add_rmsnorm_quant(int M, int H, const uint16_t *r_prev, const uint16_t *y_prev,
                           const uint16_t *w_norm, const uint16_t *mod_scale,
                           const uint16_t *mod_shift, float eps, float inv_x, uint16_t *r_out,
                           float *x_out, uint8_t *xq_out, int nthreads) {
  norm_ctx c = {H, r_prev, y_prev, w_norm, mod_scale, mod_shift, eps, inv_x, r_out, x_out, xq_out};
  parallel_for(M, nthreads, norm_range, &c);
}

/* ------------------------------------------------------------------------ */
/* Step 2: gate/up GEMM, dequant, gated activation, re-quantise.            */
/*   g = f32( f32(Ag) * alpha_g ),  u = f32( f32(Au) * alpha_u )            */
/*   GeGLU: h = f32( f32(gelu_tanh(g)) * u );  SwiGLU: silu instead;         */
/*   non-gated: h = f32( gelu_tanh(u) )                                      */
/*   hq = e4m3( f32(h * inv_h) )                                            */
/* ------------------------------------------------------------------------ */

static float gated_value(int act, float g, float u) {
  if (act == ORC_ACT_GELU_TANH) return (float)orc_gelu_tanh((double)u);
  float a = (act == ORC_ACT_SWIGLU) ? (float)orc_silu((double)g) : (float)orc_gelu_tanh((double)g);
  return a * u;
}

/* Epilogue of step 2 on given fp32 accumulators Ag, Au [M*I] (Ag unused for
   the non-gated form). */
void orc_gateup_epilogue(int64_t n, int act, const float *Ag, const float *Au, float alpha_g,
                         float alpha_u, float inv_h, float *h_out, uint8_t *hq_out) {
  for (int64_t idx = 0; idx < n; ++idx) {
    float u = Au[idx] * alpha_u;
    float g = (act != ORC_ACT_GELU_TANH) ? Ag[idx] * alpha_g : 0.0f;
    float h = gated_value(act, g, u);
    if (h_out) h_out[idx] = h;
    if (hq_out) hq_out[idx] = orc_e4m3_encode(h * inv_h);
  }
}

int orc_gateup(int M, int H, int I, int act, const uint8_t *xq, const uint8_t *qg,
               const uint8_t *qu, float alpha_g, float alpha_u, float inv_h, float *h_out,
               uint8_t *hq_out, int nthreads) {
  float *Ag = NULL, *Au = (float *)malloc(sizeof(float) * (size_t)M * I);
  if (!Au) return -2;
  if (orc_gemm_e4m3(M, I, H, xq, qu, Au, nthreads)) return free(Au), -1;
  if (act != ORC_ACT_GELU_TANH) {
    Ag = (float *)malloc(sizeof(float) * (size_t)M * I);
    if (!Ag) return free(Au), -2;
    if (orc_gemm_e4m3(M, I, H, xq, qg, Ag, nthreads)) return free(Au), free(Ag), -1;
  }
  orc_gateup_epilogue((int64_t)M * I, act, Ag, Au, alpha_g, alpha_u, inv_h, h_out, hq_out);
  free(Au);
  free(Ag);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 3: down GEMM, dequant, bf16 output.                                 */
/*   y = bf16( f32( f32(Ad) * alpha_d ) )                                   */
/* ------------------------------------------------------------------------ */

void orc_down_epilogue(int64_t n, const float *Ad, float alpha_d, uint16_t *y_out) {
  for (int64_t idx = 0; idx < n; ++idx) y_out[idx] = orc_bf16_round(Ad[idx] * alpha_d);
}

int orc_down(int M, int H, int I, const uint8_t *hq, const uint8_t *qd, float alpha_d,
             uint16_t *y_out, int nthreads) {
  float *Ad = (float *)malloc(sizeof(float) * (size_t)M * H);
  if (!Ad) return -2;
  if (orc_gemm_e4m3(M, H, I, hq, qd, Ad, nthreads)) return free(Ad), -1;
  orc_down_epilogue((int64_t)M * H, Ad, alpha_d, y_out);
  free(Ad);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* One whole block (layer): (r_prev, y_prev) -> (r_out, y_out).              */
/* Host scalars are derived exactly as the architecture doc's calibration   */
/* component describes: alpha = act_scale * weight_scale, plus the two      */
/* reciprocal activation scales used by the quantisers.                     */
/* ------------------------------------------------------------------------ */

int orc_block(int M, int H, int I, int act, float eps, const uint16_t *r_prev,
              const uint16_t *y_prev, const uint16_t *w_norm, const uint16_t *mod_scale,
              const uint16_t *mod_shift, const uint8_t *qg,
              const uint8_t *qu, const uint8_t *qd, float s_g, float s_u, float s_d, float s_x,
              float s_h, uint16_t *r_out, uint8_t *xq_out, uint8_t *hq_out, uint16_t *y_out,
              int nthreads) {
  float inv_x = 1.0f / s_x, inv_h = 1.0f / s_h;
  float alpha_g = s_x * s_g, alpha_u = s_x * s_u, alpha_d = s_h * s_d;
  uint8_t *xq = xq_out ? xq_out : (uint8_t *)malloc((size_t)M * H);
  uint8_t *hq = hq_out ? hq_out : (uint8_t *)malloc((size_t)M * I);
  int rc = 0;
  if (!xq || !hq) rc = -2;
  if (!rc)
    orc_add_rmsnorm_quant(M, H, r_prev, y_prev, w_norm, mod_scale, mod_shift, eps, inv_x, r_out, NULL, xq,
                          nthreads);
  if (!rc) rc = orc_gateup(M, H, I, act, xq, qg, qu, alpha_g, alpha_u, inv_h, NULL, hq, nthreads);
  if (!rc) rc = orc_down(M, H, I, hq, qd, alpha_d, y_out, nthreads);
  if (!xq_out) free(xq);
  if (!hq_out) free(hq);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Calibration measurement pass for one block (architecture doc,            */
/* "Calibration" (a); the predict() flow's "run 1 fwd, record amax").        */
/* Activations stay unquantised (fp32 as produced), weights are the already */
/* quantised FP8 codes times their per-tensor scale; dot products in fp64.  */
/* Returns the running maxima of |x| (gate/up GEMM input) and |h| (down     */
/* GEMM input) through amax_x / amax_h (max-accumulated, not reset).        */
/* ------------------------------------------------------------------------ */

typedef struct {
  int M, N, K;
  const float *a;   /* [M,K] fp32 activations */
  const uint8_t *b; /* [N,K] codes */
  float scale;
  double *out; /* [M,N] fp64 sums (unscaled) */
  double dec[256];
} mgemm_ctx;

static void mgemm_range(void *p, int64_t begin, int64_t end) {
  mgemm_ctx *g = (mgemm_ctx *)p;
  for (int64_t idx = begin; idx < end; ++idx) {
    int m = (int)(idx / g->N);
    int n = (int)(idx % g->N);
    const float *ar = g->a + (int64_t)m * g->K;
    const uint8_t *br = g->b + (int64_t)n * g->K;
    double acc = 0.0;
    for (int k = 0; k < g->K; ++k) acc += (double)ar[k] * g->dec[br[k]];
    g->out[idx] = acc;
  }
}

static void measure_gemm(int M, int N, int K, const float *a, const uint8_t *b, double *out,
                         int nthreads) {
  mgemm_ctx g;
  g.M = M;
  g.N = N;
  g.K = K;
  g.a = a;
  g.b = b;
  g.out = out;
  for (int c = 0; c < 256; ++c) g.dec[c] = ((c & 0x7f) == 0x7f) ? 0.0 : orc_e4m3_decode((uint8_t)c);
  parallel_for((int64_t)M * N, nthreads, mgemm_range, &g);
}

int orc_block_measure(int M, int H, int I, int act, float eps, const uint16_t *r_prev,
                      const uint16_t *y_prev, const uint16_t *w_norm, const uint16_t *mod_scale,
                      const uint16_t *mod_shift, const uint8_t *qg,
                      const uint8_t *qu, const uint8_t *qd, float s_g, float s_u, float s_d,
                      uint16_t *r_out, uint16_t *y_out, float *amax_x, float *amax_h,
                      int nthreads) {
  float *x = (float *)malloc(sizeof(float) * (size_t)M * H);
  float *h = (float *)malloc(sizeof(float) * (size_t)M * I);
  double *su = (double *)malloc(sizeof(double) * (size_t)M * I);
  double *sg = (act != ORC_ACT_GELU_TANH) ? (double *)malloc(sizeof(double) * (size_t)M * I) : NULL;
  double *sd = (double *)malloc(sizeof(double) * (size_t)M * H);
  int rc = 0;
  if (!x || !h || !su || !sd || (act != ORC_ACT_GELU_TANH && !sg)) rc = -2;
  if (!rc) {
    orc_add_rmsnorm_quant(M, H, r_prev, y_prev, w_norm, mod_scale, mod_shift, eps, 1.0f, r_out, x, NULL,
                          nthreads);
    for (int64_t i = 0; i < (int64_t)M * H; ++i)
      if (fabsf(x[i]) > *amax_x) *amax_x = fabsf(x[i]);
    measure_gemm(M, I, H, x, qu, su, nthreads);
    if (sg) measure_gemm(M, I, H, x, qg, sg, nthreads);
    for (int64_t i = 0; i < (int64_t)M * I; ++i) {
      float u = (float)((double)s_u * su[i]);
      float g = sg ? (float)((double)s_g * sg[i]) : 0.0f;
      h[i] = gated_value(act, g, u);
      if (fabsf(h[i]) > *amax_h) *amax_h = fabsf(h[i]);
    }
    measure_gemm(M, H, I, h, qd, sd, nthreads);
    for (int64_t i = 0; i < (int64_t)M * H; ++i)
      y_out[i] = orc_bf16_round((float)((double)s_d * sd[i]));
  }
  free(x);
  free(h);
  free(su);
  free(sg);
  free(sd);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Attention input: fused QKV projection, split and rotary embedding.        */
/* FlashRT architecture doc, "Kernel library" ("qkv split + RoPE" fusion);  */
/* itsolotime article section 5.2 (FusedQKV: the q, k and v projections of  */
/* a layer fused into one quantised weight, optionally with the norm weight */
/* folded in).  The rotation is the half-split form: dimension i of a head  */
/* is paired with dimension i + hd/2.                                        */
/*                                                                          */
/* Rotary table, entry (p, i) for i < hd/2:                                 */
/*   theta_i = base^(-2i/hd),  cos/sin of p * theta_i in fp64, each rounded */
/*   once to fp32; stored as [P][hd/2][2] = (cos, sin).                     */
/* ------------------------------------------------------------------------ */

void orc_rope_table(int P, int hd, double base, float *cos_sin) {
  const int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    const double theta = pow(base, -(2.0 * (double)i) / (double)hd);
    for (int p = 0; p < P; ++p) {
      const double a = (double)p * theta;
      cos_sin[((int64_t)p * half + i) * 2] = (float)cos(a);
      cos_sin[((int64_t)p * half + i) * 2 + 1] = (float)sin(a);
    }
  }
}

/* Split and rotate one row block.  A is the fp32 GEMM result [M][N] with  */
/* N = (nq + 2*nkv) * hd over the fused rows [q heads; k heads; v heads].  */
/*   v_n = f32(A[m][n] * alpha)                                            */
/* Q and K heads, d < hd/2, (c, s) = table[pos[m]][d]:                     */
/*   out[d]        = bf16( f32( f32(v_d * c) - f32(v_{d+hd/2} * s) ) )      */
/*   out[d + hd/2] = bf16( f32( f32(v_{d+hd/2} * c) + f32(v_d * s) ) )      */
/* V heads: out = bf16(v).  Outputs [M][heads][hd].  Returns -1 when a     */
/* position lies outside the table.                                        */
int orc_qkv_epilogue(int M, int nq, int nkv, int hd, const float *A, float alpha, const int32_t *pos,
                     const float *table, int P, uint16_t *q, uint16_t *k, uint16_t *v) {
  const int half = hd / 2;
  const int64_t N = (int64_t)(nq + 2 * nkv) * hd;
  for (int m = 0; m < M; ++m) {
    const int p = pos[m];
    if (p < 0 || p >= P) return -1;
    for (int head = 0; head < nq + nkv; ++head) {
      const float *a = A + (int64_t)m * N + (int64_t)head * hd;
      uint16_t *o = head < nq ? q + ((int64_t)m * nq + head) * hd : k + ((int64_t)m * nkv + (head - nq)) * hd;
      for (int d = 0; d < half; ++d) {
        const float x1 = a[d] * alpha;
        const float x2 = a[d + half] * alpha;
        const float c = table[((int64_t)p * half + d) * 2];
        const float sn = table[((int64_t)p * half + d) * 2 + 1];
        const float x1c = x1 * c, x2s = x2 * sn, x2c = x2 * c, x1s = x1 * sn;
        o[d] = orc_bf16_round(x1c - x2s);
        o[d + half] = orc_bf16_round(x2c + x1s);
      }
    }
    const float *av = A + (int64_t)m * N + (int64_t)(nq + nkv) * hd;
    for (int64_t j = 0; j < (int64_t)nkv * hd; ++j) v[(int64_t)m * nkv * hd + j] = orc_bf16_round(av[j] * alpha);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* MXFP4: the 4-bit FFN variant (itsolotime article section 7.2 describes   */
/* the NVFP4 form: AWQ pre-scale, low-bit gate/up and down GEMMs, a gated   */
/* combine that re-quantises to 4 bits, a high-precision residual).  The    */
/* format is OCP Microscaling MXFP4: blocks of 32 consecutive values along  */
/* the reduction dimension share one E8M0 scale X = 2^(e - 127); elements   */
/* are FP4 E2M1 (sign bit 3; exponent bits 2..1, bias 1; mantissa bit 0):   */
/* magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.                                    */
/*   e = floor(log2(amax)) - 2 + 127, clamped to [0, 254]; amax = 0: e = 0   */
/*   element = e2m1(v / X), round to nearest, ties to the even mantissa,     */
/*   saturating at +-6; the sign bit follows v (so -0 is kept).              */
/* Packing: element 2i in the low nibble of byte i, 2i+1 in the high one.   */
/* ------------------------------------------------------------------------ */

double orc_e2m1_decode(uint8_t c) {
  const int e = (c >> 1) & 3, m = c & 1;
  const double v = e ? ldexp(1.0 + 0.5 * m, e - 1) : 0.5 * m;
  return (c & 8) ? -v : v;
}

/* nearest of the eight magnitudes, ties to the code with mantissa bit 0;
   from 6 up (where distances to the grid would round together for huge
   inputs) the largest magnitude */
uint8_t orc_e2m1_encode(double v) {
  const double a = fabs(v);
  int best = 7;
  double bd = INFINITY;
  for (int c = 0; c < 8 && a < 6.0; ++c) {
    const double d = fabs(orc_e2m1_decode((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)(best | (signbit(v) ? 8 : 0));
}

int orc_mx_scale_exp(double amax) {
  if (!(amax > 0.0)) return 0;
  int ex;
  (void)frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2(amax)) = ex - 1 */
  int e = (ex - 1) - 2 + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

/* v [rows][cols] (cols % 32 == 0) -> codes [rows][cols/2], scales [rows][cols/32] */
void orc_mxfp4_quant_rows(const float *v, int64_t rows, int64_t cols, uint8_t *codes, uint8_t *scales) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < cols / 32; ++b) {
      const float *blk = v + r * cols + b * 32;
      double amax = 0.0;
      for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs((double)blk[j]));
      const int e = orc_mx_scale_exp(amax);
      scales[r * (cols / 32) + b] = (uint8_t)e;
      for (int j = 0; j < 32; j += 2) {
        const uint8_t lo = orc_e2m1_encode(ldexp((double)blk[j], 127 - e));
        const uint8_t hi = orc_e2m1_encode(ldexp((double)blk[j + 1], 127 - e));
        codes[r * (cols / 2) + b * 16 + j / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

/* Weights: bf16 w [rows][cols] times the bf16 column factor colw[k] (the AWQ */
/* scale; NULL = 1), an exact product, then MXFP4 along cols (rows in        */
/* parallel: each is independent).                                           */
typedef struct {
  const uint16_t *w, *colw;
  int64_t cols;
  uint8_t *codes, *scales;
  int err;
} mxq_ctx;

static void mxq_range(void *p, int64_t begin, int64_t end) {
  mxq_ctx *c = (mxq_ctx *)p;
  float *tmp = (float *)malloc(sizeof(float) * (size_t)c->cols);
  if (!tmp) {
    c->err = 1;
    return;
  }
  for (int64_t r = begin; r < end; ++r) {
    for (int64_t k = 0; k < c->cols; ++k)
      tmp[k] = orc_bf16_to_f32(c->w[r * c->cols + k]) * (c->colw ? orc_bf16_to_f32(c->colw[k]) : 1.0f);
    orc_mxfp4_quant_rows(tmp, 1, c->cols, c->codes + r * (c->cols / 2), c->scales + r * (c->cols / 32));
  }
  free(tmp);
}

int orc_mxfp4_quant_weight(const uint16_t *w, int64_t rows, int64_t cols, const uint16_t *colw, uint8_t *codes,
                           uint8_t *scales, int nthreads) {
  mxq_ctx c = {w, colw, cols, codes, scales, 0};
  parallel_for(rows, nthreads, mxq_range, &c);
  return c.err ? -2 : 0;
}

/* round v * 2^e (v a 128-bit integer) once to fp32, ties to even */
static float i128_to_f32(__int128 v, int e) {
  if (v == 0) return 0.0f;
  const int neg = v < 0;
  unsigned __int128 mag = neg ? (unsigned __int128)(-v) : (unsigned __int128)v;
  int nbits = 0;
  for (unsigned __int128 t = mag; t; t >>= 1) ++nbits;
  if (nbits > 24) {
    const int sh = nbits - 24;
    unsigned __int128 q = mag >> sh;
    const unsigned __int128 rem = mag & ((((unsigned __int128)1) << sh) - 1);
    const unsigned __int128 half = ((unsigned __int128)1) << (sh - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    mag = q;
    e += sh;
  }
  const double r = ldexp((double)(uint64_t)mag, e); /* < 2^25 * 2^e: exact in double */
  return (float)(neg ? -r : r);                      /* exact: at most 24 significant bits */
}

typedef struct {
  int M, N, K;
  const uint8_t *ac, *as, *bc, *bs;
  float *out;
  int err;
  int twice[16]; /* 2 * decode(code): an integer in [-12, 12] */
} mxgemm_ctx;

static void mxgemm_range(void *p, int64_t begin, int64_t end) {
  mxgemm_ctx *g = (mxgemm_ctx *)p;
  const int nb = g->K / 32;
  for (int64_t idx = begin; idx < end; ++idx) {
    const int m = (int)(idx / g->N), n = (int)(idx % g->N);
    int emin = 1 << 30, emax = -(1 << 30);
    for (int b = 0; b < nb; ++b) {
      const int e = (int)g->as[(int64_t)m * nb + b] + (int)g->bs[(int64_t)n * nb + b];
      if (e < emin) emin = e;
      if (e > emax) emax = e;
    }
    if (emax - emin > 100) {
      g->err = 1;
      g->out[idx] = NAN;
      continue;
    }
    __int128 acc = 0;
    for (int b = 0; b < nb; ++b) {
      long S = 0;
      for (int j = 0; j < 32; ++j) {
        const int k = b * 32 + j;
        const uint8_t ca = (g->ac[(int64_t)m * (g->K / 2) + k / 2] >> (4 * (k & 1))) & 15;
        const uint8_t cb = (g->bc[(int64_t)n * (g->K / 2) + k / 2] >> (4 * (k & 1))) & 15;
        S += (long)g->twice[ca] * (long)g->twice[cb];
      }
      const int e = (int)g->as[(int64_t)m * nb + b] + (int)g->bs[(int64_t)n * nb + b];
      acc += ((__int128)S) << (e - emin);
    }
    /* each product is (2a)(2b)/4 * 2^(ea-127) * 2^(eb-127) */
    g->out[idx] = i128_to_f32(acc, emin - 254 - 2);
  }
}

/* out [M][N] = f32( exact sum_k A[m][k] B[n][k] ) for MXFP4 operands with   */
/* K along the rows of both.  -1 when a row's scale exponents spread too far */
/* for the 128-bit accumulator (never for the workloads here).               */
int orc_mxfp4_gemm(int M, int N, int K, const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                   const uint8_t *b_scales, float *out, int nthreads) {
  if (K % 32) return -1;
  mxgemm_ctx g = {M, N, K, a_codes, a_scales, b_codes, b_scales, out, 0, {0}};
  for (int c = 0; c < 16; ++c) g.twice[c] = (int)lrint(2.0 * orc_e2m1_decode((uint8_t)c));
  parallel_for((int64_t)M * N, nthreads, mxgemm_range, &g);
  return g.err ? -1 : 0;
}

/* One MXFP4 block:                                                          */
/*   r' = bf16(r + y); x = RMSNorm (or AdaRMSNorm) as in the FP8 block;     */
/*   xs = f32(x * inv_awq[k]) (inv_awq NULL: xs = x);  XQ = MXFP4(xs)        */
/*   g, u = f32(exact MXFP4 dot products);  h = f32(act(g) * u) (or         */
/*   gelu_tanh(u));  HQ = MXFP4(h) along I;  y = bf16(f32(exact down sum))  */
int orc_block_mxfp4(int M, int H, int I, int act, float eps, const uint16_t *r_prev, const uint16_t *y_prev,
                    const uint16_t *w_norm, const uint16_t *mod_scale, const uint16_t *mod_shift,
                    const float *inv_awq, const uint8_t *gc, const uint8_t *gs, const uint8_t *uc, const uint8_t *us,
                    const uint8_t *dc, const uint8_t *ds, uint16_t *r_out, uint8_t *xq_codes, uint8_t *xq_scales,
                    uint8_t *hq_codes, uint8_t *hq_scales, uint16_t *y_out, int nthreads) {
  int rc = -2;
  float *x = (float *)malloc(sizeof(float) * (size_t)M * H);
  float *Ag = (float *)malloc(sizeof(float) * (size_t)M * I);
  float *Au = (float *)malloc(sizeof(float) * (size_t)M * I);
  float *h = (float *)malloc(sizeof(float) * (size_t)M * I);
  float *Ad = (float *)malloc(sizeof(float) * (size_t)M * H);
  if (!x || !Ag || !Au || !h || !Ad) goto done;
  orc_add_rmsnorm_quant(M, H, r_prev, y_prev, w_norm, mod_scale, mod_shift, eps, 1.0f, r_out, x, NULL, nthreads);
  if (inv_awq)
    for (int64_t i = 0; i < (int64_t)M * H; ++i) x[i] = x[i] * inv_awq[i % H];
  orc_mxfp4_quant_rows(x, M, H, xq_codes, xq_scales);
  rc = -1;
  if (act != ORC_ACT_GELU_TANH && orc_mxfp4_gemm(M, I, H, xq_codes, xq_scales, gc, gs, Ag, nthreads)) goto done;
  if (orc_mxfp4_gemm(M, I, H, xq_codes, xq_scales, uc, us, Au, nthreads)) goto done;
  orc_gateup_epilogue((int64_t)M * I, act, Ag, Au, 1.0f, 1.0f, 1.0f, h, NULL);
  orc_mxfp4_quant_rows(h, M, I, hq_codes, hq_scales);
  if (orc_mxfp4_gemm(M, H, I, hq_codes, hq_scales, dc, ds, Ad, nthreads)) goto done;
  for (int64_t i = 0; i < (int64_t)M * H; ++i) y_out[i] = orc_bf16_round(Ad[i]);
  rc = 0;
done:
  free(x);
  free(Ag);
  free(Au);
  free(h);
  free(Ad);
  return rc;
}
