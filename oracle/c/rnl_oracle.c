/*
 * rnl_oracle.c -- plain, slow CPU oracle of the fused RMSNorm -> Linear
 * projection, in C.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, by the smoke check and by the
 * cpu_baseline leg of the benchmark (through oracle/c_oracle.py); never by the
 * product path.  It shares no code, header or table with the HIP library.
 *
 * Pages this follows (cited by title and section):
 *   AT-10 page -- "PyPTO-Gym operator design pattern AT-10: RMSNorm + Linear
 *     fused (V->C layout), principle and MLAProlog practice": section 2 (the
 *     compute flow), section 3 (RMSNorm variants A "rsqrt" and B "sqrt + div",
 *     the MLA rms_norm code), section 4 (AT-09 BF16 / INT8 W8A8 / MXFP8 modes,
 *     AT-05 quant, AT-06 dequant), section 5 (MLAProlog), section 6 (the
 *     pre-attention operator: residual add, per-head norm, RoPE), section 9
 *     (the golden reference divides by the root).
 *   SK-03 page -- "SK-03 Linear Projection (Norm->MatMul)": the quant variant
 *     and the mhc_pre variant (very long reduction, FP32 compute).
 *   SK-14 page -- "SK-14 General Multi-MatMul skeleton": the
 *     QuantMatMulReduceSum dequant order; the MXFP8 layout (E4M3FN data, E8M0
 *     scale per 64 elements).
 *   Patterns page -- "PyPTO common coding patterns": section 9.17 (eps inside
 *     the root), section 9.18 point 5 (a transposed second operand).
 *
 * Arithmetic.  Built with gcc -O2 -ffp-contract=off and no fast-math: every
 * float operation below is one IEEE binary32 operation rounded to nearest
 * even, and no multiply is fused with an add.  Sums the pages leave open are
 * accumulated in double in index order and rounded once.  Products of bf16,
 * fp32 and E4M3 values are exact in double.  The integer product accumulates
 * in int64.  Every choice the pages leave open is the reading stated beside
 * it (READING).
 *
 * Every entry point works on whole rows; rows are independent, so each one
 * splits its rows over `threads` POSIX threads (threads <= 1: the caller's
 * thread only).  Splitting changes nothing in the arithmetic of a row.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------- */
/* Rows over threads                                                          */
/* ------------------------------------------------------------------------- */
typedef void (*row_fn)(void* ctx, int64_t t);

struct span {
  row_fn fn;
  void* ctx;
  int64_t t0, t1;
};

static void* run_span(void* p) {
  struct span* s = (struct span*)p;
  for (int64_t t = s->t0; t < s->t1; ++t) s->fn(s->ctx, t);
  return NULL;
}

/* Calls fn(ctx, t) once for every t in [0, T), rows split over the threads
 * (a thread that cannot be started has its rows run by the caller). */
static void for_rows(int64_t T, int threads, row_fn fn, void* ctx) {
  if (threads > T) threads = (int)T;
  if (threads <= 1) {
    for (int64_t t = 0; t < T; ++t) fn(ctx, t);
    return;
  }
  struct span* spans = (struct span*)calloc((size_t)threads, sizeof(struct span));
  pthread_t* tid = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
  char* started = (char*)calloc((size_t)threads, 1);
  for (int i = 0; i < threads; ++i) {
    spans[i].fn = fn;
    spans[i].ctx = ctx;
    spans[i].t0 = T * i / threads;
    spans[i].t1 = T * (i + 1) / threads;
  }
  for (int i = 1; i < threads; ++i) started[i] = pthread_create(&tid[i], NULL, run_span, &spans[i]) == 0;
  run_span(&spans[0]);
  for (int i = 1; i < threads; ++i) {
    if (started[i]) pthread_join(tid[i], NULL);
    else run_span(&spans[i]);
  }
  free(started);
  free(tid);
  free(spans);
}

int orc_cpu_count(void) { return (int)sysconf(_SC_NPROCESSORS_ONLN); }

/* ------------------------------------------------------------------------- */
/* bf16                                                                       */
/* ------------------------------------------------------------------------- */
/* bf16 holds the top 16 bits of a binary32: widening is exact. */
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* READING (AT-10 page section 2 casts the normed values to BF16, rounding
 * unstated): round to nearest, ties to even, on the 16 dropped bits; a NaN
 * stays a quiet NaN. */
static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) return (uint16_t)((u >> 16) | 0x0040u);
  const uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)(((uint64_t)u + 0x7FFFu + lsb) >> 16);
}

static float bf16_round(float f) { return bf16_to_f32(f32_to_bf16(f)); }

void orc_f32_to_bf16(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(x[i]);
}

void orc_bf16_to_f32(const uint16_t* x, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(x[i]);
}

/* ------------------------------------------------------------------------- */
/* RMSNorm (AT-03 as AT-10 uses it, section 3)                                */
/* ------------------------------------------------------------------------- */
/* ms = fl( fl(sum_k xf^2) * fl(1/K) ).  READING: the pages ask for fp32
 * reductions but give no order; the squares (exact in double) are summed in
 * double in k order and the sum is rounded to float once. */
static float mean_square(const uint16_t* x, int64_t K) {
  double S = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const double v = (double)bf16_to_f32(x[k]);
    S += v * v;
  }
  const float c = 1.0f / (float)K;
  return (float)S * c;
}

/* variant B: rstd = fl(1 / fl(sqrt(fl(ms + eps)))) -- eps added to the mean
 * square before the root (patterns page 9.17). */
static float rstd_b(float ms, float eps) {
  const float var = ms + eps;
  const float sd = sqrtf(var);
  return 1.0f / sd;
}

/* variant A: rsqrt(fl(ms + eps)); the hardware rsqrt has its own error, so
 * the ideal value is taken: 1/sqrt in double, rounded once. */
static float rstd_a(float ms, float eps) {
  const float var = ms + eps;
  return (float)(1.0 / sqrt((double)var));
}

struct norm_ctx {
  const uint16_t* x;
  const uint16_t* gamma;
  float eps;
  int64_t K;
  const float* rstd_in; /* when not NULL: use it (for instance the device's) */
  float* n;
  float* rstd;
  int variant; /* 0: B, 1: A */
};

static void norm_row(void* p, int64_t t) {
  struct norm_ctx* c = (struct norm_ctx*)p;
  const uint16_t* x = c->x + t * c->K;
  float r;
  if (c->rstd_in != NULL) r = c->rstd_in[t];
  else r = c->variant == 1 ? rstd_a(mean_square(x, c->K), c->eps) : rstd_b(mean_square(x, c->K), c->eps);
  c->rstd[t] = r;
  float* n = c->n + t * c->K;
  for (int64_t k = 0; k < c->K; ++k) {
    float v = bf16_to_f32(x[k]) * r;
    if (c->gamma != NULL) v = v * bf16_to_f32(c->gamma[k]); /* (x * rstd) * gamma: two roundings */
    n[k] = v;
  }
}

/* n[T,K] = fl(fl(xf * rstd) * gamma) (gamma optional), rstd[T]. */
void orc_rms_norm_rows(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T, int64_t K,
                       const float* rstd_in, int variant, float* n, float* rstd, int threads) {
  struct norm_ctx c = {x, gamma, eps, K, rstd_in, n, rstd, variant};
  for_rows(T, threads, norm_row, &c);
}

/* The ordering of the MLA rms_norm code (section 3): each square times 1/D,
 * then the sum (double, k order, one rounding); no gamma. */
void orc_rms_norm_rows_mla_order(const uint16_t* x, float eps, int64_t T, int64_t K, float* n, float* rstd) {
  const float c = 1.0f / (float)K;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * K;
    double S = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const float v = bf16_to_f32(xr[k]);
      const float sq = v * v;
      S += (double)(sq * c);
    }
    const float r = rstd_b((float)S, eps);
    rstd[t] = r;
    for (int64_t k = 0; k < K; ++k) n[t * K + k] = bf16_to_f32(xr[k]) * r;
  }
}

/* The golden reference form of section 9: x / sqrt(ms + eps). */
void orc_rms_norm_rows_golden_div(const uint16_t* x, float eps, int64_t T, int64_t K, float* n) {
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + t * K;
    const float var = mean_square(xr, K) + eps;
    const float sd = sqrtf(var);
    for (int64_t k = 0; k < K; ++k) n[t * K + k] = bf16_to_f32(xr[k]) / sd;
  }
}

/* ------------------------------------------------------------------------- */
/* Projections (AT-09, AT-10 page sections 2 and 4)                           */
/* ------------------------------------------------------------------------- */
struct proj_ctx {
  const float* a;     /* [T, K] fp32 rows (already bf16-valued for the bf16 mode) */
  const uint16_t* wb; /* [N, K] bf16 weight, or */
  const float* wf;    /* [N, K] fp32 weight */
  int64_t K, N;
  float* y;
};

/* y[t, j] = fl( sum_k a[t,k] * W[j,k] ) with the products exact in double,
 * summed in double in k order: W's rows are the output columns (b_trans). */
static void proj_row(void* p, int64_t t) {
  struct proj_ctx* c = (struct proj_ctx*)p;
  const float* a = c->a + t * c->K;
  for (int64_t j = 0; j < c->N; ++j) {
    double acc = 0.0;
    if (c->wb != NULL) {
      const uint16_t* w = c->wb + j * c->K;
      for (int64_t k = 0; k < c->K; ++k) acc += (double)a[k] * (double)bf16_to_f32(w[k]);
    } else {
      const float* w = c->wf + j * c->K;
      for (int64_t k = 0; k < c->K; ++k) acc += (double)a[k] * (double)w[k];
    }
    c->y[t * c->N + j] = (float)acc;
  }
}

/* BF16 mode: the fp32 normed rows are cast to bf16 (RNE), then multiplied by
 * the bf16 weight [N, K]; READING: fp32-or-wider accumulation with one final
 * rounding (here: double, rounded once to float). */
void orc_project_bf16(const float* n, const uint16_t* W, int64_t T, int64_t K, int64_t N, float* y, int threads) {
  float* a = (float*)malloc((size_t)(T * K) * sizeof(float));
  for (int64_t i = 0; i < T * K; ++i) a[i] = bf16_round(n[i]);
  struct proj_ctx c = {a, W, NULL, K, N, y};
  for_rows(T, threads, proj_row, &c);
  free(a);
}

/* FP32 compute of the mhc_pre variant (SK-03 page): no bf16 cast, fp32
 * weight [N, K]; fp32 x fp32 products are exact in double. */
void orc_project_fp32(const float* n, const float* W, int64_t T, int64_t K, int64_t N, float* y, int threads) {
  struct proj_ctx c = {n, NULL, W, K, N, y};
  for_rows(T, threads, proj_row, &c);
}

/* ------------------------------------------------------------------------- */
/* INT8 W8A8 (AT-09 INT8 mode, AT-05, AT-06)                                  */
/* ------------------------------------------------------------------------- */
/* q = saturate_+-127(rint(fl(n * s))).  READING (SK-03 quant variant: cast
 * with RINT, ROUND, then TRUNC with saturation): one round to the nearest
 * integer, ties to even (rintf under the default rounding mode), then the
 * symmetric clamp; the later casts leave an in-range integer unchanged. */
static int8_t quant1(float n, float s) {
  float r = rintf(n * s);
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

/* Per-token symmetric quant: amax = max |n|; s = fl(127 / amax) (AT-10 page
 * section 4); x_scale = fl(amax / 127) (SK-03 page: max/127 is the dequant
 * scale).  READING for an all-zero row: s = 0, q = 0, x_scale = 0. */
void orc_quant_rows(const float* n, int64_t T, int64_t K, int8_t* q, float* x_scale, float* s_out) {
  for (int64_t t = 0; t < T; ++t) {
    const float* r = n + t * K;
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      const float a = fabsf(r[k]);
      if (a > amax) amax = a;
    }
    const float s = amax == 0.0f ? 0.0f : 127.0f / amax;
    for (int64_t k = 0; k < K; ++k) q[t * K + k] = quant1(r[k], s);
    x_scale[t] = amax / 127.0f;
    if (s_out != NULL) s_out[t] = s;
  }
}

void orc_quant_values(const float* n, const float* s, int64_t T, int64_t K, int8_t* q) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t k = 0; k < K; ++k) q[t * K + k] = quant1(n[t * K + k], s[t]);
}

struct i8_ctx {
  const int8_t* q;
  const int8_t* w;
  int64_t K, N;
  int64_t* acc;
};

static void i8_row(void* p, int64_t t) {
  struct i8_ctx* c = (struct i8_ctx*)p;
  const int8_t* a = c->q + t * c->K;
  for (int64_t j = 0; j < c->N; ++j) {
    const int8_t* w = c->w + j * c->K;
    int64_t s = 0;
    for (int64_t k = 0; k < c->K; ++k) s += (int64_t)a[k] * (int64_t)w[k];
    c->acc[t * c->N + j] = s;
  }
}

/* acc[t, j] = sum_k q[t,k] * Wq[j,k] in int64 (INT8 mode: int8 x int8 ->
 * INT32 with b_trans).  Returns 1 when a sum does not fit int32. */
int orc_int8_gemm(const int8_t* q, const int8_t* W, int64_t T, int64_t K, int64_t N, int64_t* acc, int threads) {
  struct i8_ctx c = {q, W, K, N, acc};
  for_rows(T, threads, i8_row, &c);
  for (int64_t i = 0; i < T * N; ++i)
    if (acc[i] > 2147483647LL || acc[i] < -2147483648LL) return 1;
  return 0;
}

/* AT-06 in the order of the SK-14 page's QuantMatMulReduceSum: cast the
 * accumulator to float (nearest even), form x_scale * w_scale, multiply. */
void orc_dequant(const int64_t* acc, const float* x_scale, const float* w_scale, int64_t T, int64_t N, float* y) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < N; ++j) {
      const float a = (float)acc[t * N + j];
      const float sm = x_scale[t] * w_scale[j];
      y[t * N + j] = a * sm;
    }
}

/* ------------------------------------------------------------------------- */
/* Residual add (AT-10 page section 6)                                        */
/* ------------------------------------------------------------------------- */
/* READING: the two bf16 values are added in float (one rounding) and the sum
 * is rounded to bf16 (nearest even): the tensor the norm reads and the new
 * residual stream. */
void orc_add_residual(const uint16_t* x, const uint16_t* r, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(bf16_to_f32(x[i]) + bf16_to_f32(r[i]));
}

/* ------------------------------------------------------------------------- */
/* Per-head norm + RoPE (AT-10 page section 6)                                */
/* ------------------------------------------------------------------------- */
/* Rotate-half RoPE of one normed head of D values with the angles of its
 * token (c, s of D/2 pairs).  READING (RoPE is named, not defined): element i
 * turns with element i + D/2, in float, every product and sum rounded once:
 *   out[i]       = fl( fl(n[i] c) - fl(n[i+D/2] s) )
 *   out[i + D/2] = fl( fl(n[i+D/2] c) + fl(n[i] s) ) */
static void rope_half(float* n, int64_t D, const float* c, const float* s) {
  const int64_t h = D / 2;
  for (int64_t i = 0; i < h; ++i) {
    const float lo = n[i], hi = n[i + h];
    const float a = lo * c[i], b = hi * s[i];
    const float e = hi * c[i], f = lo * s[i];
    n[i] = a - b;
    n[i + h] = e + f;
  }
}

void orc_rope_rotate_half(const float* n, int64_t R, int64_t D, const float* cos_t, const float* sin_t, float* out) {
  for (int64_t r = 0; r < R; ++r) {
    memcpy(out + r * D, n + r * D, (size_t)D * sizeof(float));
    rope_half(out + r * D, D, cos_t + r * (D / 2), sin_t + r * (D / 2));
  }
}

/* Heads h of D columns from column col0 of y [T, ld] (bf16): each head is one
 * AT-03 row of D values (gamma [D] shared by the heads, variant B rstd), then
 * RoPE when cos/sin [T, D/2] are given, then rounded to bf16 into out (which
 * holds y's values elsewhere).  rstd [T, H]. */
void orc_head_rms_norm(const uint16_t* y, int64_t T, int64_t ld, int64_t col0, int64_t H, int64_t D,
                       const uint16_t* gamma, float eps, const float* cos_t, const float* sin_t, const float* rstd_in,
                       uint16_t* out, float* rstd) {
  float* n = (float*)malloc((size_t)D * sizeof(float));
  memcpy(out, y, (size_t)(T * ld) * sizeof(uint16_t));
  for (int64_t t = 0; t < T; ++t)
    for (int64_t h = 0; h < H; ++h) {
      const uint16_t* x = y + t * ld + col0 + h * D;
      const float r = rstd_in != NULL ? rstd_in[t * H + h] : rstd_b(mean_square(x, D), eps);
      rstd[t * H + h] = r;
      for (int64_t k = 0; k < D; ++k) {
        float v = bf16_to_f32(x[k]) * r;
        if (gamma != NULL) v = v * bf16_to_f32(gamma[k]);
        n[k] = v;
      }
      if (cos_t != NULL) rope_half(n, D, cos_t + t * (D / 2), sin_t + t * (D / 2));
      for (int64_t k = 0; k < D; ++k) out[t * ld + col0 + h * D + k] = f32_to_bf16(n[k]);
    }
  free(n);
}

/* ------------------------------------------------------------------------- */
/* MXFP8 (AT-09 MXFP8 mode; E4M3FN data, E8M0 scale per 64 -- SK-14 page)     */
/* ------------------------------------------------------------------------- */
/* E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities;
 * exponent field 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN. */
static double e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 0xF, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return (c & 0x80) ? -mag : mag;
}

void orc_e4m3_decode(const uint8_t* c, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)e4m3_value(c[i]);
}

/* E8M0 scale: 2^(code - 127); code 255 is NaN. */
void orc_e8m0_decode(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = c[i] == 255 ? NAN : ldexp(1.0, (int)c[i] - 127);
}

/* READING (the pages fix the format, not the conversion): the OCP MX rule --
 * the nearest E4M3 value, ties to the even mantissa; magnitudes past the
 * largest normal 448 clamp to it; a value that rounds to zero is +0. */
static uint8_t e4m3_of(double v) {
  const double a = fabs(v);
  if (a == 0.0) return 0;
  int E;
  frexp(a, &E);           /* a = f 2^E, f in [0.5, 1): floor(log2 a) = E - 1 */
  int q = E - 1;          /* exponent of a */
  if (q < -6) q = -6;     /* below the normals the spacing stays 2^-9 */
  q -= 3;                 /* three mantissa bits: spacing 2^(exponent - 3) */
  double r = nearbyint(ldexp(a, -q)); /* nearest even multiple of the spacing */
  r = ldexp(r, q);
  if (r > 448.0) r = 448.0;
  if (r == 0.0) return 0;
  uint8_t code;
  if (r >= ldexp(1.0, -6)) {
    int E2;
    frexp(r, &E2);
    const int e = E2 - 1;
    const int m = (int)(ldexp(r, -e) * 8.0 - 8.0);
    code = (uint8_t)(((e + 7) << 3) | m);
  } else {
    code = (uint8_t)(int)(ldexp(r, 9));
  }
  return (uint8_t)(code | (v < 0 ? 0x80 : 0));
}

void orc_e4m3_encode(const double* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_of(v[i]);
}

/* MX quant of fp32 rows n [T, K], K a multiple of 64.  READING (how the
 * activations get their scale is not stated): the OCP MX rule -- per block,
 * X = 2^(floor(log2 amax) - 8), 8 the largest E4M3 exponent, clamped to
 * E8M0's [-127, 127], -127 for an all-zero block; element = E4M3(n / X). */
void orc_mx_quant_rows(const float* n, int64_t T, int64_t K, uint8_t* codes, uint8_t* scales) {
  const int64_t nb = K / 64;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t b = 0; b < nb; ++b) {
      const float* v = n + t * K + b * 64;
      double amax = 0.0;
      for (int k = 0; k < 64; ++k)
        if (fabs((double)v[k]) > amax) amax = fabs((double)v[k]);
      int sh = -127;
      if (amax > 0.0) {
        int E;
        frexp(amax, &E);
        sh = E - 1 - 8;
      }
      if (sh < -127) sh = -127;
      if (sh > 127) sh = 127;
      for (int k = 0; k < 64; ++k) codes[t * K + b * 64 + k] = e4m3_of(ldexp((double)v[k], -sh));
      scales[t * nb + b] = (uint8_t)(sh + 127);
    }
}

/* One MX operand decoded: v[r, k] = E4M3(q[r, k]) * 2^(scale[r, k / 64] - 127)
 * in double, which holds it exactly (3-bit mantissas, power-of-two scales);
 * a NaN code or the NaN scale 255 gives NaN. */
static double* mx_decode_rows(const uint8_t* q, const uint8_t* sc, int64_t R, int64_t K) {
  const int64_t nb = K / 64;
  double* v = (double*)malloc((size_t)(R * K) * sizeof(double));
  for (int64_t r = 0; r < R; ++r)
    for (int64_t k = 0; k < K; ++k) {
      const uint8_t s = sc[r * nb + k / 64];
      v[r * K + k] = s == 255 ? NAN : ldexp(e4m3_value(q[r * K + k]), (int)s - 127);
    }
  return v;
}

struct mx_ctx {
  const double *x, *w; /* decoded operands [T, K], [N, K] */
  int64_t K, N;
  float* y;
};

/* y[t, n] = sum over 64-blocks b of Xx[t,b] Xw[n,b] sum_{k in b} x[t,k] w[n,k]
 * = sum_k (Xx x)[t,k] (Xw w)[n,k]: every scaled product is exact in double,
 * summed in double in k order and rounded once (the MXFP8 product accumulates
 * into FP32). */
static void mx_row(void* p, int64_t t) {
  struct mx_ctx* c = (struct mx_ctx*)p;
  const double* a = c->x + t * c->K;
  for (int64_t j = 0; j < c->N; ++j) {
    const double* w = c->w + j * c->K;
    double acc = 0.0;
    for (int64_t k = 0; k < c->K; ++k) acc += a[k] * w[k];
    c->y[t * c->N + j] = (float)acc;
  }
}

void orc_mx_scaled_mm(const uint8_t* qx, const uint8_t* sx, const uint8_t* qw, const uint8_t* sw, int64_t T, int64_t K,
                      int64_t N, float* y, int threads) {
  double* xd = mx_decode_rows(qx, sx, T, K);
  double* wd = mx_decode_rows(qw, sw, N, K);
  struct mx_ctx c = {xd, wd, K, N, y};
  for_rows(T, threads, mx_row, &c);
  free(wd);
  free(xd);
}
