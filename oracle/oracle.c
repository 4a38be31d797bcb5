/*
 * oracle.c -- plain, slow CPU reference of the MoE FFN layer. TEST INFRASTRUCTURE ONLY: used by
 * the tests, the smoke check and the benchmark's CPU-baseline leg, never by the GPU library.
 *
 * Each function restates one step from its definition, in double precision, with no blocking or
 * reordering beyond what that definition states. Decisions the method takes in fp32 (top-k on fp32
 * logits, quantiser codes) are taken here in fp32 as well. Build without fast-math and without
 * floating-point contraction so that every fp32 operation is a single IEEE operation.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------------------------------------- */
/* Number formats (OCP 8-bit FP spec for e4m3; OCP MX v1.0 for e2m1 and E8M0).                    */
/* ---------------------------------------------------------------------------------------------- */

/* e4m3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0. Exponent field 0 encodes
 * subnormals m * 2^-9. S.1111.111 is NaN; there are no infinities, so the largest value is 448. */
double oracle_e4m3_value(uint8_t code)
{
  int sign = code >> 7, ef = (code >> 3) & 15, m = code & 7;
  double v;
  if (ef == 15 && m == 7) return NAN;
  if (ef == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, ef - 7);
  return sign ? -v : v;
}

/* Round |v| to the nearest e4m3 value (ties to the even mantissa), saturating at 448; the sign bit
 * is copied from v (so tiny negative values give negative zero). */
uint8_t oracle_e4m3_encode(float v)
{
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7E;                 /* 1111.110 = 448 */
  if (a < ldexp(1.0, -6)) {                           /* subnormal range: steps of 2^-9 */
    double m = rint(a / ldexp(1.0, -9));              /* 0..8; 8 is the smallest normal 2^-6 */
    return sign | (uint8_t)m;                         /* m = 8 is exactly code 0001.000 */
  }
  int ex;
  frexp(a, &ex);                                      /* a = f * 2^ex, f in [0.5, 1) */
  int E = ex - 1;                                     /* a in [2^E, 2^(E+1)) */
  double m = rint(a / ldexp(1.0, E - 3));             /* 3 mantissa bits: m in [8, 16] */
  if (m == 16.0) { m = 8.0; E += 1; }
  /* a < 448 keeps E + 7 <= 15 with mantissa <= 6 at E = 8 */
  return sign | (uint8_t)(((E + 7) << 3) | ((int)m - 8));
}

/* e2m1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_value(uint8_t nib)
{
  int sign = (nib >> 3) & 1, ef = (nib >> 1) & 3, m = nib & 1;
  double v = (ef == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, ef - 1);
  return sign ? -v : v;
}

/* Nearest of the eight magnitudes, ties to the even code, saturating at 6; sign copied from v. */
uint8_t oracle_e2m1_encode(float v)
{
  uint8_t sign = signbit(v) ? 0x8 : 0x0;
  double a = fabs((double)v);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double d = fabs(a - oracle_e2m1_value((uint8_t)c));
    if (d < best_d || (d == best_d && (c & 1) == 0)) { best = c; best_d = d; }
  }
  return sign | (uint8_t)best;
}

/* bf16 keeps the top 16 bits of an fp32 value: 8 exponent bits and 7 mantissa bits. Rounding to
 * the nearest of the two bf16 neighbours of v, ties to the one with an even last mantissa bit. */
float oracle_bf16_round(float v)
{
  int ex;
  double a = fabs((double)v);
  if (a == 0.0) return v;
  frexp(a, &ex);                                      /* a in [2^(ex-1), 2^ex) */
  double step = ldexp(1.0, ex - 1 - 7);               /* spacing of bf16 values in this binade */
  if (ex - 1 < -126) step = ldexp(1.0, -126 - 7);     /* subnormal range: fixed spacing */
  double q = rint(a / step) * step;                   /* rint: nearest, ties to even multiple */
  return (float)(signbit(v) ? -q : q);
}

double oracle_e8m0_value(uint8_t code)
{
  if (code == 255) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* ---------------------------------------------------------------------------------------------- */
/* Quantisers                                                                                      */
/* ---------------------------------------------------------------------------------------------- */

void oracle_quant_fp8(int rows, int cols, int bn, int bk, const float* src, uint8_t* codes,
                      float* scales)
{
  int nbr = (rows + bn - 1) / bn, nbc = (cols + bk - 1) / bk;
#pragma omp parallel for collapse(2) schedule(static)
  for (int bi = 0; bi < nbr; ++bi)
    for (int bj = 0; bj < nbc; ++bj) {
      int r1 = (bi + 1) * bn < rows ? (bi + 1) * bn : rows;
      int c1 = (bj + 1) * bk < cols ? (bj + 1) * bk : cols;
      float amax = 0.0f;
      for (int r = bi * bn; r < r1; ++r)
        for (int c = bj * bk; c < c1; ++c) {
          float a = fabsf(src[(size_t)r * cols + c]);
          if (a > amax) amax = a;
        }
      float s = amax > 0.0f ? amax / 448.0f : 1.0f;   /* fp32 division */
      scales[(size_t)bi * nbc + bj] = s;
      for (int r = bi * bn; r < r1; ++r)
        for (int c = bj * bk; c < c1; ++c) {
          float q = src[(size_t)r * cols + c] / s;    /* fp32 division */
          codes[(size_t)r * cols + c] = oracle_e4m3_encode(q);
        }
    }
}

void oracle_quant_mx4(int rows, int cols, const float* src, uint8_t* packed, uint8_t* scales)
{
  int ng = cols / 32;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r)
    for (int g = 0; g < ng; ++g) {
      const float* v = src + (size_t)r * cols + (size_t)g * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i)
        if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
      int e;
      if (amax == 0.0f) {
        e = -127;
      } else {
        int ex;
        frexpf(amax, &ex);            /* floor(log2(amax)) = ex - 1 */
        e = (ex - 1) - 2;             /* largest e2m1 exponent is 2 */
        if (e < -127) e = -127;
        if (e > 127) e = 127;
      }
      scales[(size_t)r * ng + g] = (uint8_t)(e + 127);
      float mul = ldexpf(1.0f, -e);   /* exact power of two */
      uint8_t* out = packed + (size_t)r * (cols / 2) + (size_t)g * 16;
      for (int i = 0; i < 16; ++i) {
        uint8_t lo = oracle_e2m1_encode(v[2 * i] * mul);
        uint8_t hi = oracle_e2m1_encode(v[2 * i + 1] * mul);
        out[i] = (uint8_t)(lo | (hi << 4));
      }
    }
}

/* The MX shared exponent of one group: floor(log2(amax)) minus the element format's largest
 * exponent (2 for e2m1, 8 for e4m3), clamped to the E8M0 range; -127 for an all-zero group. */
static int mx_shared_exp(float amax, int emax_elem)
{
  if (amax == 0.0f) return -127;
  int ex;
  frexpf(amax, &ex);                  /* floor(log2(amax)) = ex - 1 */
  int e = (ex - 1) - emax_elem;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

void oracle_quant_mx8(int rows, int cols, const float* src, uint8_t* codes, uint8_t* scales)
{
  int ng = cols / 32;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r)
    for (int g = 0; g < ng; ++g) {
      const float* v = src + (size_t)r * cols + (size_t)g * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i)
        if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
      int e = mx_shared_exp(amax, 8);
      scales[(size_t)r * ng + g] = (uint8_t)(e + 127);
      float mul = ldexpf(1.0f, -e);   /* exact power of two */
      uint8_t* out = codes + (size_t)r * cols + (size_t)g * 32;
      for (int i = 0; i < 32; ++i) out[i] = oracle_e4m3_encode(v[i] * mul);
    }
}

/* NVFP4: two levels of scale. The row scale g maps the row's absolute maximum onto the largest
 * product of the two formats (6 * 448), so each 16-element block's own scale (its absolute maximum
 * over 6, relative to g) uses the full e4m3 range; elements are then e2m1 codes of v / (s * g). */
void oracle_quant_nv4(int rows, int cols, const float* src, uint8_t* packed, uint8_t* bscales,
                      float* rscales)
{
  int nb = cols / 16;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const float* row = src + (size_t)r * cols;
    float amax = 0.0f;
    for (int c = 0; c < cols; ++c)
      if (fabsf(row[c]) > amax) amax = fabsf(row[c]);
    float g = amax / 2688.0f;                          /* fp32 division */
    if (!(g > 0.0f)) g = 1.0f;                         /* amax = 0 (or below 2688 * 2^-149) */
    float d6 = 6.0f * g;                               /* fp32 product  */
    rscales[r] = g;
    for (int b = 0; b < nb; ++b) {
      const float* v = row + (size_t)b * 16;
      float bamax = 0.0f;
      for (int i = 0; i < 16; ++i)
        if (fabsf(v[i]) > bamax) bamax = fabsf(v[i]);
      uint8_t sc = oracle_e4m3_encode(bamax / d6);
      bscales[(size_t)r * nb + b] = sc;
      float d = (float)oracle_e4m3_value(sc) * g;      /* exact e4m3 value times g, fp32 product */
      uint8_t* out = packed + (size_t)r * (cols / 2) + (size_t)b * 8;
      for (int i = 0; i < 8; ++i) {
        uint8_t lo, hi;
        if (d == 0.0f) {
          lo = signbit(v[2 * i]) ? 0x8 : 0x0;
          hi = signbit(v[2 * i + 1]) ? 0x8 : 0x0;
        } else {
          lo = oracle_e2m1_encode(v[2 * i] / d);
          hi = oracle_e2m1_encode(v[2 * i + 1] / d);
        }
        out[i] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

double oracle_mat_at(const oracle_mat* m, int g, int n, int kk)
{
  size_t row = (size_t)g * m->N + n;
  switch (m->fmt) {
  case ORACLE_F32:
    return (double)((const float*)m->q)[row * m->K + kk];
  case ORACLE_FP8: {
    int nbn = (m->N + m->bn - 1) / m->bn, nbk = (m->K + m->bk - 1) / m->bk;
    uint8_t c = ((const uint8_t*)m->q)[row * m->K + kk];
    float s = ((const float*)m->s)[((size_t)g * nbn + n / m->bn) * nbk + kk / m->bk];
    return oracle_e4m3_value(c) * (double)s;
  }
  case ORACLE_MX4: {
    uint8_t b = ((const uint8_t*)m->q)[row * (m->K / 2) + kk / 2];
    uint8_t nib = (kk & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
    uint8_t sc = ((const uint8_t*)m->s)[row * (m->K / 32) + kk / 32];
    return oracle_e2m1_value(nib) * oracle_e8m0_value(sc);
  }
  case ORACLE_MX8: {
    uint8_t c = ((const uint8_t*)m->q)[row * m->K + kk];
    uint8_t sc = ((const uint8_t*)m->s)[row * (m->K / 32) + kk / 32];
    return oracle_e4m3_value(c) * oracle_e8m0_value(sc);
  }
  case ORACLE_NV4: {
    uint8_t b = ((const uint8_t*)m->q)[row * (m->K / 2) + kk / 2];
    uint8_t nib = (kk & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
    uint8_t sc = ((const uint8_t*)m->s)[row * (m->K / 16) + kk / 16];
    double gr = (double)((const float*)m->r)[row];
    return oracle_e2m1_value(nib) * oracle_e4m3_value(sc) * gr;   /* exact in double */
  }
  default:
    return NAN;
  }
}

void oracle_mat_dequant(const oracle_mat* m, double* out)
{
#pragma omp parallel for collapse(2) schedule(static)
  for (int g = 0; g < m->G; ++g)
    for (int n = 0; n < m->N; ++n)
      for (int kk = 0; kk < m->K; ++kk)
        out[((size_t)g * m->N + n) * m->K + kk] = oracle_mat_at(m, g, n, kk);
}

/* row n of matrix g as doubles */
static void mat_row(const oracle_mat* m, int g, int n, double* dst)
{
  if (m->fmt == ORACLE_F32) {
    const float* p = (const float*)m->q + ((size_t)g * m->N + n) * m->K;
    for (int kk = 0; kk < m->K; ++kk) dst[kk] = (double)p[kk];
  } else {
    for (int kk = 0; kk < m->K; ++kk) dst[kk] = oracle_mat_at(m, g, n, kk);
  }
}

/* ---------------------------------------------------------------------------------------------- */
/* Routing                                                                                         */
/* ---------------------------------------------------------------------------------------------- */

void oracle_logits(int T, int H, int E, const float* x, const float* w_r, const float* bias,
                   int n_tok, const int32_t* tok, double* logits, double* absdot)
{
  int n = tok ? n_tok : T;
#pragma omp parallel for collapse(2) schedule(static)
  for (int i = 0; i < n; ++i)
    for (int e = 0; e < E; ++e) {
      int t = tok ? tok[i] : i;
      double s = 0.0, a = 0.0;
      for (int h = 0; h < H; ++h) {
        double p = (double)x[(size_t)t * H + h] * (double)w_r[(size_t)e * H + h];
        s += p;
        a += fabs(p);
      }
      if (bias) { s += (double)bias[e]; a += fabs((double)bias[e]); }
      if (logits) logits[(size_t)i * E + e] = s;
      if (absdot) absdot[(size_t)i * E + e] = a;
    }
}

/* Gate of the shared expert for token t: one logit z = x_t . w_sg (double), then the logistic
 * function 1 / (1 + exp(-z)). */
static double shared_gate_row(int H, const float* x, const float* w_sg, int t)
{
  double z = 0.0;
  for (int h = 0; h < H; ++h) z += (double)x[(size_t)t * H + h] * (double)w_sg[h];
  return 1.0 / (1.0 + exp(-z));
}

void oracle_shared_gate(int T, int H, const float* x, const float* w_sg, int n_tok,
                        const int32_t* tok, double* g)
{
  int n = tok ? n_tok : T;
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i) g[i] = shared_gate_row(H, x, w_sg, tok ? tok[i] : i);
}

/* Selection of the k largest fp32 logits: repeatedly take the largest remaining value, the lowest
 * index among equal values (C comparison treats +0 and -0 as equal). This equals a full sort by
 * (value descending, index ascending) cut after k entries. */
static void topk_row(int E, int k, const float* L, int scoring, int renormalize, int32_t* ids,
                     double* w, char* taken)
{
  memset(taken, 0, (size_t)E);
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || L[e] > L[best]) best = e;
    }
    taken[best] = 1;
    ids[j] = best;
  }
  if (scoring == ORACLE_SOFTMAX) {
    /* softmax over all E experts, restricted to the chosen ones; with renormalisation this is
     * the softmax over the chosen logits alone */
    double mx = (double)L[ids[0]];
    double z = 0.0;
    if (renormalize) {
      for (int j = 0; j < k; ++j) z += exp((double)L[ids[j]] - mx);
    } else {
      for (int e = 0; e < E; ++e) z += exp((double)L[e] - mx);
    }
    for (int j = 0; j < k; ++j) w[j] = exp((double)L[ids[j]] - mx) / z;
  } else {
    double z = 0.0;
    for (int j = 0; j < k; ++j) {
      w[j] = 1.0 / (1.0 + exp(-(double)L[ids[j]]));
      z += w[j];
    }
    if (renormalize)
      for (int j = 0; j < k; ++j) w[j] /= z;
  }
}

void oracle_topk(int T, int E, int k, const float* logits, int scoring, int renormalize,
                 int32_t* ids, double* w)
{
#pragma omp parallel
  {
    char* taken = (char*)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t)
      topk_row(E, k, logits + (size_t)t * E, scoring, renormalize, ids + (size_t)t * k,
               w + (size_t)t * k, taken);
    free(taken);
  }
}

/* ---------------------------------------------------------------------------------------------- */
/* Dispatch: counts per expert, offsets, a unique row per local slot                              */
/* ---------------------------------------------------------------------------------------------- */

int oracle_permute(int T, int k, int e0, int E_loc, const int32_t* ids, int32_t* counts,
                   int32_t* offsets, int32_t* slot_to_row, int32_t* row_to_flat)
{
  for (int f = 0; f < T * k; ++f) slot_to_row[f] = -1;
  int r = 0;
  for (int el = 0; el < E_loc; ++el) {
    offsets[el] = r;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (ids[t * k + j] == e0 + el) {
          row_to_flat[r] = t * k + j;
          slot_to_row[t * k + j] = r;
          ++r;
        }
    counts[el] = r - offsets[el];
  }
  offsets[E_loc] = r;
  return r;
}

/* ---------------------------------------------------------------------------------------------- */
/* Expert FFN (SwiGLU) and the layer                                                               */
/* ---------------------------------------------------------------------------------------------- */

static void quantise_h(int act_fmt, int I, double* h)
{
  if (act_fmt == ORACLE_BF16 || act_fmt == ORACLE_NV4) {
    /* the down projection of a bf16 or NVFP4 layer reads h as a bf16 tensor (rounded from fp32) */
    for (int i = 0; i < I; ++i) h[i] = (double)oracle_bf16_round((float)h[i]);
  } else if (act_fmt == ORACLE_FP8) {
    /* 1 x 128 blocks along the intermediate dimension */
    for (int b = 0; b < I; b += 128) {
      int e = b + 128 < I ? b + 128 : I;
      float amax = 0.0f;
      for (int i = b; i < e; ++i) {
        float a = fabsf((float)h[i]);
        if (a > amax) amax = a;
      }
      float s = amax > 0.0f ? amax / 448.0f : 1.0f;
      for (int i = b; i < e; ++i)
        h[i] = oracle_e4m3_value(oracle_e4m3_encode((float)h[i] / s)) * (double)s;
    }
  } else if (act_fmt == ORACLE_MX4) {
    float* hf = (float*)calloc((size_t)I, sizeof(float));
    uint8_t* pk = (uint8_t*)malloc((size_t)I / 2);
    uint8_t* sc = (uint8_t*)malloc((size_t)I / 32);
    for (int i = 0; i < I; ++i) hf[i] = (float)h[i];
    oracle_quant_mx4(1, I, hf, pk, sc);
    oracle_mat m = {ORACLE_MX4, 1, 1, I, 0, 0, pk, sc, NULL};
    for (int i = 0; i < I; ++i) h[i] = oracle_mat_at(&m, 0, 0, i);
    free(hf); free(pk); free(sc);
  } else if (act_fmt == ORACLE_MX8) {
    /* 1 x 32 groups along the intermediate dimension, decisions on the fp32 value of h */
    float* hf = (float*)calloc((size_t)I, sizeof(float));
    uint8_t* cd = (uint8_t*)malloc((size_t)I);
    uint8_t* sc = (uint8_t*)malloc((size_t)I / 32);
    for (int i = 0; i < I; ++i) hf[i] = (float)h[i];
    oracle_quant_mx8(1, I, hf, cd, sc);
    oracle_mat m = {ORACLE_MX8, 1, 1, I, 0, 0, cd, sc, NULL};
    for (int i = 0; i < I; ++i) h[i] = oracle_mat_at(&m, 0, 0, i);
    free(hf); free(cd); free(sc);
  }
}

void oracle_ffn_row(const oracle_desc* d, int I, const double* a, const oracle_mat* gate,
                    const oracle_mat* up, const oracle_mat* down, int g, double* y)
{
  int H = d->H;
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  double* wrow = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
  for (int i = 0; i < I; ++i) {
    double gs = 0.0, us = 0.0;
    mat_row(gate, g, i, wrow);
    for (int c = 0; c < H; ++c) gs += a[c] * wrow[c];
    mat_row(up, g, i, wrow);
    for (int c = 0; c < H; ++c) us += a[c] * wrow[c];
    h[i] = gs / (1.0 + exp(-gs)) * us;          /* silu(g) * u */
  }
  quantise_h(d->act_fmt, I, h);
  for (int c = 0; c < H; ++c) {
    double s = 0.0;
    mat_row(down, g, c, wrow);
    for (int i = 0; i < I; ++i) s += h[i] * wrow[i];
    y[c] = s;
  }
  free(h);
  free(wrow);
}

/* out row o[H] of token t for a given routing (sel, wt of k slots): the weighted sum of the local
 * experts' FFN outputs in slot order, then the shared expert times its gate */
static void expert_sum(const oracle_desc* d, const float* x, const oracle_mat* xa,
                       const oracle_mat* gate, const oracle_mat* up, const oracle_mat* down,
                       const oracle_mat* sh_gate, const oracle_mat* sh_up,
                       const oracle_mat* sh_down, const float* w_sg, int t, const int32_t* sel,
                       const double* wt, double* a, double* y, double* o)
{
  int H = d->H;
  mat_row(xa, 0, t, a);
  for (int c = 0; c < H; ++c) o[c] = 0.0;
  for (int j = 0; j < d->k; ++j) {
    int el = sel[j] - d->e0;
    if (el < 0 || el >= d->E_loc) continue;   /* not on this GPU: contributes nothing here */
    oracle_ffn_row(d, d->I, a, gate, up, down, el, y);
    for (int c = 0; c < H; ++c) o[c] += wt[j] * y[c];
  }
  if (d->I_s > 0) {
    double gs = w_sg ? shared_gate_row(H, x, w_sg, t) : 1.0;
    oracle_ffn_row(d, d->I_s, a, sh_gate, sh_up, sh_down, 0, y);
    for (int c = 0; c < H; ++c) o[c] += gs * y[c];
  }
}

void oracle_moe_layer(const oracle_desc* d, const float* x, const float* w_r, const float* bias,
                      const oracle_mat* xa, const oracle_mat* gate, const oracle_mat* up,
                      const oracle_mat* down, const oracle_mat* sh_gate, const oracle_mat* sh_up,
                      const oracle_mat* sh_down, const float* w_sg, int n_tok,
                      const int32_t* tok, double* out, double* logits64, float* logits32,
                      int32_t* ids, double* w)
{
  int n = tok ? n_tok : d->T;
  int H = d->H, E = d->E, k = d->k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n; ++i) {
    int t = tok ? tok[i] : i;
    double* L64 = (double*)malloc(sizeof(double) * (size_t)E);
    float* L32 = (float*)malloc(sizeof(float) * (size_t)E);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* wt = (double*)malloc(sizeof(double) * (size_t)k);
    char* taken = (char*)malloc((size_t)E);
    double* a = (double*)malloc(sizeof(double) * (size_t)H);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);

    oracle_logits(d->T, H, E, x, w_r, bias, 1, &t, L64, NULL);
    for (int e = 0; e < E; ++e) L32[e] = (float)L64[e];
    topk_row(E, k, L32, d->scoring, d->renormalize, sel, wt, taken);
    expert_sum(d, x, xa, gate, up, down, sh_gate, sh_up, sh_down, w_sg, t, sel, wt, a, y,
               out + (size_t)i * H);

    if (logits64) memcpy(logits64 + (size_t)i * E, L64, sizeof(double) * (size_t)E);
    if (logits32) memcpy(logits32 + (size_t)i * E, L32, sizeof(float) * (size_t)E);
    if (ids) memcpy(ids + (size_t)i * k, sel, sizeof(int32_t) * (size_t)k);
    if (w) memcpy(w + (size_t)i * k, wt, sizeof(double) * (size_t)k);
    free(L64); free(L32); free(sel); free(wt); free(taken); free(a); free(y);
  }
}

void oracle_moe_layer_routed(const oracle_desc* d, const float* x, const oracle_mat* xa,
                             const oracle_mat* gate, const oracle_mat* up,
                             const oracle_mat* down, const oracle_mat* sh_gate,
                             const oracle_mat* sh_up, const oracle_mat* sh_down,
                             const float* w_sg, int n_tok, const int32_t* tok,
                             const int32_t* ids, const float* w, double* out)
{
  int H = d->H, k = d->k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n_tok; ++i) {
    double* wt = (double*)malloc(sizeof(double) * (size_t)k);
    double* a = (double*)malloc(sizeof(double) * (size_t)H);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    for (int j = 0; j < k; ++j) wt[j] = (double)w[(size_t)i * k + j];
    expert_sum(d, x, xa, gate, up, down, sh_gate, sh_up, sh_down, w_sg, tok[i],
               ids + (size_t)i * k, wt, a, y, out + (size_t)i * H);
    free(wt); free(a); free(y);
  }
}

/* ---------------------------------------------------------------------------------------------- */
/* The grouped GEMM and the combine as separate steps                                             */
/* ---------------------------------------------------------------------------------------------- */

void oracle_grouped_gemm(int G, const int32_t* offsets, const oracle_mat* A, const int32_t* a_rows,
                         int a_row_div, const oracle_mat* B, const oracle_mat* B2,
                         const float* bias, double* out)
{
  int K = B->K, N = B->N;
  int rows = offsets[G];
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)K);
    double* b = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
    for (int r = 0; r < rows; ++r) {
      int g = 0;
      while (offsets[g + 1] <= r) ++g;              /* group of row r */
      int src = a_rows ? a_rows[r] / a_row_div : r;
      mat_row(A, 0, src, a);
      for (int n = 0; n < N; ++n) {
        double d = 0.0;
        mat_row(B, g, n, b);
        for (int kk = 0; kk < K; ++kk) d += a[kk] * b[kk];
        if (bias) d += (double)bias[n];
        if (B2) {
          double u = 0.0;
          mat_row(B2, g, n, b);
          for (int kk = 0; kk < K; ++kk) u += a[kk] * b[kk];
          d = d / (1.0 + exp(-d)) * u;
        }
        out[(size_t)r * N + n] = d;
      }
    }
    free(a);
    free(b);
  }
}

void oracle_combine(int T, int H, int k, const float* y, const float* w, const int32_t* slot_to_row,
                    const float* shared, const float* shared_w, double* out)
{
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    double* o = out + (size_t)t * H;
    for (int c = 0; c < H; ++c) o[c] = 0.0;
    for (int j = 0; j < k; ++j) {
      int r = slot_to_row[t * k + j];
      if (r < 0) continue;
      for (int c = 0; c < H; ++c) o[c] += (double)w[t * k + j] * (double)y[(size_t)r * H + c];
    }
    if (shared) {
      double gs = shared_w ? (double)shared_w[t] : 1.0;
      for (int c = 0; c < H; ++c) o[c] += gs * (double)shared[(size_t)t * H + c];
    }
  }
}
