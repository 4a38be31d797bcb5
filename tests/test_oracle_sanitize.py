"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): oracle.c built with
gcc -fsanitize=address,undefined and a small C driver that runs every oracle routine on small,
ragged inputs (odd row counts, partial fp8 blocks, empty groups, tokens with no local expert,
every expert format as weights and as activations). Any out-of-bounds access, leak or undefined
operation aborts the driver."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")

DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include "oracle.h"

static unsigned long long st = 88172645463325252ull;
static float rnd(void) {                       /* xorshift64, uniform in [-1, 1) */
  st ^= st << 13; st ^= st >> 7; st ^= st << 17;
  return (float)((st >> 11) * (1.0 / 9007199254740992.0)) * 2.0f - 1.0f;
}
static float* frand(size_t n, float s) { float* p = malloc(n * sizeof(float)); for (size_t i = 0; i < n; ++i) p[i] = rnd() * s; return p; }

/* a quantised stack [G, N, K] of fmt from float values; fills m, returns the buffers to free */
static void quant(int fmt, int G, int N, int K, const float* w, oracle_mat* m, void** q, void** s, void** r) {
  memset(m, 0, sizeof(*m));
  m->fmt = fmt; m->G = G; m->N = N; m->K = K; m->bn = 128; m->bk = 128;
  *q = *s = *r = NULL;
  if (fmt == ORACLE_F32) { *q = malloc((size_t)G * N * K * 4); memcpy(*q, w, (size_t)G * N * K * 4); }
  if (fmt == ORACLE_FP8) {
    int nbn = (N + 127) / 128, nbk = (K + 127) / 128;
    *q = malloc((size_t)G * N * K); *s = malloc((size_t)G * nbn * nbk * 4);
    for (int g = 0; g < G; ++g)
      oracle_quant_fp8(N, K, 128, 128, w + (size_t)g * N * K, (uint8_t*)*q + (size_t)g * N * K,
                       (float*)*s + (size_t)g * nbn * nbk);
  }
  if (fmt == ORACLE_MX4) {
    *q = malloc((size_t)G * N * K / 2); *s = malloc((size_t)G * N * K / 32);
    oracle_quant_mx4(G * N, K, w, *q, *s);
  }
  if (fmt == ORACLE_MX8) {
    *q = malloc((size_t)G * N * K); *s = malloc((size_t)G * N * K / 32);
    oracle_quant_mx8(G * N, K, w, *q, *s);
  }
  if (fmt == ORACLE_NV4) {
    *q = malloc((size_t)G * N * K / 2); *s = malloc((size_t)G * N * K / 16); *r = malloc((size_t)G * N * 4);
    oracle_quant_nv4(G * N, K, w, *q, *s, *r);
  }
  m->q = *q; m->s = *s; m->r = *r;
}

int main(void) {
  /* codecs on special values */
  const float sp[] = {0.0f, -0.0f, 1e-30f, -1e-30f, 0.25f, 0.75f, 5.0f, 6.5f, 448.0f, 1e6f, -1e6f, 2.5f};
  for (unsigned i = 0; i < sizeof(sp) / sizeof(sp[0]); ++i) {
    (void)oracle_e4m3_value(oracle_e4m3_encode(sp[i]));
    (void)oracle_e2m1_value(oracle_e2m1_encode(sp[i]));
    (void)oracle_bf16_round(sp[i]);
  }
  for (int c = 0; c < 256; ++c) { (void)oracle_e4m3_value((uint8_t)c); (void)oracle_e8m0_value((uint8_t)c); }
  for (int c = 0; c < 16; ++c) (void)oracle_e2m1_value((uint8_t)c);

  /* layers: tiny shapes, every format; one token routes only to non-local experts */
  const int T = 7, H = 256, E = 12, k = 3, I = 128, Is = 128, E_loc = 5, e0 = 4;
  const int fmts[] = {ORACLE_F32, ORACLE_FP8, ORACLE_MX4, ORACLE_MX8, ORACLE_NV4};
  float* x = frand((size_t)T * H, 1.0f);
  float* wr = frand((size_t)E * H, 0.05f);
  float* bias = frand(E, 1.0f);
  for (int e = e0; e < e0 + E_loc; ++e) bias[e] = -1.0f;
  float* wsg = frand(H, 0.05f);
  float* wg = frand((size_t)E_loc * I * H, 0.05f), *wu = frand((size_t)E_loc * I * H, 0.05f);
  float* wd = frand((size_t)E_loc * H * I, 0.05f);
  float* sg = frand((size_t)Is * H, 0.05f), *su = frand((size_t)Is * H, 0.05f), *sd = frand((size_t)H * Is, 0.05f);
  for (unsigned f = 0; f < sizeof(fmts) / sizeof(fmts[0]); ++f) {
    const int fmt = fmts[f];
    oracle_mat xa, g, u, d, shg, shu, shd;
    void* b[21];
    quant(fmt, 1, T, H, x, &xa, &b[0], &b[1], &b[2]);
    quant(fmt, E_loc, I, H, wg, &g, &b[3], &b[4], &b[5]);
    quant(fmt, E_loc, I, H, wu, &u, &b[6], &b[7], &b[8]);
    quant(fmt, E_loc, H, I, wd, &d, &b[9], &b[10], &b[11]);
    quant(fmt, 1, Is, H, sg, &shg, &b[12], &b[13], &b[14]);
    quant(fmt, 1, Is, H, su, &shu, &b[15], &b[16], &b[17]);
    quant(fmt, 1, H, Is, sd, &shd, &b[18], &b[19], &b[20]);
    oracle_desc ds = {T, H, E, e0, E_loc, I, k, Is, f % 2 ? ORACLE_SIGMOID : ORACLE_SOFTMAX, 1,
                      fmt == ORACLE_F32 ? ORACLE_BF16 : fmt};
    double* out = malloc((size_t)T * H * 8);
    double* l64 = malloc((size_t)T * E * 8);
    float* l32 = malloc((size_t)T * E * 4);
    int32_t* ids = malloc((size_t)T * k * 4);
    double* w = malloc((size_t)T * k * 8);
    oracle_moe_layer(&ds, x, wr, bias, &xa, &g, &u, &d, &shg, &shu, &shd, wsg, T, NULL, out, l64, l32, ids, w);
    int32_t tok[2] = {6, 0};
    float w32[6];
    for (int i = 0; i < 6; ++i) w32[i] = (float)w[i];
    oracle_moe_layer_routed(&ds, x, &xa, &g, &u, &d, &shg, &shu, &shd, NULL, 2, tok, ids, w32, out);
    /* the dispatch maps, the grouped GEMM (with an empty group) and the combine on their own */
    int32_t counts[5], offsets[6], s2r[21], r2f[21];
    int R = oracle_permute(T, k, e0, E_loc, ids, counts, offsets, s2r, r2f);
    int32_t offg[4] = {0, R / 2, R / 2, R};
    double* y = malloc((size_t)(R + 1) * H * 8);
    oracle_grouped_gemm(3, offg, &xa, r2f, k, &d, NULL, NULL, y);
    double* h = malloc((size_t)(R + 1) * I * 8);
    oracle_grouped_gemm(3, offg, &xa, r2f, k, &g, &u, NULL, h);
    float* yf = frand((size_t)(R + 1) * H, 1.0f), *shf = frand((size_t)T * H, 1.0f), *gw = frand(T, 1.0f);
    float wf[21];
    for (int i = 0; i < T * k; ++i) wf[i] = (float)w[i];
    oracle_combine(T, H, k, yf, wf, s2r, shf, gw, out);
    double* dq = malloc((size_t)E_loc * I * H * 8);
    oracle_mat_dequant(&g, dq);
    double gs[7];
    oracle_shared_gate(T, H, x, wsg, 2, tok, gs);
    free(out); free(l64); free(l32); free(ids); free(w); free(y); free(h); free(yf); free(shf); free(gw); free(dq);
    for (int i = 0; i < 21; ++i) free(b[i]);
  }
  /* fp8 quantiser with partial blocks (rows and columns not multiples of 128) */
  float* q = frand(200 * 384, 3.0f);
  uint8_t* qc = malloc(200 * 384);
  float* qs = malloc(2 * 3 * 4);
  oracle_quant_fp8(200, 384, 128, 128, q, qc, qs);
  float* qs1 = malloc(200 * 3 * 4);
  oracle_quant_fp8(200, 384, 1, 128, q, qc, qs1);
  /* top-k with every logit equal */
  float* tie = calloc(5 * 64, sizeof(float));
  int32_t tids[5 * 64]; double tw[5 * 64];
  oracle_topk(5, 64, 64, tie, ORACLE_SOFTMAX, 1, tids, tw);
  oracle_topk(5, 64, 7, tie, ORACLE_SIGMOID, 0, tids, tw);
  free(q); free(qc); free(qs); free(qs1); free(tie);
  free(x); free(wr); free(bias); free(wsg); free(wg); free(wu); free(wd); free(sg); free(su); free(sd);
  printf("sanitized oracle run complete\n");
  return 0;
}
"""


def _gcc_sanitizers_work(tmp):
    src = os.path.join(tmp, "probe.c")
    open(src, "w").write("int main(void){return 0;}\n")
    r = subprocess.run(["gcc", "-fsanitize=address,undefined", src, "-o", os.path.join(tmp, "probe")],
                       capture_output=True, text=True)
    return r.returncode == 0


def test_oracle_under_asan_ubsan():
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        if not _gcc_sanitizers_work(tmp):
            pytest.skip("gcc has no ASan/UBSan runtime here")
        drv = os.path.join(tmp, "driver.c")
        open(drv, "w").write(DRIVER)
        exe = os.path.join(tmp, "driver")
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", ORACLE,
               os.path.join(ORACLE, "oracle.c"), drv, "-lm", "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        assert "sanitized oracle run complete" in r.stdout
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
