/* Drives every entry point of the CPU oracle (oracle/bao_ref.c) once over
 * small inputs of every kind it takes (fp16 / bf16, both row normalisers,
 * no bias, dense fp32 and fp16 biases shared and per batch, relative-position
 * biases with and without a prefix token, given scales, row windows, every
 * optional output), so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer sees every code path. Test infrastructure: the
 * sanitizer test builds and runs it; exits 0 when every call returned as
 * expected. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "bao_ref.h"

static uint32_t rng_state = 12345u;
static uint32_t rnd(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return rng_state;
}
/* a random finite 16-bit value of moderate size */
static uint16_t r16(int dtype) {
  const uint16_t sign = (rnd() & 1u) << 15;
  return dtype == BAO_F16 ? (uint16_t)(sign | (0x3000u + (rnd() % 0x1000u)))
                          : (uint16_t)(sign | (0x3E00u + (rnd() % 0x200u)));
}

static int run_case(int dtype, int B, int H, int N, int d, int bias_kind, int bias_dtype, int per_batch,
                    int gh, int gw, int npre, int given_mu, int norm) {
  const int64_t nt = (int64_t)B * H * N, ne = nt * d;
  uint16_t* q = malloc(2 * ne);
  uint16_t* k = malloc(2 * ne);
  uint16_t* v = malloc(2 * ne);
  for (int64_t i = 0; i < ne; ++i) { q[i] = r16(dtype); k[i] = r16(dtype); v[i] = r16(dtype); }
  bao_bias bias = {BAO_BIAS_NONE, NULL, BAO_F32, 0, 0, 0, 0};
  void* bdata = NULL;
  if (bias_kind == BAO_BIAS_DENSE) {
    const int64_t n = (per_batch ? B : 1) * (int64_t)H * N * N;
    if (bias_dtype == BAO_F32) {
      float* b = malloc(4 * n);
      for (int64_t i = 0; i < n; ++i) b[i] = (float)(rnd() % 1000) * 1e-4f - 0.05f;
      bdata = b;
    } else {
      uint16_t* b = malloc(2 * n);
      for (int64_t i = 0; i < n; ++i) b[i] = r16(BAO_F16);
      bdata = b;
    }
    bias = (bao_bias){BAO_BIAS_DENSE, bdata, bias_dtype, per_batch ? (int64_t)H * N * N : 0, 0, 0, 0};
  } else if (bias_kind == BAO_BIAS_RELPOS) {
    const int64_t n = (int64_t)H * (2 * gh - 1) * (2 * gw - 1);
    float* b = malloc(4 * n);
    for (int64_t i = 0; i < n; ++i) b[i] = (float)(rnd() % 1000) * 1e-4f - 0.05f;
    bdata = b;
    bias = (bao_bias){BAO_BIAS_RELPOS, bdata, BAO_F32, 0, gh, gw, npre};
  }
  float* mu = NULL;
  if (given_mu) {
    mu = malloc(4 * nt);
    for (int64_t i = 0; i < nt; ++i) mu[i] = (float)(rnd() % 100) * 0.02f;
  }
  /* a window of heads and rows: the last head, rows 1 .. N-1 */
  const int bh0 = B * H - 1, nbh = 1, row0 = N > 1 ? 1 : 0, nrows = N - row0;
  const int64_t no = (int64_t)nbh * nrows;
  double* out = malloc(8 * no * d);
  uint16_t* bits = malloc(2 * no * d);
  double* m = malloc(8 * no);
  double* l = malloc(8 * no);
  uint8_t* p8 = malloc(no * N);
  int64_t* acc = malloc(8 * no * d);
  double* e255 = malloc(8 * no * N);
  double* fp = malloc(8 * no * d);
  double* prob = malloc(8 * no * N);
  int rc = bao_attention_mu(q, k, v, dtype, B, H, N, d, &bias, mu, mu, norm, bh0, nbh, row0, nrows, dtype, out,
                            bits, m, l, p8, acc, e255);
  rc |= bao_attention_mu(q, k, v, dtype, B, H, N, d, &bias, NULL, NULL, norm, 0, B * H, 0, N, BAO_BF16, NULL, NULL,
                         NULL, NULL, NULL, NULL, NULL) == 0 ? 0 : 1;
  rc |= bao_attention_fp_mu(q, k, v, dtype, B, H, N, d, &bias, mu, NULL, bh0, nbh, row0, nrows, fp, prob);
  rc |= bao_attention(q, k, v, dtype, B, H, N, d, &bias, norm, 0, 1, 0, 1, dtype, out, NULL, NULL, NULL, NULL, NULL);
  rc |= bao_attention_fp(q, k, v, dtype, B, H, N, d, &bias, 0, 1, 0, 1, fp, NULL);
  /* pack, quantise and the similarity on their own */
  const int W = bao_words(d);
  uint32_t* qb = malloc(4 * nt * W);
  uint32_t* kb = malloc(4 * nt * W);
  float* qm = malloc(4 * nt);
  int8_t* vq = malloc(ne);
  float* vs = malloc(4 * (int64_t)B * H * d);
  int32_t* sg = malloc(4 * (int64_t)B * H * N * N);
  bao_pack(q, dtype, nt, d, qb, qm);
  bao_pack(k, dtype, nt, d, kb, qm);
  bao_quant_v(v, dtype, (int64_t)B * H, N, d, vq, vs);
  bao_hamming(qb, kb, N, d, 0, B * H, 0, N, sg);
  free(q); free(k); free(v); free(bdata); free(mu); free(out); free(bits); free(m); free(l); free(p8); free(acc);
  free(e255); free(fp); free(prob); free(qb); free(kb); free(qm); free(vq); free(vs); free(sg);
  return rc;
}

int main(void) {
  int fails = 0;
  /* number formats: every 16-bit pattern, and roundings at the edges */
  uint16_t all[65536];
  float dec[65536];
  for (int i = 0; i < 65536; ++i) all[i] = (uint16_t)i;
  bao_decode16(all, BAO_F16, 65536, dec);
  bao_decode16(all, BAO_BF16, 65536, dec);
  const double edge[] = {0.0, -0.0, 1e-40, -1e-8, 65504.0, 65520.0, 1e38, -3.4e38, 5.9604644775390625e-08};
  for (unsigned i = 0; i < sizeof edge / sizeof edge[0]; ++i) {
    (void)bao_round16(edge[i], BAO_F16);
    (void)bao_round16(edge[i], BAO_BF16);
  }
  /*           dt        B  H  N   d   bias              bias dt   pb gh gw pre mu norm */
  fails += run_case(BAO_F16, 1, 2, 37, 64, BAO_BIAS_NONE, BAO_F32, 0, 0, 0, 0, 0, BAO_NORM_P8);
  fails += run_case(BAO_BF16, 2, 1, 33, 72, BAO_BIAS_DENSE, BAO_F32, 0, 0, 0, 0, 1, BAO_NORM_FLOAT);
  fails += run_case(BAO_BF16, 2, 2, 20, 5, BAO_BIAS_DENSE, BAO_F16, 1, 0, 0, 0, 0, BAO_NORM_P8);
  fails += run_case(BAO_F16, 1, 3, 13, 128, BAO_BIAS_RELPOS, BAO_F32, 0, 3, 4, 1, 0, BAO_NORM_P8);
  fails += run_case(BAO_F16, 2, 1, 16, 33, BAO_BIAS_RELPOS, BAO_F32, 0, 4, 4, 0, 1, BAO_NORM_FLOAT);
  fails += run_case(BAO_BF16, 1, 1, 1, 1, BAO_BIAS_NONE, BAO_F32, 0, 0, 0, 0, 0, BAO_NORM_P8);
  /* rejected arguments return -1 without touching memory */
  uint16_t x[8] = {0};
  double o[8];
  bao_bias bad = {BAO_BIAS_RELPOS, NULL, BAO_F32, 0, 2, 3, 0};
  fails += bao_attention(x, x, x, BAO_F32, 1, 1, 1, 8, NULL, BAO_NORM_P8, 0, 1, 0, 1, BAO_F16, o, NULL, NULL, NULL,
                         NULL, NULL) != -1;
  fails += bao_attention(x, x, x, BAO_F16, 1, 1, 1, 8, &bad, BAO_NORM_P8, 0, 1, 0, 1, BAO_F16, o, NULL, NULL, NULL,
                         NULL, NULL) != -1;
  fails += bao_attention(x, x, x, BAO_F16, 1, 1, 1, 8, NULL, 7, 0, 1, 0, 1, BAO_F16, o, NULL, NULL, NULL, NULL,
                         NULL) != -1;
  fails += bao_attention_fp(x, x, x, BAO_F16, 1, 1, 1, 8, NULL, 0, 2, 0, 1, o, NULL) != -1;
  printf("oracle driver: %d failure(s)\n", fails);
  return fails != 0;
}
