/*
 * bao_ref.c — CPU oracle for the BinaryAttention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY (see bao_ref.h). Written step by step from the
 * technical summaries of "BinaryAttention: One-Bit QK-Attention for Vision
 * and Diffusion Transformers" on gist.science (pages zh, nl, it, fr, pt).
 * Each function names the section it follows. Where the pages leave a step
 * open, the reading taken is stated at the function.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math):
 * single-precision steps are then plain IEEE float operations and the
 * double-precision steps are plain IEEE double operations.
 */
#include "bao_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int bao_words(int d) { return (d + 31) / 32; }

int bao_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- number formats (not part of the method; exact by construction) ---- */

static float decode_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1.m) * 2^(e-15) */
  return (float)(s ? -v : v);
}

static float decode_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float decode1(const uint16_t* x, int dtype, int64_t i) {
  return dtype == BAO_F16 ? decode_f16(x[i]) : decode_bf16(x[i]);
}

void bao_decode16(const uint16_t* x, int dtype, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = decode1(x, dtype, i);
}

/* Round x to the nearest value with `mant` fraction bits and minimum normal
 * exponent `emin` (ties to even), then encode. One rounding from double. */
uint16_t bao_round16(double x, int dtype) {
  const int mant = dtype == BAO_F16 ? 10 : 7;
  const int emin = dtype == BAO_F16 ? -14 : -126;
  const int emax = dtype == BAO_F16 ? 15 : 127;
  const int ebits = dtype == BAO_F16 ? 5 : 8;
  const int bias = (1 << (ebits - 1)) - 1;
  uint16_t sign = signbit(x) ? (uint16_t)(1u << 15) : 0;
  double a = fabs(x);
  if (isnan(x)) return (uint16_t)(sign | (((1u << ebits) - 1) << mant) | 1u);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;         /* exponent of the leading bit */
  if (e < emin) e = emin; /* subnormal range: fixed quantum */
  double quantum = ldexp(1.0, e - mant);
  double r = rint(a / quantum) * quantum; /* a/quantum is exact */
  if (r == 0.0) return sign;
  frexp(r, &e2);
  e = e2 - 1;
  if (e > emax) return (uint16_t)(sign | (((1u << ebits) - 1) << mant)); /* inf */
  if (e < emin) { /* still subnormal after rounding */
    uint32_t m = (uint32_t)(r / ldexp(1.0, emin - mant));
    return (uint16_t)(sign | m);
  }
  uint32_t m = (uint32_t)(r / ldexp(1.0, e - mant)) - (1u << mant);
  return (uint16_t)(sign | ((uint32_t)(e + bias) << mant) | m);
}

/* ---- step 1: scaled binary representation of Q and K ----
 * BinaryAttention (gist.science/zh) technical summary, section 2.2 item 1;
 * (nl) Methodologie 2; (it) section 2B; (fr) section 2B; (pt) section 2B.
 * Each query/key vector is replaced by its sign vector times a magnitude
 * scalar. Readings: the sign of +0 and -0 is +1 (bit = value < 0); the
 * scalar is per token, the mean absolute value over the d channels. */
static void pack_one(const uint16_t* x, int dtype, int64_t off, int d,
                     uint32_t* bits, float* mu) {
  const int W = bao_words(d);
  for (int w = 0; w < W; ++w) bits[w] = 0;
  double asum = 0.0;
  for (int c = 0; c < d; ++c) {
    float v = decode1(x, dtype, off + c);
    if (v < 0.0f) bits[c / 32] |= 1u << (c % 32);
    asum += fabs((double)v);
  }
  *mu = (float)(asum / d);
}

void bao_pack(const uint16_t* x, int dtype, int64_t ntok, int d,
              uint32_t* bits, float* mu) {
  const int W = bao_words(d);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < ntok; ++t)
    pack_one(x, dtype, t * d, d, bits + t * W, mu + t);
}

/* ---- channel-wise 8-bit V ----
 * (zh) section 2.2 item 3; (nl) Methodologie 2 (hybrid quantisation with a
 * channel-specific scale). Reading: symmetric, one scale per (head, channel)
 * taken over the N tokens, 127 levels, round to nearest even, float32
 * arithmetic: inv = 127/amax, q = rint(v*inv), scale = amax/127. */
static void quant_head(const uint16_t* v, int dtype, int64_t base, int N,
                       int d, int8_t* vq, float* vscale) {
  for (int c = 0; c < d; ++c) {
    float amax = 0.0f;
    for (int j = 0; j < N; ++j) {
      float a = fabsf(decode1(v, dtype, base + (int64_t)j * d + c));
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      vscale[c] = 0.0f;
      for (int j = 0; j < N; ++j) vq[(int64_t)j * d + c] = 0;
      continue;
    }
    const float inv = 127.0f / amax; /* float32 IEEE division */
    vscale[c] = amax / 127.0f;
    for (int j = 0; j < N; ++j) {
      float r = rintf(decode1(v, dtype, base + (int64_t)j * d + c) * inv);
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      vq[(int64_t)j * d + c] = (int8_t)r;
    }
  }
}

void bao_quant_v(const uint16_t* v, int dtype, int64_t nbh, int N, int d,
                 int8_t* vq, float* vscale) {
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < nbh; ++bh)
    quant_head(v, dtype, bh * (int64_t)N * d, N, d,
               vq + bh * (int64_t)N * d, vscale + bh * d);
}

/* ---- step 2: Hamming similarity ----
 * (zh) sections 2.1 and 2.2 item 1; (it) section 2A; (fr) section 2A: the
 * dot product of two sign vectors equals d minus twice their Hamming
 * distance, computed with bitwise ops and a population count. */
static int popcount32(uint32_t x) {
  int n = 0;
  while (x) { x &= x - 1; ++n; }
  return n;
}

static int32_t sigma_of(const uint32_t* a, const uint32_t* b, int W, int d) {
  int h = 0;
  for (int w = 0; w < W; ++w) h += popcount32(a[w] ^ b[w]);
  return d - 2 * h;
}

void bao_hamming(const uint32_t* qbits, const uint32_t* kbits, int N, int d,
                 int bh0, int nbh, int row0, int nrows, int32_t* sigma) {
  const int W = bao_words(d);
#pragma omp parallel for collapse(2) schedule(static)
  for (int hh = 0; hh < nbh; ++hh)
    for (int r = 0; r < nrows; ++r) {
      const int64_t bh = bh0 + hh;
      const uint32_t* qi = qbits + (bh * N + row0 + r) * W;
      int32_t* out = sigma + ((int64_t)hh * nrows + r) * N;
      for (int j = 0; j < N; ++j)
        out[j] = sigma_of(qi, kbits + (bh * N + j) * W, W, d);
    }
}

/* ---- step 3: additive bias b_ij ----
 * (zh) section 2.2 item 2; (nl) Methodologie 2 (bias enhancement): the bias
 * may be dense or position-sensitive. Readings: dense is [H,N,N] per batch
 * slice; the position-sensitive form is a relative-position table indexed by
 * the grid offset between the two tokens, zero when either token is a prefix
 * token without a grid position. */
static double bias_at(const bao_bias* bias, int N, int b, int h, int i,
                      int j) {
  if (!bias || bias->kind == BAO_BIAS_NONE) return 0.0;
  if (bias->kind == BAO_BIAS_DENSE) {
    int64_t off = (int64_t)b * bias->batch_stride + ((int64_t)h * N + i) * N + j;
    if (bias->dtype == BAO_F32) return ((const float*)bias->data)[off];
    return decode_f16(((const uint16_t*)bias->data)[off]);
  }
  /* relative position */
  const int p = bias->n_prefix, gh = bias->grid_h, gw = bias->grid_w;
  if (i < p || j < p) return 0.0;
  const int ri = (i - p) / gw, ci = (i - p) % gw;
  const int rj = (j - p) / gw, cj = (j - p) % gw;
  const int64_t T = (int64_t)(2 * gh - 1) * (2 * gw - 1);
  const int64_t idx = (int64_t)(ri - rj + gh - 1) * (2 * gw - 1) + (ci - cj + gw - 1);
  return ((const float*)bias->data)[h * T + idx];
}

static int check_args(int dtype, int B, int H, int N, int d,
                      const bao_bias* bias, int bh0, int nbh, int row0,
                      int nrows) {
  if (dtype != BAO_F16 && dtype != BAO_BF16) return -1;
  if (B < 1 || H < 1 || N < 1 || d < 1 || d > 256) return -1;
  if (bh0 < 0 || nbh < 0 || bh0 + nbh > B * H) return -1;
  if (row0 < 0 || nrows < 0 || row0 + nrows > N) return -1;
  if (bias && bias->kind == BAO_BIAS_RELPOS &&
      bias->n_prefix + bias->grid_h * bias->grid_w != N)
    return -1;
  return 0;
}

/* Scores of one query row against all N keys of its head:
 * s_j = mu_q * mu_k_j * sigma_j / sqrt(d) + b_ij, in double.
 * (zh) section 2.2 items 1-2. Reading: temperature 1/sqrt(d) with the real
 * d; the bias is added after scaling. */
static void score_row(const uint32_t* qb, float qmu, const uint32_t* kb,
                      const float* kmu, int W, int N, int d,
                      const bao_bias* bias, int b, int h, int i, double* s) {
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  for (int j = 0; j < N; ++j) {
    int32_t sg = sigma_of(qb, kb + (int64_t)j * W, W, d);
    s[j] = (double)qmu * (double)kmu[j] * (double)sg * inv_sqrt_d +
           bias_at(bias, N, b, h, i, j);
  }
}

/* ---- step 4: softmax over the keys ----
 * (zh) section 2.3 (online softmax inside a FlashAttention2-style kernel).
 * The oracle takes the plain, unblocked definition: m = exact row max,
 * p~_j = exp(s_j - m) in (0, 1], l = sum_j p~_j (unquantised). */
static void softmax_row(const double* s, int N, double* pt, double* m_out,
                        double* l_out) {
  double m = s[0];
  for (int j = 1; j < N; ++j) if (s[j] > m) m = s[j];
  double l = 0.0;
  for (int j = 0; j < N; ++j) { pt[j] = exp(s[j] - m); l += pt[j]; }
  *m_out = m;
  *l_out = l;
}

/* Per-head working set: packed K, quantised V for all N keys. */
typedef struct {
  uint32_t* kbits;
  float* kmu;
  int8_t* vq;
  float* vscale;
} head_ws;

static int head_prepare(const uint16_t* k, const uint16_t* v, int dtype,
                        int64_t bh, int N, int d, int want_v,
                        const float* kmu_in, head_ws* ws) {
  const int W = bao_words(d);
  ws->kbits = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)N * W);
  ws->kmu = (float*)malloc(sizeof(float) * (size_t)N);
  ws->vq = want_v ? (int8_t*)malloc((size_t)N * d) : NULL;
  ws->vscale = want_v ? (float*)malloc(sizeof(float) * (size_t)d) : NULL;
  if (!ws->kbits || !ws->kmu || (want_v && (!ws->vq || !ws->vscale))) return -1;
  const int64_t base = bh * (int64_t)N * d;
  for (int j = 0; j < N; ++j) {
    pack_one(k, dtype, base + (int64_t)j * d, d, ws->kbits + (int64_t)j * W,
             ws->kmu + j);
    if (kmu_in) ws->kmu[j] = kmu_in[bh * N + j];  /* a given key scale */
  }
  if (want_v) quant_head(v, dtype, base, N, d, ws->vq, ws->vscale);
  return 0;
}

static void head_release(head_ws* ws) {
  free(ws->kbits); free(ws->kmu); free(ws->vq); free(ws->vscale);
}

/* ---- steps 5-6: 8-bit P, integer aggregation, dequantisation ----
 * (zh) section 2.2 item 3 and section 2.3; (nl) Methodologie 2-3. The
 * unnormalised probabilities become unsigned 8-bit over [0,1]
 * (p8 = rne(255 p~)), V is the channel-wise int8 above, P.V is summed in
 * integers and dequantised: O_ic = A_ic * scale_c / (255 * l_i).
 * The pages do not say what l is. Reading (BAO_NORM_FLOAT): the float sum
 * of the unquantised values, l = sum_j p~_ij, so the rows of the
 * real-valued P sum to 1 before quantisation and keys whose p8 rounds to 0
 * still count in l. BAO_NORM_P8 keeps the alternative l = sum_j p8_ij / 255
 * (the integer row sum of the quantised weights; then 255 l = sum_j p8_ij
 * exactly), which renormalises over the keys that survive quantisation. */
int bao_attention_mu(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int dtype, int B, int H, int N, int d, const bao_bias* bias,
                     const float* qmu_in, const float* kmu_in, int norm,
                     int bh0, int nbh, int row0, int nrows, int out_dtype,
                     double* out_f64, uint16_t* out_bits, double* row_m,
                     double* row_l, uint8_t* p8, int64_t* acc, double* e255) {
  if (check_args(dtype, B, H, N, d, bias, bh0, nbh, row0, nrows)) return -1;
  if (out_dtype != BAO_F16 && out_dtype != BAO_BF16) return -1;
  if (norm != BAO_NORM_P8 && norm != BAO_NORM_FLOAT) return -1;
  const int W = bao_words(d);
  int status = 0;
  for (int hh = 0; hh < nbh; ++hh) {
    const int64_t bh = bh0 + hh;
    const int b = (int)(bh / H), h = (int)(bh % H);
    head_ws ws;
    if (head_prepare(k, v, dtype, bh, N, d, 1, kmu_in, &ws)) { head_release(&ws); return -1; }
#pragma omp parallel
    {
      double* s = (double*)malloc(sizeof(double) * (size_t)N);
      double* pt = (double*)malloc(sizeof(double) * (size_t)N);
      uint8_t* q8 = (uint8_t*)malloc((size_t)N);
      int64_t* A = (int64_t*)malloc(sizeof(int64_t) * (size_t)d);
      uint32_t qb[8];
      float qmu;
#pragma omp for schedule(static)
      for (int r = 0; r < nrows; ++r) {
        const int i = row0 + r;
        pack_one(q, dtype, (bh * N + i) * (int64_t)d, d, qb, &qmu);
        if (qmu_in) qmu = qmu_in[bh * N + i];  /* a given query scale */
        score_row(qb, qmu, ws.kbits, ws.kmu, W, N, d, bias, b, h, i, s);
        double m, l;
        softmax_row(s, N, pt, &m, &l);
        int64_t psum = 0; /* sum_j p8_ij */
        for (int j = 0; j < N; ++j) {
          double x = rint(255.0 * pt[j]);
          if (x < 0.0) x = 0.0;
          if (x > 255.0) x = 255.0;
          q8[j] = (uint8_t)x;
          psum += q8[j];
        }
        /* 255 * l: the integer row sum of P, or 255 times the float one */
        const double den = norm == BAO_NORM_P8 ? (double)psum : 255.0 * l;
        for (int c = 0; c < d; ++c) A[c] = 0;
        for (int j = 0; j < N; ++j) {
          const int64_t pj = q8[j];
          if (!pj) continue;
          const int8_t* vj = ws.vq + (int64_t)j * d;
          for (int c = 0; c < d; ++c) A[c] += pj * vj[c];
        }
        const int64_t o = ((int64_t)hh * nrows + r);
        for (int c = 0; c < d; ++c) {
          if (A[c] > INT32_MAX || A[c] < INT32_MIN) {
#pragma omp atomic write
            status = -2;
          }
          double out = (double)A[c] * (double)ws.vscale[c] / den;
          if (out_f64) out_f64[o * d + c] = out;
          if (out_bits) out_bits[o * d + c] = bao_round16(out, out_dtype);
          if (acc) acc[o * d + c] = A[c];
        }
        if (row_m) row_m[o] = m;
        if (row_l) row_l[o] = den / 255.0;
        if (p8) memcpy(p8 + o * N, q8, (size_t)N);
        if (e255)
          for (int j = 0; j < N; ++j) e255[o * N + j] = 255.0 * pt[j];
      }
      free(s); free(pt); free(q8); free(A);
    }
    head_release(&ws);
  }
  return status;
}

/* Unquantised reference (no P or V quantisation): O_ic = sum_j p~_ij v_jc / l_i
 * with the same binary scores and bias. */
int bao_attention_fp_mu(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        int dtype, int B, int H, int N, int d,
                        const bao_bias* bias, const float* qmu_in,
                        const float* kmu_in, int bh0, int nbh, int row0,
                        int nrows, double* out_f64, double* prob) {
  if (check_args(dtype, B, H, N, d, bias, bh0, nbh, row0, nrows)) return -1;
  const int W = bao_words(d);
  for (int hh = 0; hh < nbh; ++hh) {
    const int64_t bh = bh0 + hh;
    const int b = (int)(bh / H), h = (int)(bh % H);
    head_ws ws;
    if (head_prepare(k, v, dtype, bh, N, d, 0, kmu_in, &ws)) { head_release(&ws); return -1; }
    const int64_t base = bh * (int64_t)N * d;
#pragma omp parallel
    {
      double* s = (double*)malloc(sizeof(double) * (size_t)N);
      double* pt = (double*)malloc(sizeof(double) * (size_t)N);
      uint32_t qb[8];
      float qmu;
#pragma omp for schedule(static)
      for (int r = 0; r < nrows; ++r) {
        const int i = row0 + r;
        pack_one(q, dtype, (bh * N + i) * (int64_t)d, d, qb, &qmu);
        if (qmu_in) qmu = qmu_in[bh * N + i];  /* a given query scale */
        score_row(qb, qmu, ws.kbits, ws.kmu, W, N, d, bias, b, h, i, s);
        double m, l;
        softmax_row(s, N, pt, &m, &l);
        const int64_t o = ((int64_t)hh * nrows + r);
        for (int c = 0; c < d; ++c) {
          double a = 0.0;
          for (int j = 0; j < N; ++j)
            a += pt[j] * (double)decode1(v, dtype, base + (int64_t)j * d + c);
          out_f64[o * d + c] = a / l;
        }
        if (prob)
          for (int j = 0; j < N; ++j) prob[o * N + j] = pt[j] / l;
      }
      free(s); free(pt);
    }
    head_release(&ws);
  }
  return 0;
}

/* The scales mu are an input of the attention step (zh section 2.2 item 1
 * calls them learnable; reading R1 computes them per token). These two
 * forms take them as given arrays [B,H,N] (either may be NULL: then the
 * per-token mean |x| as in bao_pack), e.g. a per-head scalar. */
int bao_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  int dtype, int B, int H, int N, int d, const bao_bias* bias,
                  int norm, int bh0, int nbh, int row0, int nrows, int out_dtype,
                  double* out_f64, uint16_t* out_bits, double* row_m,
                  double* row_l, uint8_t* p8, int64_t* acc) {
  return bao_attention_mu(q, k, v, dtype, B, H, N, d, bias, NULL, NULL, norm, bh0,
                          nbh, row0, nrows, out_dtype, out_f64, out_bits, row_m,
                          row_l, p8, acc, NULL);
}

int bao_attention_fp(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int dtype, int B, int H, int N, int d,
                     const bao_bias* bias, int bh0, int nbh, int row0,
                     int nrows, double* out_f64, double* prob) {
  return bao_attention_fp_mu(q, k, v, dtype, B, H, N, d, bias, NULL, NULL, bh0,
                             nbh, row0, nrows, out_f64, prob);
}
