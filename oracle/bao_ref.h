/*
 * bao_ref.h — CPU oracle for the BinaryAttention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, obviously-correct
 * implementation of what the method computes, written from the technical
 * summaries of "BinaryAttention: One-Bit QK-Attention for Vision and
 * Diffusion Transformers" (gist.science pages zh, nl, it, fr, pt). Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it. It shares no code, header, table or helper with the GPU library.
 *
 * Conventions (all arrays host memory, row-major, caller-owned):
 *   dtype codes: 0 = fp16, 1 = bf16, 2 = fp32 (the 16-bit inputs are passed
 *   as raw uint16 bit patterns).
 *   Q, K, V: [B, H, N, d] tokens; a "head" index bh = b*H + h.
 *   Packed sign bits: uint32 [.., W] with W = ceil(d/32), channel c in word
 *   c/32 at bit c%32, bit = 1 iff the value is < 0 (so +0 and -0 give +1),
 *   pad bits zero.
 *   Softmax and scores in double; integer arithmetic where the method is
 *   integer; exp() is the host libm routine.
 */
#ifndef BAO_REF_H
#define BAO_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { BAO_F16 = 0, BAO_BF16 = 1, BAO_F32 = 2 };
enum { BAO_BIAS_NONE = 0, BAO_BIAS_DENSE = 1, BAO_BIAS_RELPOS = 2 };
/* The row normaliser l_i that the integer P.V sum is divided by (the pages
 * leave it open):
 *   BAO_NORM_FLOAT l_i = sum_j exp(s_ij - m_i): the unquantised row sum (the
 *                  reading the library follows);
 *   BAO_NORM_P8    l_i = (sum_j p8_ij) / 255: the sum of the quantised
 *                  weights that multiply V (an alternative: it drops the
 *                  mass of keys whose p8 rounds to 0 from the normaliser). */
enum { BAO_NORM_FLOAT = 0, BAO_NORM_P8 = 1 };

typedef struct {
  int kind;              /* BAO_BIAS_*                                        */
  const void* data;      /* DENSE: [H,N,N] per batch slice; RELPOS: [H,T]      */
  int dtype;             /* DENSE: BAO_F32 or BAO_F16; RELPOS: BAO_F32         */
  int64_t batch_stride;  /* DENSE: elements between batch slices (0 = shared) */
  int grid_h, grid_w;    /* RELPOS: token grid; T = (2gh-1)(2gw-1)             */
  int n_prefix;          /* RELPOS: leading tokens without a grid position    */
} bao_bias;

int bao_words(int d);

/* Exact widening of fp16 / bf16 bit patterns to float. */
void bao_decode16(const uint16_t* x, int dtype, int64_t n, float* out);

/* Round a double to fp16 / bf16 (round to nearest even, one rounding). */
uint16_t bao_round16(double x, int dtype);

/* Sign bits and per-token scale mu = mean_c |x_c| for ntok tokens of d. */
void bao_pack(const uint16_t* x, int dtype, int64_t ntok, int d,
              uint32_t* bits, float* mu);

/* Channel-wise int8 quantisation of V over the N tokens of each head. */
void bao_quant_v(const uint16_t* v, int dtype, int64_t nbh, int N, int d,
                 int8_t* vq, float* vscale);

/* Integer similarity sigma = d - 2*popcount(q xor k) for a window of heads
 * [bh0, bh0+nbh) and query rows [row0, row0+nrows); output [nbh,nrows,N]. */
void bao_hamming(const uint32_t* qbits, const uint32_t* kbits, int N, int d,
                 int bh0, int nbh, int row0, int nrows, int32_t* sigma);

/* Quantised BinaryAttention forward for heads [bh0,bh0+nbh) and query rows
 * [row0,row0+nrows), from the raw 16-bit Q, K, V, with the row normaliser
 * `norm` (BAO_NORM_*). Any output pointer may be NULL. Shapes:
 * out_f64/out_bits/acc [nbh,nrows,d]; row_m/row_l [nbh,nrows]; p8 and e255
 * [nbh,nrows,N] (e255: the unrounded 255 * p~ that p8 rounds). Returns 0, or
 * -1 on an argument error, -2 if an integer accumulator would leave int32
 * range. */
int bao_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  int dtype, int B, int H, int N, int d, const bao_bias* bias,
                  int norm, int bh0, int nbh, int row0, int nrows, int out_dtype,
                  double* out_f64, uint16_t* out_bits, double* row_m,
                  double* row_l, uint8_t* p8, int64_t* acc);

/* Unquantised reference: same scores and softmax, then P V with the decoded
 * float V (no P or V quantisation). out_f64 [nbh,nrows,d]; prob, if not
 * NULL, receives the normalised probabilities [nbh,nrows,N]. */
int bao_attention_fp(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int dtype, int B, int H, int N, int d,
                     const bao_bias* bias, int bh0, int nbh, int row0,
                     int nrows, double* out_f64, double* prob);

/* The same two computations with the scales mu given instead of computed:
 * qmu_in, kmu_in float [B,H,N] (either may be NULL: computed as in
 * bao_pack). mu is an input of the attention step (a learnable scale in
 * zh section 2.2 item 1), so e.g. a per-head scalar passes through here. */
int bao_attention_mu(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int dtype, int B, int H, int N, int d, const bao_bias* bias,
                     const float* qmu_in, const float* kmu_in, int norm,
                     int bh0, int nbh, int row0, int nrows, int out_dtype,
                     double* out_f64, uint16_t* out_bits, double* row_m,
                     double* row_l, uint8_t* p8, int64_t* acc, double* e255);
int bao_attention_fp_mu(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        int dtype, int B, int H, int N, int d,
                        const bao_bias* bias, const float* qmu_in,
                        const float* kmu_in, int bh0, int nbh, int row0,
                        int nrows, double* out_f64, double* prob);

/* Number of OpenMP threads the oracle will use. */
int bao_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
