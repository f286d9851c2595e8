/*
 * binattn.h — C ABI of the MI355X (gfx950) BinaryAttention forward library.
 *
 * The method (BinaryAttention: One-Bit QK-Attention for Vision and Diffusion
 * Transformers; technical summaries on gist.science, pages zh, nl, it, fr,
 * pt) replaces each query and key by its sign vector and a magnitude scale,
 * scores query/key pairs through a Hamming distance of the sign bits, adds a
 * learnable bias, applies softmax, quantises the unnormalised probabilities
 * to unsigned 8 bit and V to channel-wise int8, and aggregates P.V in
 * integers before dequantising. The calls below follow that statement of the
 * problem: pack Q/K, quantise V, then the fused attention; a debug call
 * exposes the integer similarity.
 *
 * Conventions shared by every call
 *  - Memory: every pointer argument is DEVICE memory allocated by the caller
 *    (e.g. a torch tensor's data_ptr()). The library allocates nothing, keeps
 *    no pointer after a call returns, and fully overwrites its outputs.
 *    Outputs must not alias inputs. Buffers must stay alive until the work
 *    queued on `stream` has finished.
 *  - Stream: `stream` is a hipStream_t passed as void* (NULL = the default
 *    stream). Every call only enqueues work; none synchronises.
 *  - Layouts: dense, row-major. Tokens are [B, H, N, d] (head index
 *    bh = b*H + h). W = ba_packed_words(d) = ceil(d/32). The two *_strided
 *    calls also read Q/K/V from, and write the output to, strided views
 *    (ba_strides); every layout the library writes besides that output is
 *    dense.
 *  - Errors: arguments are validated before any HIP call. A rejected call
 *    returns BA_ERR_INVALID_ARG (null or misaligned pointer, size < 1,
 *    inconsistent bias description) or BA_ERR_UNSUPPORTED (d outside
 *    [1,128], N above BA_MAX_TOKENS, a dtype not listed for that argument)
 *    and enqueues nothing. A failed kernel launch returns BA_ERR_HIP. Device
 *    faults surface at the caller's next synchronisation. No C++ exception
 *    crosses this interface. The library is stateless and re-entrant.
 *  - Alignment: bits / vq / out / Q / K / V pointers 16-byte aligned; mu,
 *    vscale and bias pointers 4-byte aligned (fp16 bias: 2-byte).
 */
#ifndef BINATTN_H
#define BINATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BA_OK = 0,
  BA_ERR_INVALID_ARG = 1,
  BA_ERR_UNSUPPORTED = 2,
  BA_ERR_HIP = 3
} ba_status;

typedef enum { BA_F16 = 0, BA_BF16 = 1, BA_F32 = 2 } ba_dtype;

typedef enum {
  BA_BIAS_NONE = 0,   /* no bias                                            */
  BA_BIAS_DENSE = 1,  /* b[h,i,j] from a dense [H,N,N] slice per batch entry */
  BA_BIAS_RELPOS = 2  /* b[h,i,j] = table[h, idx(i,j)], relative position     */
} ba_bias_kind;

/* Largest N accepted: the integer P.V sum must stay inside int32
 * (255 * 127 * N < 2^31). */
#define BA_MAX_TOKENS 65536

/* Element strides of a [B, H, N, d] view of 16-bit values whose d channels
 * are contiguous: element (b, h, n, c) sits at
 * base + b*batch + h*head + n*token + c (in elements, not bytes). Strides are
 * non-negative. The dense layout is {H*N*d, N*d, d}; the per-head slices of
 * a fused QKV projection output [B, N, 3, H, d] are {3*N*H*d, d, 3*H*d}
 * (from the q, k and v bases 0, H*d and 2*H*d). */
typedef struct {
  int64_t batch, head, token;
} ba_strides;

/* Additive bias b_ij on the scores (bias enhancement: zh technical summary
 * section 2.2 item 2; nl Methodologie 2; it/fr/pt section 2B). The pages
 * allow a dense, a position-sensitive or a context-aware bias; a context-
 * aware bias computed elsewhere can be passed as a per-batch DENSE bias.
 *
 *  DENSE : data = [H,N,N] elements for batch entry 0, entry b starts at
 *          data + b*batch_stride elements (batch_stride 0 = one slice shared
 *          by the whole batch, else >= H*N*N). dtype BA_F32 or BA_F16.
 *  RELPOS: data = fp32 table [H, (2*grid_h-1)*(2*grid_w-1)]. Tokens
 *          t >= n_prefix sit on a grid_h x grid_w grid at row
 *          (t-n_prefix)/grid_w, column (t-n_prefix)%grid_w; the bias of
 *          query i and key j is table[h, (r_i-r_j+grid_h-1)*(2*grid_w-1)
 *          + (c_i-c_j+grid_w-1)], and 0 when i or j < n_prefix. Requires
 *          N == n_prefix + grid_h*grid_w. dtype must be BA_F32;
 *          grid_w <= 256 (else BA_ERR_UNSUPPORTED).
 */
typedef struct {
  ba_bias_kind kind;
  const void* data;
  ba_dtype dtype;
  int64_t batch_stride;
  int32_t grid_h, grid_w, n_prefix;
} ba_bias;

/* W = ceil(d/32): 32-bit words per packed token. Returns 0 for d < 1. */
int ba_packed_words(int d);

/* Scaled binary representation of Q and K (zh technical summary section 2.2
 * item 1; nl Methodologie 2; it section 2B; fr section 2B; pt section 2B):
 * each token x (d channels) becomes sign bits and one scale.
 *   bits[t, w] bit c%32 of word w = c/32 is 1 iff x_c < 0 (so +0 and -0
 *   count as +1); bits for c >= d are 0.
 *   mu[t] = (sum_c |x_c|) / d  (one scale per token).
 * q, k: [B,H,N,d] fp16 or bf16 (dt), device. qbits, kbits: uint32
 * [B,H,N,W]; qmu, kmu: float [B,H,N]. */
ba_status ba_pack_qk(const void* q, const void* k, ba_dtype dt, int B, int H,
                     int N, int d, uint32_t* qbits, float* qmu,
                     uint32_t* kbits, float* kmu, void* stream);

/* Channel-wise 8-bit V (zh section 2.2 item 3; nl Methodologie 2): for each
 * (b,h,c), amax = max_j |v_jc| over the N tokens; vq = clamp(rne(v * (127 /
 * amax)), -127, 127) in float32; vscale = amax / 127; an all-zero channel
 * gives vq = 0 and vscale = 0.
 * v: [B,H,N,d] fp16 or bf16; vq: int8 [B,H,N,d]; vscale: float [B,H,d].
 * vq and vscale must not overlap each other or v. */
ba_status ba_quant_v(const void* v, ba_dtype dt, int B, int H, int N, int d,
                     int8_t* vq, float* vscale, void* stream);

/* ba_pack_qk and ba_quant_v in one call, for callers that run both before
 * ba_attention_fwd (as every forward pass does): the same outputs, bit for
 * bit, with the same layouts, alignment and error rules as the two calls
 * (q, k, v all [B,H,N,d] of dt). Where d % 8 == 0 and a head fits the
 * register-resident V quantiser whole (N <= 10 * 1024 / (d / 8)) or in up
 * to four parts (each part's block then reads the whole head for the
 * channel maxima itself), it is a single launch in which the V heads and
 * the Q/K token blocks run side by side; with longer heads the packing
 * launch also clears vscale and the V quantiser's two passes follow;
 * otherwise it enqueues the two calls' kernels in turn. No output may
 * overlap another output or an input. */
ba_status ba_pack_qk_quant_v(const void* q, const void* k, const void* v, ba_dtype dt, int B, int H,
                             int N, int d, uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu,
                             int8_t* vq, float* vscale, void* stream);

/* ba_pack_qk_quant_v with q, k and v read through strided views that share
 * in_strides (typically the head slices of one QKV projection output, so no
 * head-split copy is needed; zh technical summary section 4 measures the
 * method inside whole transformer layers). The outputs are the dense ones
 * of ba_pack_qk_quant_v, bit for bit equal to packing a dense copy. q, k, v
 * need 2-byte alignment only; where d % 8 == 0, every stride is a multiple
 * of 8 and q, k, v are 16-byte aligned, the 16-byte-load kernels run. The
 * views may overlap one another (they are only read) but no output may
 * overlap the span of any view. in_strides NULL or negative, or a view
 * spanning more than about 2^40 elements: BA_ERR_INVALID_ARG. */
ba_status ba_pack_qk_quant_v_strided(const void* q, const void* k, const void* v, const ba_strides* in_strides,
                                     ba_dtype dt, int B, int H, int N, int d, uint32_t* qbits, float* qmu,
                                     uint32_t* kbits, float* kmu, int8_t* vq, float* vscale, void* stream);

/* Fused BinaryAttention forward (zh sections 2.1-2.3; nl Methodologie 1-3;
 * it section 2; fr section 2B; pt section 2B-2C), non-causal, self-attention
 * (N queries and N keys per head). For each head and query i:
 *   sigma_ij = d - 2*popcount(qbits_i XOR kbits_j)
 *   s_ij     = qmu_i * kmu_j * sigma_ij / sqrt(d) + b_ij
 *   m_i      = max_j s_ij,  p_ij = exp(s_ij - m_i)
 *   p8_ij    = rne(255 * p_ij)                  (unsigned 8 bit over [0,1])
 *   A_ic     = sum_j p8_ij * vq_jc              (exact, int32)
 *   l_i      = sum_j p_ij                       (fp32, the unquantised p)
 *   out_ic   = A_ic * vscale_c / (255 * l_i)    rounded to out_dt
 * i.e. the row normaliser is the softmax denominator of the unquantised
 * probabilities, so the mass of keys whose p8 rounds to 0 still counts.
 * m_i is the exact row maximum (the kernel finds it in a first pass over the
 * keys), so p8 matches the plain definition up to float rounding. The
 * kernel uses no scratch memory and allocates nothing.
 * Any int8 vq with any non-negative scales is accepted (the outputs of
 * ba_pack_qk / ba_quant_v or equivalent data; e.g. a learned mu); the
 * kernel needs nothing besides these arrays.
 * bias: NULL or kind BA_BIAS_NONE for no bias.
 * out: [B,H,N,d] of out_dt, which must be BA_F16 or BA_BF16. */
ba_status ba_attention_fwd(const uint32_t* qbits, const float* qmu,
                           const uint32_t* kbits, const float* kmu,
                           const int8_t* vq, const float* vscale,
                           const ba_bias* bias,
                           int B, int H, int N, int d,
                           void* out, ba_dtype out_dt, void* stream);

/* Extension (not one of the four calls): the same attention in one pass
 * over the keys with a running row maximum, the FlashAttention-2 order that
 * the pages' kernel keeps (zh section 2.3; nl Methodologie 3). Keys go in
 * blocks of 32 in index order; for query i and a key j of block b, p8_ij =
 * rne(255 * exp(s_ij - m_ib)) where m_ib is the maximum of s_i over blocks
 * 0..b, and the sums gathered so far are scaled by exp(m_old - m_new) (in
 * fp32) whenever the maximum grows. p8 therefore depends on the key order
 * and differs from that of ba_attention_fwd, which quantises against the
 * exact row maximum; the two outputs agree within 2e-2 * max|V|, the bound
 * that covers this blocking. On MI355X this form is the slower one (its
 * rescales cost more vector work than the maximum pass of the two-pass
 * kernel); it is kept for comparison. d <= 64 only (BA_ERR_UNSUPPORTED
 * otherwise); arguments, layouts and errors as ba_attention_fwd. */
ba_status ba_attention_fwd_online(const uint32_t* qbits, const float* qmu,
                                  const uint32_t* kbits, const float* kmu,
                                  const int8_t* vq, const float* vscale,
                                  const ba_bias* bias,
                                  int B, int H, int N, int d,
                                  void* out, ba_dtype out_dt, void* stream);

/* ba_attention_fwd writing the output through a strided view: element
 * (b, h, i, c) of the result goes to out + b*batch + h*head + i*token + c
 * (e.g. {N*H*d, d, H*d} writes [B, N, H, d], the input layout of an output
 * projection, with no head-merge copy). The same values as
 * ba_attention_fwd, bit for bit; elements outside the view are not
 * touched. out needs 2-byte alignment (8-byte stores where d and the
 * strides are multiples of 4 and out is 8-byte aligned). The view must not
 * map two elements to one address and its span must not overlap an input:
 * BA_ERR_INVALID_ARG otherwise, as for NULL or negative strides or a span
 * above about 2^40 elements; a head or token stride above 2^31 - 1:
 * BA_ERR_UNSUPPORTED. */
ba_status ba_attention_fwd_strided(const uint32_t* qbits, const float* qmu,
                                   const uint32_t* kbits, const float* kmu,
                                   const int8_t* vq, const float* vscale,
                                   const ba_bias* bias,
                                   int B, int H, int N, int d, void* out,
                                   const ba_strides* out_strides, ba_dtype out_dt,
                                   void* stream);

/* Extension: the path with Q packed inside the attention (zh technical
 * summary section 2.3: the steps fused into one kernel; section 2.2 item 1
 * for the packing itself). Each query row is read once, by the workgroup
 * that owns it, so binarising it in the attention's prologue repeats no
 * work; K and V rows are read by every query block of their head, so they
 * are still packed and quantised first, by ba_pack_k_quant_v.
 *
 * ba_pack_k_quant_v: the K and V half of ba_pack_qk_quant_v (kbits, kmu,
 * vq, vscale bit for bit as that call writes them; same layouts, alignment
 * and error rules, k and v [B,H,N,d] of dt, no output overlapping another
 * output or an input). */
ba_status ba_pack_k_quant_v(const void* k, const void* v, ba_dtype dt, int B, int H, int N, int d,
                            uint32_t* kbits, float* kmu, int8_t* vq, float* vscale, void* stream);

/* ba_attention_fwd_q16: ba_attention_fwd with Q given as 16-bit values q
 * [B,H,N,d] of q_dt (BA_F16 or BA_BF16; 16-byte aligned, dense), packed by
 * the attention kernel into the same sign bits and scales that ba_pack_qk
 * forms (same arithmetic: bit = x < 0; scale = float64 sum of |x| in
 * channel order / d, rounded to float once); the output equals
 * ba_pack_qk followed by ba_attention_fwd bit for bit. d % 8 == 0 only
 * (BA_ERR_UNSUPPORTED otherwise); the other arguments, layouts and errors
 * as ba_attention_fwd; out must not overlap q. */
ba_status ba_attention_fwd_q16(const void* q, ba_dtype q_dt,
                               const uint32_t* kbits, const float* kmu,
                               const int8_t* vq, const float* vscale,
                               const ba_bias* bias,
                               int B, int H, int N, int d,
                               void* out, ba_dtype out_dt, void* stream);

/* ba_attention_fwd_qkv16: the whole forward pass in one launch, for short
 * heads: Q, K and V given as 16-bit values [B,H,N,d] of dt (16-byte
 * aligned, dense), each workgroup binarising its queries and its head's
 * keys and quantising its head's V itself, with the arithmetic of
 * ba_pack_qk and ba_quant_v, straight into on-chip memory (zh technical
 * summary section 2.3: one fused kernel; section 2.2 items 1 and 3). The
 * output equals ba_pack_qk + ba_quant_v + ba_attention_fwd bit for bit; no
 * packed or quantised array is written. It applies where a head's keys all
 * stay on chip at once: N <= 256, d % 8 == 0 and d <= 96, and no bias, a
 * relative-position table, or a dense fp32 bias with 16-byte rows (N % 4 ==
 * 0, batch stride % 4 == 0, 16-byte aligned); except a relative-position
 * table over grid rows that are multiples of 16 tokens wide with no leading
 * tokens at 33..64 channels (that kernel runs four workgroups per CU and
 * has no room for a whole head); BA_ERR_UNSUPPORTED otherwise, with nothing
 * enqueued. Each head's K and V are read by each of its (at
 * most two) query blocks. Other arguments, layouts and errors as
 * ba_attention_fwd; out must not overlap q, k or v. */
ba_status ba_attention_fwd_qkv16(const void* q, const void* k, const void* v, ba_dtype dt,
                                 const ba_bias* bias, int B, int H, int N, int d,
                                 void* out, ba_dtype out_dt, void* stream);

/* Integer Hamming similarity for inspection (zh sections 2.1 and 2.2 item 1;
 * it section 2A; fr section 2A): for heads [bh_begin, bh_begin+bh_count) and
 * query rows [row_begin, row_begin+row_count),
 *   sigma[hb, r, j] = d - 2*popcount(qbits[bh_begin+hb, row_begin+r] XOR
 *                                    kbits[bh_begin+hb, j])
 * sigma: int32 [bh_count, row_count, N], device. The window must lie inside
 * [0, B*H) x [0, N).
 * The values come from the fused attention kernel's own Q.K code, every
 * route it has for that d: the staged-tile route writes them, then the
 * route without staging (and, at 65..96 channels, the raw-word route)
 * recompute them and overwrite any element they disagree on with
 * 0x7FFFFFFF, which no similarity equals. */
ba_status ba_debug_hamming_scores(const uint32_t* qbits, const uint32_t* kbits,
                                  int B, int H, int N, int d, int bh_begin,
                                  int bh_count, int row_begin, int row_count,
                                  int32_t* sigma, void* stream);

/* Static description of a status code. */
const char* ba_status_string(ba_status s);

#ifdef __cplusplus
}
#endif
#endif /* BINATTN_H */
