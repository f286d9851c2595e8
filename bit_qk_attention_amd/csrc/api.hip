// api.hip — the extern "C" entry points declared in include/binattn.h:
// argument validation (before any HIP call), dispatch to the gfx950
// launchers, and status mapping. No C++ exception crosses this layer.
#include <stdint.h>
#include <string.h>

#include "common.h"

namespace {

using namespace binattn;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The value a caller passed for an enum argument or field, as an int. C
// callers may pass any int there; loading such a value as the C++ enum type
// is undefined, so its bytes are copied out instead.
template <class E>
int raw(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "the ABI's enums are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

bool dtype16(int dt) { return dt == BA_F16 || dt == BA_BF16; }

// Shape checks shared by every call. Returns BA_OK or the status to report.
ba_status check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return BA_ERR_INVALID_ARG;
  if (d > 128 || N > BA_MAX_TOKENS) return BA_ERR_UNSUPPORTED;
  if ((int64_t)B * H > 0x7FFFFFFF / 2) return BA_ERR_UNSUPPORTED;
  return BA_OK;
}

// [p, p+bytes) and [q, q+qbytes) overlap
bool overlap(const void* p, int64_t bytes, const void* q, int64_t qbytes) {
  if (!p || !q) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + (uintptr_t)qbytes && b < a + (uintptr_t)bytes;
}

ba_status from_hip(hipError_t e) { return e == hipSuccess ? BA_OK : BA_ERR_HIP; }

// Elements spanned by a [B, H, N, d] view with these strides (first to last
// element, plus one).
int64_t view_extent(const ba_strides& st, int B, int H, int N, int d) {
  return (int64_t)(B - 1) * st.batch + (int64_t)(H - 1) * st.head + (int64_t)(N - 1) * st.token + d;
}

// Non-negative strides whose view spans at most 2^40 elements (so no
// offset computed from them overflows).
bool strides_valid(const ba_strides* st, int B, int H, int N) {
  if (!st || st->batch < 0 || st->head < 0 || st->token < 0) return false;
  const int64_t lim = (int64_t)1 << 38;  // per dimension: 4 x 2^38 <= 2^40
  return st->batch <= lim / (B > 1 ? B - 1 : 1) && st->head <= lim / (H > 1 ? H - 1 : 1) &&
         st->token <= lim / (N > 1 ? N - 1 : 1);
}

// No two elements of the view share an address: with the dimensions of size
// > 1 in increasing stride order (channels first, stride 1), each stride
// exceeds the span of the dimensions inside it.
bool view_disjoint(const ba_strides& st, int B, int H, int N, int d) {
  int64_t dim[4][2] = {{1, d}, {st.token, N}, {st.head, H}, {st.batch, B}};
  for (int i = 1; i < 4; ++i)  // insertion sort of the outer three by stride
    for (int j = i; j > 1 && dim[j][0] < dim[j - 1][0]; --j)
      for (int e = 0; e < 2; ++e) { const int64_t t = dim[j][e]; dim[j][e] = dim[j - 1][e]; dim[j - 1][e] = t; }
  int64_t span = d;  // elements spanned by the dimensions so far
  for (int i = 1; i < 4; ++i) {
    if (dim[i][1] == 1) continue;
    if (dim[i][0] < span) return false;
    span += (dim[i][1] - 1) * dim[i][0];
  }
  return true;
}

// ba_pack_qk_quant_v on the view `in` (validated here); in_elems = the
// elements each of q, k, v spans.
// with_q false: K and V only (q, qbits, qmu unused).
ba_status prepass_checked(const void* q, const void* k, const void* v, const InView& in, int64_t in_elems,
                          int in_align, int dt, int B, int H, int N, int d, uint32_t* qbits, float* qmu,
                          uint32_t* kbits, float* kmu, int8_t* vq, float* vscale, void* stream,
                          bool with_q = true) {
  if (!with_q) q = nullptr, qbits = nullptr, qmu = nullptr;
  if ((with_q && (!q || !qbits || !qmu)) || !k || !v || !kbits || !kmu || !vq || !vscale)
    return BA_ERR_INVALID_ARG;
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (!dtype16(dt)) return BA_ERR_UNSUPPORTED;
  if (!aligned(q, in_align) || !aligned(k, in_align) || !aligned(v, in_align) || !aligned(qbits, 16) ||
      !aligned(kbits, 16) || !aligned(vq, 16) || !aligned(qmu, 4) || !aligned(kmu, 4) || !aligned(vscale, 4))
    return BA_ERR_INVALID_ARG;
  const int64_t ntok = (int64_t)B * H * N;
  const int64_t W = (d + 31) / 32;
  const int64_t nc = (int64_t)B * H * d * 4;  // bytes of vscale
  const void* outs[6] = {qbits, qmu, kbits, kmu, vq, vscale};
  const int64_t osz[6] = {ntok * W * 4, ntok * 4, ntok * W * 4, ntok * 4, ntok * d, nc};
  for (int i = 0; i < 6; ++i) {
    if (overlap(outs[i], osz[i], q, in_elems * 2) || overlap(outs[i], osz[i], k, in_elems * 2) ||
        overlap(outs[i], osz[i], v, in_elems * 2))
      return BA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j])) return BA_ERR_INVALID_ARG;
  }
  return from_hip(launch_prepass(q, k, v, (ba_dtype)dt, in, B * H, N, d, qbits, qmu, kbits, kmu, vq, vscale,
                                 static_cast<hipStream_t>(stream)));
}

// q16 != nullptr: Q given as 16-bit values of type q16_dt (qbits, qmu unused);
// kv16: K and V too, as k16 and v16 of the same type (kbits, kmu, vq, vscale
// unused).
ba_status attention_checked(const uint32_t* qbits, const float* qmu, const uint32_t* kbits, const float* kmu,
                            const int8_t* vq, const float* vscale, const ba_bias* bias, int B,
                            int H, int N, int d, void* out, const ba_strides& ost, int out_align, int out_dt,
                            void* stream, int online = 0, const void* q16 = nullptr, int q16_dt = -1,
                            bool kv16 = false, const void* k16 = nullptr, const void* v16 = nullptr) {
  if (q16) qbits = nullptr, qmu = nullptr;
  if (kv16) {
    kbits = nullptr, kmu = nullptr, vq = nullptr, vscale = nullptr;
    if (!q16 || !k16 || !v16 || !out) return BA_ERR_INVALID_ARG;
  } else if ((!q16 && (!qbits || !qmu)) || !kbits || !kmu || !vq || !vscale || !out) {
    return BA_ERR_INVALID_ARG;
  }
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (online && d > 64) return BA_ERR_UNSUPPORTED;
  if (!dtype16(out_dt)) return BA_ERR_UNSUPPORTED;
  if (q16 && (!dtype16(q16_dt) || d % 8 != 0)) return BA_ERR_UNSUPPORTED;
  if (!aligned(qbits, 16) || !aligned(kbits, 16) || !aligned(vq, 16) || !aligned(out, out_align) ||
      !aligned(qmu, 4) || !aligned(kmu, 4) || !aligned(vscale, 4) || !aligned(q16, 16) || !aligned(k16, 16) ||
      !aligned(v16, 16))
    return BA_ERR_INVALID_ARG;
  const int64_t ntok = (int64_t)B * H * N;
  const int64_t W = (d + 31) / 32;
  AttnArgs a = {};
  a.qbits = qbits; a.qmu = qmu; a.kbits = kbits; a.kmu = kmu; a.vq = vq; a.vscale = vscale;
  a.q16 = q16; a.q16_dt = q16_dt; a.k16 = k16; a.v16 = v16;
  a.B = B; a.H = H; a.N = N; a.d = d; a.out = out; a.out_dt = out_dt; a.online = online;
  a.out_sb = ost.batch; a.out_sh = ost.head; a.out_sn = ost.token;
  a.bias_kind = BA_BIAS_NONE;
  int64_t bias_bytes = 0;
  const int kind = bias ? raw(bias->kind) : BA_BIAS_NONE;
  const int bdt = bias ? raw(bias->dtype) : BA_F32;
  if (kind != BA_BIAS_NONE) {
    if (!bias->data) return BA_ERR_INVALID_ARG;
    if (kind == BA_BIAS_DENSE) {
      if (bdt != BA_F32 && bdt != BA_F16) return BA_ERR_UNSUPPORTED;
      const int64_t slice = (int64_t)H * N * N;
      if (bias->batch_stride != 0 && bias->batch_stride < slice) return BA_ERR_INVALID_ARG;
      const int esz = bdt == BA_F32 ? 4 : 2;
      if (!aligned(bias->data, esz)) return BA_ERR_INVALID_ARG;
      bias_bytes = ((int64_t)(B - 1) * bias->batch_stride + slice) * esz;
      a.bias_kind = BA_BIAS_DENSE;
      a.bias_dtype = bdt;
      a.bias_bstride = bias->batch_stride;
    } else if (kind == BA_BIAS_RELPOS) {
      if (bdt != BA_F32) return BA_ERR_UNSUPPORTED;
      if (bias->grid_h < 1 || bias->grid_w < 1 || bias->n_prefix < 0) return BA_ERR_INVALID_ARG;
      if (bias->grid_w > 256) return BA_ERR_UNSUPPORTED;  // table window must fit LDS
      if ((int64_t)bias->n_prefix + (int64_t)bias->grid_h * bias->grid_w != N) return BA_ERR_INVALID_ARG;
      if (!aligned(bias->data, 4)) return BA_ERR_INVALID_ARG;
      bias_bytes = (int64_t)H * (2 * bias->grid_h - 1) * (2 * bias->grid_w - 1) * 4;
      a.bias_kind = BA_BIAS_RELPOS;
      a.grid_h = bias->grid_h; a.grid_w = bias->grid_w; a.n_prefix = bias->n_prefix;
    } else {
      return BA_ERR_INVALID_ARG;
    }
    a.bias = bias->data;
  }
  const int64_t out_bytes = view_extent(ost, B, H, N, d) * 2;
  const void* ins[10] = {qbits, qmu, kbits, kmu, vq, vscale, a.bias, q16, k16, v16};
  const int64_t isz[10] = {ntok * W * 4, ntok * 4, ntok * W * 4, ntok * 4, ntok * d,
                           (int64_t)B * H * d * 4, bias_bytes, ntok * d * 2, ntok * d * 2, ntok * d * 2};
  for (int i = 0; i < 10; ++i)
    if (overlap(out, out_bytes, ins[i], isz[i])) return BA_ERR_INVALID_ARG;
  const hipError_t e = launch_attention(a, static_cast<hipStream_t>(stream));
  // (16-bit K and V outside the resident mode: refused before any launch)
  return (kv16 && e == hipErrorNotSupported) ? BA_ERR_UNSUPPORTED : from_hip(e);
}

}  // namespace

extern "C" {

int ba_packed_words(int d) { return d < 1 ? 0 : (d + 31) / 32; }

const char* ba_status_string(ba_status s) {
  switch (raw(s)) {
    case BA_OK: return "ok";
    case BA_ERR_INVALID_ARG: return "invalid argument";
    case BA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case BA_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

ba_status ba_pack_qk(const void* q, const void* k, ba_dtype dt, int B, int H, int N, int d,
                     uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu, void* stream) {
  if (!q || !k || !qbits || !qmu || !kbits || !kmu) return BA_ERR_INVALID_ARG;
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (!dtype16(raw(dt))) return BA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(qbits, 16) || !aligned(kbits, 16) ||
      !aligned(qmu, 4) || !aligned(kmu, 4))
    return BA_ERR_INVALID_ARG;
  const int64_t ntok = (int64_t)B * H * N;
  const int64_t W = (d + 31) / 32;
  const void* outs[4] = {qbits, qmu, kbits, kmu};
  const int64_t osz[4] = {ntok * W * 4, ntok * 4, ntok * W * 4, ntok * 4};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], osz[i], q, ntok * d * 2) || overlap(outs[i], osz[i], k, ntok * d * 2))
      return BA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j])) return BA_ERR_INVALID_ARG;
  }
  return from_hip(launch_pack_qk(q, k, dt, dense_view(H, N, d), B * H, N, d, qbits, qmu, kbits, kmu,
                                 static_cast<hipStream_t>(stream)));
}

ba_status ba_quant_v(const void* v, ba_dtype dt, int B, int H, int N, int d, int8_t* vq,
                     float* vscale, void* stream) {
  if (!v || !vq || !vscale) return BA_ERR_INVALID_ARG;
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (!dtype16(raw(dt))) return BA_ERR_UNSUPPORTED;
  if (!aligned(v, 16) || !aligned(vq, 16) || !aligned(vscale, 4)) return BA_ERR_INVALID_ARG;
  const int64_t n = (int64_t)B * H * N * d;
  const int64_t nc = (int64_t)B * H * d * 4;  // bytes of vscale
  if (overlap(vq, n, v, 2 * n) || overlap(vscale, nc, v, 2 * n) || overlap(vq, n, vscale, nc))
    return BA_ERR_INVALID_ARG;
  return from_hip(launch_quant_v(v, dt, dense_view(H, N, d), B * H, N, d, vq, vscale,
                                 static_cast<hipStream_t>(stream)));
}

ba_status ba_pack_qk_quant_v(const void* q, const void* k, const void* v, ba_dtype dt, int B, int H,
                             int N, int d, uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu,
                             int8_t* vq, float* vscale, void* stream) {
  const ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  return prepass_checked(q, k, v, dense_view(H, N, d), (int64_t)B * H * N * d, 16, raw(dt), B, H, N, d, qbits, qmu,
                         kbits, kmu, vq, vscale, stream);
}

ba_status ba_pack_qk_quant_v_strided(const void* q, const void* k, const void* v, const ba_strides* in_strides,
                                     ba_dtype dt, int B, int H, int N, int d, uint32_t* qbits, float* qmu,
                                     uint32_t* kbits, float* kmu, int8_t* vq, float* vscale, void* stream) {
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (!strides_valid(in_strides, B, H, N)) return BA_ERR_INVALID_ARG;
  InView in;
  in.sb = in_strides->batch;
  in.sh = in_strides->head;
  in.sn = in_strides->token;
  in.H = H;
  in.vec = d % 8 == 0 && in.sb % 8 == 0 && in.sh % 8 == 0 && in.sn % 8 == 0 && aligned(q, 16) &&
           aligned(k, 16) && aligned(v, 16);
  return prepass_checked(q, k, v, in, view_extent(*in_strides, B, H, N, d), 2, raw(dt), B, H, N, d, qbits, qmu, kbits,
                         kmu, vq, vscale, stream);
}

ba_status ba_pack_k_quant_v(const void* k, const void* v, ba_dtype dt, int B, int H, int N, int d,
                            uint32_t* kbits, float* kmu, int8_t* vq, float* vscale, void* stream) {
  const ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  return prepass_checked(nullptr, k, v, dense_view(H, N, d), (int64_t)B * H * N * d, 16, raw(dt), B, H, N, d,
                         nullptr, nullptr, kbits, kmu, vq, vscale, stream, false);
}

ba_status ba_attention_fwd_q16(const void* q, ba_dtype q_dt, const uint32_t* kbits, const float* kmu,
                               const int8_t* vq, const float* vscale, const ba_bias* bias, int B, int H,
                               int N, int d, void* out, ba_dtype out_dt, void* stream) {
  if (!q) return BA_ERR_INVALID_ARG;
  const ba_strides dense = {(int64_t)H * N * d, (int64_t)N * d, (int64_t)d};
  return attention_checked(nullptr, nullptr, kbits, kmu, vq, vscale, bias, B, H, N, d, out, dense, 16,
                           raw(out_dt), stream, 0, q, raw(q_dt));
}

ba_status ba_attention_fwd_qkv16(const void* q, const void* k, const void* v, ba_dtype dt, const ba_bias* bias,
                                 int B, int H, int N, int d, void* out, ba_dtype out_dt, void* stream) {
  if (!q || !k || !v) return BA_ERR_INVALID_ARG;
  const ba_strides dense = {(int64_t)H * N * d, (int64_t)N * d, (int64_t)d};
  return attention_checked(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, bias, B, H, N, d, out, dense, 16,
                           raw(out_dt), stream, 0, q, raw(dt), true, k, v);
}

ba_status ba_attention_fwd(const uint32_t* qbits, const float* qmu, const uint32_t* kbits,
                           const float* kmu, const int8_t* vq, const float* vscale,
                           const ba_bias* bias, int B, int H, int N,
                           int d, void* out, ba_dtype out_dt, void* stream) {
  // head and token strides of a dense output (N * d <= 2^23) fit 32 bits
  const ba_strides dense = {(int64_t)H * N * d, (int64_t)N * d, (int64_t)d};
  return attention_checked(qbits, qmu, kbits, kmu, vq, vscale, bias, B, H, N, d, out, dense, 16, raw(out_dt),
                           stream);
}

ba_status ba_attention_fwd_online(const uint32_t* qbits, const float* qmu, const uint32_t* kbits,
                                  const float* kmu, const int8_t* vq, const float* vscale,
                                  const ba_bias* bias, int B, int H, int N,
                                  int d, void* out, ba_dtype out_dt, void* stream) {
  const ba_strides dense = {(int64_t)H * N * d, (int64_t)N * d, (int64_t)d};
  return attention_checked(qbits, qmu, kbits, kmu, vq, vscale, bias, B, H, N, d, out, dense, 16, raw(out_dt),
                           stream, 1);
}

ba_status ba_attention_fwd_strided(const uint32_t* qbits, const float* qmu, const uint32_t* kbits,
                                   const float* kmu, const int8_t* vq, const float* vscale,
                                   const ba_bias* bias, int B, int H, int N,
                                   int d, void* out, const ba_strides* out_strides, ba_dtype out_dt,
                                   void* stream) {
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (!strides_valid(out_strides, B, H, N) || !view_disjoint(*out_strides, B, H, N, d)) return BA_ERR_INVALID_ARG;
  if (out_strides->head > 0x7FFFFFFF || out_strides->token > 0x7FFFFFFF) return BA_ERR_UNSUPPORTED;
  return attention_checked(qbits, qmu, kbits, kmu, vq, vscale, bias, B, H, N, d, out, *out_strides, 2,
                           raw(out_dt), stream);
}

ba_status ba_debug_hamming_scores(const uint32_t* qbits, const uint32_t* kbits, int B, int H,
                                  int N, int d, int bh_begin, int bh_count, int row_begin,
                                  int row_count, int32_t* sigma, void* stream) {
  if (!qbits || !kbits || !sigma) return BA_ERR_INVALID_ARG;
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (bh_count < 1 || row_count < 1 || bh_begin < 0 || row_begin < 0) return BA_ERR_INVALID_ARG;
  if ((int64_t)bh_begin + bh_count > (int64_t)B * H || (int64_t)row_begin + row_count > N)
    return BA_ERR_INVALID_ARG;
  if (!aligned(qbits, 16) || !aligned(kbits, 16) || !aligned(sigma, 4)) return BA_ERR_INVALID_ARG;
  const int64_t ntok = (int64_t)B * H * N;
  const int64_t W = (d + 31) / 32;
  const int64_t ssz = (int64_t)bh_count * row_count * N * 4;
  if (overlap(sigma, ssz, qbits, ntok * W * 4) || overlap(sigma, ssz, kbits, ntok * W * 4))
    return BA_ERR_INVALID_ARG;
  return from_hip(launch_hamming(qbits, kbits, N, d, bh_begin, bh_count, row_begin, row_count,
                                 sigma, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
