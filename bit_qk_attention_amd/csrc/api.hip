// api.hip — the extern "C" entry points declared in include/binattn.h:
// argument validation (before any HIP call), dispatch to the gfx950
// launchers, and status mapping. No C++ exception crosses this layer.
#include <stdint.h>

#include "common.h"

namespace {

using namespace binattn;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool dtype16(ba_dtype dt) { return dt == BA_F16 || dt == BA_BF16; }

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

}  // namespace

extern "C" {

int ba_packed_words(int d) { return d < 1 ? 0 : (d + 31) / 32; }

const char* ba_status_string(ba_status s) {
  switch (s) {
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
  if (!dtype16(dt)) return BA_ERR_UNSUPPORTED;
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
  return from_hip(launch_pack_qk(q, k, dt, ntok, d, qbits, qmu, kbits, kmu,
                                 static_cast<hipStream_t>(stream)));
}

ba_status ba_quant_v(const void* v, ba_dtype dt, int B, int H, int N, int d, int8_t* vq,
                     float* vscale, int32_t* vsum, void* stream) {
  if (!v || !vq || !vscale || !vsum) return BA_ERR_INVALID_ARG;
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (!dtype16(dt)) return BA_ERR_UNSUPPORTED;
  if (!aligned(v, 16) || !aligned(vq, 16) || !aligned(vscale, 4) || !aligned(vsum, 4))
    return BA_ERR_INVALID_ARG;
  const int64_t n = (int64_t)B * H * N * d;
  const int64_t nc = (int64_t)B * H * d * 4;  // bytes of vscale, of vsum
  const void* outs[3] = {vq, vscale, vsum};
  const int64_t osz[3] = {n, nc, nc};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], osz[i], v, 2 * n)) return BA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j])) return BA_ERR_INVALID_ARG;
  }
  return from_hip(launch_quant_v(v, dt, B * H, N, d, vq, vscale, vsum, static_cast<hipStream_t>(stream)));
}

ba_status ba_pack_qk_quant_v(const void* q, const void* k, const void* v, ba_dtype dt, int B, int H,
                             int N, int d, uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu,
                             int8_t* vq, float* vscale, int32_t* vsum, void* stream) {
  if (!q || !k || !v || !qbits || !qmu || !kbits || !kmu || !vq || !vscale || !vsum) return BA_ERR_INVALID_ARG;
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (!dtype16(dt)) return BA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(qbits, 16) || !aligned(kbits, 16) ||
      !aligned(vq, 16) || !aligned(qmu, 4) || !aligned(kmu, 4) || !aligned(vscale, 4) || !aligned(vsum, 4))
    return BA_ERR_INVALID_ARG;
  const int64_t ntok = (int64_t)B * H * N;
  const int64_t W = (d + 31) / 32;
  const int64_t nc = (int64_t)B * H * d * 4;  // bytes of vscale, of vsum
  const void* outs[7] = {qbits, qmu, kbits, kmu, vq, vscale, vsum};
  const int64_t osz[7] = {ntok * W * 4, ntok * 4, ntok * W * 4, ntok * 4, ntok * d, nc, nc};
  for (int i = 0; i < 7; ++i) {
    if (overlap(outs[i], osz[i], q, ntok * d * 2) || overlap(outs[i], osz[i], k, ntok * d * 2) ||
        overlap(outs[i], osz[i], v, ntok * d * 2))
      return BA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 7; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j])) return BA_ERR_INVALID_ARG;
  }
  return from_hip(launch_prepass(q, k, v, dt, B * H, N, d, qbits, qmu, kbits, kmu, vq, vscale, vsum,
                                 static_cast<hipStream_t>(stream)));
}

ba_status ba_attention_fwd(const uint32_t* qbits, const float* qmu, const uint32_t* kbits,
                           const float* kmu, const int8_t* vq, const float* vscale,
                           const int32_t* vsum, const ba_bias* bias, int B, int H, int N,
                           int d, void* out, ba_dtype out_dt, void* stream) {
  if (!qbits || !qmu || !kbits || !kmu || !vq || !vscale || !vsum || !out) return BA_ERR_INVALID_ARG;
  ba_status st = check_shape(B, H, N, d);
  if (st != BA_OK) return st;
  if (!dtype16(out_dt)) return BA_ERR_UNSUPPORTED;
  if (!aligned(qbits, 16) || !aligned(kbits, 16) || !aligned(vq, 16) || !aligned(out, 16) ||
      !aligned(qmu, 4) || !aligned(kmu, 4) || !aligned(vscale, 4) || !aligned(vsum, 4))
    return BA_ERR_INVALID_ARG;
  const int64_t ntok = (int64_t)B * H * N;
  const int64_t W = (d + 31) / 32;
  AttnArgs a = {};
  a.qbits = qbits; a.qmu = qmu; a.kbits = kbits; a.kmu = kmu; a.vq = vq; a.vscale = vscale;
  a.vsum = vsum;
  a.B = B; a.H = H; a.N = N; a.d = d; a.out = out; a.out_dt = out_dt;
  a.bias_kind = BA_BIAS_NONE;
  int64_t bias_bytes = 0;
  if (bias && bias->kind != BA_BIAS_NONE) {
    if (!bias->data) return BA_ERR_INVALID_ARG;
    if (bias->kind == BA_BIAS_DENSE) {
      if (bias->dtype != BA_F32 && bias->dtype != BA_F16) return BA_ERR_UNSUPPORTED;
      const int64_t slice = (int64_t)H * N * N;
      if (bias->batch_stride != 0 && bias->batch_stride < slice) return BA_ERR_INVALID_ARG;
      const int esz = bias->dtype == BA_F32 ? 4 : 2;
      if (!aligned(bias->data, esz)) return BA_ERR_INVALID_ARG;
      bias_bytes = ((int64_t)(B - 1) * bias->batch_stride + slice) * esz;
      a.bias_kind = BA_BIAS_DENSE;
      a.bias_dtype = bias->dtype;
      a.bias_bstride = bias->batch_stride;
    } else if (bias->kind == BA_BIAS_RELPOS) {
      if (bias->dtype != BA_F32) return BA_ERR_UNSUPPORTED;
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
  const int64_t out_bytes = ntok * d * 2;
  const void* ins[8] = {qbits, qmu, kbits, kmu, vq, vscale, vsum, a.bias};
  const int64_t isz[8] = {ntok * W * 4, ntok * 4, ntok * W * 4, ntok * 4, ntok * d,
                          (int64_t)B * H * d * 4, (int64_t)B * H * d * 4, bias_bytes};
  for (int i = 0; i < 8; ++i)
    if (overlap(out, out_bytes, ins[i], isz[i])) return BA_ERR_INVALID_ARG;
  return from_hip(launch_attention(a, static_cast<hipStream_t>(stream)));
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
