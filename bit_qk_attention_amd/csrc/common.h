// common.h — internal declarations shared by the gfx950 kernels and the
// C-ABI layer of the BinaryAttention library. Not a public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "binattn.h"

namespace binattn {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

// ---- 16-bit formats -------------------------------------------------------

// Widen an fp16 / bf16 bit pattern to float (exact).
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, h);
  return (float)x;
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}
template <int DT>
__device__ __forceinline__ float to_f32(uint16_t h) {
  return DT == BA_F16 ? f16_to_f32(h) : bf16_to_f32(h);
}

// True iff the 16-bit value is < 0 (negative, non-zero, not NaN), i.e. its
// sign is -1 under the convention sign(+0) = sign(-0) = +1.
template <int DT>
__device__ __forceinline__ uint32_t neg_bit(uint16_t h) {
  const uint32_t mag = h & 0x7FFFu;
  const uint32_t inf = DT == BA_F16 ? 0x7C00u : 0x7F80u;
  return (h >> 15) & (uint32_t)(mag != 0u) & (uint32_t)(mag <= inf);
}

// Round float to fp16 / bf16, nearest even.
__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- channel-wise int8 V ---------------------------------------------------

// The int8 codes clamp(rne(x * inv), -127, 127) of 8 values (16-bit
// patterns in 4 dwords, channel e with its inv[e] = 127 / amax_e in float32,
// or 0), as two dwords of bytes. The product is rounded to float32, then
// 1.5 * 2^23 is added: that sum has a unit spacing of 1, so it is the
// product rounded once to an integer (ties to even, as rintf) plus 1.5 * 2^23,
// and its bit pattern is 0x4B400000 + that integer, whose low byte is the
// integer's two's-complement code. For |x| <= amax, |x * inv| <= 127 (1 +
// 2^-24)^2 < 127.5, so the integer lies in [-127, 127] and the clamp never
// acts. Contraction into a fused multiply-add is off (it would round the
// exact product and the sum once, not the product first).
template <int DT>
__device__ __forceinline__ uint2 quant8_codes(const u4v& raw, const float* inv) {
#pragma clang fp contract(off)
  uint32_t u[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = to_f32<DT>((uint16_t)(raw[e >> 1] >> ((e & 1) * 16))) * inv[e];
    u[e] = __float_as_uint(t + 12582912.0f);
  }
  const uint32_t lo = __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0400u) | __builtin_amdgcn_perm(u[3], u[2], 0x04000c0cu);
  const uint32_t hi = __builtin_amdgcn_perm(u[5], u[4], 0x0c0c0400u) | __builtin_amdgcn_perm(u[7], u[6], 0x04000c0cu);
  return make_uint2(lo, hi);
}

// ---- launchers (host side; arguments already validated) -------------------

// Element strides of a [B, H, N, d] view of 16-bit Q, K or V with contiguous
// channels: token (b, h, n) starts at b*sb + h*sh + n*sn. vec: every token
// row starts 16-byte aligned (d % 8 == 0, strides % 8 == 0, aligned bases),
// so the kernels may load whole 16-byte pieces.
struct InView {
  int64_t sb, sh, sn;
  int H;
  bool vec;
  bool dense(int N, int d) const { return sn == d && sh == (int64_t)N * d && sb == (int64_t)H * sh; }
};
InView dense_view(int H, int N, int d);

// zero, nzero: a buffer of nzero words the packing launch also zeroes.
// q == nullptr (launch_pack_qk, launch_prepass): K (and V) only.
hipError_t launch_pack_qk(const void* q, const void* k, ba_dtype dt, const InView& in, int nbh, int N,
                          int d, uint32_t* qbits, float* qmu, uint32_t* kbits,
                          float* kmu, hipStream_t s, uint32_t* zero = nullptr, int64_t nzero = 0);
hipError_t launch_quant_v(const void* v, ba_dtype dt, const InView& in, int nbh, int N, int d,
                          int8_t* vq, float* vscale, hipStream_t s);
hipError_t launch_prepass(const void* q, const void* k, const void* v, ba_dtype dt, const InView& in, int nbh,
                          int N, int d, uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu, int8_t* vq,
                          float* vscale, hipStream_t s);
// The integer similarity of a window, computed by the attention kernel's own
// Q.K routes (attention.hip).
hipError_t launch_hamming(const uint32_t* qbits, const uint32_t* kbits, int N,
                          int d, int bh_begin, int bh_count, int row_begin,
                          int row_count, int32_t* sigma, hipStream_t s);

struct AttnArgs {
  const uint32_t* qbits;
  const float* qmu;
  const uint32_t* kbits;
  const float* kmu;
  const int8_t* vq;
  const float* vscale;
  int bias_kind;           // ba_bias_kind
  const void* bias;
  int bias_dtype;          // dense: BA_F32 / BA_F16
  int64_t bias_bstride;    // dense: elements between batch slices
  int grid_h, grid_w, n_prefix;
  int B, H, N, d;
  void* out;
  int out_dt;
  int64_t out_sb, out_sh, out_sn;  // element strides of out's [B, H, N, d] view
  int online;                      // one pass with a running maximum (d <= 64)
  const void* q16;                 // Q as 16-bit values [B,H,N,d] (d % 8 == 0), packed by the
  int q16_dt;                      // attention kernel itself; then qbits and qmu are unused
  const void* k16;                 // K and V as 16-bit values of q16_dt, binarised and quantised
  const void* v16;                 // in the resident mode (heads of at most 256 tokens; the launch
                                   // returns hipErrorNotSupported where it does not apply)
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

}  // namespace binattn
