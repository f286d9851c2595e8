// prepass.hip — gfx950 kernels for the steps before the fused attention:
// sign/scale packing of Q and K, channel-wise int8 quantisation of V, and
// the integer Hamming-score debug view.
//
// Method: BinaryAttention (gist.science summaries). Scaled binary Q/K: zh
// technical summary section 2.2 item 1 (nl Methodologie 2, it/fr/pt section
// 2B). Channel-wise 8-bit V: zh section 2.2 item 3 (nl Methodologie 2).
// Hamming similarity: zh sections 2.1 and 2.2 item 1.
//
// All three are memory-bound; the kernels aim at coalesced 16-byte accesses
// and an XCD-aware block order where blocks share cache lines.
#include <algorithm>

#include "common.h"

namespace binattn {

// ---------------------------------------------------------------------------
// pack_qk, any d: one thread per token. Loads the token's d 16-bit values,
// sets bit c iff x_c < 0, and computes mu = sum|x| / d with a float64 sum
// (exact for fp16/bf16 inputs of ordinary range) and one float64 division
// rounded once to float.
// grid.y selects Q (0) or K (1). Tokens are read through the view `in`
// (any strides, 2-byte aligned).
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void pack_qk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, InView in, int N, int64_t ntok,
    int d, uint32_t* __restrict__ qbits, float* __restrict__ qmu,
    uint32_t* __restrict__ kbits, float* __restrict__ kmu) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= ntok) return;
  const int64_t bh = t / N, n = t - bh * N;
  const uint16_t* x = (blockIdx.y == 0 ? q : k) + (bh / in.H) * in.sb + (bh % in.H) * in.sh + n * in.sn;
  uint32_t* bits = (blockIdx.y == 0 ? qbits : kbits);
  float* mu = (blockIdx.y == 0 ? qmu : kmu);
  const int W = (d + 31) >> 5;
  double asum = 0.0;
  for (int w = 0; w < W; ++w) {
    uint32_t word = 0;
    const int c0 = w * 32;
    const int nc = min(32, d - c0);
    for (int c = 0; c < nc; ++c) {
      const uint16_t h = x[c0 + c];
      word |= neg_bit<DT>(h) << c;
      asum += (double)fabsf(to_f32<DT>(h));
    }
    bits[t * W + w] = word;
  }
  mu[t] = (float)(asum / (double)d);
}

// pack_qk for d % 8 == 0: the threads of a block cooperate on whole tokens.
// The block's token range is a contiguous run of 16-byte chunks (8 channels
// each, P = d/8 per token); thread i loads chunks i + 256u, u < kPackU (each
// load of the block one fully coalesced 4 KB run, kPackU of them in flight
// per thread), forms each chunk's 8 sign bits and a float64 partial sum of
// |x|. The pieces are combined through LDS: each 32-bit word from its 4
// chunks, mu from the P partial sums in channel order.
constexpr int kPackU = 4;
// One block of NT threads packs tokens [blk * TB, blk * TB + TB) of x.
// bits_s and sum_s hold NT * kPackU entries. STR: token t of x starts at
// x + t * sx (sx % 8 == 0) instead of x + t * d, so a block's chunks are
// runs of P pieces, one run per token.
template <int DT, int NT, bool STR = false>
__device__ __forceinline__ void pack_block(const uint16_t* __restrict__ x, int64_t ntok, int d, int64_t blk,
                                           uint32_t* __restrict__ bits, float* __restrict__ mu,
                                           uint32_t* bits_s, double* sum_s, int64_t sx = 0) {
  const int P = d >> 3;                  // chunks per token (1..16)
  const int TB = NT * kPackU / P;        // whole tokens per block
  const int W = (d + 31) >> 5;
  const int64_t tok0 = blk * TB;
  const int nchunk = (int)min((int64_t)TB, ntok - tok0) * P;  // valid chunks of this block
  const int i = threadIdx.x;
  // c / P for c < 4096 and P <= 16 as (c * ceil(2^16 / P)) >> 16 (exact there)
  const uint32_t pmag = STR ? (65536u + P - 1) / P : 0u;
  u4v raw[kPackU];
#pragma unroll
  for (int u = 0; u < kPackU; ++u) {
    const int c = i + NT * u;
    const uint16_t* src;
    if constexpr (STR) {
      const int tl = (int)(__umul24((uint32_t)c, pmag) >> 16);
      src = x + (tok0 + tl) * sx + 8 * (c - tl * P);
    } else {
      src = x + tok0 * d + 8 * c;
    }
    raw[u] = c < nchunk ? *reinterpret_cast<const u4v*>(src) : (u4v){0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kPackU; ++u) {
    uint32_t b8 = 0;
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // x < 0 as a float compare: false for -0 and NaN, true for -inf
      const float xf = to_f32<DT>((uint16_t)(raw[u][e >> 1] >> ((e & 1) * 16)));
      b8 |= xf < 0.0f ? (1u << e) : 0u;
      s += (double)fabsf(xf);
    }
    bits_s[i + NT * u] = b8;
    sum_s[i + NT * u] = s;
  }
  __syncthreads();
  const int ntb = nchunk / P;  // valid tokens of this block
  for (int j = i; j < ntb * W; j += NT) {
    const int tl = j / W, w = j % W;
    uint32_t word = 0;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int pc = 4 * w + pp;
      if (pc < P) word |= bits_s[tl * P + pc] << (8 * pp);
    }
    bits[(tok0 + tl) * W + w] = word;
  }
  for (int tl = i; tl < ntb; tl += NT) {
    double acc = 0.0;
    for (int pc = 0; pc < P; ++pc) acc += sum_s[tl * P + pc];
    mu[tok0 + tl] = (float)(acc / (double)d);
  }
}

// Dense inputs: the blocks take consecutive runs of the B*H*N tokens. A
// strided view (STR): nbph blocks per head, each within one head.
template <int DT, bool STR>
__global__ __launch_bounds__(256) void pack_qk_coop_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, InView in, int N, int64_t nbph,
    int64_t ntok, int d, uint32_t* __restrict__ qbits, float* __restrict__ qmu,
    uint32_t* __restrict__ kbits, float* __restrict__ kmu) {
  __shared__ uint32_t bits_s[256 * kPackU];
  __shared__ double sum_s[256 * kPackU];
  if constexpr (STR) {
    const bool isk = blockIdx.y != 0;
    const int64_t bh = blockIdx.x / nbph, tb = blockIdx.x - bh * nbph;
    const int W = (d + 31) >> 5;
    pack_block<DT, 256, true>((isk ? k : q) + (bh / in.H) * in.sb + (bh % in.H) * in.sh, N, d, tb,
                              (isk ? kbits : qbits) + bh * N * W, (isk ? kmu : qmu) + bh * N, bits_s, sum_s,
                              in.sn);
  } else if (blockIdx.y == 0) {
    pack_block<DT, 256>(q, ntok, d, blockIdx.x, qbits, qmu, bits_s, sum_s);
  } else {
    pack_block<DT, 256>(k, ntok, d, blockIdx.x, kbits, kmu, bits_s, sum_s);
  }
}

InView dense_view(int H, int N, int d) {
  InView v;
  v.sn = d;
  v.sh = (int64_t)N * d;
  v.sb = (int64_t)H * v.sh;
  v.H = H;
  v.vec = d % 8 == 0;
  return v;
}

hipError_t launch_pack_qk(const void* q, const void* k, ba_dtype dt, const InView& in, int nbh, int N,
                          int d, uint32_t* qbits, float* qmu, uint32_t* kbits,
                          float* kmu, hipStream_t s) {
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const int64_t ntok = (int64_t)nbh * N;
  if (in.vec) {
    const int TB = 256 * kPackU / (d / 8);
    const bool str = !in.dense(N, d);
    const int64_t nbph = (N + TB - 1) / TB;
    const int64_t nblk = str ? nbh * nbph : (ntok + TB - 1) / TB;
    if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nblk, 2);
    auto kern = dt == BA_F16 ? (str ? pack_qk_coop_kernel<BA_F16, true> : pack_qk_coop_kernel<BA_F16, false>)
                             : (str ? pack_qk_coop_kernel<BA_BF16, true> : pack_qk_coop_kernel<BA_BF16, false>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, q16, k16, in, N, nbph, ntok, d, qbits, qmu, kbits, kmu);
    return hipGetLastError();
  }
  if ((ntok + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((ntok + 255) / 256), 2);
  if (dt == BA_F16)
    hipLaunchKernelGGL(pack_qk_kernel<BA_F16>, grid, dim3(256), 0, s, q16, k16, in, N, ntok, d, qbits, qmu, kbits, kmu);
  else
    hipLaunchKernelGGL(pack_qk_kernel<BA_BF16>, grid, dim3(256), 0, s, q16, k16, in, N, ntok, d, qbits, qmu, kbits, kmu);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// quant_v, element path (d % 8 != 0, or rows of a strided view that are not
// 16-byte aligned): one block per head, one thread per (row, channel)
// element with scalar accesses. Pass 1 takes the per-channel max |v| (an
// LDS atomic max on the float bits, valid because the values are
// non-negative), pass 2 quantises with inv = 127/amax, writes int8 and
// gathers the channel sums of the int8 values (LDS atomic adds).
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void quant_v_kernel(
    const uint16_t* __restrict__ v, InView in, int N, int d,
    int8_t* __restrict__ vq, float* __restrict__ vscale, int32_t* __restrict__ vsum) {
  __shared__ uint32_t amax_bits[128];
  __shared__ float inv_s[128];
  __shared__ int32_t sum_s[128];
  const int bh = blockIdx.x;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    amax_bits[i] = 0u;
    sum_s[i] = 0;
  }
  __syncthreads();
  const uint16_t* vh = v + (int64_t)(bh / in.H) * in.sb + (int64_t)(bh % in.H) * in.sh;  // row j at j * in.sn
  int8_t* qh = vq + (int64_t)bh * N * d;
  for (int idx = threadIdx.x; idx < N * d; idx += blockDim.x) {
    const int j = idx / d, c = idx % d;
    atomicMax(&amax_bits[c], __float_as_uint(fabsf(to_f32<DT>(vh[(int64_t)j * in.sn + c]))));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float a = __uint_as_float(amax_bits[i]);
    inv_s[i] = a > 0.0f ? 127.0f / a : 0.0f;
    vscale[(int64_t)bh * d + i] = a / 127.0f;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < N * d; idx += blockDim.x) {
    const int j = idx / d, c = idx % d;
    float y = __builtin_rintf(to_f32<DT>(vh[(int64_t)j * in.sn + c]) * inv_s[c]);
    y = fminf(fmaxf(y, -127.0f), 127.0f);
    qh[(int64_t)j * d + c] = (int8_t)(int)y;
    atomicAdd(&sum_s[c], (int)y);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < d; i += blockDim.x) vsum[(int64_t)bh * d + i] = sum_s[i];
}

// quant_v for heads that fit in registers (d % 8 == 0): a block of 1024
// threads quantises HB heads (HB = 1024 / T, T threads per head, a power of
// two chosen so that no thread holds more than kQvRows rows), reading each
// head once. A head is row-major N x d, so thread t < R*P of its group
// (P = d/8 16-byte pieces per row, R = T/P rows per sweep) owns piece t % P
// of rows t / P + k*R: every load of the group is one contiguous run of
// 16*R*P bytes. Channel maxima go through an LDS atomic max on the float
// bits (non-negative), then the held values are quantised and written as
// int8, and their channel sums gathered with LDS atomic adds.
constexpr int kQvRows = 12;  // rows per thread held in registers
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
// heads bh0 .. bh0 + HB - 1 (those below nbh) by one block of 1024
// threads; smem holds 3 * 128 words per head
template <int DT>
__device__ __forceinline__ void quant_heads_block(const uint16_t* __restrict__ v, const InView& in, int N, int d,
                                                  int64_t bh0,
                                                  int64_t nbh, int HB, int8_t* __restrict__ vq,
                                                  float* __restrict__ vscale, int32_t* __restrict__ vsum,
                                                  uint32_t* smem) {
  const int T = 1024 / HB;
  const int hs = threadIdx.x / T, t = threadIdx.x % T;
  const int64_t bh = bh0 + hs;
  const bool hvalid = bh < nbh;
  uint32_t* amax_bits = smem + 384 * hs;
  float* inv_s = reinterpret_cast<float*>(amax_bits + 128);
  int32_t* sum_s = reinterpret_cast<int32_t*>(amax_bits + 256);
  const int P = d >> 3, R = T / P;
  const int piece = t % P, r0 = t / P;
  const bool active = hvalid && r0 < R;
  if (t < d) {
    amax_bits[t] = 0u;
    sum_s[t] = 0;
  }
  __syncthreads();
  const uint16_t* vh = v + (hvalid ? (bh / in.H) * in.sb + (bh % in.H) * in.sh : 0) + 8 * piece;
  int8_t* qh = vq + (hvalid ? bh * N * d : 0) + 8 * piece;
  u4v x[kQvRows];
#pragma unroll
  for (int k = 0; k < kQvRows; ++k) {
    const int r = r0 + k * R;
    x[k] = (active && r < N) ? *reinterpret_cast<const u4v*>(vh + (int64_t)r * in.sn) : (u4v){0u, 0u, 0u, 0u};
  }
  // max |v| per channel on the 16-bit patterns: for finite fp16 / bf16
  // values the magnitude bits (sign cleared) order like |v|, so a packed
  // 16-bit integer max over the rows gives the pattern of the maximum
  us2 mb[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
#pragma unroll
  for (int k = 0; k < kQvRows; ++k)
#pragma unroll
    for (int w = 0; w < 4; ++w)
      mb[w] = __builtin_elementwise_max(mb[w], __builtin_bit_cast(us2, x[k][w] & 0x7FFF7FFFu));
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = to_f32<DT>(mb[e >> 1][e & 1]);
  if (active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) atomicMax(&amax_bits[8 * piece + e], __float_as_uint(m[e]));
  }
  __syncthreads();
  if (hvalid && t < d) {
    const float a = __uint_as_float(amax_bits[t]);
    inv_s[t] = a > 0.0f ? 127.0f / a : 0.0f;
    vscale[bh * d + t] = a / 127.0f;
  }
  __syncthreads();
  float inv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) inv[e] = inv_s[8 * piece + e];
  int csum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < kQvRows; ++k) {
    const int r = r0 + k * R;
    if (active && r < N) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float y = __builtin_rintf(to_f32<DT>((uint16_t)(x[k][e >> 1] >> ((e & 1) * 16))) * inv[e]);
        y = fminf(fmaxf(y, -127.0f), 127.0f);
        csum[e] += (int)y;
        const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)y;
        if (e < 4) lo |= b << (8 * e); else hi |= b << (8 * (e - 4));
      }
      *reinterpret_cast<uint2*>(qh + (int64_t)r * d) = make_uint2(lo, hi);
    }
  }
  if (active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) atomicAdd(&sum_s[8 * piece + e], csum[e]);
  }
  __syncthreads();
  if (hvalid && t < d) vsum[bh * d + t] = sum_s[t];
}

// Heads per 1024-thread block for the register-resident quantiser: the most
// (a power of two, at most 8) whose T = 1024 / HB threads per head still
// hold at most 8 rows each (kQvRows when one head takes the whole block),
// while leaving at least 64 blocks; with fewer heads than that, one head
// per block keeps each head's rows spread over all 1024 threads.
int quant_heads_per_block(int nbh, int N, int d) {
  const int P = d / 8;
  for (int hb = 8; hb > 1; hb >>= 1) {
    const int T = 1024 / hb;
    if (T >= P && (int64_t)N <= 8 * (int64_t)(T / P) && nbh >= 64 * hb) return hb;
  }
  return 1;
}

template <int DT>
__global__ __launch_bounds__(1024) void quant_v_head_kernel(
    const uint16_t* __restrict__ v, InView in, int nbh, int N, int d, int HB, int8_t* __restrict__ vq,
    float* __restrict__ vscale, int32_t* __restrict__ vsum) {
  __shared__ uint32_t smem[8 * 3 * 128];
  quant_heads_block<DT>(v, in, N, d, (int64_t)blockIdx.x * HB, nbh, HB, vq, vscale, vsum, smem);
}

// Pack Q and K and quantise V in one launch (d % 8 == 0, heads that fit the
// register-resident quantiser): blocks 0 .. nvb-1 quantise HB heads each
// (the long-running ones, dispatched first), the rest pack npb blocks of
// tokens of Q, then npb of K, all with 1024 threads. STR (a strided view):
// the pack blocks are nbph per head, each within one head.
template <int DT, bool STR>
__global__ __launch_bounds__(1024) void prepass_fused_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, InView in,
    int nbh, int N, int d, int HB, int64_t nvb, int64_t npb, int64_t nbph, uint32_t* __restrict__ qbits,
    float* __restrict__ qmu, uint32_t* __restrict__ kbits, float* __restrict__ kmu, int8_t* __restrict__ vq,
    float* __restrict__ vscale, int32_t* __restrict__ vsum) {
  __shared__ uint32_t bits_s[1024 * kPackU];
  __shared__ double sum_s[1024 * kPackU];
  const int64_t ntok = (int64_t)nbh * N;
  const int64_t b = blockIdx.x;
  if (b < nvb) {
    quant_heads_block<DT>(v, in, N, d, b * HB, nbh, HB, vq, vscale, vsum, bits_s);
  } else if constexpr (STR) {
    const bool isk = b - nvb >= npb;
    const int64_t pb = b - nvb - (isk ? npb : 0);
    const int64_t bh = pb / nbph, tb = pb - bh * nbph;
    const int W = (d + 31) >> 5;
    pack_block<DT, 1024, true>((isk ? k : q) + (bh / in.H) * in.sb + (bh % in.H) * in.sh, N, d, tb,
                               (isk ? kbits : qbits) + bh * N * W, (isk ? kmu : qmu) + bh * N, bits_s, sum_s,
                               in.sn);
  } else if (b - nvb < npb) {
    pack_block<DT, 1024>(q, ntok, d, b - nvb, qbits, qmu, bits_s, sum_s);
  } else {
    pack_block<DT, 1024>(k, ntok, d, b - nvb - npb, kbits, kmu, bits_s, sum_s);
  }
}

// quant_v for long heads (16-byte rows, heads past the register-resident
// quantiser): the rows of each head are split over S blocks so that the whole
// chip streams V. After a zero fill of vscale and vsum, pass A takes each
// block's channel maxima of |v| and combines them with a global atomic max
// on the float bits kept in vscale (valid for non-negative values); pass B
// reads them back, quantises with inv = 127 / amax, writes int8 and combines
// the channel sums with global atomic adds into vsum; a last pass turns the
// maxima into vscale = amax / 127. The arithmetic is that of the one-block
// quantisers, so the outputs are the same bit for bit.
__global__ __launch_bounds__(256) void zero2_kernel(uint32_t* __restrict__ a, int32_t* __restrict__ b, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    a[i] = 0u;
    b[i] = 0;
  }
}

__global__ __launch_bounds__(256) void amax_to_scale_kernel(float* __restrict__ vscale, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) vscale[i] = vscale[i] / 127.0f;  // amax, held as its float bits, to the scale
}

// Block x: head x / S, rows [s * RB, min(N, s * RB + RB)) with s = x % S.
// QUANT false: pass A (maxima into amax_bits); true: pass B.
template <int DT, bool QUANT>
__global__ __launch_bounds__(256) void quant_v_split_kernel(
    const uint16_t* __restrict__ v, InView in, int N, int d, int S, int RB, int8_t* __restrict__ vq,
    uint32_t* __restrict__ amax_bits, int32_t* __restrict__ vsum) {
  __shared__ uint32_t red[128];  // channel maxima (pass A) or sums (pass B)
  __shared__ float inv_s[128];
  const int64_t bh = blockIdx.x / S;
  const int r_begin = (int)(blockIdx.x - bh * S) * RB, r_end = min(N, r_begin + RB);
  const int P = d >> 3, rows = 256 / P;  // 16-byte pieces per row, rows per sweep
  const int piece = threadIdx.x % P, r0 = threadIdx.x / P;
  const bool active = r0 < rows;
  if (threadIdx.x < d) {
    red[threadIdx.x] = 0u;
    if (QUANT) {
      const float a = __uint_as_float(amax_bits[bh * d + threadIdx.x]);
      inv_s[threadIdx.x] = a > 0.0f ? 127.0f / a : 0.0f;
    }
  }
  __syncthreads();
  const uint16_t* vh = v + (bh / in.H) * in.sb + (bh % in.H) * in.sh + 8 * piece;  // row j at j * in.sn
  if constexpr (!QUANT) {
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto take = [&](const u4v& raw) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        m[e] = fmaxf(m[e], fabsf(to_f32<DT>((uint16_t)(raw[e >> 1] >> ((e & 1) * 16)))));
    };
    if (active) {
      int j = r_begin + r0;
      for (; j + 7 * rows < r_end; j += 8 * rows) {  // 8 rows in flight per thread
        u4v raw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) raw[u] = *reinterpret_cast<const u4v*>(vh + (int64_t)(j + u * rows) * in.sn);
#pragma unroll
        for (int u = 0; u < 8; ++u) take(raw[u]);
      }
      for (; j < r_end; j += rows) take(*reinterpret_cast<const u4v*>(vh + (int64_t)j * in.sn));
#pragma unroll
      for (int e = 0; e < 8; ++e) atomicMax(&red[8 * piece + e], __float_as_uint(m[e]));
    }
    __syncthreads();
    if (threadIdx.x < d && red[threadIdx.x] != 0u) atomicMax(&amax_bits[bh * d + threadIdx.x], red[threadIdx.x]);
  } else {
    float inv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) inv[e] = inv_s[8 * piece + e];
    int csum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto quant8 = [&](const u4v& raw) -> uint2 {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float y = __builtin_rintf(to_f32<DT>((uint16_t)(raw[e >> 1] >> ((e & 1) * 16))) * inv[e]);
        y = fminf(fmaxf(y, -127.0f), 127.0f);
        csum[e] += (int)y;
        const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)y;
        if (e < 4) lo |= b << (8 * e); else hi |= b << (8 * (e - 4));
      }
      return make_uint2(lo, hi);
    };
    int8_t* qh = vq + bh * N * d + 8 * piece;
    if (active) {
      int j = r_begin + r0;
      for (; j + 7 * rows < r_end; j += 8 * rows) {
        u4v raw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) raw[u] = *reinterpret_cast<const u4v*>(vh + (int64_t)(j + u * rows) * in.sn);
#pragma unroll
        for (int u = 0; u < 8; ++u) *reinterpret_cast<uint2*>(qh + (int64_t)(j + u * rows) * d) = quant8(raw[u]);
      }
      for (; j < r_end; j += rows)
        *reinterpret_cast<uint2*>(qh + (int64_t)j * d) = quant8(*reinterpret_cast<const u4v*>(vh + (int64_t)j * in.sn));
#pragma unroll
      for (int e = 0; e < 8; ++e) atomicAdd(reinterpret_cast<int32_t*>(&red[8 * piece + e]), csum[e]);
    }
    __syncthreads();
    const int32_t sum = (int32_t)red[threadIdx.x < d ? threadIdx.x : 0];
    if (threadIdx.x < d && sum != 0) atomicAdd(&vsum[bh * d + threadIdx.x], sum);
  }
}

template <int DT>
hipError_t launch_quant_v_split(const uint16_t* v, const InView& in, int nbh, int N, int d, int8_t* vq,
                                float* vscale, int32_t* vsum, hipStream_t s) {
  const int rows = 256 / (d / 8);
  // about four blocks per CU, each with at least one full sweep of 8 rows per thread
  const int64_t want = (1024 + (int64_t)nbh - 1) / nbh;
  const int64_t cap = std::max<int64_t>(1, N / (8 * rows));
  const int S0 = (int)std::min(want, cap);
  const int RB = (N + S0 - 1) / S0;
  const int S = (N + RB - 1) / RB;
  const int64_t nblk = (int64_t)nbh * S, n = (int64_t)nbh * d;
  if (nblk > 0x7FFFFFFF || (n + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(vscale);
  const unsigned nz = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(zero2_kernel, dim3(nz), dim3(256), 0, s, amax_bits, vsum, n);
  hipLaunchKernelGGL((quant_v_split_kernel<DT, false>), dim3((unsigned)nblk), dim3(256), 0, s, v, in, N, d, S, RB, vq,
                     amax_bits, vsum);
  hipLaunchKernelGGL((quant_v_split_kernel<DT, true>), dim3((unsigned)nblk), dim3(256), 0, s, v, in, N, d, S, RB, vq,
                     amax_bits, vsum);
  hipLaunchKernelGGL(amax_to_scale_kernel, dim3(nz), dim3(256), 0, s, vscale, n);
  return hipGetLastError();
}

hipError_t launch_quant_v(const void* v, ba_dtype dt, const InView& in, int nbh, int N, int d,
                          int8_t* vq, float* vscale, int32_t* vsum, hipStream_t s) {
  if (in.vec && (int64_t)N <= (int64_t)kQvRows * (1024 / (d / 8))) {
    const uint16_t* v16 = static_cast<const uint16_t*>(v);
    const int HB = quant_heads_per_block(nbh, N, d);
    const unsigned nvb = (unsigned)((nbh + HB - 1) / HB);
    if (dt == BA_F16)
      hipLaunchKernelGGL(quant_v_head_kernel<BA_F16>, dim3(nvb), dim3(1024), 0, s, v16, in, nbh, N, d, HB, vq, vscale,
                         vsum);
    else
      hipLaunchKernelGGL(quant_v_head_kernel<BA_BF16>, dim3(nvb), dim3(1024), 0, s, v16, in, nbh, N, d, HB, vq, vscale,
                         vsum);
    return hipGetLastError();
  }
  if (in.vec) {
    const uint16_t* v16 = static_cast<const uint16_t*>(v);
    return dt == BA_F16 ? launch_quant_v_split<BA_F16>(v16, in, nbh, N, d, vq, vscale, vsum, s)
                        : launch_quant_v_split<BA_BF16>(v16, in, nbh, N, d, vq, vscale, vsum, s);
  }
  // element path (d % 8 != 0 or rows not 16-byte aligned): one block per head
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  if (dt == BA_F16)
    hipLaunchKernelGGL(quant_v_kernel<BA_F16>, dim3((unsigned)nbh), dim3(256), 0, s, v16, in, N, d, vq, vscale, vsum);
  else
    hipLaunchKernelGGL(quant_v_kernel<BA_BF16>, dim3((unsigned)nbh), dim3(256), 0, s, v16, in, N, d, vq, vscale, vsum);
  return hipGetLastError();
}

bool prepass_fusable(int N, int d) {
  return d % 8 == 0 && (int64_t)N <= (int64_t)kQvRows * (1024 / (d / 8));
}

hipError_t launch_prepass(const void* q, const void* k, const void* v, ba_dtype dt, const InView& in, int nbh,
                          int N, int d, uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu, int8_t* vq,
                          float* vscale, int32_t* vsum, hipStream_t s) {
  const int64_t ntok = (int64_t)nbh * N;
  if (!in.vec || !prepass_fusable(N, d)) {
    hipError_t e = launch_pack_qk(q, k, dt, in, nbh, N, d, qbits, qmu, kbits, kmu, s);
    if (e != hipSuccess) return e;
    return launch_quant_v(v, dt, in, nbh, N, d, vq, vscale, vsum, s);
  }
  const int TB = 1024 * kPackU / (d / 8);
  const bool str = !in.dense(N, d);
  const int64_t nbph = (N + TB - 1) / TB;
  const int64_t npb = str ? nbh * nbph : (ntok + TB - 1) / TB;
  const int HB = quant_heads_per_block(nbh, N, d);
  const int64_t nvb = (nbh + HB - 1) / HB;
  const int64_t nblk = nvb + 2 * npb;
  if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  auto kern = dt == BA_F16 ? (str ? prepass_fused_kernel<BA_F16, true> : prepass_fused_kernel<BA_F16, false>)
                           : (str ? prepass_fused_kernel<BA_BF16, true> : prepass_fused_kernel<BA_BF16, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(1024), 0, s, q16, k16, v16, in, nbh, N, d, HB, nvb, npb, nbph,
                     qbits, qmu, kbits, kmu, vq, vscale, vsum);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Hamming debug view: sigma = d - 2*popcount(q xor k), one thread per key.
// Grid: x = key blocks of 256, y = query rows of the window, z = heads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void hamming_kernel(
    const uint32_t* __restrict__ qbits, const uint32_t* __restrict__ kbits, int N,
    int d, int W, int bh_begin, int row_begin, int row_count, int32_t* __restrict__ sigma) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int r = blockIdx.y;
  const int hb = blockIdx.z;
  if (j >= N) return;
  const int64_t bh = bh_begin + hb;
  const uint32_t* qi = qbits + (bh * N + row_begin + r) * W;
  const uint32_t* kj = kbits + (bh * N + j) * W;
  int h = 0;
  for (int w = 0; w < W; ++w) h += __builtin_popcount(qi[w] ^ kj[w]);
  sigma[((int64_t)hb * row_count + r) * N + j] = d - 2 * h;
}

hipError_t launch_hamming(const uint32_t* qbits, const uint32_t* kbits, int N,
                          int d, int bh_begin, int bh_count, int row_begin,
                          int row_count, int32_t* sigma, hipStream_t s) {
  const int W = (d + 31) / 32;
  // grid.y is limited to 65535 rows per launch; split larger windows
  for (int r0 = 0; r0 < row_count; r0 += 65535) {
    const int rc = min(65535, row_count - r0);
    for (int h0 = 0; h0 < bh_count; h0 += 65535) {
      const int hc = min(65535, bh_count - h0);
      hipLaunchKernelGGL(hamming_kernel, dim3((N + 255) / 256, rc, hc), dim3(256), 0, s,
                         qbits, kbits, N, d, W, bh_begin + h0, row_begin + r0, row_count,
                         sigma + ((int64_t)h0 * row_count + r0) * N);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace binattn
