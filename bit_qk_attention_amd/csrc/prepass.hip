// prepass.hip — gfx950 kernels for the steps before the fused attention:
// sign/scale packing of Q and K and channel-wise int8 quantisation of V.
//
// Method: BinaryAttention (gist.science summaries). Scaled binary Q/K: zh
// technical summary section 2.2 item 1 (nl Methodologie 2, it/fr/pt section
// 2B). Channel-wise 8-bit V: zh section 2.2 item 3 (nl Methodologie 2).
//
// Both are memory-bound; the kernels aim at coalesced 16-byte accesses
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
// each, P = d/8 per token); thread i loads chunks i + 256u, u < U (each
// load of the block one fully coalesced 4 KB run, U of them in flight
// per thread), forms each chunk's 8 sign bits and a float64 partial sum of
// |x|. The pieces are combined through LDS: each 32-bit word from its 4
// chunks, mu from the P partial sums in channel order.
constexpr int kPackUCoop = 2;
// U (chunks per thread) is 2 for the standalone packer (4096 tokens: 18.3 ->
// 17.6 us for the pre-pass against 4) and for the fused pre-pass (two
// blocks per CU: DiT-512 14.2 -> 13.8 us against 4, 16.0 with 1).
constexpr int kPackUFused = 2;
// One block of NT threads packs tokens [blk * TB, blk * TB + TB) of x.
// bits_s and sum_s hold NT * U entries. STR: token t of x starts at
// x + t * sx (sx % 8 == 0) instead of x + t * d, so a block's chunks are
// runs of P pieces, one run per token.
template <int DT, int NT, int U, bool STR = false>
__device__ __forceinline__ void pack_block(const uint16_t* __restrict__ x, int64_t ntok, int d, int64_t blk,
                                           uint32_t* __restrict__ bits, float* __restrict__ mu,
                                           uint32_t* bits_s, double* sum_s, int64_t sx = 0) {
  const int P = d >> 3;                  // chunks per token (1..16)
  const int TB = NT * U / P;             // whole tokens per block
  const int W = (d + 31) >> 5;
  const int64_t tok0 = blk * TB;
  const int nchunk = (int)min((int64_t)TB, ntok - tok0) * P;  // valid chunks of this block
  const int i = threadIdx.x;
  // c / P for c < 4096 and P <= 16 as (c * ceil(2^16 / P)) >> 16 (exact there)
  const uint32_t pmag = STR ? (65536u + P - 1) / P : 0u;
  u4v raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
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
  for (int u = 0; u < U; ++u) {
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
// zero[0 .. nzero) is zeroed on the side (the split V quantiser's start).
template <int DT, bool STR>
__global__ __launch_bounds__(256) void pack_qk_coop_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, InView in, int N, int64_t nbph,
    int64_t ntok, int d, uint32_t* __restrict__ qbits, float* __restrict__ qmu,
    uint32_t* __restrict__ kbits, float* __restrict__ kmu, uint32_t* __restrict__ zero, int64_t nzero) {
  __shared__ uint32_t bits_s[256 * kPackUCoop];
  __shared__ double sum_s[256 * kPackUCoop];
  if (blockIdx.y == 0)
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nzero; i += (int64_t)gridDim.x * 256) zero[i] = 0u;
  if constexpr (STR) {
    const bool isk = blockIdx.y != 0;
    const int64_t bh = blockIdx.x / nbph, tb = blockIdx.x - bh * nbph;
    const int W = (d + 31) >> 5;
    pack_block<DT, 256, kPackUCoop, true>((isk ? k : q) + (bh / in.H) * in.sb + (bh % in.H) * in.sh, N, d, tb,
                              (isk ? kbits : qbits) + bh * N * W, (isk ? kmu : qmu) + bh * N, bits_s, sum_s,
                              in.sn);
  } else if (blockIdx.y == 0) {
    pack_block<DT, 256, kPackUCoop>(q, ntok, d, blockIdx.x, qbits, qmu, bits_s, sum_s);
  } else {
    pack_block<DT, 256, kPackUCoop>(k, ntok, d, blockIdx.x, kbits, kmu, bits_s, sum_s);
  }
}

__global__ void zero_kernel(uint32_t* __restrict__ a, int64_t n);

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
                          float* kmu, hipStream_t s, uint32_t* zero, int64_t nzero) {
  // q == nullptr: K alone (grid.y 0 then selects K)
  const unsigned ny = q ? 2 : 1;
  if (!q) {
    q = k;
    qbits = kbits;
    qmu = kmu;
  }
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const int64_t ntok = (int64_t)nbh * N;
  if (in.vec) {
    const int TB = 256 * kPackUCoop / (d / 8);
    const bool str = !in.dense(N, d);
    const int64_t nbph = (N + TB - 1) / TB;
    const int64_t nblk = str ? nbh * nbph : (ntok + TB - 1) / TB;
    if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nblk, ny);
    auto kern = dt == BA_F16 ? (str ? pack_qk_coop_kernel<BA_F16, true> : pack_qk_coop_kernel<BA_F16, false>)
                             : (str ? pack_qk_coop_kernel<BA_BF16, true> : pack_qk_coop_kernel<BA_BF16, false>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, q16, k16, in, N, nbph, ntok, d, qbits, qmu, kbits, kmu, zero,
                       nzero);
    return hipGetLastError();
  }
  if (nzero > 0) {
    if ((nzero + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((nzero + 255) / 256)), dim3(256), 0, s, zero, nzero);
  }
  if ((ntok + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((ntok + 255) / 256), ny);
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
// non-negative), pass 2 quantises with inv = 127/amax and writes int8.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void quant_v_kernel(
    const uint16_t* __restrict__ v, InView in, int N, int d,
    int8_t* __restrict__ vq, float* __restrict__ vscale) {
  __shared__ uint32_t amax_bits[128];
  __shared__ float inv_s[128];
  const int bh = blockIdx.x;
  for (int i = threadIdx.x; i < d; i += blockDim.x) amax_bits[i] = 0u;
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
  }
}

// quant_v for heads that fit in registers (d % 8 == 0): a block of 1024
// threads quantises HB heads (HB = 1024 / T, T threads per head, a power of
// two chosen so that no thread holds more than kQvRows rows), reading each
// head once. A head is row-major N x d, so thread t < R*P of its group
// (P = d/8 16-byte pieces per row, R = T/P rows per sweep) owns piece t % P
// of rows t / P + k*R: every load of the group is one contiguous run of
// 16*R*P bytes. Channel maxima go through an LDS atomic max on the float
// bits (non-negative), then the held values are quantised and written as
// int8.
// rows per thread held in registers: 10 keeps the fused pre-pass within 64
// VGPRs, so two of its 1024-thread blocks share a CU
constexpr int kQvRows = 10;
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
// heads bh0 .. bh0 + HB - 1 (those below nbh) by one block of 1024
// threads; smem holds 2 * 128 words per head
template <int DT>
__device__ __forceinline__ void quant_heads_block(const uint16_t* __restrict__ v, const InView& in, int N, int d,
                                                  int64_t bh0,
                                                  int64_t nbh, int HB, int8_t* __restrict__ vq,
                                                  float* __restrict__ vscale, uint32_t* smem) {
  const int T = 1024 / HB;
  const int hs = threadIdx.x / T, t = threadIdx.x % T;
  const int64_t bh = bh0 + hs;
  const bool hvalid = bh < nbh;
  uint32_t* amax_bits = smem + 256 * hs;
  float* inv_s = reinterpret_cast<float*>(amax_bits + 128);
  const int P = d >> 3, R = T / P;
  const int piece = t % P, r0 = t / P;
  const bool active = hvalid && r0 < R;
  if (t < d) amax_bits[t] = 0u;
  __syncthreads();
  const uint16_t* vh = v + (hvalid ? (bh / in.H) * in.sb + (bh % in.H) * in.sh : 0) + 8 * piece;
  int8_t* qh = vq + (hvalid ? bh * N * d : 0) + 8 * piece;
  // rows r0, r0 + R, ... below N: this thread holds the first cnt of them;
  // the row addresses are stepped, not kept per row (register pressure)
  const int cnt = active && r0 < N ? min(kQvRows, (N - r0 + R - 1) / R) : 0;
  u4v x[kQvRows];
  {
    const uint16_t* src = vh + (int64_t)r0 * in.sn;
    const int64_t step = (int64_t)R * in.sn;
#pragma unroll
    for (int k = 0; k < kQvRows; ++k, src += step)
      x[k] = k < cnt ? *reinterpret_cast<const u4v*>(src) : (u4v){0u, 0u, 0u, 0u};
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
  int8_t* dst = qh + (int64_t)r0 * d;
#pragma unroll
  for (int k = 0; k < kQvRows; ++k, dst += (int64_t)R * d) {
    if (k < cnt) *reinterpret_cast<uint2*>(dst) = quant8_codes<DT>(x[k], inv);
  }
}

// quant_v for heads split over S blocks of 1024 threads, each part's rows
// held in registers as in quant_heads_block (2 <= S <= kQvMaxParts): every
// block takes the channel maxima over ALL N rows of its head itself,
// streaming them once (eight 16-byte loads in flight per thread), so no
// block depends on another and no zero fill or second launch is needed;
// then it loads its own rows [s RB, s RB + RB), quantises them and writes
// int8, and part 0 stores the scales. The maximum and the float32
// arithmetic are those of the other quantisers, so the outputs are the same
// bit for bit. Block b takes head 8 (i / S) + b % 8, part i % S, with
// i = b / 8: the parts of a head run on one XCD (blocks are dealt to the
// XCDs in turn) and share its L2 for the repeated reads. Blocks whose head
// is past nbh do nothing.
constexpr int kQvMaxParts = 4;
template <int DT>
__device__ __forceinline__ void quant_head_part_block(const uint16_t* __restrict__ v, const InView& in, int N,
                                                      int d, int64_t nbh, int S, int RB, int64_t b,
                                                      int8_t* __restrict__ vq, float* __restrict__ vscale,
                                                      uint32_t* smem) {
  const int64_t i = b >> 3;
  const int part = (int)(i % S);
  const int64_t bh = 8 * (i / S) + (b & 7);
  if (bh >= nbh) return;  // (the whole block)
  uint32_t* amax_bits = smem;
  float* inv_s = reinterpret_cast<float*>(smem + 128);
  const int P = d >> 3, R = 1024 / P;
  const int piece = threadIdx.x % P, r0 = threadIdx.x / P;
  const bool active = r0 < R;
  if (threadIdx.x < d) amax_bits[threadIdx.x] = 0u;
  const uint16_t* vh = v + (bh / in.H) * in.sb + (bh % in.H) * in.sh + 8 * piece;
  // channel maxima of |v| over the head on the 16-bit patterns (magnitude
  // bits order like |v| for finite values)
  us2 mb[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
  auto take = [&](const u4v& raw) {
#pragma unroll
    for (int w = 0; w < 4; ++w) mb[w] = __builtin_elementwise_max(mb[w], __builtin_bit_cast(us2, raw[w] & 0x7FFF7FFFu));
  };
  if (active) {
    int j = r0;
    for (; j + 7 * R < N; j += 8 * R) {
      u4v raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) raw[u] = *reinterpret_cast<const u4v*>(vh + (int64_t)(j + u * R) * in.sn);
#pragma unroll
      for (int u = 0; u < 8; ++u) take(raw[u]);
    }
    for (; j < N; j += R) take(*reinterpret_cast<const u4v*>(vh + (int64_t)j * in.sn));
  }
  __syncthreads();  // (the zeroed maxima)
  if (active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) atomicMax(&amax_bits[8 * piece + e], __float_as_uint(to_f32<DT>(mb[e >> 1][e & 1])));
  }
  __syncthreads();
  if (threadIdx.x < d) {
    const float a = __uint_as_float(amax_bits[threadIdx.x]);
    inv_s[threadIdx.x] = a > 0.0f ? 127.0f / a : 0.0f;
    if (part == 0) vscale[bh * d + threadIdx.x] = a / 127.0f;
  }
  __syncthreads();
  // this part's rows: r_begin + r0, + R, ... below r_end, held in registers
  const int r_begin = part * RB, r_end = min(N, r_begin + RB);
  const int cnt = active && r_begin + r0 < r_end ? min(kQvRows, (r_end - r_begin - r0 + R - 1) / R) : 0;
  u4v x[kQvRows];
  {
    const uint16_t* src = vh + (int64_t)(r_begin + r0) * in.sn;
    const int64_t step = (int64_t)R * in.sn;
#pragma unroll
    for (int k = 0; k < kQvRows; ++k, src += step)
      x[k] = k < cnt ? *reinterpret_cast<const u4v*>(src) : (u4v){0u, 0u, 0u, 0u};
  }
  float inv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) inv[e] = inv_s[8 * piece + e];
  int8_t* dst = vq + bh * N * d + 8 * piece + (int64_t)(r_begin + r0) * d;
#pragma unroll
  for (int k = 0; k < kQvRows; ++k, dst += (int64_t)R * d) {
    if (k < cnt) *reinterpret_cast<uint2*>(dst) = quant8_codes<DT>(x[k], inv);
  }
}

// Parts per head for quant_head_part_block: 0 where one block holds a head
// (or the rows are not 16-byte pieces), and where more than kQvMaxParts
// would be needed (the split quantiser then takes the head).
int quant_parts(int N, int d) {
  if (d % 8 != 0) return 0;
  const int64_t cap = (int64_t)kQvRows * (1024 / (d / 8));  // rows one block holds
  if (N <= cap) return 0;
  const int64_t S = (N + cap - 1) / cap;
  return S <= kQvMaxParts ? (int)S : 0;
}
// V blocks (XCD-dealt, see quant_head_part_block) and rows per part
int64_t quant_part_blocks(int64_t nbh, int S) { return 8 * (int64_t)S * ((nbh + 7) / 8); }
int quant_part_rows(int N, int S) { return (N + S - 1) / S; }

template <int DT>
__global__ __launch_bounds__(1024) void quant_v_parts_kernel(
    const uint16_t* __restrict__ v, InView in, int nbh, int N, int d, int S, int RB, int8_t* __restrict__ vq,
    float* __restrict__ vscale) {
  __shared__ uint32_t smem[2 * 128];
  quant_head_part_block<DT>(v, in, N, d, nbh, S, RB, blockIdx.x, vq, vscale, smem);
}

// Heads per 1024-thread block for the register-resident quantiser: the most
// (a power of two, at most 8) whose T = 1024 / HB threads per head still
// hold at most kQvRows rows each, while leaving at least 64 blocks; with
// fewer heads than that, one head per block keeps each head's rows spread
// over all 1024 threads. (At most 8 rows per thread for several heads per
// block measured slower: DiT-256 pre-pass 18.3 against 15.5 us, two heads
// per block against four.)
int quant_heads_per_block(int nbh, int N, int d) {
  const int P = d / 8;
  for (int hb = 8; hb > 1; hb >>= 1) {
    const int T = 1024 / hb;
    if (T >= P && (int64_t)N <= kQvRows * (int64_t)(T / P) && nbh >= 64 * hb) return hb;
  }
  return 1;
}

template <int DT>
__global__ __launch_bounds__(1024) void quant_v_head_kernel(
    const uint16_t* __restrict__ v, InView in, int nbh, int N, int d, int HB, int8_t* __restrict__ vq,
    float* __restrict__ vscale) {
  __shared__ uint32_t smem[8 * 2 * 128];
  quant_heads_block<DT>(v, in, N, d, (int64_t)blockIdx.x * HB, nbh, HB, vq, vscale, smem);
}

// Pack Q and K and quantise V in one launch (d % 8 == 0, heads that fit the
// register-resident quantiser, whole or in S parts): blocks 0 .. nvb-1
// quantise HB heads each, or S > 0 parts of heads (the long-running ones,
// dispatched first), the rest pack npq blocks of
// tokens of Q (npb, or 0 when Q is left to the attention), then npb of K,
// all with 1024 threads. STR (a strided view):
// the pack blocks are nbph per head, each within one head. At most 64 VGPRs
// (eight waves per SIMD), so two blocks share a CU: a packing block runs
// beside a quantising one instead of after it (DiT-512 15.5 -> 13.8 us,
// DiT-256 15.4 -> 14.1, DeiT-Small 9.3 -> 8.4).
template <int DT, bool STR, int U>
__global__ __launch_bounds__(1024, 8) void prepass_fused_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, InView in,
    int nbh, int N, int d, int HB, int S, int RB, int64_t nvb, int64_t npq, int64_t npb, int64_t nbph,
    uint32_t* __restrict__ qbits, float* __restrict__ qmu, uint32_t* __restrict__ kbits, float* __restrict__ kmu,
    int8_t* __restrict__ vq, float* __restrict__ vscale) {
  __shared__ uint32_t bits_s[1024 * U];
  __shared__ double sum_s[1024 * U];
  const int64_t ntok = (int64_t)nbh * N;
  const int64_t b = blockIdx.x;
  if (b < nvb) {
    if (S > 0) quant_head_part_block<DT>(v, in, N, d, nbh, S, RB, b, vq, vscale, bits_s);
    else quant_heads_block<DT>(v, in, N, d, b * HB, nbh, HB, vq, vscale, bits_s);
  } else if constexpr (STR) {
    const bool isk = b - nvb >= npq;
    const int64_t pb = b - nvb - (isk ? npq : 0);
    const int64_t bh = pb / nbph, tb = pb - bh * nbph;
    const int W = (d + 31) >> 5;
    pack_block<DT, 1024, U, true>((isk ? k : q) + (bh / in.H) * in.sb + (bh % in.H) * in.sh, N, d, tb,
                               (isk ? kbits : qbits) + bh * N * W, (isk ? kmu : qmu) + bh * N, bits_s, sum_s,
                               in.sn);
  } else if (b - nvb < npq) {
    pack_block<DT, 1024, U>(q, ntok, d, b - nvb, qbits, qmu, bits_s, sum_s);
  } else {
    pack_block<DT, 1024, U>(k, ntok, d, b - nvb - npq, kbits, kmu, bits_s, sum_s);
  }
}

// quant_v for long heads (16-byte rows, heads past the register-resident
// quantiser): the rows of each head are split over S blocks so that the whole
// chip streams V, in two passes after a zero fill of vscale (folded into the
// packing launch when ba_pack_qk_quant_v runs it).
//  * Pass A: each block takes the channel maxima of |v| over its rows and
//    combines them into vscale with a global atomic max on the float bits
//    with the top bit set (unsigned order = order of the non-negative
//    values; the set bit marks "a maximum, not yet a scale").
//  * Pass B: each block reads the head's maxima, quantises its rows with
//    inv = 127 / amax, writes int8, and stores vscale = amax / 127. Every
//    block of the head stores the same value, and a block that reads a word
//    already turned into a scale recovers amax exactly as the 16-bit
//    rounding of scale * 127 (amax is a 16-bit value and the two float
//    roundings move it by far less than half a 16-bit step; exhaustively
//    true for every finite fp16 and bf16 value), so no block depends on
//    which form it finds.
// The arithmetic is that of the one-block quantisers, so the outputs are the
// same bit for bit.
constexpr uint32_t kAmaxMark = 0x80000000u;

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ a, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) a[i] = 0u;
}

// amax of a channel from its vscale word (either form, see above)
template <int DT>
__device__ __forceinline__ float amax_of_word(uint32_t w) {
  if (w & kAmaxMark) return __uint_as_float(w & ~kAmaxMark);
  const float y = __uint_as_float(w) * 127.0f;
  return DT == BA_F16 ? f16_to_f32(f32_to_f16(y)) : bf16_to_f32(f32_to_bf16(y));
}

// Block x: head x / S, rows [s * RB, min(N, s * RB + RB)) with s = x % S.
// QUANT false: pass A; true: pass B.
template <int DT, bool QUANT>
__global__ __launch_bounds__(256) void quant_v_split_kernel(
    const uint16_t* __restrict__ v, InView in, int N, int d, int S, int RB, int8_t* __restrict__ vq,
    uint32_t* __restrict__ vs_bits) {
  __shared__ uint32_t red[128];  // channel maxima (pass A)
  __shared__ float inv_s[128];
  const int64_t bh = blockIdx.x / S;
  const int r_begin = (int)(blockIdx.x - bh * S) * RB, r_end = min(N, r_begin + RB);
  const int P = d >> 3, rows = 256 / P;  // 16-byte pieces per row, rows per sweep
  const int piece = threadIdx.x % P, r0 = threadIdx.x / P;
  const bool active = r0 < rows;
  float amax = 0.0f;
  if (threadIdx.x < d) {
    red[threadIdx.x] = 0u;
    if (QUANT) {
      amax = amax_of_word<DT>(vs_bits[bh * d + threadIdx.x]);
      inv_s[threadIdx.x] = amax > 0.0f ? 127.0f / amax : 0.0f;
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
    if (threadIdx.x < d) atomicMax(&vs_bits[bh * d + threadIdx.x], red[threadIdx.x] | kAmaxMark);
  } else {
    float inv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) inv[e] = inv_s[8 * piece + e];
    auto quant8 = [&](const u4v& raw) -> uint2 { return quant8_codes<DT>(raw, inv); };
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
    }
    // the scale, the same value from every block of the head
    if (threadIdx.x < d) vs_bits[bh * d + threadIdx.x] = __float_as_uint(amax / 127.0f);
  }
}

// rows per block of the split quantiser: about four blocks per CU, each with
// at least one full sweep of 8 rows per thread
void split_shape(int nbh, int N, int d, int& S, int& RB) {
  const int rows = 256 / (d / 8);
  const int64_t want = (1024 + (int64_t)nbh - 1) / nbh;
  const int64_t cap = std::max<int64_t>(1, N / (8 * rows));
  const int S0 = (int)std::min(want, cap);
  RB = (N + S0 - 1) / S0;
  S = (N + RB - 1) / RB;
}

// passes A and B (vscale already zero)
template <int DT>
hipError_t launch_quant_v_split_ab(const uint16_t* v, const InView& in, int nbh, int N, int d, int8_t* vq,
                                   float* vscale, hipStream_t s) {
  int S, RB;
  split_shape(nbh, N, d, S, RB);
  const int64_t nblk = (int64_t)nbh * S;
  if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
  uint32_t* vs_bits = reinterpret_cast<uint32_t*>(vscale);
  hipLaunchKernelGGL((quant_v_split_kernel<DT, false>), dim3((unsigned)nblk), dim3(256), 0, s, v, in, N, d, S, RB,
                     vq, vs_bits);
  hipLaunchKernelGGL((quant_v_split_kernel<DT, true>), dim3((unsigned)nblk), dim3(256), 0, s, v, in, N, d, S, RB,
                     vq, vs_bits);
  return hipGetLastError();
}

bool quant_in_registers(int N, int d) {
  return d % 8 == 0 && (int64_t)N <= (int64_t)kQvRows * (1024 / (d / 8));
}

hipError_t launch_quant_v(const void* v, ba_dtype dt, const InView& in, int nbh, int N, int d,
                          int8_t* vq, float* vscale, hipStream_t s) {
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  if (in.vec && quant_in_registers(N, d)) {
    const int HB = quant_heads_per_block(nbh, N, d);
    const unsigned nvb = (unsigned)((nbh + HB - 1) / HB);
    if (dt == BA_F16)
      hipLaunchKernelGGL(quant_v_head_kernel<BA_F16>, dim3(nvb), dim3(1024), 0, s, v16, in, nbh, N, d, HB, vq, vscale);
    else
      hipLaunchKernelGGL(quant_v_head_kernel<BA_BF16>, dim3(nvb), dim3(1024), 0, s, v16, in, nbh, N, d, HB, vq, vscale);
    return hipGetLastError();
  }
  if (in.vec && quant_parts(N, d) > 0) {
    const int S = quant_parts(N, d), RB = quant_part_rows(N, S);
    const int64_t nvb = quant_part_blocks(nbh, S);
    if (nvb > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (dt == BA_F16)
      hipLaunchKernelGGL(quant_v_parts_kernel<BA_F16>, dim3((unsigned)nvb), dim3(1024), 0, s, v16, in, nbh, N, d, S, RB,
                         vq, vscale);
    else
      hipLaunchKernelGGL(quant_v_parts_kernel<BA_BF16>, dim3((unsigned)nvb), dim3(1024), 0, s, v16, in, nbh, N, d, S,
                         RB, vq, vscale);
    return hipGetLastError();
  }
  if (in.vec) {
    const int64_t n = (int64_t)nbh * d;
    if ((n + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(vscale), n);
    return dt == BA_F16 ? launch_quant_v_split_ab<BA_F16>(v16, in, nbh, N, d, vq, vscale, s)
                        : launch_quant_v_split_ab<BA_BF16>(v16, in, nbh, N, d, vq, vscale, s);
  }
  // element path (d % 8 != 0 or rows not 16-byte aligned): one block per head
  if (dt == BA_F16)
    hipLaunchKernelGGL(quant_v_kernel<BA_F16>, dim3((unsigned)nbh), dim3(256), 0, s, v16, in, N, d, vq, vscale);
  else
    hipLaunchKernelGGL(quant_v_kernel<BA_BF16>, dim3((unsigned)nbh), dim3(256), 0, s, v16, in, N, d, vq, vscale);
  return hipGetLastError();
}

hipError_t launch_prepass(const void* q, const void* k, const void* v, ba_dtype dt, const InView& in, int nbh,
                          int N, int d, uint32_t* qbits, float* qmu, uint32_t* kbits, float* kmu, int8_t* vq,
                          float* vscale, hipStream_t s) {
  const int64_t ntok = (int64_t)nbh * N;
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  if (!in.vec) {
    hipError_t e = launch_pack_qk(q, k, dt, in, nbh, N, d, qbits, qmu, kbits, kmu, s);
    if (e != hipSuccess) return e;
    return launch_quant_v(v, dt, in, nbh, N, d, vq, vscale, s);
  }
  const int S = quant_in_registers(N, d) ? 0 : quant_parts(N, d);
  if (!quant_in_registers(N, d) && S == 0) {
    // long heads: the packing launch also zeroes vscale, then the split
    // quantiser's two passes
    hipError_t e = launch_pack_qk(q, k, dt, in, nbh, N, d, qbits, qmu, kbits, kmu, s,
                                  reinterpret_cast<uint32_t*>(vscale), (int64_t)nbh * d);
    if (e != hipSuccess) return e;
    return dt == BA_F16 ? launch_quant_v_split_ab<BA_F16>(v16, in, nbh, N, d, vq, vscale, s)
                        : launch_quant_v_split_ab<BA_BF16>(v16, in, nbh, N, d, vq, vscale, s);
  }
  const bool str = !in.dense(N, d);
  const int HB = S > 0 ? 1 : quant_heads_per_block(nbh, N, d);
  const int RB = S > 0 ? quant_part_rows(N, S) : 0;
  const int64_t nvb = S > 0 ? quant_part_blocks(nbh, S) : (nbh + HB - 1) / HB;
  const int TB = 1024 * kPackUFused / (d / 8);  // tokens per packing block
  const int64_t nbph = (N + TB - 1) / TB;
  const int64_t npb = str ? nbh * nbph : (ntok + TB - 1) / TB;
  const int64_t npq = q ? npb : 0;  // (no Q: packed by the attention)
  const int64_t nblk = nvb + npq + npb;
  if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
  constexpr int U = kPackUFused;
  auto kern = dt == BA_F16 ? (str ? prepass_fused_kernel<BA_F16, true, U> : prepass_fused_kernel<BA_F16, false, U>)
                           : (str ? prepass_fused_kernel<BA_BF16, true, U> : prepass_fused_kernel<BA_BF16, false, U>);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(1024), 0, s, q16, k16, v16, in, nbh, N, d, HB, S, RB, nvb, npq,
                     npb, nbph,
                     qbits, qmu, kbits, kmu, vq, vscale);
  return hipGetLastError();
}

}  // namespace binattn
