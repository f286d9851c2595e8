// attention.hip — fused BinaryAttention forward for gfx950 (MI355X).
//
// Method (BinaryAttention: One-Bit QK-Attention for Vision and Diffusion
// Transformers, gist.science summaries): zh technical summary section 2.1
// (sign-vector dot product as Hamming distance), section 2.2 items 1-3
// (scaled binary Q/K, additive bias, u8 P and channel-wise int8 V with
// integer aggregation), section 2.3 (fused, tiled kernel). Same content in
// nl Methodologie 1-3 and it/fr/pt section 2.
//
// Design on CDNA4 (not the pages' A100 design, which used 1-bit and u8 x s8
// tensor-core MMAs that gfx950 does not have):
//
//  * One workgroup = 4 waves = 128 queries of one (batch, head); each wave
//    owns 32 queries. Keys stream through LDS in tiles of 64.
//  * Q.K similarity on the matrix cores: the +-1 sign vectors are encoded as
//    fp4 (e2m1: +1 = 0x2, -1 = 0xA, 0 = 0x0) and multiplied with
//    v_mfma_f32_32x32x64_f8f6f4 (fp4 runs at twice the int8 rate). The sums
//    are integers |sigma| <= 128, exact in fp32, and equal
//    d - 2*popcount(q xor k) because padding channels are encoded as 0 on
//    the query side. The product is formed transposed, S^T = K Q^T, so each
//    lane holds 16 keys of ONE query: the row max and row sum are in-lane
//    reductions, and the probabilities already sit in the int8 MFMA operand
//    layout needed for the next product.
//  * Two passes over the keys: pass 1 finds the exact row max m_i, pass 2
//    forms p8 = rne(255 * exp(s - m)), the float row sum, and P.V. There is
//    no rescaling of the integer accumulator at all, and p8 follows the
//    plain (unblocked) definition up to float rounding.
//  * P.V on v_mfma_i32_32x32x32_i8, computed as O^T = V^T P^T. gfx950 int8
//    MFMA is signed x signed, so the u8 probabilities enter as p8 - 128 (a
//    byte XOR 0x80) and 128 * sum_j v8_jc is added back at the end (exact in
//    int32). V tiles are transposed into LDS while staged; the per-channel
//    sums come from the same pass with v_dot4.
//  * Softmax in base 2: x = s*log2(e) - m*log2(e) + log2(255), so a single
//    v_exp_f32 gives 255*exp(s - m); v_cvt_pk_u8_f32 rounds to nearest even
//    and clamps to [0, 255].
#include "common.h"

namespace binattn {

namespace {

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kQW = 32;            // queries per wave
constexpr int kQB = kWaves * kQW;  // queries per workgroup
constexpr int kBC = 64;            // keys per LDS tile (two 32-key MFMA blocks)
constexpr int kVStride = kBC + 16; // bytes per transposed V row in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_255 = 7.9943534368588578f;

enum { BIAS_NONE = 0, BIAS_DENSE_F32 = 1, BIAS_DENSE_F16 = 2, BIAS_RELPOS = 3 };

struct Params {
  const uint32_t* qbits;
  const float* qmu;
  const uint32_t* kbits;
  const float* kmu;
  const int8_t* vq;
  const float* vscale;
  const void* bias;
  int64_t bias_bstride;
  int grid_h, grid_w, n_prefix;
  int B, H, N, d, W;
  int nqb;          // query blocks per head
  float inv_sqrt_d;
  void* out;
};

// fp4 expansion of 32 sign bits. Dword m (0..3) holds the channels
// 32w + m + 4p at nibble p (0..7); the same channel order is used for the
// query and the key operand, so the dot product is unchanged.
__device__ __forceinline__ uint32_t fp4_signs(uint32_t bits, int m) {
  return (((bits >> m) & 0x11111111u) << 3) | 0x22222222u;
}

// LDS swizzle of the 16-byte fp4 slots of one key row (avoids bank
// conflicts between the lanes that read the A operand together).
template <int NKB>
__device__ __forceinline__ int kslot(int key, int slot) {
  if (NKB == 1) return slot ^ ((key >> 4) & 1);
  return slot ^ (((key >> 1) & 1) | ((key >> 3) & 2));
}

// Key (within a 32-key block) that row position p of S^T holds: chosen so
// that lane group g ends up with the 16 consecutive keys 16g..16g+15.
__device__ __forceinline__ int key_of_pos(int p) {
  return 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3);
}

// Value held by the partner lane (lane ^ 32). v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second;
// with both operands = x, lanes 0-31 find the partner value in the second
// result and lanes 32-63 in the first.
__device__ __forceinline__ float partner32(float x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

template <int OUTDT>
__device__ __forceinline__ uint16_t to_out(float x) {
  return OUTDT == BA_F16 ? f32_to_f16(x) : f32_to_bf16(x);
}

template <int NKB, int NCB, int BIAS, int OUTDT>
__global__ __launch_bounds__(256) void attn_fwd_kernel(Params p) {
  constexpr int DV = 32 * NCB;
  constexpr int KROW = 32 * NKB;  // bytes of fp4 per key row
  __shared__ __attribute__((aligned(16))) uint8_t kx_s[kBC * KROW];
  __shared__ __attribute__((aligned(16))) uint8_t vt_s[DV * kVStride];
  __shared__ __attribute__((aligned(16))) float muk_s[kBC];
  __shared__ int colsum_s[DV];

  const int N = p.N, d = p.d, W = p.W;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, g = lane >> 5;

  // ---- work item: (b, h, query block), XCD-aware order ----
  const int nblk = gridDim.x;
  int u = blockIdx.x;
  if ((nblk & 7) == 0) u = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  int b, h, qb;
  if (BIAS == BIAS_DENSE_F32 || BIAS == BIAS_DENSE_F16) {
    // batch innermost: the B workgroups that read the same bias rows run
    // together on one XCD
    b = u % p.B;
    const int r = u / p.B;
    qb = r % p.nqb;
    h = r / p.nqb;
  } else {
    qb = u % p.nqb;
    const int r = u / p.nqb;
    h = r % p.H;
    b = r / p.H;
  }
  const int64_t bh = (int64_t)b * p.H + h;
  const int qi = qb * kQB + wave * kQW + ql;
  const bool qvalid = qi < N;

  // ---- prologue: query operand (fp4 signs, padding channels zero) ----
  v8i qop[NKB];
#pragma unroll
  for (int kk = 0; kk < NKB; ++kk) {
    const int w = 2 * kk + g;
    const uint32_t bits = (qvalid && w < W) ? p.qbits[(bh * N + qi) * W + w] : 0u;
    v8i o = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t e = fp4_signs(bits, m);
      uint32_t mask = 0;
#pragma unroll
      for (int pp = 0; pp < 8; ++pp)
        if (32 * w + m + 4 * pp < d) mask |= 0xFu << (4 * pp);
      o[m] = (int)(e & mask);
    }
    qop[kk] = o;
  }
  const float qmu = qvalid ? p.qmu[bh * N + qi] : 0.0f;
  const float c0 = qmu * p.inv_sqrt_d;  // natural-log units (bias path)
  const float cq = c0 * kLog2e;         // base-2 units (no-bias path)

  int rp = 0, cp = 0;  // relative-position grid coordinates of the query
  if (BIAS == BIAS_RELPOS && qvalid && qi >= p.n_prefix) {
    rp = (qi - p.n_prefix) / p.grid_w;
    cp = (qi - p.n_prefix) % p.grid_w;
  }
  const int T = (2 * p.grid_h - 1) * (2 * p.grid_w - 1);

  const int ntiles = (N + kBC - 1) / kBC;
  const bool ragged = (N % kBC) != 0;

  // stage one key tile: fp4 signs of K and mu_k
  auto stage_k = [&](int t) {
    for (int idx = tid; idx < kBC * 2 * NKB; idx += 256) {
      const int key = idx / (2 * NKB), w = idx % (2 * NKB);
      const int j = t * kBC + key;
      const uint32_t bits = (j < N && w < W) ? p.kbits[(bh * N + j) * W + w] : 0u;
      u4v o;
      if (w < W) {
        o[0] = fp4_signs(bits, 0); o[1] = fp4_signs(bits, 1);
        o[2] = fp4_signs(bits, 2); o[3] = fp4_signs(bits, 3);
      } else {
        o[0] = o[1] = o[2] = o[3] = 0u;
      }
      *reinterpret_cast<u4v*>(kx_s + key * KROW + kslot<NKB>(key, w) * 16) = o;
    }
    if (tid < kBC) {
      const int j = t * kBC + tid;
      muk_s[tid] = j < N ? p.kmu[bh * N + j] : 0.0f;
    }
  };

  // S^T block (32 keys x 32 queries) of key block kb of the staged tile
  auto qk_block = [&](int kb) -> v16f {
    const int key = kb * 32 + key_of_pos(ql);
    v16f s = {};
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const u4v a4 = *reinterpret_cast<const u4v*>(kx_s + key * KROW + kslot<NKB>(key, 2 * kk + g) * 16);
      v8i a = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], 0, 0, 0, 0};
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qop[kk], s, 4, 4, 0, 0, 0, 0);
    }
    return s;
  };

  // score in the units used by the max: t = sigma*mu_k (no bias) or
  // u = t*c0 + b (natural-log units, bias)
  auto scores = [&](int t, int kb, const v16f& sig, float* out16) {
    const int jb = t * kBC + kb * 32 + 16 * g;  // first key of this lane's 16
    float mk[16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4 v = *reinterpret_cast<const float4*>(muk_s + kb * 32 + 16 * g + 4 * r);
      mk[4 * r] = v.x; mk[4 * r + 1] = v.y; mk[4 * r + 2] = v.z; mk[4 * r + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) out16[i] = sig[i] * mk[i];
    if (BIAS == BIAS_DENSE_F32 || BIAS == BIAS_DENSE_F16) {
      const int64_t row = (int64_t)b * p.bias_bstride + ((int64_t)h * N + (qvalid ? qi : 0)) * N;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = min(jb + i, N - 1);
        float bv;
        if (BIAS == BIAS_DENSE_F32) bv = static_cast<const float*>(p.bias)[row + j];
        else bv = f16_to_f32(static_cast<const uint16_t*>(p.bias)[row + j]);
        out16[i] = __builtin_fmaf(out16[i], c0, bv);
      }
    } else if (BIAS == BIAS_RELPOS) {
      const float* tab = static_cast<const float*>(p.bias) + (int64_t)h * T;
      const int gw = p.grid_w, npre = p.n_prefix;
      int jr = 0, jc = 0;
      if (jb >= npre) { jr = (jb - npre) / gw; jc = (jb - npre) % gw; }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = jb + i;
        float bv = 0.0f;
        if (qvalid && qi >= npre && j >= npre && j < N) {
          bv = tab[(rp - jr + p.grid_h - 1) * (2 * gw - 1) + (cp - jc + gw - 1)];
        }
        if (j >= npre) { if (++jc == gw) { jc = 0; ++jr; } }
        out16[i] = __builtin_fmaf(out16[i], c0, bv);
      }
    }
  };

  // keys past N in the last (ragged) tile get -inf
  auto mask_tail = [&](int t, int kb, float* v16) {
    if (ragged && t == ntiles - 1) {
      const int jb = t * kBC + kb * 32 + 16 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (jb + i >= N) v16[i] = -INFINITY;
    }
  };

  // ================= pass 1: exact row maximum =================
  float mrun = -INFINITY;
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    stage_k(t);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const v16f sig = qk_block(kb);
      float sc[16];
      scores(t, kb, sig, sc);
      mask_tail(t, kb, sc);
#pragma unroll
      for (int i = 0; i < 16; i += 2) mrun = fmaxf(mrun, fmaxf(sc[i], sc[i + 1]));
    }
  }
  mrun = fmaxf(mrun, partner32(mrun, lane));
  // x = score*scale + negm gives log2(255 * exp(s - m))
  const float scale2 = (BIAS == BIAS_NONE) ? cq : kLog2e;
  const float negm = __builtin_fmaf(-scale2, mrun, kLog2_255);

  // ================= pass 2: u8 P, row sum, integer P.V =================
  for (int i = tid; i < DV; i += 256) colsum_s[i] = 0;
  // channels >= d of the transposed V tile stay zero
  for (int i = tid; i < DV * kVStride / 4; i += 256) reinterpret_cast<uint32_t*>(vt_s)[i] = 0u;
  float lrun = 0.0f;
  v16i acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = (v16i){};
  int csum[3][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  const int d4 = (d + 3) / 4;
  const int nblk4 = (kBC / 4) * d4;
  const bool dword_v = (d % 4) == 0;

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    stage_k(t);
    // V tile: 4 keys x 4 channels per thread, transposed into vt_s[c][key]
#pragma unroll
    for (int rr = 0; rr < 3; ++rr) {
      const int blk = tid + 256 * rr;
      if (blk < nblk4) {
        const int kg = blk / d4, cg = blk % d4;
        uint32_t r4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = t * kBC + kg * 4 + k;
          const int8_t* src = p.vq + (bh * N + j) * d + cg * 4;
          uint32_t wv = 0u;
          if (j < N) {
            if (dword_v) {
              wv = *reinterpret_cast<const uint32_t*>(src);
            } else {
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (cg * 4 + c < d) wv |= (uint32_t)(uint8_t)src[c] << (8 * c);
            }
          }
          r4[k] = wv;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t o = ((r4[0] >> (8 * c)) & 0xFFu) | (((r4[1] >> (8 * c)) & 0xFFu) << 8) |
                             (((r4[2] >> (8 * c)) & 0xFFu) << 16) | (((r4[3] >> (8 * c)) & 0xFFu) << 24);
          const int ch = cg * 4 + c;
          if (ch < DV) *reinterpret_cast<uint32_t*>(vt_s + ch * kVStride + kg * 4) = o;
          csum[rr][c] = __builtin_amdgcn_sdot4((int)o, 0x01010101, csum[rr][c], false);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const v16f sig = qk_block(kb);
      float sc[16];
      scores(t, kb, sig, sc);
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = __builtin_fmaf(sc[i], scale2, negm);
      mask_tail(t, kb, sc);  // after the scaling: -inf * 0 would be NaN
      uint32_t pw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t wd = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ex = __builtin_amdgcn_exp2f(sc[4 * r + e]);
          lrun += ex;
          wd = __builtin_amdgcn_cvt_pk_u8_f32(ex, e, wd);
        }
        pw[r] = wd ^ 0x80808080u;  // u8 -> s8 (p8 - 128)
      }
      const v4i bop = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const u4v a4 = *reinterpret_cast<const u4v*>(vt_s + (cb * 32 + ql) * kVStride + kb * 32 + 16 * g);
        const v4i a = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3]};
        acc[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bop, acc[cb], 0, 0, 0);
      }
    }
  }

  // ================= epilogue =================
#pragma unroll
  for (int rr = 0; rr < 3; ++rr) {
    const int blk = tid + 256 * rr;
    if (blk < nblk4) {
      const int cg = blk % d4;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (cg * 4 + c < DV) atomicAdd(&colsum_s[cg * 4 + c], csum[rr][c]);
    }
  }
  lrun += partner32(lrun, lane);
  __syncthreads();
  if (!qvalid) return;
  const float inv_l = 1.0f / lrun;
  uint16_t* outp = static_cast<uint16_t*>(p.out) + (bh * N + qi) * d;
  const float* vs = p.vscale + bh * d;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = cb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
      if (c < d) {
        const int a = acc[cb][i] + 128 * colsum_s[c];
        outp[c] = to_out<OUTDT>((float)a * vs[c] * inv_l);
      }
    }
  }
}

template <int NKB, int NCB, int BIAS>
hipError_t launch_t(const Params& p, int nblocks, int out_dt, hipStream_t s) {
  if (out_dt == BA_F16)
    hipLaunchKernelGGL((attn_fwd_kernel<NKB, NCB, BIAS, BA_F16>), dim3(nblocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<NKB, NCB, BIAS, BA_BF16>), dim3(nblocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int NKB, int NCB>
hipError_t launch_bias(const Params& p, int bias, int nblocks, int out_dt, hipStream_t s) {
  switch (bias) {
    case BIAS_NONE: return launch_t<NKB, NCB, BIAS_NONE>(p, nblocks, out_dt, s);
    case BIAS_DENSE_F32: return launch_t<NKB, NCB, BIAS_DENSE_F32>(p, nblocks, out_dt, s);
    case BIAS_DENSE_F16: return launch_t<NKB, NCB, BIAS_DENSE_F16>(p, nblocks, out_dt, s);
    default: return launch_t<NKB, NCB, BIAS_RELPOS>(p, nblocks, out_dt, s);
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  Params p;
  p.qbits = a.qbits; p.qmu = a.qmu; p.kbits = a.kbits; p.kmu = a.kmu;
  p.vq = a.vq; p.vscale = a.vscale;
  p.bias = a.bias; p.bias_bstride = a.bias_bstride;
  p.grid_h = a.grid_h; p.grid_w = a.grid_w; p.n_prefix = a.n_prefix;
  p.B = a.B; p.H = a.H; p.N = a.N; p.d = a.d; p.W = (a.d + 31) / 32;
  p.nqb = (a.N + kQB - 1) / kQB;
  p.inv_sqrt_d = (float)(1.0 / sqrt((double)a.d));
  p.out = a.out;
  int bias = BIAS_NONE;
  if (a.bias_kind == BA_BIAS_DENSE) bias = a.bias_dtype == BA_F32 ? BIAS_DENSE_F32 : BIAS_DENSE_F16;
  else if (a.bias_kind == BA_BIAS_RELPOS) bias = BIAS_RELPOS;
  const int64_t nblocks = (int64_t)p.nqb * a.B * a.H;
  if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int ncb = (a.d + 31) / 32;
  switch (ncb) {
    case 1: return launch_bias<1, 1>(p, bias, (int)nblocks, a.out_dt, s);
    case 2: return launch_bias<1, 2>(p, bias, (int)nblocks, a.out_dt, s);
    case 3: return launch_bias<2, 3>(p, bias, (int)nblocks, a.out_dt, s);
    default: return launch_bias<2, 4>(p, bias, (int)nblocks, a.out_dt, s);
  }
}

}  // namespace binattn
