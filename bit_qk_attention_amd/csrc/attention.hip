// attention.hip — fused BinaryAttention forward for gfx950 (MI355X).
//
// Method (BinaryAttention: One-Bit QK-Attention for Vision and Diffusion
// Transformers, gist.science summaries): zh technical summary section 2.1
// (sign-vector dot product as a Hamming distance), section 2.2 items 1-3
// (scaled binary Q/K, additive bias, u8 P and channel-wise int8 V with
// integer aggregation), section 2.3 (fused, tiled kernel). Same content in
// nl Methodologie 1-3 and it/fr/pt section 2.
//
// Design on CDNA4 (not the pages' A100 design, which used 1-bit and u8 x s8
// tensor-core MMAs that gfx950 does not have):
//
//  * One workgroup = 4 waves = 128 queries of one (batch, head); each wave
//    owns 32 queries. Keys stream through LDS in tiles of 64, double
//    buffered: the next tile's global loads are in flight while the current
//    tile is computed, and there is one barrier per tile.
//  * Q.K similarity on the matrix cores: the +-1 sign vectors are encoded as
//    fp4 (e2m1: +1 = 0x2, -1 = 0xA, 0 = 0x0) and multiplied with
//    v_mfma_f32_32x32x64_f8f6f4 (fp4 runs at twice the int8 rate). The sums
//    are integers |sigma| <= 128, exact in fp32, equal to
//    d - 2*popcount(q xor k) because padding channels are 0 on the query
//    side. The product is formed transposed, S^T = K Q^T, so each lane holds
//    16 keys of ONE query: the row max and row sum are in-lane reductions
//    and the probabilities already sit in the int8 MFMA operand layout of the
//    next product.
//  * Two passes over the keys: pass 1 finds the exact row max m_i, pass 2
//    forms p8 = rne(255 * exp(s - m)), the float row sum and P.V. The integer
//    accumulator is never rescaled, and p8 follows the plain (unblocked)
//    definition up to float rounding.
//  * P.V on v_mfma_i32_32x32x32_i8 as O^T = V^T P^T. The V^T operand comes
//    straight from row-major V in LDS through the transposing LDS read
//    (ds_read_b64_tr_b8: in each 16-lane group, output lane 8h+b receives
//    byte b of the 8-byte rows addressed by lanes 2k+h, k = 0..7). gfx950
//    int8 MFMA is signed x signed and p8 reaches 255, so each block adds
//    V^T (127 - p8) (127 - p8 = p8 XOR 0x7F as a signed byte) and then
//    V^T (-127); the accumulator ends at -sum_j p8_j v8_j, exact in int32.
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
constexpr int kTblMax = 2048;      // floats of relative-position window per tile

// Workgroups per CU the register allocation must allow (4 waves each; 2 ->
// up to 256 VGPRs per wave, 3 -> 168, 4 -> 128), per instantiation, from
// measurements on MI355X: without a bias and d <= 64 the extra occupancy
// wins even though a few values spill outside the key loops; the relative-
// position gather prefers 3; the dense-bias loads need the registers.
template <int NCB, int BIAS>
constexpr int min_blocks() {
  return BIAS == 3 ? 3 : (BIAS == 0 ? (NCB <= 2 ? 4 : 3) : 2);
}
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
  int bias_vec;     // dense bias rows are 16-byte aligned (vector loads)
  int v_dma;        // V tiles go global -> LDS directly (16-byte pieces)
  int v_swz_shift;  // 16-byte chunk swizzle of V rows: -1 none, else shift
  int relpos_fast;  // relative-position rows never wrap inside 16 keys
  void* out;
};

// fp4 expansion of 32 sign bits. Dword m (0..3) holds the channels
// 32w + m + 4p at nibble p (0..7); the same channel order is used for the
// query and the key operand, so the dot product is unchanged.
__device__ __forceinline__ uint32_t fp4_signs(uint32_t bits, int m) {
  return (((bits >> m) & 0x11111111u) << 3) | 0x22222222u;
}

// LDS swizzle of the 16-byte fp4 slots of one key row (spreads the lanes
// that read the A operand together over the LDS banks).
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

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

template <int V>
struct IntC {
  static constexpr int value = V;
};

// One LDS tile buffer. The kernel keeps two as separate __shared__ objects
// and selects them at compile time, so the compiler can tell a DMA into one
// from reads of the other and does not wait for the prefetch.
template <int NKB, int NCB, int BIAS>
struct TileBuf {
  static constexpr int DV = 32 * NCB;  // V channels padded to the MFMA block
  static constexpr int KROW = 32 * NKB;
  static constexpr int VS = DV + 8;    // bytes per V row, generic (byte-copy) layout
  static constexpr int NT = BIAS == BIAS_RELPOS ? kTblMax : 1;
  uint8_t kx[kBC * KROW];
  uint8_t vr[kBC * VS];  // also holds a 64 x d tile at stride d (d <= DV)
  float mk[kBC];
  float tbl[NT];
};

template <int NKB, int NCB, int BIAS, int OUTDT>
__global__ __launch_bounds__(256, (min_blocks<NCB, BIAS>())) void attn_fwd_kernel(Params p) {
  using S = TileBuf<NKB, NCB, BIAS>;
  constexpr int KROW = S::KROW, VS = S::VS;
  constexpr bool DENSE = BIAS == BIAS_DENSE_F32 || BIAS == BIAS_DENSE_F16;
  __shared__ __attribute__((aligned(16))) S sb0;
  __shared__ __attribute__((aligned(16))) S sb1;
  auto pick = [&](auto bufc) -> S& {
    if constexpr (decltype(bufc)::value == 0) return sb0;
    else return sb1;
  };

  const int N = p.N, d = p.d, W = p.W;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, g = lane >> 5;

  // ---- work item: (b, h, query block), XCD-aware order ----
  const int nblk = gridDim.x;
  int u = blockIdx.x;
  if ((nblk & 7) == 0) u = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  int b, h, qb;
  if (DENSE) {
    // batch innermost: the B workgroups that read the same bias rows run
    // back to back on one XCD
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
  const int qc = qvalid ? qi : N - 1;  // clamped query index for addressing

  // ---- query operand: fp4 signs, padding channels zero ----
  v8i qop[NKB];
#pragma unroll
  for (int kk = 0; kk < NKB; ++kk) {
    const int w = 2 * kk + g;
    const uint32_t bits = (qvalid && w < W) ? p.qbits[(bh * N + qi) * W + w] : 0u;
    v8i o = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t mask = 0;
#pragma unroll
      for (int pp = 0; pp < 8; ++pp)
        if (32 * w + m + 4 * pp < d) mask |= 0xFu << (4 * pp);
      o[m] = (int)(fp4_signs(bits, m) & mask);
    }
    qop[kk] = o;
  }
  const float qmu = qvalid ? p.qmu[bh * N + qi] : 0.0f;
  const float c0 = qmu * p.inv_sqrt_d;  // natural-log units (bias path)
  const float cq = c0 * kLog2e;         // base-2 units (no-bias path)

  const int ntiles = (N + kBC - 1) / kBC;
  const bool ragged = (N % kBC) != 0;

  // ---- relative-position bookkeeping ----
  const int gh = p.grid_h, gw = p.grid_w, npre = p.n_prefix;
  const int T2 = 2 * gw - 1;
  int q_rr = 0, q_cc = 0;  // grid row/column of this lane's query
  bool q_grid = false;     // query has a grid position
  if (BIAS == BIAS_RELPOS && qc >= npre) {
    q_grid = true;
    q_rr = (qc - npre) / gw;
    q_cc = (qc - npre) % gw;
  }
  // grid rows spanned by this workgroup's queries
  int wq_lo = 0, wq_hi = -1;
  if (BIAS == BIAS_RELPOS) {
    const int q0 = qb * kQB, q1 = min(qb * kQB + kQB - 1, N - 1);
    if (q1 >= npre) {
      wq_lo = (max(q0, npre) - npre) / gw;
      wq_hi = (q1 - npre) / gw;
    }
  }
  // table rows dr_lo.. of the window tile t needs, and its size in floats
  auto tbl_window = [&](int t, int& dr_lo, int& count) {
    const int j0 = t * kBC, j1 = min(t * kBC + kBC - 1, N - 1);
    dr_lo = 0;
    count = 0;
    if (wq_hi < wq_lo || j1 < npre) return;
    const int rk_lo = (max(j0, npre) - npre) / gw, rk_hi = (j1 - npre) / gw;
    dr_lo = wq_lo - rk_hi + gh - 1;
    count = ((wq_hi - rk_lo + gh - 1) - dr_lo + 1) * T2;
  };

  // ---- staging ----
  // Full tiles: V, the key scales and the relative-position window rows go
  // global -> LDS with global_load_lds (no registers, no VALU); wave 0 loads
  // the K sign words into registers a tile ahead and expands them to fp4 in
  // LDS. The ragged last tile is staged synchronously with bounds checks.
  //
  // V layout in LDS (v_dma): row stride d; with v_swz_shift >= 0 the 16-byte
  // chunks of row r are permuted, chunk c stored at c ^ vswz(r), so that the
  // 8 consecutive rows one transposing read touches fall in distinct banks.
  // The permutation is applied on the global side (each lane of a DMA picks
  // its source chunk). Generic d (not v_dma): stride VS, no swizzle.
  const int vstride = p.v_dma ? d : VS;
  const int nchk = d >> 4;  // 16-byte chunks per row (swizzled layouts)
  auto vswz = [&](int row) -> int {
    return p.v_swz_shift >= 0 ? ((row >> p.v_swz_shift) & (nchk - 1)) : 0;
  };
  auto vaddr = [&](int row, int col) -> int {  // LDS byte offset of V[row][col]
    return p.v_swz_shift >= 0 ? row * vstride + 16 * ((col >> 4) ^ vswz(row)) + (col & 15)
                              : row * vstride + col;
  };
  // DMA sources: wave w fills the 1 KB LDS chunks w and w + 4 of the tile
  int v_src[2];
  bool v_on[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int dst = 1024 * (wave + 4 * i) + 16 * lane;  // LDS byte of this lane
    v_on[i] = dst < kBC * d;
    const int row = dst / max(d, 1), pc = (dst % max(d, 1)) >> 4;
    v_src[i] = p.v_swz_shift >= 0 ? row * d + 16 * (pc ^ vswz(row)) : dst;
  }
  typedef __attribute__((address_space(1))) const void gptr_t;
  typedef __attribute__((address_space(3))) void lptr_t;

  uint32_t st_k[2 * NKB];
  auto load_k = [&](int t) {
    if (wave == 0) {
      const bool last = ragged && t == ntiles - 1;
      const int j = t * kBC + lane;
      const uint32_t* src = p.kbits + (bh * N + j) * W;
#pragma unroll
      for (int w = 0; w < 2 * NKB; ++w) st_k[w] = (w < W && (!last || j < N)) ? src[w] : 0u;
    }
  };
  auto store_k = [&](auto bufc) {
    S& sb = pick(bufc);
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < 2 * NKB; ++w) {
        u4v o;
        o[0] = fp4_signs(st_k[w], 0); o[1] = fp4_signs(st_k[w], 1);
        o[2] = fp4_signs(st_k[w], 2); o[3] = fp4_signs(st_k[w], 3);
        *reinterpret_cast<u4v*>(sb.kx + lane * KROW + kslot<NKB>(lane, w) * 16) = o;
      }
    }
  };
  // relative-position window rows of tile t (always in bounds of the table)
  auto dma_tbl = [&](int t, auto bufc) {
    S& sb = pick(bufc);
    if (BIAS == BIAS_RELPOS) {
      int dr_lo, count;
      tbl_window(t, dr_lo, count);
      const float* src = static_cast<const float*>(p.bias) + (int64_t)h * T2 * (2 * gh - 1) + (int64_t)dr_lo * T2;
#pragma unroll
      for (int i = 0; i < kTblMax / 256; ++i) {
        const int x0 = 64 * (wave + 4 * i);
        if (x0 + lane < count)
          __builtin_amdgcn_global_load_lds((gptr_t*)(src + x0 + lane), (lptr_t*)(sb.tbl + x0), 4, 0, 0);
      }
    }
  };
  // full tile t (all keys < N): V, mu_k and the table window by DMA
  auto dma_tile = [&](int t, auto bufc, bool with_v) {
    S& sb = pick(bufc);
    const int j0 = t * kBC;
    if (with_v && p.v_dma) {
      const int8_t* src = p.vq + (bh * N + j0) * d;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (v_on[i])
          __builtin_amdgcn_global_load_lds((gptr_t*)(src + v_src[i]), (lptr_t*)(sb.vr + 1024 * (wave + 4 * i)), 16, 0, 0);
    }
    if (wave == 1)
      __builtin_amdgcn_global_load_lds((gptr_t*)(p.kmu + bh * N + j0 + lane), (lptr_t*)(sb.mk), 4, 0, 0);
    dma_tbl(t, bufc);
  };
  // V tile t through registers, rows past N zero (ragged tile; any d)
  auto copy_v_checked = [&](int t, auto bufc) {
    S& sb = pick(bufc);
    const int j0 = t * kBC;
    if (p.v_dma) {
      for (int x = tid; x < kBC * d / 8; x += 256) {
        const int off = 8 * x, row = off / d, col = off % d;
        uint2 v = make_uint2(0u, 0u);
        if (j0 + row < N) v = *reinterpret_cast<const uint2*>(p.vq + (bh * N + j0) * d + off);
        *reinterpret_cast<uint2*>(sb.vr + vaddr(row, col)) = v;
      }
    } else {
      for (int x = tid; x < kBC * d; x += 256) {
        const int row = x / d, col = x % d;
        const int j = j0 + row;
        sb.vr[row * VS + col] = j < N ? (uint8_t)p.vq[(bh * N + j) * d + col] : (uint8_t)0;
      }
    }
  };
  // synchronous staging of tile t with bounds checks (the ragged tile)
  auto stage_checked = [&](int t, auto bufc, bool with_v) {
    S& sb = pick(bufc);
    load_k(t);
    store_k(bufc);
    if (wave == 1) {
      const int j = t * kBC + lane;
      sb.mk[lane] = j < N ? p.kmu[bh * N + j] : 0.0f;
    }
    if (with_v) copy_v_checked(t, bufc);
    dma_tbl(t, bufc);
  };
  auto wait_dma = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)

  // S^T block (32 keys x 32 queries) of key block kb of the selected buffer
  auto qk_block = [&](auto bufc, int kb) -> v16f {
    S& sb = pick(bufc);
    const int key = kb * 32 + key_of_pos(ql);
    v16f s = {};
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const u4v a4 = *reinterpret_cast<const u4v*>(sb.kx + key * KROW + kslot<NKB>(key, 2 * kk + g) * 16);
      const v8i a = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], 0, 0, 0, 0};
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qop[kk], s, 4, 4, 0, 0, 0, 0);
    }
    return s;
  };

  // Scores of this lane's 16 keys in key block kb of tile t:
  // sigma * mu_k (no bias; the query scale is applied later) or
  // sigma * mu_k * mu_q / sqrt(d) + b (natural-log units, with bias).
  // TAIL: the last tile when N is not a multiple of the tile; keys past N
  // get -inf.
  auto scores = [&](auto tail, int t, auto bufc, int kb, const v16f& sig, float* sc) {
    S& sb = pick(bufc);
    constexpr bool TAIL = decltype(tail)::value;
    const bool last = ragged && t == ntiles - 1;  // keys past N in this tile
    const int jl = kb * 32 + 16 * g;  // first key of the lane's 16, in the tile
    const int jb = t * kBC + jl;
    const float4* mkp = reinterpret_cast<const float4*>(sb.mk + jl);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4 m4 = mkp[r];
      sc[4 * r + 0] = sig[4 * r + 0] * m4.x;
      sc[4 * r + 1] = sig[4 * r + 1] * m4.y;
      sc[4 * r + 2] = sig[4 * r + 2] * m4.z;
      sc[4 * r + 3] = sig[4 * r + 3] * m4.w;
    }
    if (DENSE) {
      const int64_t row = (int64_t)b * p.bias_bstride + ((int64_t)h * N + qc) * N;
      float bv[16];
      if (!last && p.bias_vec) {
        if (BIAS == BIAS_DENSE_F32) {
          const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(p.bias) + row + jb);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float4 v = src[r];
            bv[4 * r] = v.x; bv[4 * r + 1] = v.y; bv[4 * r + 2] = v.z; bv[4 * r + 3] = v.w;
          }
        } else {
          const u4v* src = reinterpret_cast<const u4v*>(static_cast<const uint16_t*>(p.bias) + row + jb);
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const u4v v = src[r];
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[8 * r + e] = f16_to_f32((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = min(jb + i, N - 1);
          bv[i] = BIAS == BIAS_DENSE_F32 ? static_cast<const float*>(p.bias)[row + j]
                                         : f16_to_f32(static_cast<const uint16_t*>(p.bias)[row + j]);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = __builtin_fmaf(sc[i], c0, bv[i]);
    } else if (BIAS == BIAS_RELPOS) {
      int dr_lo, count;
      tbl_window(t, dr_lo, count);
      // local window index = aq - (r_j*T2 + c_j)
      const int aq = (q_rr + gh - 1 - dr_lo) * T2 + q_cc + gw - 1;
      const float* tb = sb.tbl;
      float bv[16];
      const bool wave_grid = qb * kQB + wave * kQW >= npre;  // no prefix query in this wave
      if (!last && p.relpos_fast && wave_grid && jb >= npre) {
        // 16 keys on one grid row: a contiguous, reversed window
        const int g0 = jb - npre;
        const int base = aq - ((g0 / gw) * T2 + g0 % gw);
#pragma unroll
        for (int i = 0; i < 16; ++i) bv[i] = tb[base - i];
      } else {
        int rj = 0, cj = 0;
        if (jb >= npre) { rj = (jb - npre) / gw; cj = (jb - npre) % gw; }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = jb + i;
          const bool on = q_grid && j >= npre && j < N;
          bv[i] = on ? tb[aq - (rj * T2 + cj)] : 0.0f;
          if (j >= npre) { if (++cj == gw) { cj = 0; ++rj; } }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = __builtin_fmaf(sc[i], c0, bv[i]);
    }
    if (TAIL) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (jb + i >= N) sc[i] = -INFINITY;
    }
  };

  // ================= pass 1: exact row maximum =================
  float m0 = -INFINITY, m1 = -INFINITY;
  auto max16 = [&](const float* sc) {
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      m0 = fmaxf(fmaxf(m0, sc[i]), sc[i + 1]);
      m1 = fmaxf(fmaxf(m1, sc[i + 2]), sc[i + 3]);
    }
  };
  auto pass1_tile = [&](auto tail, int t, auto bufc) {
    const v16f sig0 = qk_block(bufc, 0);
    const v16f sig1 = qk_block(bufc, 1);
    float sc[16];
    scores(tail, t, bufc, 0, sig0, sc);
    max16(sc);
    scores(tail, t, bufc, 1, sig1, sc);
    max16(sc);
  };
  const int nfull = ragged ? ntiles - 1 : ntiles;
  // tile 0 -> buffer 0
  auto stage_first = [&](bool with_v) {
    if (nfull > 0) {
      dma_tile(0, IntC<0>(), with_v);
      if (with_v && !p.v_dma) copy_v_checked(0, IntC<0>());
      load_k(0);
      store_k(IntC<0>());
    } else {
      stage_checked(0, IntC<0>(), with_v);
    }
    wait_dma();
    __syncthreads();
  };
  // Full tiles alternate between the buffers (tile t in buffer t % 2, the
  // loop unrolled by two so the buffer is known at compile time); the next
  // full tile is staged while this one is computed. Then the ragged tile,
  // staged synchronously.
  auto run_pass = [&](bool with_v, auto body) {
    stage_first(with_v);
    auto step = [&](int t, auto cur, auto nxt) {
      const bool next_full = t + 1 < nfull;
      if (next_full) {
        dma_tile(t + 1, nxt, with_v);
        load_k(t + 1);
      }
      body(BoolC<false>(), t, cur);
      if (next_full) {
        store_k(nxt);
        if (with_v && !p.v_dma) copy_v_checked(t + 1, nxt);
      }
      wait_dma();
      __syncthreads();
    };
    for (int t = 0; t < nfull; t += 2) {
      step(t, IntC<0>(), IntC<1>());
      if (t + 1 < nfull) step(t + 1, IntC<1>(), IntC<0>());
    }
    if (ragged) {
      const int t = ntiles - 1;
      auto tail = [&](auto cur) {
        if (nfull > 0) {
          stage_checked(t, cur, with_v);
          wait_dma();
          __syncthreads();
        }
        body(BoolC<true>(), t, cur);
      };
      if (t & 1) tail(IntC<1>());
      else tail(IntC<0>());
    }
  };
  run_pass(false, pass1_tile);

  float mrun = fmaxf(m0, m1);
  mrun = fmaxf(mrun, partner32(mrun, lane));
  // x = score * scale2 + negm is log2(255 * exp(s - m))
  const float scale2 = (BIAS == BIAS_NONE) ? cq : kLog2e;
  const float negm = __builtin_fmaf(-scale2, mrun, kLog2_255);

  // ================= pass 2: u8 P, row sum, integer P.V =================
  float l0 = 0.0f, l1 = 0.0f, l2 = 0.0f, l3 = 0.0f;
  v16i acc[NCB];  // ends at -sum_j p8_j v8_j
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = (v16i){};
  const v4i m127 = {(int)0x81818181, (int)0x81818181, (int)0x81818181, (int)0x81818181};  // -127 bytes
  // transposing-read address of this lane for the V^T operand: row
  // 16*(lane/32) + (lane%16)/2 (+8 for the upper half), column
  // 16*((lane/16)%2) + 8*(lane%2) (+32 per channel block)
  const int tr_row = 16 * (lane >> 5) + ((lane & 15) >> 1);
  const int tr_col = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);

  // u8 probabilities of one key block, as the s8 MFMA operand 127 - p8.
  // Tail keys (past N) are masked after the scaling: -inf * 0 would be NaN.
  auto probs = [&](auto tail, int t, int kb, float* sc) -> v4i {
    constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = __builtin_fmaf(sc[i], scale2, negm);
    if (TAIL) {
      const int jb = t * kBC + kb * 32 + 16 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (jb + i >= N) sc[i] = -INFINITY;
    }
    uint32_t pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e0 = __builtin_amdgcn_exp2f(sc[4 * r + 0]);
      const float e1 = __builtin_amdgcn_exp2f(sc[4 * r + 1]);
      const float e2 = __builtin_amdgcn_exp2f(sc[4 * r + 2]);
      const float e3 = __builtin_amdgcn_exp2f(sc[4 * r + 3]);
      l0 += e0; l1 += e1; l2 += e2; l3 += e3;
      uint32_t wd = __builtin_amdgcn_cvt_pk_u8_f32(e0, 0, 0u);
      wd = __builtin_amdgcn_cvt_pk_u8_f32(e1, 1, wd);
      wd = __builtin_amdgcn_cvt_pk_u8_f32(e2, 2, wd);
      wd = __builtin_amdgcn_cvt_pk_u8_f32(e3, 3, wd);
      pw[r] = wd ^ 0x7F7F7F7Fu;  // u8 p8 -> s8 (127 - p8)
    }
    return (v4i){(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};
  };
  // P.V of one key block: acc += V^T (127 - p8) + V^T (-127)
  auto pv = [&](auto bufc, int kb, const v4i& bop) {
    S& sb = pick(bufc);
    const uint8_t* vb = sb.vr;
    const int r0 = kb * 32 + tr_row, r1 = r0 + 8;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vb + vaddr(r0, tr_col + 32 * cb)));
      const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vb + vaddr(r1, tr_col + 32 * cb)));
      const v4i a = {lo[0], lo[1], hi[0], hi[1]};
      acc[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bop, acc[cb], 0, 0, 0);
      acc[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, m127, acc[cb], 0, 0, 0);
    }
  };
  auto pass2_tile = [&](auto tail, int t, auto bufc) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const v16f sig = qk_block(bufc, kb);
      float sc[16];
      scores(BoolC<false>(), t, bufc, kb, sig, sc);
      const v4i pk = probs(tail, t, kb, sc);
      pv(bufc, kb, pk);
    }
  };

  __syncthreads();  // pass 1 is done with both buffers
  run_pass(true, pass2_tile);

  // ================= epilogue =================
  float lrun = (l0 + l1) + (l2 + l3);
  lrun += partner32(lrun, lane);
  if (!qvalid) return;
  const float ninv_l = -1.0f / lrun;  // the accumulator holds -A
  uint16_t* outp = static_cast<uint16_t*>(p.out) + (bh * N + qi) * d;
  const float* vs = p.vscale + bh * d;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = cb * 32 + 8 * r + 4 * g;  // 4 consecutive channels c..c+3
      uint16_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = (c + e < d) ? to_out<OUTDT>((float)acc[cb][4 * r + e] * vs[c + e] * ninv_l) : (uint16_t)0;
      }
      if (c + 3 < d && (d & 3) == 0) {
        *reinterpret_cast<uint2*>(outp + c) =
            make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < d) outp[c + e] = o[e];
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
  // V tiles by DMA: 16-byte pieces must be 16-byte aligned in global memory
  // (tile starts are (bh*N + 64t)*d bytes from a 16-byte aligned base)
  p.v_dma = (a.d % 16 == 0) || (a.d % 8 == 0 && a.N % 2 == 0);
  p.v_swz_shift = -1;
  if (p.v_dma && (a.d == 32 || a.d == 64 || a.d == 128)) p.v_swz_shift = a.d == 32 ? 2 : a.d == 64 ? 1 : 0;
  p.out = a.out;
  int bias = BIAS_NONE;
  p.bias_vec = 0;
  p.relpos_fast = 0;
  if (a.bias_kind == BA_BIAS_DENSE) {
    bias = a.bias_dtype == BA_F32 ? BIAS_DENSE_F32 : BIAS_DENSE_F16;
    const int per16 = a.bias_dtype == BA_F32 ? 4 : 8;  // elements per 16 bytes
    p.bias_vec = (a.N % per16 == 0) && (a.bias_bstride % per16 == 0) &&
                 (reinterpret_cast<uintptr_t>(a.bias) % 16 == 0);
  } else if (a.bias_kind == BA_BIAS_RELPOS) {
    bias = BIAS_RELPOS;
    p.relpos_fast = (a.grid_w % 16 == 0) && (a.n_prefix % 16 == 0);
  }
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
