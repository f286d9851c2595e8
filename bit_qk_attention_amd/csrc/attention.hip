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
//    owns 32 queries. Keys stream through LDS in tiles of 64 over two or
//    three stages: later tiles' global loads are in flight while the
//    current tile is computed, and there is one barrier per tile.
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
//    int8 MFMA is signed x signed and p8 reaches 255, so the product uses
//    the signed byte 127 - p8 (= p8 XOR 0x7F): the accumulator ends at
//    sum_j (127 - p8_j) v8_j, and sum_j p8_j v8_j = 127 * vsum - that, with
//    vsum the channel sums of v8. The kernel forms vsum itself from the V^T
//    operand it already holds (one v_dot4 per 4 keys, each wave taking a
//    quarter of the key blocks). Exact in int32.
//  * Softmax in base 2: x = s*log2(e) - m*log2(e) + log2(255), so a single
//    v_exp_f32 gives 255*exp(s - m); v_cvt_pk_u8_f32 rounds to nearest even
//    and clamps to [0, 255]. The row normaliser is the float sum of the
//    unquantised values (so the mass of keys whose p8 rounds to 0 still
//    counts).
//  * A sigma mode of the same kernel writes the integer similarity that its
//    Q.K path produces (the staged-tile route, the raw-word route and the
//    pass-1 route straight from global memory), for inspection.
//  * The queries may come as 16-bit values, binarised in the prologue with
//    the packing kernels' arithmetic (each query row belongs to one
//    workgroup); for heads whose keys all stay on chip, the keys and values
//    too (the resident mode binarises and quantises them into its stages).
//    The outputs are those of the packed-input path bit for bit.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace binattn {

namespace {

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kQW = 32;            // queries per wave
constexpr int kQB = kWaves * kQW;  // queries per workgroup
constexpr int kBC = 64;            // keys per LDS tile (two 32-key MFMA blocks)
constexpr int kTblMax = 2048;      // floats of relative-position window per tile
constexpr int kCUs = 256;          // compute units of an MI355X

// Bias variants. Dense rows that allow 16-byte vector access take the
// specialised paths (fp32: vector loads; fp16: tiles staged in LDS by DMA);
// any other dense bias takes per-element bounds-checked loads.
// Relative-position bias: BIAS_RELPOS_ROW when no tokens precede the grid
// and its width is a multiple of 16 (every run of 16 keys of a full tile
// lies on one grid row: a contiguous window of the table), else BIAS_RELPOS.
enum { BIAS_NONE = 0, BIAS_DENSE_F32 = 1, BIAS_DENSE_F16 = 2, BIAS_RELPOS = 3, BIAS_DENSE_ANY = 4,
       BIAS_RELPOS_ROW = 5 };
constexpr bool is_relpos(int bias) { return bias == BIAS_RELPOS || bias == BIAS_RELPOS_ROW; }

// What the kernel produces. MODE_ATTN: the attention output, two passes
// over the keys (the exact row maximum, then P and P.V). MODE_ONLINE: the
// same attention in one pass with a running row maximum (see the online
// pass below; d <= 64). The sigma
// modes (no bias, no softmax) produce the integer similarity of a window of
// query rows, each through one Q.K route of the attention:
//  MODE_SIGMA       the staged-tile route (K words DMA'd into LDS and
//                   expanded to fp4 once per tile), written out;
//  MODE_SIGMA_RAW   the raw-word route (each wave expands the staged words
//                   itself, as with the fp16 dense bias at 65..96 channels);
//  MODE_SIGMA_SPLIT the pass-1 route without a bias (K words straight from
//                   global memory into registers, four query groups);
// the last two compare their result with what is already in the output and
// overwrite every element that differs with kSigmaPoison.
enum { MODE_ATTN = 0, MODE_SIGMA = 1, MODE_SIGMA_RAW = 2, MODE_SIGMA_SPLIT = 3, MODE_ONLINE = 4 };
constexpr bool is_attn(int mode) { return mode == MODE_ATTN || mode == MODE_ONLINE; }
constexpr int32_t kSigmaPoison = 0x7FFFFFFF;  // never a similarity (|sigma| <= 128)

// Workgroups per CU the register allocation must allow (4 waves each; 2 ->
// up to 256 VGPRs per wave, 3 -> 168, 4 -> 128), per instantiation, from
// measurements on MI355X. At d <= 64 without a bias or with the row-run
// relative-position bias, four (with the lean pass-2 tile) beat three even
// though some values spill. Three: the general relative-position bias and
// the fp16 dense bias (staged in LDS) at d <= 64, and d <= 96 without a bias
// or with the fp16 dense bias (lean tile; with the bias the waves expand raw
// K words to make room in LDS); the third workgroup wins even where values
// of the ragged-tile code spill. Two: the fp32 and unaligned dense-bias
// loads go through registers, and d > 96.
template <int NCB, int BIAS, int MODE = MODE_ATTN>
constexpr int min_blocks() {
  // the online pass holds an fp32 output and two int32 accumulators
  if (MODE == MODE_ONLINE) return NCB <= 2 ? 3 : 2;
  if ((BIAS == BIAS_NONE || BIAS == BIAS_RELPOS_ROW) && NCB <= 2) return 4;
  return ((BIAS == BIAS_NONE || is_relpos(BIAS) || BIAS == BIAS_DENSE_F16) && NCB <= 2) ||
                 ((BIAS == BIAS_NONE || BIAS == BIAS_DENSE_F16) && NCB == 3)
             ? 3
             : 2;
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_255 = 7.9943534368588578f;

struct Params {
  const uint32_t* qbits;
  const float* qmu;
  const uint16_t* q16;  // Q as 16-bit values, packed in the prologue (then qbits, qmu unused)
  int q16_f16;          // q16, k16, v16 are fp16 (else bf16)
  const uint16_t* k16;  // resident mode only: K and V as 16-bit values, binarised and quantised
  const uint16_t* v16;  // by the workgroup itself (then kbits, kmu, vq, vscale unused)
  const uint32_t* kbits;
  const float* kmu;
  const int8_t* vq;
  const float* vscale;
  const void* bias;
  int64_t bias_bstride;
  int grid_h, grid_w, n_prefix;
  uint32_t gw_magic;  // ceil(2^32 / grid_w) for grid_w >= 2, else 0
  int B, H, N, d, W;
  int nqb;          // query blocks per head
  float inv_sqrt_d;
  int bias_f16;     // dense bias element type (BIAS_DENSE_ANY): fp16, else fp32
  int bias_al4;     // BIAS_DENSE_ANY: 1 every bias row starts 4-byte aligned; 2 only the
                    // base is (fp16 rows at 2-byte alignment); 0 neither
  int out_mode;     // bit 0: fp16 output (else bf16); bit 1: 8-byte row stores
                    // (d and the output strides % 4 == 0, 8-byte aligned base)
  int v_dma;        // V tiles go global -> LDS directly (16-byte pieces)
  int v_swz_shift;  // 16-byte chunk swizzle of V rows: -1 none, else shift
  int balance;      // wave priority policy: 1 the whole grid is resident at once, 2 it takes several rounds
  int slots;        // workgroups the chip holds at once (256 CUs x occupancy)
  int mk_vec;       // key scales of a head start 16-byte aligned (N % 4 == 0)
  int64_t out_sb;              // element strides of the output's [B, H, N, d] view
  int out_sh, out_sn;
  void* out;
  // sigma modes: query rows [row0, row0 + nrows) of each head are written to
  // sigma[head][row - row0][key]; the workgroups cover query blocks qb0 ..
  int32_t* sigma;
  int row0, nrows, qb0;
};

// fp4 expansion of 32 sign bits. Dword m (0..3) holds the channels
// 32w + m + 4p at nibble p (0..7); the same channel order is used for the
// query and the key operand, so the dot product is unchanged.
__device__ __forceinline__ uint32_t fp4_signs(uint32_t bits, int m) {
  // ((bits << (3 - m)) & 0x88888888) | 0x22222222 as one three-input
  // bitwise op (truth table 0xEA = (a & b) | c) after the shift
  return __builtin_amdgcn_bitop3_b32(bits << (3 - m), 0x88888888u, 0x22222222u, 0xEA);
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

// x / gw for 0 <= x < 65536 (every token offset), gw the grid width, by one
// high multiply with m = ceil(2^32 / gw): x * m / 2^32 = x / gw +
// x * e / (gw * 2^32) with e = m * gw - 2^32 < gw <= 256, and x * e < 2^24, so
// the floor is the exact quotient (checked for all x and gw in that range).
// m == 0 stands for gw == 1.
__device__ __forceinline__ int div_gw(int x, uint32_t m) {
  return m ? (int)__umulhi((uint32_t)x, m) : x;
}

// Raw buffer descriptor over [base, base + bytes): stride 0, so an access's
// offset is a byte offset, and one at or past `bytes` reads zero. Word 3 is
// the untyped 32-bit data format the gfx9 buffer unit expects.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Value held by the partner lane (lane ^ 32). v_permlane32_swap exchanges
// the upper half of its first operand with the lower half of its second;
// with both operands = x, lanes 0-31 find the partner value in the second
// result and lanes 32-63 in the first.
__device__ __forceinline__ float partner32(float x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}
__device__ __forceinline__ uint32_t partner32u(uint32_t x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return lane < 32 ? r[1] : r[0];
}
__device__ __forceinline__ double partner64(double x, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint64_t lo = partner32u((uint32_t)u, lane), hi = partner32u((uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, (hi << 32) | lo);
}


// Value of lane I of this lane's 16-lane row (DPP row_newbcast; the
// compiler folds it into the consuming VALU instruction).
template <int I>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + I, 0xF, 0xF, true));
}
// sc[i] = sig[i] * (lane i of the row's value of mrow). In the S^T layout
// register i of lane l holds key 16*(l/32) + i of the block, so with lane l
// holding the scale of key 16*(l/32) + l%16 this is sig * mu_k per key.
template <int... I>
__device__ __forceinline__ void mul_key_scales(float* sc, const v16f& sig, float mrow, std::integer_sequence<int, I...>) {
  ((sc[I] = sig[I] * row_bcast<I>(mrow)), ...);
}

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

template <int V>
struct IntC {
  static constexpr int value = V;
};

// LDS stages. Key-side data of one 64-key tile and its V rows live in
// separate __shared__ objects, one per stage, selected at compile time: the
// compiler then tells a DMA into one stage from reads of another and does
// not wait for the prefetch before reading.
// TBL: the stage holds its tile's relative-position table window (the
// resident mode keeps one window for all keys instead).
template <int NKB, int BIAS, bool RAWK, bool TBL = is_relpos(BIAS)>
struct KeyStage {
  static constexpr int KROW = 32 * NKB;
  static constexpr int NT = TBL ? kTblMax + 4 : 4;  // [0]: a 0.0 slot, then the window
  static constexpr int NB = BIAS == BIAS_DENSE_F16 ? kQB * kBC : 8;
  static constexpr int NKO = is_relpos(BIAS) ? kBC : 4;
  uint8_t kx[RAWK ? 16 : kBC * KROW];  // fp4 K operand (unused when the waves expand raw words)
  int koff[NKO];           // relative position: key part of the table-window index
  uint32_t kraw[256];      // K sign words as loaded, one per thread
  uint16_t bt[NB];         // fp16 dense bias tile: 128 query rows x 64 keys
  float mk[kBC];
  float tbl[NT];
};
template <int NCB>
struct VStage {
  static constexpr int DV = 32 * NCB;  // V channels padded to the MFMA block
  static constexpr int VS = DV + 8;    // bytes per V row, generic (byte-copy) layout
  uint8_t vr[kBC * VS];  // also holds a 64 x d tile at stride d (d <= DV)
};
// Stages per pass: pass 1 cycles through three (loads two tiles ahead);
// pass 2, which also stages V, through three where the LDS budget of the
// target occupancy allows, else two (one tile ahead).
// fp16 dense bias with three channel blocks: the waves expand the raw K
// words themselves (no fp4 copy in LDS), so that three workgroups fit a CU
template <int NCB, int BIAS, int MODE>
constexpr bool raw_k() {
  return (BIAS == BIAS_DENSE_F16 && NCB == 3) || MODE == MODE_SIGMA_RAW;
}
// Resident mode (heads of at most kResTiles tiles, N <= 256): every tile
// has a stage of its own, all staged at the start, and both passes read
// them with no further wait or barrier. For the instantiations whose LDS
// allows it at their occupancy: no bias, dense fp32, relative position.
constexpr int kResTiles = 4;
template <int NKB, int NCB, int BIAS, int MODE>
constexpr bool res_fits() {
  if (MODE != MODE_ATTN || NCB > 3) return false;
  if (!(BIAS == BIAS_NONE || BIAS == BIAS_DENSE_F32 || is_relpos(BIAS))) return false;
  constexpr int bytes = kResTiles * ((int)sizeof(KeyStage<NKB, BIAS, raw_k<NCB, BIAS, MODE>(), false>) +
                                     (int)sizeof(VStage<NCB>)) +
                        (is_relpos(BIAS) ? 4 * (kTblMax + 4) : 0) + 2048 + 512 + 512;
  return bytes <= 160 * 1024 / min_blocks<NCB, BIAS, MODE>();
}
template <int NKB, int NCB, int BIAS, int MODE>
struct StageCfg {
  static constexpr int KS = (int)sizeof(KeyStage<NKB, BIAS, raw_k<NCB, BIAS, MODE>()>);
  static constexpr int VSZ = (int)sizeof(VStage<NCB>);
  // less the pass-1 reduction buffer, the channel sums and scales
  static constexpr int BUDGET = 160 * 1024 / min_blocks<NCB, BIAS, MODE>() - 2048 - 512 - 512;
  static constexpr int NS2 = 3 * KS + 3 * VSZ <= BUDGET ? 3 : 2;
  static constexpr int NS1 = 3 * KS + NS2 * VSZ <= BUDGET ? 3 : 2;
};

// 16-byte chunk (8 keys) permutation of the fp16 bias rows in LDS: the 16
// consecutive rows that one 16-lane read group touches land in distinct
// 16-byte bank groups.
__device__ __forceinline__ int bswz(int row) { return (row ^ (row >> 3)) & 7; }

template <int NKB, int NCB, int BIAS, int MODE, bool RES>
__global__ __launch_bounds__(256, (min_blocks<NCB, BIAS, MODE>())) void attn_fwd_kernel(Params p) {
  constexpr bool RAWK = raw_k<NCB, BIAS, MODE>();
  static_assert(!RAWK || NKB == 2, "raw K words: four per key");
  static_assert(is_attn(MODE) || BIAS == BIAS_NONE, "the sigma modes take no bias");
  static_assert(MODE != MODE_ONLINE || NCB <= 2, "the online pass takes d <= 64");
  static_assert(!RES || res_fits<NKB, NCB, BIAS, MODE>(), "resident mode outside its instantiations");
  using KS = KeyStage<NKB, BIAS, RAWK, is_relpos(BIAS) && !RES>;
  using VSt = VStage<NCB>;
  using Cfg = StageCfg<NKB, NCB, BIAS, MODE>;
  constexpr int KROW = KS::KROW, VS = VSt::VS;
  constexpr int NS1 = Cfg::NS1, NS2 = Cfg::NS2;
  constexpr bool DENSE = BIAS == BIAS_DENSE_F32 || BIAS == BIAS_DENSE_F16 || BIAS == BIAS_DENSE_ANY;
  // pass 1 with the keys split over the waves (no staging) when there is no
  // bias; with a bias, staged tiles (a dense bias read row-wise per wave
  // would touch half-used 128-byte lines)
  constexpr bool P1_SPLIT = BIAS == BIAS_NONE && !RES;
  __shared__ float p1red[4][4][kQW];  // per-wave partial row maxima (pass 1 split)
  __shared__ int32_t vtot[32 * NCB];  // channel sums of v8 over the head's keys
  __shared__ float vscl[128];         // the head's V channel scales (DMA'd ahead of the epilogue)
  __shared__ __attribute__((aligned(16))) KS ks0;
  __shared__ __attribute__((aligned(16))) KS ks1;
  __shared__ __attribute__((aligned(16))) KS ks2;
  __shared__ __attribute__((aligned(16))) VSt vs0;
  __shared__ __attribute__((aligned(16))) VSt vs1;
  __shared__ __attribute__((aligned(16))) VSt vs2;
  // resident mode: tile t in stage t (a runtime index), one table window
  using KSR = std::conditional_t<RES, KS, char>;
  using VSR = std::conditional_t<RES, VSt, char>;
  __shared__ __attribute__((aligned(16))) KSR ksr[RES ? kResTiles : 1];
  __shared__ __attribute__((aligned(16))) VSR vsr[RES ? kResTiles : 1];
  __shared__ float tblr[(RES && is_relpos(BIAS)) ? kTblMax + 4 : 1];
  auto pick = [&](auto bufc) -> KS& {
    if constexpr (std::is_integral_v<decltype(bufc)>) {
      return ksr[bufc];
    } else {
      constexpr int i = decltype(bufc)::value;
      if constexpr (i == 0) return ks0;
      else if constexpr (i == 1) return ks1;
      else return ks2;
    }
  };
  // the stage's relative-position table window (slot 0 holds 0.0)
  auto tbl_of = [&](KS& sb) -> float* {
    if constexpr (RES) return tblr;
    else return sb.tbl;
  };
  auto pick_v = [&](auto bufc) -> VSt& {
    if constexpr (std::is_integral_v<decltype(bufc)>) {
      return vsr[bufc];
    } else {
      constexpr int i = decltype(bufc)::value;
      if constexpr (i == 0) return vs0;
      else if constexpr (i == 1) return vs1;
      else return vs2;
    }
  };

  const int N = p.N, d = p.d, W = p.W;
  const int tid = threadIdx.x;
  // the wave index is uniform: keep it in a scalar register so that the
  // per-wave staging branches are scalar branches, not exec-mask regions
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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
    qb = p.qb0 + u % p.nqb;
    const int r = u / p.nqb;
    h = r % p.H;
    b = r / p.H;
  }
  const int64_t bh = (int64_t)b * p.H + h;
  const int qi = qb * kQB + wave * kQW + ql;
  const bool qvalid = qi < N;
  // a wave whose 32 queries are all past N (the last query block of a head)
  // skips the score work of pass 1 and of the interleaved pass-2 tile: it
  // still stages its share of the tiles and adds its share of the V channel
  // sums
  const bool wave_live = qb * kQB + wave * kQW < N;
  const int qc = qvalid ? qi : N - 1;  // clamped query index for addressing

  // ---- query operand: fp4 signs, padding channels zero ----
  // Word w of a query covers channels 32w..32w+31; of those, the first
  // min(max(d - 32w, 0), 32) are real. Dword m of the fp4 operand holds
  // channel 32w + m + 4p at nibble p, so its nibble mask is bit m + 4p of
  // the real-channel mask spread to four bits. wb[kk] is word 2 kk + g.
  auto q_operand_w = [&](const uint32_t* wb, v8i* op) {
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const int w = 2 * kk + g;
      const int nv = min(max(d - 32 * w, 0), 32);
      const uint32_t vm = nv >= 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u);
      v8i o = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < 4; ++m) o[m] = (int)(fp4_signs(wb[kk], m) & (((vm >> m) & 0x11111111u) * 0xFu));
      op[kk] = o;
    }
  };
  auto q_operand = [&](int q, bool valid, v8i* op) {
    uint32_t wb[NKB];
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const int w = 2 * kk + g;
      wb[kk] = (valid && w < W) ? p.qbits[(bh * N + q) * W + w] : 0u;
    }
    q_operand_w(wb, op);
  };
  // Q given as 16-bit values (d % 8 == 0): the two lanes of a query pack it
  // here with the arithmetic of the packing kernels, so bits and scale are
  // those ba_pack_qk writes. Lane g takes the words 2 kk + g: sign bits from
  // a float compare (x < 0), a float64 sum of |x| per 8-channel piece. The
  // scale adds the piece sums in channel order (the running sum passes
  // between the two lanes word by word), divides by d in float64 and rounds
  // to float once. raw: the lane's 16-byte pieces (zero past d).
  auto pack_q16 = [&](auto dtc, const u4v (&raw)[NKB][4], bool valid, uint32_t* wb, float& mu)
      __attribute__((always_inline)) {
    constexpr int DT = decltype(dtc)::value;
    double ps[NKB][4];
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      uint32_t word = 0;
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        double s = 0.0;
        // (uniform: pieces past d for lane 0 are past d for lane 1 too)
        if (64 * kk + 8 * pc < d) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xf = to_f32<DT>((uint16_t)(raw[kk][pc][e >> 1] >> ((e & 1) * 16)));
            word |= xf < 0.0f ? (1u << (8 * pc + e)) : 0u;
            s += (double)fabsf(xf);
          }
        }
        ps[kk][pc] = s;
      }
      wb[kk] = valid ? word : 0u;
    }
    double acc = 0.0;
#pragma unroll
    for (int w = 0; w < 2 * NKB; ++w) {
      if (w < W) {  // (uniform)
        const bool own = (w & 1) == g;
        double mine = acc;
        if (own) {
#pragma unroll
          for (int pc = 0; pc < 4; ++pc)
            if (32 * w + 8 * pc < d) mine += ps[w >> 1][pc];
        }
        const double other = partner64(mine, lane);
        acc = own ? mine : other;
      }
    }
    mu = valid ? (float)(acc / (double)d) : 0.0f;
  };
  v8i qop[NKB];
  float c0 = 0.0f;  // mu_q / sqrt(d): natural-log units (bias path)
  float cq = 0.0f;  // c0 * log2(e): base-2 units (no-bias path)
  // The query operand and scale (the sigma modes take no scales), in two
  // steps: issue_q starts the loads (16-bit rows, or sign words and scale),
  // finish_q forms the operand. The staged and resident passes start the
  // first tiles' DMA in between, so the two memory latencies overlap and
  // the packing runs while the tiles land. Packed here from 16-bit Q, the
  // key-split pass 1 also needs the other waves' queries: each wave leaves
  // its signs and scales in the first V stage (unused until pass 2).
  const bool q_from16 = MODE == MODE_ATTN && p.q16 != nullptr;
  u4v qraw[NKB][4];
  uint32_t qwb[NKB];
  float qmu_ld = 0.0f;
  auto issue_q = [&]() __attribute__((always_inline)) {
    if (q_from16) {
      const uint16_t* row = p.q16 + (bh * N + qc) * d;
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
        for (int pc = 0; pc < 4; ++pc) {
          const int c = 32 * (2 * kk + g) + 8 * pc;
          qraw[kk][pc] = c < d ? *reinterpret_cast<const u4v*>(row + c) : (u4v){0u, 0u, 0u, 0u};
        }
    } else {
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const int w = 2 * kk + g;
        qwb[kk] = (qvalid && w < W) ? p.qbits[(bh * N + qi) * W + w] : 0u;
      }
      qmu_ld = (is_attn(MODE) && qvalid) ? p.qmu[bh * N + qi] : 0.0f;
    }
  };
  auto finish_q = [&]() __attribute__((always_inline)) {
    float qmu = qmu_ld;
    if (q_from16) {
      uint32_t wb[NKB];
      if (p.q16_f16) pack_q16(IntC<BA_F16>(), qraw, qvalid, wb, qmu);
      else pack_q16(IntC<BA_BF16>(), qraw, qvalid, wb, qmu);
      q_operand_w(wb, qop);
      if constexpr (P1_SPLIT) {
        uint32_t* tw = reinterpret_cast<uint32_t*>(vs0.vr);
        const int qr = wave * kQW + ql;
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
          if (2 * kk + g < W) tw[qr * W + 2 * kk + g] = wb[kk];
        if (g == 0) reinterpret_cast<float*>(tw + kQB * W)[qr] = qmu;
      }
    } else {
      q_operand_w(qwb, qop);
    }
    c0 = qmu * p.inv_sqrt_d;
    cq = c0 * kLog2e;
  };
  // the staged pass 1 of the attention and the resident mode split the two
  // steps around their first DMA; every other form loads the queries here
  constexpr bool Q_SPLIT = MODE == MODE_ATTN && !P1_SPLIT;
  if constexpr (!Q_SPLIT) {
    issue_q();
    finish_q();
  } else if constexpr (!RES) {
    issue_q();
  }

  const int ntiles = (N + kBC - 1) / kBC;
  const bool ragged = (N % kBC) != 0;
  // Wave priorities. The arbiter issues from the oldest ready wave, so of
  // the workgroups that share a CU the first one runs ahead and the last one
  // ends alone, one wave per SIMD, with little latency hidden.
  //  * Whole grid resident at once (policy 1): each wave runs at priority 1
  //    until three quarters of its pass-2 tiles are done and at 0 after, so
  //    the leaders wait for the others near the end (4096 tokens: the 4
  //    workgroups of a CU otherwise finish 73 us apart; 7-9% faster).
  //  * Several rounds (policy 2): the first workgroup each CU receives runs
  //    at priority 3 and ends early, the workgroups of the later rounds at 2
  //    and the rest at 0, so the later rounds start sooner and overlap the
  //    first (1024 workgroups on 768 slots: 6-7% faster).
  const bool balance = p.balance == 1;
  if (balance) {
    __builtin_amdgcn_s_setprio(1);
  } else if (p.balance == 2) {
    if (blockIdx.x < kCUs) __builtin_amdgcn_s_setprio(3);
    else if ((int)blockIdx.x >= p.slots) __builtin_amdgcn_s_setprio(2);
  }
  bool prio_high = balance;
  auto progress = [&](int done) {  // pass-2 tiles done
    if (prio_high && 4 * done >= 3 * ntiles) {
      prio_high = false;
      __builtin_amdgcn_s_setprio(0);
    }
  };
  if (MODE == MODE_ATTN && tid < 32 * NCB) vtot[tid] = 0;

  // sigma modes: this lane's 16 similarities of query q, keys key0 .. key0 +
  // 15 (those < N), written (CHECK false) or compared with the output, an
  // element that differs being overwritten with kSigmaPoison (CHECK true)
  auto put_sigma = [&](auto check, int q, int key0, const v16f& sg) {
    constexpr bool CHECK = decltype(check)::value;
    if (q < p.row0 || q >= p.row0 + p.nrows) return;
    int32_t* row = p.sigma + ((int64_t)bh * p.nrows + (q - p.row0)) * N;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + i;
      if (key < N) {
        const int32_t sv = (int32_t)sg[i];  // an exact integer
        if constexpr (CHECK) {
          if (row[key] != sv) row[key] = kSigmaPoison;
        } else {
          row[key] = sv;
        }
      }
    }
  };

  // ---- relative-position bookkeeping ----
  const int gh = p.grid_h, gw = p.grid_w, npre = p.n_prefix;
  const int T2 = 2 * gw - 1;
  int q_rr = 0, q_cc = 0;  // grid row/column of this lane's query
  bool q_grid = false;     // query has a grid position
  const uint32_t gwm = p.gw_magic;
  if (is_relpos(BIAS) && qc >= npre) {
    q_grid = true;
    q_rr = div_gw(qc - npre, gwm);
    q_cc = qc - npre - q_rr * gw;
  }
  // grid rows spanned by this workgroup's queries
  int wq_lo = 0, wq_hi = -1;
  if (is_relpos(BIAS)) {
    const int q0 = qb * kQB, q1 = min(qb * kQB + kQB - 1, N - 1);
    if (q1 >= npre) {
      wq_lo = div_gw(max(q0, npre) - npre, gwm);
      wq_hi = div_gw(q1 - npre, gwm);
    }
  }
  // table rows dr_lo.. of the window tile t needs (in the resident mode,
  // all keys), and its size in floats
  auto tbl_window = [&](int t, int& dr_lo, int& count) {
    const int j0 = RES ? 0 : t * kBC, j1 = RES ? N - 1 : min(t * kBC + kBC - 1, N - 1);
    dr_lo = 0;
    count = 0;
    if (wq_hi < wq_lo || j1 < npre) return;
    const int rk_lo = div_gw(max(j0, npre) - npre, gwm), rk_hi = div_gw(j1 - npre, gwm);
    dr_lo = wq_lo - rk_hi + gh - 1;
    count = ((wq_hi - rk_lo + gh - 1) - dr_lo + 1) * T2;
  };
  // Window index of (query, key) = qwin - koff[key]: qwin = (r_i + gh - 1) * T2
  // + c_i + gw - 1 depends on the query only, koff = (r_j + dr_lo) * T2 + c_j
  // on the key and the tile's window start dr_lo. The window sits at slot 1
  // of the stage's table, slot 0 holds 0.0, and the slot of a pair is the
  // unsigned saturating difference qwin1 - koff with qwin1 = qwin + 1 for a
  // query on the grid, 0 for one off it, and koff = kKoffNone for a key off
  // the grid or past N: both land on slot 0 (bias 0), every pair on the grid
  // on slot >= 1. Both terms are kept in bytes (x 4), so the difference is
  // the slot's byte offset in the table and needs no shift. koff is written
  // by wave 2 while the tile is staged (plain LDS stores, visible after the
  // step's barrier).
  constexpr int kKoffNone = 0x3FFFFFFF;
  const int qwin1 = q_grid ? 4 * ((q_rr + gh - 1) * T2 + q_cc + gw) : 0;
  if (is_relpos(BIAS) && tid == 0) {  // the 0.0 slot of each stage's table window
    if constexpr (RES) {
      tblr[0] = 0.0f;
    } else {
      ks0.tbl[0] = 0.0f;
      ks1.tbl[0] = 0.0f;
      if constexpr (NS1 == 3 || NS2 == 3) ks2.tbl[0] = 0.0f;
    }
  }
  auto stage_koff = [&](int t, auto bufc) {
    if (is_relpos(BIAS) && wave == 2) {
      int dr_lo, count;
      tbl_window(t, dr_lo, count);
      const int j = t * kBC + lane;
      int ko = kKoffNone;
      if (j >= npre && j < N) {
        const int r = div_gw(j - npre, gwm);
        ko = 4 * ((r + dr_lo) * T2 + (j - npre - r * gw));
      }
      pick(bufc).koff[lane] = ko;
    }
  };

  // ---- staging ----
  // Full tiles go global -> LDS by buffer loads with the LDS destination (no
  // registers): V, the key scales and the relative-position window rows
  // first, then the K sign words and the fp16 bias tile, a fixed number of
  // instructions per wave, so that a wait for all but that last group leaves
  // only the newest tile in flight. Each thread DMAs one K word and, once
  // its own load has landed, expands it to the fp4 operand (no barrier
  // between the two); where the raw words are kept, the waves expand them
  // where they use them. The ragged last tile is staged synchronously with
  // bounds checks.
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
  // DMA sources: wave w fills the 1 KB LDS chunks w and w + 4 of the tile.
  // Every per-tile DMA is a buffer load: a descriptor for this (batch, head)
  // slice in scalar registers, a per-lane 32-bit byte offset that does not
  // change from tile to tile, and the tile's offset as a scalar, so the loop
  // carries no 64-bit address arithmetic.
  uint32_t v_src[2];
  bool v_on[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int dst = 1024 * (wave + 4 * i) + 16 * lane;  // LDS byte of this lane
    v_on[i] = dst < kBC * d;
    const int row = dst / max(d, 1), pc = (dst % max(d, 1)) >> 4;
    v_src[i] = p.v_swz_shift >= 0 ? row * d + 16 * (pc ^ vswz(row)) : dst;
  }
  typedef __attribute__((address_space(3))) void lptr_t;
  const auto rs_v = make_rsrc(p.vq + bh * N * d, (uint32_t)N * d);
  const auto rs_kmu = make_rsrc(p.kmu + bh * N, 4u * N);
  const auto rs_kbits = make_rsrc(p.kbits + bh * N * W, 4u * N * W);

  // K sign words of a tile, spread over all 256 threads: thread tid expands
  // word kw_w of key kw_key (NKB == 2: all four 16-byte fp4 slots of the
  // key, one per thread; NKB == 1: two threads share a word, 8 bytes each).
  // Padding words (kw_w >= W) expand whatever was loaded: the query operand
  // is zero in those channels.
  // With raw words kept (RAWK) slot s of key j holds word s ^ ((j >> 3) & 3),
  // so that the lanes reading one word of 32 keys hit 32 distinct banks; the
  // words a wave loads stay those of 16 consecutive keys.
  const int kw_key = tid >> 2;
  const int kw_w = RAWK ? ((tid & 3) ^ ((kw_key >> 3) & 3)) : NKB == 2 ? (tid & 3) : ((tid >> 1) & 1);
  const int kw_half = NKB == 2 ? 0 : (tid & 1);
  const int kw_src = 4 * (kw_key * W + min(kw_w, W - 1));  // byte offset within a full tile
  auto expand_k = [&](auto bufc, uint32_t bits) {
    KS& sb = pick(bufc);
    if constexpr (RAWK) {
      sb.kraw[tid] = bits;
      return;
    }
    uint8_t* dst = sb.kx + kw_key * KROW + kslot<NKB>(kw_key, kw_w) * 16;
    if (NKB == 2) {
      u4v o;
      o[0] = fp4_signs(bits, 0); o[1] = fp4_signs(bits, 1);
      o[2] = fp4_signs(bits, 2); o[3] = fp4_signs(bits, 3);
      *reinterpret_cast<u4v*>(dst) = o;
    } else {
      const int m = 2 * kw_half;
      *reinterpret_cast<uint2*>(dst + 8 * kw_half) = make_uint2(fp4_signs(bits, m), fp4_signs(bits, m + 1));
    }
  };
  // this thread's K word of a full tile, DMA'd into the stage (needs the
  // thread's own vmcnt wait only)
  auto finish_k = [&](auto bufc) {
    if constexpr (!RAWK) expand_k(bufc, pick(bufc).kraw[tid]);
  };
  // relative-position window rows of tile t (always in bounds of the table)
  auto dma_tbl = [&](int t, auto bufc) {
    float* tb = tbl_of(pick(bufc));
    if (is_relpos(BIAS) && (!RES || t == 0)) {  // (resident mode: one window, with tile 0)
      int dr_lo, count;
      tbl_window(t, dr_lo, count);
      const auto rs = make_rsrc(static_cast<const float*>(p.bias) + (int64_t)h * T2 * (2 * gh - 1),
                                4u * T2 * (2 * gh - 1));
#pragma unroll
      for (int i = 0; i < kTblMax / 256; ++i) {
        const int x0 = 64 * (wave + 4 * i);
        if (x0 >= count) break;  // uniform: the wave's later rows are past the window
        // lanes past the window reload its last entry into slots past it
        // (inside tbl, never read), so no lane is masked off
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t*)(tb + 1 + x0), 4, 4 * min(x0 + lane, count - 1),
                                                 4 * dr_lo * T2, 0, 0);
      }
    }
  };
  // V rows of tile t by DMA (v_dma layouts): a full tile (CHECKED false,
  // the tile's offset as a scalar) or the ragged one (CHECKED true, the
  // offset in the per-lane part, which the descriptor's range check covers)
  auto dma_v = [&](auto checked, int t, auto bufc) {
    constexpr bool CHECKED = decltype(checked)::value;
    VSt& vb = pick_v(bufc);
    const int j0 = t * kBC;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (v_on[i])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_v, (lptr_t*)(vb.vr + 1024 * (wave + 4 * i)), 16,
                                                 CHECKED ? v_src[i] + j0 * d : v_src[i], CHECKED ? 0 : j0 * d, 0,
                                                 0);
  };
  // the head's V channel scales into vscl (wave 0; entries past d read 0)
  auto dma_vscale = [&]() {
    if (wave == 0) {
      const auto rs = make_rsrc(p.vscale + bh * d, 4u * d);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t*)(vscl + 64 * i), 4, 4 * lane, 256 * i, 0, 0);
    }
  };
  // full tile t (all keys < N), all by DMA: V, mu_k and the table window,
  // then the last group (kLastGroup instructions in every wave): the K words
  // and the fp16 bias tile
  constexpr int kLastGroup = 1 + (BIAS == BIAS_DENSE_F16 ? 4 : 0);
  auto dma_tile = [&](int t, auto bufc, bool with_v) {
    KS& sb = pick(bufc);
    const int j0 = t * kBC;
    if (with_v && p.v_dma) dma_v(BoolC<false>(), t, bufc);
    if (is_attn(MODE) && wave == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_kmu, (lptr_t*)(sb.mk), 4, 4 * lane, 4 * j0, 0, 0);
    dma_tbl(t, bufc);
    stage_koff(t, bufc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_kbits, (lptr_t*)(sb.kraw + 64 * wave), 4, kw_src, 4 * j0 * W, 0, 0);
    if (BIAS == BIAS_DENSE_F16) {
      // wave w fills its own 32 query rows, 8 rows (1 KB) per instruction;
      // the descriptor covers this block's query rows
      const auto rs = make_rsrc(static_cast<const uint16_t*>(p.bias) + (int64_t)b * p.bias_bstride +
                                    ((int64_t)h * N + qb * kQB) * N,
                                2u * N * min(kQB, N - qb * kQB));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wave * kQW + 8 * i + (lane >> 3);
        const int chunk = (lane & 7) ^ bswz(row);
        const int qr = min(qb * kQB + row, N - 1) - qb * kQB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t*)(sb.bt + (wave * kQW + 8 * i) * kBC), 16,
                                                 2 * (qr * N + 8 * chunk), 2 * j0, 0, 0);
      }
    }
  };
  // V tile t through registers, rows past N zero (tiles of V without the
  // DMA layout; any d)
  auto copy_v_checked = [&](int t, auto bufc) {
    VSt& sb = pick_v(bufc);
    const int j0 = t * kBC;
    for (int x = tid; x < kBC * d; x += 256) {
      const int row = x / d, col = x % d;
      const int j = j0 + row;
      sb.vr[row * VS + col] = j < N ? (uint8_t)p.vq[(bh * N + j) * d + col] : (uint8_t)0;
    }
  };
  // The ragged tile, staged after the full ones by the same DMA but with the
  // tile's offset in the per-lane offset, which each descriptor's range check
  // covers: every access past the head's keys is dropped. Whatever those
  // lanes leave in LDS is never used (scores of keys past N are masked, and
  // their P.V operand bytes zeroed). The caller waits, expands the K words
  // and synchronises.
  auto stage_checked = [&](int t, auto bufc, bool with_v) {
    KS& sb = pick(bufc);
    const int j0 = t * kBC;
    if (with_v) {
      if (p.v_dma) dma_v(BoolC<true>(), t, bufc);
      else copy_v_checked(t, bufc);
    }
    if (is_attn(MODE) && wave == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_kmu, (lptr_t*)(sb.mk), 4, 4 * (lane + j0), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_kbits, (lptr_t*)(sb.kraw + 64 * wave), 4, kw_src + 4 * j0 * W, 0,
                                             0, 0);
    dma_tbl(t, bufc);
    stage_koff(t, bufc);
  };
  // s_waitcnt vmcnt(n) (gfx9 encoding; expcnt and lgkmcnt not waited for)
  auto wait_vm0 = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };
  auto wait_vm_last = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70 | kLastGroup); };

  // fp4 K operand (NKB x 16 bytes per lane) of key block kb of the selected
  // buffer, and the S^T block (32 keys x 32 queries) it gives
  // stage slots of this lane's words g and g + 2 in key block 0
  int kraw_at[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int kp = key_of_pos(ql);
    kraw_at[kk] = 4 * kp + ((2 * kk + g) ^ ((kp >> 3) & 3));
  }
  auto k_operand = [&](auto bufc, int kb, u4v* a) {
    KS& sb = pick(bufc);
    const int key = kb * 32 + key_of_pos(ql);
    if constexpr (RAWK) {
      // the key's words g and g + 2, expanded here
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const uint32_t x = sb.kraw[kb * 128 + kraw_at[kk]];
        a[kk] = (u4v){fp4_signs(x, 0), fp4_signs(x, 1), fp4_signs(x, 2), fp4_signs(x, 3)};
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
        a[kk] = *reinterpret_cast<const u4v*>(sb.kx + key * KROW + kslot<NKB>(key, 2 * kk + g) * 16);
    }
  };
  auto qk_mfma = [&](const u4v* a) -> v16f {
    v16f s = {};
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const v8i op = {(int)a[kk][0], (int)a[kk][1], (int)a[kk][2], (int)a[kk][3], 0, 0, 0, 0};
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op, qop[kk], s, 4, 4, 0, 0, 0, 0);
    }
    return s;
  };
  auto qk_block = [&](auto bufc, int kb) -> v16f {
    u4v a[NKB];
    k_operand(bufc, kb, a);
    return qk_mfma(a);
  };

  // Scores of this lane's 16 keys in key block kb of tile t:
  // sigma * mu_k (no bias; the query scale is applied later) or
  // sigma * mu_k * mu_q / sqrt(d) + b (natural-log units, with bias).
  // TAIL: the last tile when N is not a multiple of the tile (bias loads are
  // bounds-checked); MASK: keys past N get -inf.
  auto scores = [&](auto tail, auto mask, int t, auto bufc, int kb, const v16f& sig, float* sc) {
    KS& sb = pick(bufc);
    constexpr bool TAIL = decltype(tail)::value;
    constexpr bool MASK = decltype(mask)::value;
    const int jl = kb * 32 + 16 * g;  // first key of the lane's 16, in the tile
    const int jb = t * kBC + jl;
    if constexpr (BIAS == BIAS_RELPOS || BIAS == BIAS_DENSE_ANY) {
      // (the product feeds two bias paths here; a row broadcast would not
      // fold into it, so the 16 scales are read as vectors)
      const float4* mkp = reinterpret_cast<const float4*>(sb.mk + jl);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 m4 = mkp[r];
        sc[4 * r + 0] = sig[4 * r + 0] * m4.x;
        sc[4 * r + 1] = sig[4 * r + 1] * m4.y;
        sc[4 * r + 2] = sig[4 * r + 2] * m4.z;
        sc[4 * r + 3] = sig[4 * r + 3] * m4.w;
      }
    } else {
      mul_key_scales(sc, sig, sb.mk[jl + (lane & 15)], std::make_integer_sequence<int, 16>{});
    }
    if (DENSE) {
      const int64_t row = (int64_t)b * p.bias_bstride + ((int64_t)h * N + qc) * N;
      float bv[16];
      if ((BIAS == BIAS_DENSE_F16 || BIAS == BIAS_DENSE_F32) && !TAIL) {
        if (BIAS == BIAS_DENSE_F16) {
          // staged in LDS by dma_tile
          const int rl = wave * kQW + ql;
          const u4v* src = reinterpret_cast<const u4v*>(sb.bt + rl * kBC);
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const u4v v = src[(4 * kb + 2 * g + r) ^ bswz(rl)];
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[8 * r + e] = f16_to_f32((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
          }
        } else if (BIAS == BIAS_DENSE_F32) {
          const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(p.bias) + row + jb);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float4 v = src[r];
            bv[4 * r] = v.x; bv[4 * r + 1] = v.y; bv[4 * r + 2] = v.z; bv[4 * r + 3] = v.w;
          }
        }
      } else if (BIAS == BIAS_DENSE_ANY && !TAIL && p.bias_al4 == 1) {
        // rows 4-byte but not 16-byte aligned: 16-byte loads at 4-byte
        // alignment (gfx950 global loads accept them), not one load per value
        typedef float f4a4 __attribute__((ext_vector_type(4), aligned(4)));
        typedef unsigned u4a4 __attribute__((ext_vector_type(4), aligned(4)));
        if (p.bias_f16) {
          const u4a4* src = reinterpret_cast<const u4a4*>(static_cast<const uint16_t*>(p.bias) + row + jb);
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const u4a4 v = src[r];
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[8 * r + e] = f16_to_f32((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
          }
        } else {
          const f4a4* src = reinterpret_cast<const f4a4*>(static_cast<const float*>(p.bias) + row + jb);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const f4a4 v = src[r];
            bv[4 * r] = v.x; bv[4 * r + 1] = v.y; bv[4 * r + 2] = v.z; bv[4 * r + 3] = v.w;
          }
        }
      } else if (BIAS == BIAS_DENSE_ANY && !TAIL && p.bias_al4 == 2) {
        // fp16 rows only 2-byte aligned (a 4-byte aligned base): the 4-byte words around the lane's 16
        // values (a ninth word only when they start mid-word, so nothing past
        // the last value's word is read), realigned by a funnel shift
        typedef unsigned u4a4 __attribute__((ext_vector_type(4), aligned(4)));
        const int64_t o = row + jb;
        const uint32_t* w = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.bias) + (o & ~(int64_t)1));
        const uint32_t sh = 16u * (uint32_t)(o & 1);
        const u4a4 w0 = reinterpret_cast<const u4a4*>(w)[0], w1 = reinterpret_cast<const u4a4*>(w)[1];
        const uint32_t w8 = sh ? w[8] : 0u;
        const uint32_t ws[9] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3], w8};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t pr = __builtin_amdgcn_alignbit(ws[k + 1], ws[k], sh);
          bv[2 * k] = f16_to_f32((uint16_t)pr);
          bv[2 * k + 1] = f16_to_f32((uint16_t)(pr >> 16));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = min(jb + i, N - 1);
          const bool f16 = BIAS == BIAS_DENSE_F16 || (BIAS == BIAS_DENSE_ANY && p.bias_f16);
          bv[i] = f16 ? f16_to_f32(static_cast<const uint16_t*>(p.bias)[row + j])
                      : static_cast<const float*>(p.bias)[row + j];
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = __builtin_fmaf(sc[i], c0, bv[i]);
    } else if (is_relpos(BIAS)) {
      const float* tb = tbl_of(sb);
      float bv[16];
      if constexpr (BIAS == BIAS_RELPOS_ROW && !TAIL) {
        // 16 keys on one grid row: a contiguous, reversed window. Its lowest
        // entry's address is formed once and kept opaque, so that the 16
        // reads take small immediate offsets from it (the window's offset
        // inside the stage would not fit the paired read's offset fields,
        // and the compiler would add it per pair).
        typedef __attribute__((address_space(3))) const float lds_f32;
        lds_f32* lo = (lds_f32*)(reinterpret_cast<const char*>(tb) + (qwin1 - sb.koff[jl])) - 15;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int i = 0; i < 16; ++i) bv[i] = lo[15 - i];
      } else {
        const int4* kop = reinterpret_cast<const int4*>(sb.koff + jl);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int4 ko = kop[r];
          const int k4[4] = {ko.x, ko.y, ko.z, ko.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            bv[4 * r + e] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(tb) +
                                                            __builtin_elementwise_sub_sat((uint32_t)qwin1, (uint32_t)k4[e]));
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = __builtin_fmaf(sc[i], c0, bv[i]);
    }
    if (MASK) {
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
  // key scales and fp16 bias words of this lane's 16 keys in block kb, read
  // from the stage ahead of use (full tiles of the fp16 dense-bias path)
  struct KeyVals {
    float mk;  // scale of key 16 * g + lane % 16 of the block
    u4v bb[2];
  };
  auto load_keyvals = [&](auto bufc, int kb, KeyVals& r) {
    KS& sb = pick(bufc);
    r.mk = sb.mk[kb * 32 + 16 * g + (lane & 15)];
    const int rl = wave * kQW + ql;
    const u4v* src = reinterpret_cast<const u4v*>(sb.bt + rl * kBC);
#pragma unroll
    for (int i = 0; i < 2; ++i) r.bb[i] = src[(4 * kb + 2 * g + i) ^ bswz(rl)];
  };
  auto scores_kv = [&](const v16f& sig, const KeyVals& r, float* sc) {
    mul_key_scales(sc, sig, r.mk, std::make_integer_sequence<int, 16>{});
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t wd = r.bb[e >> 3][(e >> 1) & 3];
      sc[e] = __builtin_fmaf(sc[e], c0, f16_to_f32((uint16_t)(wd >> (16 * (e & 1)))));
    }
  };
  auto pass1_tile = [&](auto tail, int t, auto bufc) {
    constexpr bool TAIL = decltype(tail)::value;
    float sc[16];
    if constexpr (BIAS == BIAS_DENSE_F16 && !TAIL) {
      // every LDS read of the tile is issued first (K operands, then key
      // scales and bias), so one wait covers them rather than one per use
      u4v a0[NKB], a1[NKB];
      k_operand(bufc, 0, a0);
      k_operand(bufc, 1, a1);
      KeyVals kv0, kv1;
      load_keyvals(bufc, 0, kv0);
      load_keyvals(bufc, 1, kv1);
      __builtin_amdgcn_sched_barrier(0);
      const v16f sig0 = qk_mfma(a0);
      const v16f sig1 = qk_mfma(a1);
      scores_kv(sig0, kv0, sc);
      max16(sc);
      scores_kv(sig1, kv1, sc);
      max16(sc);
    } else if (TAIL && t * kBC + 32 >= N) {
      // the ragged tile's second block holds no key < N
      const v16f sig0 = qk_block(bufc, 0);
      scores(tail, tail, t, bufc, 0, sig0, sc);
      max16(sc);
    } else {
      const v16f sig0 = qk_block(bufc, 0);
      const v16f sig1 = qk_block(bufc, 1);
      scores(tail, tail, t, bufc, 0, sig0, sc);
      max16(sc);
      scores(tail, tail, t, bufc, 1, sig1, sc);
      max16(sc);
    }
    // keep the running max here, ahead of the end-of-tile wait, rather than
    // let the compiler sink it past the wait
    const float ma = m0, mb = m1;
    asm volatile("" ::"v"(ma), "v"(mb));
  };
  const int nfull = ragged ? ntiles - 1 : ntiles;
  // Full tiles cycle through NS stages (tile t in stage t % NS, the loop
  // unrolled by NS so the stage is known at compile time): tile t + NS - 1
  // is loaded while tile t is computed, and the end of step t waits only
  // for tile t + 1. Then the ragged tile, staged synchronously.
  // pre: work done while the first tiles' DMA is in flight
  auto run_pass = [&](auto nsc, bool with_v, auto body, auto pre) {
    // (with_v: pass 2, whose progress sets the issue priority)
    constexpr int NS = decltype(nsc)::value;
    if (nfull > 0) {
      dma_tile(0, IntC<0>(), with_v);
      if constexpr (NS == 3) {
        if (nfull > 1) dma_tile(1, IntC<1>(), with_v);
      }
      pre();
      if (NS == 3 && nfull > 1) wait_vm_last();
      else wait_vm0();
      finish_k(IntC<0>());
      if (with_v && !p.v_dma) copy_v_checked(0, IntC<0>());
    } else {
      stage_checked(0, IntC<0>(), with_v);
      pre();
      wait_vm0();
      finish_k(IntC<0>());
    }
    __syncthreads();
    auto step = [&](int t, auto cur) {
      constexpr int c = decltype(cur)::value;
      constexpr int nx = (c + 1) % NS, far = (c + NS - 1) % NS;
      const bool issue = t + NS - 1 < nfull;
      if (issue) dma_tile(t + NS - 1, IntC<far>(), with_v);
      body(BoolC<false>(), t, cur);
      if (with_v) progress(t + 1);
      if (t + 1 < nfull) {
        if (NS == 3 && issue) wait_vm_last();
        else wait_vm0();
        finish_k(IntC<nx>());
        if (with_v && !p.v_dma) copy_v_checked(t + 1, IntC<nx>());
      }
      __syncthreads();
    };
    for (int t = 0; t < nfull; t += NS) {
      step(t, IntC<0>());
      if (t + 1 < nfull) step(t + 1, IntC<1>());
      if constexpr (NS == 3) {
        if (t + 2 < nfull) step(t + 2, IntC<2>());
      }
    }
    if (ragged) {
      const int t = ntiles - 1;
      auto tail = [&](auto cur) {
        if (nfull > 0) {
          stage_checked(t, cur, with_v);
          wait_vm0();
          finish_k(cur);
          __syncthreads();
        }
        body(BoolC<true>(), t, cur);
      };
      const int sidx = t % NS;
      if (sidx == 0) tail(IntC<0>());
      else if (sidx == 1) tail(IntC<1>());
      else if constexpr (NS == 3) tail(IntC<2>());
    }
  };
  // Resident mode: every tile into a stage of its own. The query loads and
  // then the key side of all tiles (K words, key scales, table window) are
  // issued, and the query operand formed while they land; one wait, then the V rows of all tiles and the
  // channel scales are started and pass 1 runs while they land; a second
  // wait before pass 2. Neither pass waits or synchronises per tile.
  // Resident mode from 16-bit K and V (p.k16, p.v16; d % 8 == 0): the
  // workgroup binarises and quantises its head's keys and values itself,
  // with the pre-pass kernels' arithmetic, straight into the stages, so the
  // packed arrays never go through HBM (each head is read by its nqb <= 2
  // query blocks). Thread j packs key j: the row's 16-byte pieces, sign bits
  // by a float compare, float64 piece sums of |x| added in channel order,
  // one float64 division by d; the fp4 operand goes to the slots expand_k
  // uses. V: channel maxima of |v| (a 16-bit magnitude max per thread, an
  // LDS max on the float bits), inv = 127 / amax and scale = amax / 127 in
  // float32, then a second read of the rows quantised into the V stage
  // layout; the scales stay in LDS for the epilogue. Keys and V rows past N
  // are left unwritten: their scores are masked and their P.V operand bytes
  // and channel-sum bytes zeroed, as for the ragged tile's DMA.
  auto res_stage16 = [&](auto dtc) __attribute__((always_inline)) {
    constexpr int DT = decltype(dtc)::value;
    if constexpr (RES && MODE == MODE_ATTN) {
    static_assert(!RAWK, "the resident mode keeps the fp4 K operand in LDS");
    issue_q();
    for (int t = 0; t < ntiles; ++t) {
      dma_tbl(t, t);
      stage_koff(t, t);
    }
    // vscl holds the maxima' float bits, then 127 / amax while the rows are
    // quantised, then the scales amax / 127 (thread c keeps amax of channel c)
    uint32_t* vamax = reinterpret_cast<uint32_t*>(vscl);
    if (tid < d) vamax[tid] = 0u;
    if (tid < N) {
      const uint16_t* row = p.k16 + (bh * N + tid) * d;
      uint32_t wb[2 * NKB];
#pragma unroll
      for (int w = 0; w < 2 * NKB; ++w) wb[w] = 0u;
      double acc = 0.0;
#pragma unroll
      for (int pc = 0; pc < 8 * NKB; ++pc) {
        if (8 * pc < d) {
          const u4v raw = *reinterpret_cast<const u4v*>(row + 8 * pc);
          uint32_t b8 = 0;
          double sm = 0.0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xf = to_f32<DT>((uint16_t)(raw[e >> 1] >> ((e & 1) * 16)));
            b8 |= xf < 0.0f ? (1u << e) : 0u;
            sm += (double)fabsf(xf);
          }
          wb[pc >> 2] |= b8 << (8 * (pc & 3));
          acc += sm;
        }
      }
      KS& sb = ksr[tid >> 6];
      const int kl = tid & 63;
#pragma unroll
      for (int w = 0; w < 2 * NKB; ++w)
        *reinterpret_cast<u4v*>(sb.kx + kl * KROW + kslot<NKB>(kl, w) * 16) =
            (u4v){fp4_signs(wb[w], 0), fp4_signs(wb[w], 1), fp4_signs(wb[w], 2), fp4_signs(wb[w], 3)};
      sb.mk[kl] = (float)(acc / (double)d);
    }
    // V: thread tid takes 16-byte piece tid % P of rows tid / P + k R
    const int P = d >> 3, R = 256 / P;
    const int piece = tid % P, r0 = tid / P;
    const bool vact = r0 < R;
    const uint16_t* vh = p.v16 + bh * N * d + 8 * piece;
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 mb[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
    auto take = [&](const u4v& raw) __attribute__((always_inline)) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        mb[w] = __builtin_elementwise_max(mb[w], __builtin_bit_cast(us2, raw[w] & 0x7FFF7FFFu));
    };
    if (vact) {
      int j = r0;
      for (; j + 3 * R < N; j += 4 * R) {
        u4v raw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) raw[u] = *reinterpret_cast<const u4v*>(vh + (int64_t)(j + u * R) * d);
#pragma unroll
        for (int u = 0; u < 4; ++u) take(raw[u]);
      }
      for (; j < N; j += R) take(*reinterpret_cast<const u4v*>(vh + (int64_t)j * d));
    }
    __syncthreads();  // (the zeroed maxima)
    if (vact) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        atomicMax(&vamax[8 * piece + e], __float_as_uint(to_f32<DT>(mb[e >> 1][e & 1])));
    }
    __syncthreads();
    float amax_c = 0.0f;
    if (tid < d) {
      amax_c = __uint_as_float(vamax[tid]);
      vscl[tid] = amax_c > 0.0f ? 127.0f / amax_c : 0.0f;
    }
    __syncthreads();
    if (vact) {
      float inv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) inv[e] = vscl[8 * piece + e];
      auto quant8 = [&](const u4v& raw, int j) __attribute__((always_inline)) {
        *reinterpret_cast<uint2*>(vsr[j >> 6].vr + vaddr(j & 63, 8 * piece)) = quant8_codes<DT>(raw, inv);
      };
      int j = r0;
      for (; j + 3 * R < N; j += 4 * R) {
        u4v raw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) raw[u] = *reinterpret_cast<const u4v*>(vh + (int64_t)(j + u * R) * d);
#pragma unroll
        for (int u = 0; u < 4; ++u) quant8(raw[u], j + u * R);
      }
      for (; j < N; j += R) quant8(*reinterpret_cast<const u4v*>(vh + (int64_t)j * d), j);
    }
    finish_q();
    wait_vm0();
    __syncthreads();  // (every thread has read its 127 / amax)
    if (tid < d) vscl[tid] = amax_c / 127.0f;
    __syncthreads();
    }
  };
  auto res_stage = [&]() __attribute__((always_inline)) {
    if constexpr (RES && MODE == MODE_ATTN) {
      if (p.k16) {
        if (p.q16_f16) res_stage16(IntC<BA_F16>());
        else res_stage16(IntC<BA_BF16>());
        return;
      }
    }
    if constexpr (RES) {
      issue_q();
      for (int t = 0; t < ntiles; ++t) {
        if (t < nfull) dma_tile(t, t, false);
        else stage_checked(t, t, false);
      }
      finish_q();
      wait_vm0();
      for (int t = 0; t < ntiles; ++t) {
        finish_k(t);
        if (!p.v_dma) copy_v_checked(t, t);
        else if (t < nfull) dma_v(BoolC<false>(), t, t);
        else dma_v(BoolC<true>(), t, t);
      }
      dma_vscale();
      __syncthreads();
    }
  };
  auto res_pass = [&](bool with_v, auto body) {
    for (int t = 0; t < nfull; ++t) {
      body(BoolC<false>(), t, t);
      if (with_v) progress(t + 1);
    }
    if (ragged) body(BoolC<true>(), ntiles - 1, ntiles - 1);
  };
  if constexpr (MODE == MODE_SIGMA || MODE == MODE_SIGMA_RAW) {
    // the Q.K of every staged tile, as pass 2 forms it, written out
    // (MODE_SIGMA) or compared (MODE_SIGMA_RAW, after MODE_SIGMA wrote it)
    auto sigma_tile = [&](auto tail, int t, auto bufc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u4v a[NKB];
        k_operand(bufc, kb, a);
        put_sigma(BoolC<MODE == MODE_SIGMA_RAW>(), qi, t * kBC + kb * 32 + 16 * g, qk_mfma(a));
      }
    };
    run_pass(IntC<Cfg::NS2>(), false, sigma_tile, [] {});
    return;
  }
  if constexpr (MODE == MODE_ONLINE) {
    // ======== one pass with a running row maximum (FlashAttention-2 order) ========
    // The keys stream once. Per 32-key block a lane takes the block maximum
    // of its query (its 16 keys and the partner lane's 16); when the running
    // maximum m of any query of the wave grows, every lane folds: O <- (O +
    // A) * exp(m_old - m_new), l <- l * exp(m_old - m_new), A <- 0 (O and A
    // both hold sums taken against m_old; for a query whose maximum did not
    // grow the factor is exactly 1). Then p8 =
    // rne(255 * exp(s - m)) with the current m, l += 255 * exp(s - m), and A
    // += p8 v8 on the int8 matrix cores. p8 reaches 255 while the int8 MFMA
    // is signed, and A must fold exactly at any point, so the product takes
    // p8 as two nibble operands (0..15): A = 16 A_hi + A_lo, both exact.
    // At the end out = (O + A) * vscale / l.
    const float sc2 = (BIAS == BIAS_NONE) ? cq : kLog2e;  // score -> base-2 units
    float mo = -INFINITY;   // running maximum (score units of the pass-1 code)
    float ngm = 0.0f;       // log2(255) - m * sc2
    float ls = 0.0f;        // 255 * running sum over this lane's keys
    v16i ah[NCB], al[NCB];  // A_hi and A_lo since the last fold
    float of[NCB][16];      // folded output, fp32
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      ah[cb] = (v16i){};
      al[cb] = (v16i){};
#pragma unroll
      for (int i = 0; i < 16; ++i) of[cb][i] = 0.0f;
    }
    const int tr_row = 16 * (lane >> 5) + ((lane & 15) >> 1);  // transposing read, as in pass 2
    const int tr_col = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
    auto fold = [&](float alpha) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) of[cb][i] = (of[cb][i] + (float)(16 * ah[cb][i] + al[cb][i])) * alpha;
        ah[cb] = (v16i){};
        al[cb] = (v16i){};
      }
    };
    auto oblock = [&](auto tail, int t, auto bufc, int kb) {
      u4v a[NKB];
      k_operand(bufc, kb, a);
      const v16f sig = qk_mfma(a);
      float sc[16];
      scores(tail, tail, t, bufc, kb, sig, sc);  // keys past N: -inf
      float b0 = -INFINITY, b1 = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        b0 = fmaxf(fmaxf(b0, sc[i]), sc[i + 1]);
        b1 = fmaxf(fmaxf(b1, sc[i + 2]), sc[i + 3]);
      }
      float bm = fmaxf(b0, b1);
      bm = fmaxf(bm, partner32(bm, lane));
      const float mn = fmaxf(mo, bm);
      if (__builtin_amdgcn_ballot_w64(mn > mo) != 0) {  // wave-uniform
        const float alpha = mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mo - mn) * sc2);
        fold(alpha);
        ls *= alpha;
        mo = mn;
        ngm = __builtin_fmaf(-sc2, mo, kLog2_255);
      }
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          e[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * r + k], sc2, ngm));
          ls += e[k];
        }
        uint32_t wd = __builtin_amdgcn_cvt_pk_u8_f32(e[0], 0, 0u);
        wd = __builtin_amdgcn_cvt_pk_u8_f32(e[1], 1, wd);
        wd = __builtin_amdgcn_cvt_pk_u8_f32(e[2], 2, wd);
        wd = __builtin_amdgcn_cvt_pk_u8_f32(e[3], 3, wd);
        hi[r] = (wd >> 4) & 0x0F0F0F0Fu;  // keys past N: p8 = 0 in both
        lo[r] = wd & 0x0F0F0F0Fu;
      }
      const v4i bhi = (v4i){(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      const v4i blo = (v4i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
      const uint8_t* vb = pick_v(bufc).vr;
      const int r0 = kb * 32 + tr_row, r1 = r0 + 8;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const v2i vlo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vb + vaddr(r0, tr_col + 32 * cb)));
        const v2i vhi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vb + vaddr(r1, tr_col + 32 * cb)));
        const v4i vt = (v4i){vlo[0], vlo[1], vhi[0], vhi[1]};
        ah[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(vt, bhi, ah[cb], 0, 0, 0);
        al[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(vt, blo, al[cb], 0, 0, 0);
      }
    };
    auto otile = [&](auto tail, int t, auto bufc) {
      constexpr bool TAIL = decltype(tail)::value;
      oblock(tail, t, bufc, 0);
      if (!(TAIL && t * kBC + 32 >= N)) oblock(tail, t, bufc, 1);  // (a block holding a key < N)
    };
    run_pass(IntC<NS2>(), true, otile, [] {});
    fold(1.0f);
    const float lr = ls + partner32(ls, lane);  // 255 l over both halves of the keys
    if (!qvalid) return;
    const float inv_l = 1.0f / lr;
    uint16_t* outp = static_cast<uint16_t*>(p.out) + b * p.out_sb + (int64_t)h * p.out_sh + (int64_t)qi * p.out_sn;
    const float* vs = p.vscale + bh * d;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = cb * 32 + 8 * r + 4 * g;  // channels c .. c + 3 of acc[cb][4 r ..]
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = of[cb][4 * r + e] * (vs[min(c + e, d - 1)] * inv_l);
          o[e] = (c + e < d) ? ((p.out_mode & 1) ? f32_to_f16(x) : f32_to_bf16(x)) : (uint16_t)0;
        }
        if (p.out_mode & 2) {
          if (c < d)
            *reinterpret_cast<uint2*>(outp + c) =
                make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < d) outp[c + e] = o[e];
        }
      }
    }
    return;
  }
  float mrun;
  if constexpr (P1_SPLIT) {
    // Pass 1 splits the keys, not the queries, over the waves: wave w takes
    // the 32-key blocks w, w + 4, ... against all 128 queries of the
    // workgroup (four MFMA query groups), straight from global memory into
    // registers: no shared staging and no barrier, and each block's K words
    // are expanded once for four query groups. A wave's next block is loaded
    // while the current one is computed. The four partial maxima of each
    // query are combined through LDS at the end.
    v8i qop4[4][NKB];
    float c04[4];
    if (MODE == MODE_ATTN && p.q16) {
      // the workgroup's query signs and scales as the waves packed them
      // (finish_q); the stage is not touched again before pass 2's barrier
      static_assert((2 * NKB + 1) * kQB * 4 <= (int)sizeof(VSt::vr), "query table fits the first V stage");
      __syncthreads();
      const uint32_t* tw = reinterpret_cast<const uint32_t*>(vs0.vr);
      const float* tm = reinterpret_cast<const float*>(tw + kQB * W);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int qr = kQW * q + ql;
        uint32_t wb[NKB];
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) wb[kk] = 2 * kk + g < W ? tw[qr * W + 2 * kk + g] : 0u;
        q_operand_w(wb, qop4[q]);
        c04[q] = tm[qr] * p.inv_sqrt_d;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int qq = qb * kQB + kQW * q + ql;
        q_operand(qq, qq < N, qop4[q]);
        c04[q] = (MODE == MODE_ATTN && qq < N) ? p.qmu[bh * N + qq] * p.inv_sqrt_d : 0.0f;
      }
    }
    struct Blk {
      uint32_t kw[NKB];
      float4 mk[4];  // scales of keys 16 * g .. 16 * g + 15 of the block
      u4v bb[BIAS == BIAS_DENSE_F16 ? 4 : 1][2];
    };
    const float* kmu_bh = p.kmu + bh * N;
    const uint16_t* bias_bh = static_cast<const uint16_t*>(p.bias) + (int64_t)b * p.bias_bstride + (int64_t)h * N * N;
    // full block: every key < N
    auto load_blk = [&](int blk, Blk& r) {
      const int k0 = blk * 32;
      const int myk = k0 + key_of_pos(ql);  // key of this lane's A-operand row
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const int w = 2 * kk + g;
        r.kw[kk] = w < W ? p.kbits[(bh * N + myk) * W + w] : 0u;
      }
      if constexpr (MODE != MODE_ATTN) return;  // the sigma modes take no scales
      if (p.mk_vec) {
        const float4* src = reinterpret_cast<const float4*>(kmu_bh + k0 + 16 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.mk[i] = src[i];
      } else {
        const float* src = kmu_bh + k0 + 16 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) r.mk[i] = make_float4(src[4 * i], src[4 * i + 1], src[4 * i + 2], src[4 * i + 3]);
      }
      if constexpr (BIAS == BIAS_DENSE_F16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = min(qb * kQB + kQW * q + ql, N - 1);
          const u4v* src = reinterpret_cast<const u4v*>(bias_bh + (int64_t)row * N + k0 + 16 * g);
          r.bb[q][0] = src[0];
          r.bb[q][1] = src[1];
        }
      }
    };
    // the ragged last block: loads clamped to key N - 1 (those keys are masked)
    auto load_blk_tail = [&](int blk, Blk& r) {
      const int k0 = blk * 32;
      const int myk = min(k0 + key_of_pos(ql), N - 1);
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const int w = 2 * kk + g;
        r.kw[kk] = w < W ? p.kbits[(bh * N + myk) * W + w] : 0u;
      }
      if constexpr (MODE != MODE_ATTN) return;
      float mv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) mv[i] = kmu_bh[min(k0 + 16 * g + i, N - 1)];
#pragma unroll
      for (int i = 0; i < 4; ++i) r.mk[i] = make_float4(mv[4 * i], mv[4 * i + 1], mv[4 * i + 2], mv[4 * i + 3]);
      if constexpr (BIAS == BIAS_DENSE_F16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = min(qb * kQB + kQW * q + ql, N - 1);
          const uint16_t* src = bias_bh + (int64_t)row * N;
          uint32_t hw[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            hw[e] = (uint32_t)src[min(k0 + 16 * g + 2 * e, N - 1)] | ((uint32_t)src[min(k0 + 16 * g + 2 * e + 1, N - 1)] << 16);
          r.bb[q][0] = (u4v){hw[0], hw[1], hw[2], hw[3]};
          r.bb[q][1] = (u4v){hw[4], hw[5], hw[6], hw[7]};
        }
      }
    };
    float mx[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) mx[q][0] = mx[q][1] = -INFINITY;
    // ALLQ: all four query groups hold a query < N (only the last query
    // block of a head may have groups past N, which are skipped)
    auto comp_blk = [&](auto allq, auto tail, int blk, const Blk& r) __attribute__((always_inline)) {
      constexpr bool ALLQ = decltype(allq)::value;
      constexpr bool TAIL = decltype(tail)::value;
      v8i a[NKB];
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk)
        a[kk] = (v8i){(int)fp4_signs(r.kw[kk], 0), (int)fp4_signs(r.kw[kk], 1), (int)fp4_signs(r.kw[kk], 2),
                      (int)fp4_signs(r.kw[kk], 3), 0, 0, 0, 0};
      const int jb = blk * 32 + 16 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!ALLQ && qb * kQB + kQW * q >= N) continue;  // no query of the group < N
        v16f sg = {};
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
          sg = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[kk], qop4[q][kk], sg, 4, 4, 0, 0, 0, 0);
        if constexpr (MODE == MODE_SIGMA_SPLIT) {
          put_sigma(BoolC<true>(), qb * kQB + kQW * q + ql, jb, sg);
          continue;
        }
        float sc[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[4 * i + 0] = sg[4 * i + 0] * r.mk[i].x;
          sc[4 * i + 1] = sg[4 * i + 1] * r.mk[i].y;
          sc[4 * i + 2] = sg[4 * i + 2] * r.mk[i].z;
          sc[4 * i + 3] = sg[4 * i + 3] * r.mk[i].w;
        }
        if constexpr (BIAS == BIAS_DENSE_F16) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t wd = r.bb[q][e >> 3][(e >> 1) & 3];
            sc[e] = __builtin_fmaf(sc[e], c04[q], f16_to_f32((uint16_t)(wd >> (16 * (e & 1)))));
          }
        }
        if (TAIL) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (jb + i >= N) sc[i] = -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          mx[q][0] = fmaxf(fmaxf(mx[q][0], sc[i]), sc[i + 1]);
          mx[q][1] = fmaxf(fmaxf(mx[q][1], sc[i + 2]), sc[i + 3]);
        }
      }
    };
    const int nfb = N >> 5;  // full 32-key blocks
    auto split_pass = [&](auto allq) {
      Blk ra, rb;
      if (wave < nfb) load_blk(wave, ra);
      for (int blk = wave; blk < nfb; blk += 8) {
        const bool hb = blk + 4 < nfb;
        if (hb) load_blk(blk + 4, rb);
        comp_blk(allq, BoolC<false>(), blk, ra);
        if (hb) {
          if (blk + 8 < nfb) load_blk(blk + 8, ra);
          comp_blk(allq, BoolC<false>(), blk + 4, rb);
        }
      }
      if ((N & 31) != 0 && wave == (nfb & 3)) {
        Blk rt;
        load_blk_tail(nfb, rt);
        comp_blk(allq, BoolC<true>(), nfb, rt);
      }
    };
    if (qb * kQB + kQB <= N) split_pass(BoolC<true>());
    else split_pass(BoolC<false>());
    if constexpr (MODE == MODE_SIGMA_SPLIT) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v = fmaxf(mx[q][0], mx[q][1]);
      v = fmaxf(v, partner32(v, lane));
      if (g == 0) p1red[wave][q][ql] = v;
    }
    __syncthreads();
    mrun = fmaxf(fmaxf(p1red[0][wave][ql], p1red[1][wave][ql]), fmaxf(p1red[2][wave][ql], p1red[3][wave][ql]));
  } else {
    if constexpr (RES) {
      res_stage();
      if (wave_live) res_pass(false, pass1_tile);
    } else {
      // (a wave with no live query stages its share of the tiles only;
      // every wave meets the same barriers)
      if (wave_live) run_pass(IntC<NS1>(), false, pass1_tile, finish_q);
      else run_pass(IntC<NS1>(), false, [](auto, int, auto) {}, finish_q);
    }
    mrun = fmaxf(m0, m1);
    mrun = fmaxf(mrun, partner32(mrun, lane));
  }
  // x = score * scale2 + negm is log2(255 * exp(s - m))
  const float scale2 = (BIAS == BIAS_NONE) ? cq : kLog2e;
  const float negm = __builtin_fmaf(-scale2, mrun, kLog2_255);

  // ================= pass 2: u8 P, row sum, integer P.V =================
  float l0 = 0.0f, l1 = 0.0f, l2 = 0.0f, l3 = 0.0f;  // 255 * row sum of exp(s - m)
  v16i acc[NCB];      // ends at sum_j (127 - p8_j) v8_j
  int vsacc[NCB];     // channel 32 cb + lane % 32: sum of v8 over this wave's key blocks
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) vsacc[cb] = 0;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = (v16i){};
  // transposing-read address of this lane for the V^T operand: row
  // 16*(lane/32) + (lane%16)/2 (+8 for the upper half), column
  // 16*((lane/16)%2) + 8*(lane%2) (+32 per channel block)
  const int tr_row = 16 * (lane >> 5) + ((lane & 15) >> 1);
  const int tr_col = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);

  // byte masks of this lane's 16 keys of block kb in tile t (dword r, byte
  // e: key 16 g + 4 r + e), set where the key is < N
  auto key_keep = [&](int t, int kb, uint32_t* keep) {
    const int jb = t * kBC + kb * 32 + 16 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      keep[r] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) keep[r] |= (jb + 4 * r + e < N ? 0xFFu : 0u) << (8 * e);
    }
  };
  // u8 probabilities of one key block, as the s8 MFMA operand 127 - p8, and
  // the float row sum. Tail keys (past N) are masked after the scaling:
  // -inf * 0 would be NaN.
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
    if (TAIL) {
      // keys past N: operand 0, so the (unused) V rows staged for them add
      // nothing (their p8 is already 0: exp2(-inf))
      uint32_t keep[4];
      key_keep(t, kb, keep);
#pragma unroll
      for (int r = 0; r < 4; ++r) pw[r] &= keep[r];
    }
    return (v4i){(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]};
  };
  // Channel sums of v8 from the V^T operand of key block kb of tile t: lane
  // l holds channel 32 cb + l % 32 of the keys 16 (l / 32) .. + 15, so four
  // v_dot4 against 0x01010101 add them. Wave w takes the blocks whose index
  // over the head is w mod 4 (a uniform branch); the waves' sums meet in
  // LDS after the pass. Tail keys past N are masked: their V rows in LDS are
  // stale.
  auto vsum_blk = [&](auto tail, int t, int kb, const v4i* vt) {
    constexpr bool TAIL = decltype(tail)::value;
    if (((2 * t + kb) & 3) != wave) return;
    uint32_t keep[4] = {~0u, ~0u, ~0u, ~0u};
    if (TAIL) key_keep(t, kb, keep);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vsacc[cb] = __builtin_amdgcn_sdot4((int)((uint32_t)vt[cb][r] & keep[r]), 0x01010101, vsacc[cb], false);
  };
  // V^T operand (NCB x 16 bytes per lane) of key block kb, read from LDS
  auto read_vt = [&](auto bufc, int kb, v4i* vt) {
    VSt& sb = pick_v(bufc);
    const uint8_t* vb = sb.vr;
    const int r0 = kb * 32 + tr_row, r1 = r0 + 8;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vb + vaddr(r0, tr_col + 32 * cb)));
      const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vb + vaddr(r1, tr_col + 32 * cb)));
      vt[cb] = (v4i){lo[0], lo[1], hi[0], hi[1]};
    }
  };
  // pass-2 u8 probabilities of key block kb
  auto probs2 = [&](auto tail, int t, auto bufc, int kb, const v16f& sig) -> v4i {
    float sc[16];
    scores(tail, BoolC<false>(), t, bufc, kb, sig, sc);
    return probs(tail, t, kb, sc);
  };
  // P.V of one key block: acc += V^T (127 - p8)
  auto pv_regs = [&](const v4i* vt, const v4i& bop) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      acc[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(vt[cb], bop, acc[cb], 0, 0, 0);
  };
  // A wave issues in order, so the matrix products of a tile are spread
  // through the VALU work that does not depend on them: block 1's Q.K and
  // the previous tile's deferred P.V run under block 0's softmax, block 0's
  // P.V under block 1's. Block 1's P.V is deferred to the next tile, its
  // operands carried in registers across the barrier (zero at the start:
  // the first deferred product adds 0).
  v4i vt_held[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) vt_held[cb] = (v4i){0, 0, 0, 0};
  v4i p_held = (v4i){0, 0, 0, 0};
  constexpr int kValuPerMfma = 10;
  // a wave with no live query: its share of the channel sums only
  auto vsum_only = [&](auto tail, int t, auto bufc) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (((2 * t + kb) & 3) != wave) continue;
      v4i vt[NCB];
      read_vt(bufc, kb, vt);
      vsum_blk(tail, t, kb, vt);
    }
  };
  auto pass2_tile = [&](auto tail, int t, auto bufc) {
    constexpr bool TAIL = decltype(tail)::value;
    if (!wave_live) {
      vsum_only(tail, t, bufc);
      return;
    }
    if (TAIL && t * kBC + 32 >= N) {
      // ragged tile with no key < N in its second block: the deferred
      // product of the previous tile, then block 0 alone (nothing deferred)
      pv_regs(vt_held, p_held);
      u4v a0[NKB];
      k_operand(bufc, 0, a0);
      const v16f sig0 = qk_mfma(a0);
      v4i vt0[NCB];
      read_vt(bufc, 0, vt0);
      vsum_blk(tail, t, 0, vt0);
      const v4i p0 = probs2(tail, t, bufc, 0, sig0);
      pv_regs(vt0, p0);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) vt_held[cb] = (v4i){0, 0, 0, 0};
      p_held = (v4i){0, 0, 0, 0};
      return;
    }
    u4v a0[NKB], a1[NKB];
    k_operand(bufc, 0, a0);
    k_operand(bufc, 1, a1);
    const v16f sig0 = qk_mfma(a0);
    __builtin_amdgcn_sched_barrier(0);
    const v16f sig1 = qk_mfma(a1);
    pv_regs(vt_held, p_held);
    v4i vt0[NCB];
    read_vt(bufc, 0, vt0);
    vsum_blk(tail, t, 0, vt0);
    __builtin_amdgcn_sched_barrier(0);
    const v4i p0 = probs2(tail, t, bufc, 0, sig0);
#pragma unroll
    for (int i = 0; i < NKB + NCB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);    // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    pv_regs(vt0, p0);
    p_held = probs2(tail, t, bufc, 1, sig1);
    read_vt(bufc, 1, vt_held);
#pragma unroll
    for (int i = 0; i < NCB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
    // block 1's probabilities (and the row sum) are consumed only in the
    // next tile: pin their computation here, beside block 0's P.V, rather
    // than let it sink past the end-of-tile wait
    asm volatile("" ::"v"(p_held), "v"(l0), "v"(l1), "v"(l2), "v"(l3));
    __builtin_amdgcn_sched_barrier(0);
    vsum_blk(tail, t, 1, vt_held);
  };

  // Lean tile: the two key blocks one after the other, nothing carried
  // across the barrier. Fewer live registers: it lets three workgroups share
  // a CU at three channel blocks and four at one or two (at three
  // workgroups and one or two blocks it measures the same as the
  // interleaved tile, which is kept there).
  auto pass2_tile_lean = [&](auto tail, int t, auto bufc) {
    constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (TAIL && kb == 1 && t * kBC + 32 >= N) break;  // no key < N in the block
      u4v a[NKB];
      k_operand(bufc, kb, a);
      const v16f sig = qk_mfma(a);
      const v4i pk = probs2(tail, t, bufc, kb, sig);
      v4i vt[NCB];
      read_vt(bufc, kb, vt);
      pv_regs(vt, pk);
      vsum_blk(tail, t, kb, vt);
    }
  };
  constexpr bool LEAN = (NCB == 3 && min_blocks<NCB, BIAS>() == 3) || min_blocks<NCB, BIAS>() == 4;
  if constexpr (RES) {
    // (the stages stay as pass 1 left them; V and the scales have landed)
    wait_vm0();
    __syncthreads();
    if constexpr (LEAN) {
      res_pass(true, pass2_tile_lean);
    } else {
      res_pass(true, pass2_tile);
      pv_regs(vt_held, p_held);
    }
  } else if constexpr (LEAN) {
    __syncthreads();  // pass 1 is done with both buffers
    dma_vscale();     // (landed by the first tile's wait)
    // (a wave with no live query runs the lean tile on clamped queries and
    // stores nothing: a check per tile or a second copy of the pass measured
    // slower on the four-workgroup kernels than the wasted work)
    run_pass(IntC<NS2>(), true, pass2_tile_lean, [] {});
  } else {
    __syncthreads();  // pass 1 is done with both buffers
    dma_vscale();
    run_pass(IntC<NS2>(), true, pass2_tile, [] {});
    pv_regs(vt_held, p_held);
  }

  // ================= epilogue =================
  // the channel sums: lanes l and l ^ 32 hold the two halves of each
  // block's keys; the four waves' sums meet in LDS (zeroed at the start)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int v = vsacc[cb] + (int)__float_as_uint(partner32(__uint_as_float((uint32_t)vsacc[cb]), lane));
    if (g == 0) atomicAdd(&vtot[32 * cb + ql], v);
  }
  __syncthreads();
  float lrun = (l0 + l1) + (l2 + l3);  // 255 l over both halves of the keys
  lrun += partner32(lrun, lane);
  if (!qvalid) return;
  const float inv_l = 1.0f / lrun;
  uint16_t* outp = static_cast<uint16_t*>(p.out) + b * p.out_sb + (int64_t)h * p.out_sh + (int64_t)qi * p.out_sn;
  const float* vs = vscl;
  const int32_t* vsm = vtot;
  if (p.out_mode & 2) {
    // whole groups of 4 channels: channel parameters at fixed offsets from
    // this lane's base, two elements per packed 16-bit conversion (rounding
    // to nearest even, as the scalar conversions); |vsum| <= 127 N < 2^23,
    // so 127 vsum is a 24-bit multiply. x = A * scale / (255 l).
    const float* vsl = vs + 4 * g;
    const int32_t* vsml = vsm + 4 * g;
    uint16_t* outl = outp + 4 * g;
    auto pack2 = [&](float x0, float x1) -> uint32_t {
      return (p.out_mode & 1) ? __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){x0, x1}, v2h))
                       : __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){x0, x1}, v2bf));
    };
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c0l = cb * 32 + 8 * r;  // channels c0l + 4g .. + 3
        if (c0l + 4 * g < d) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[e] = (float)(__mul24(vsml[c0l + e], 127) - acc[cb][4 * r + e]) * (vsl[c0l + e] * inv_l);
          *reinterpret_cast<uint2*>(outl + c0l) = make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
        }
      }
    }
    return;
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = cb * 32 + 8 * r + 4 * g;  // 4 consecutive channels c..c+3
      uint16_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ce = min(c + e, d - 1);
        const int a = 127 * vsm[ce] - acc[cb][4 * r + e];  // sum_j p8_j v8_j
        const float x = (float)a * (vs[ce] * inv_l);      // rounded as on the 8-byte path
        o[e] = (c + e < d) ? ((p.out_mode & 1) ? f32_to_f16(x) : f32_to_bf16(x)) : (uint16_t)0;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c + e < d) outp[c + e] = o[e];
    }
  }
}

template <int NKB, int NCB, int BIAS, int MODE = MODE_ATTN, bool RES = false>
hipError_t launch_t(const Params& p, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<NKB, NCB, BIAS, MODE, RES>), dim3(nblocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Whether the resident mode takes this launch: at most kResTiles tiles, and
// for a relative-position bias, the window of table rows that any query
// block needs against all keys fits the LDS table (as tbl_window computes
// it on the device).
bool res_takes(const Params& p, bool relpos) {
  if (p.N > kResTiles * kBC) return false;
  if (!relpos) return true;
  const int gw = p.grid_w, npre = p.n_prefix, N = p.N;
  if (N - 1 < npre) return true;  // no grid token: an empty window
  const int T2 = 2 * gw - 1;
  const int rk_hi = (N - 1 - npre) / gw;
  for (int qb = 0; qb < p.nqb; ++qb) {
    const int q0 = qb * kQB, q1 = std::min(q0 + kQB - 1, N - 1);
    if (q1 < npre) continue;
    const int wq_lo = (std::max(q0, npre) - npre) / gw, wq_hi = (q1 - npre) / gw;
    if ((int64_t)(wq_hi - wq_lo + rk_hi + 1) * T2 > kTblMax) return false;
  }
  return true;
}

// Workgroups of an instantiation that the chip holds at once: the CUs times
// the occupancy its register budget allows.
template <int NKB, int NCB, int BIAS, int MODE>
hipError_t launch_b(Params p, int nblocks, hipStream_t s) {
  p.slots = kCUs * min_blocks<NCB, BIAS, MODE>();
  p.balance = nblocks <= p.slots ? 1 : 2;
  if constexpr (res_fits<NKB, NCB, BIAS, MODE>()) {
    if (res_takes(p, is_relpos(BIAS))) return launch_t<NKB, NCB, BIAS, MODE, true>(p, nblocks, s);
  }
  if (p.k16) return hipErrorNotSupported;  // (16-bit K and V: the resident mode only)
  return launch_t<NKB, NCB, BIAS, MODE>(p, nblocks, s);
}

template <int NKB, int NCB, int MODE = MODE_ATTN>
hipError_t launch_bias(const Params& p, int bias, int nblocks, hipStream_t s) {
  switch (bias) {
    case BIAS_NONE: return launch_b<NKB, NCB, BIAS_NONE, MODE>(p, nblocks, s);
    case BIAS_DENSE_F32: return launch_b<NKB, NCB, BIAS_DENSE_F32, MODE>(p, nblocks, s);
    case BIAS_DENSE_F16: return launch_b<NKB, NCB, BIAS_DENSE_F16, MODE>(p, nblocks, s);
    case BIAS_DENSE_ANY: return launch_b<NKB, NCB, BIAS_DENSE_ANY, MODE>(p, nblocks, s);
    case BIAS_RELPOS_ROW: return launch_b<NKB, NCB, BIAS_RELPOS_ROW, MODE>(p, nblocks, s);
    default: return launch_b<NKB, NCB, BIAS_RELPOS, MODE>(p, nblocks, s);
  }
}

}  // namespace

// Sigma modes for one window (the pointers already offset to its first
// head, which the kernel sees as batch 0, heads 0 .. H - 1): the staged-tile
// route writes every element, then the pass-1 route (and, at three channel
// blocks, the raw-word route) compares and poisons what differs.
template <int NKB, int NCB>
hipError_t launch_sigma_routes(const Params& p, int nblocks, hipStream_t s) {
  hipError_t e = launch_t<NKB, NCB, BIAS_NONE, MODE_SIGMA>(p, nblocks, s);
  if (e == hipSuccess) e = launch_t<NKB, NCB, BIAS_NONE, MODE_SIGMA_SPLIT>(p, nblocks, s);
  if constexpr (NCB == 3) {
    if (e == hipSuccess) e = launch_t<NKB, NCB, BIAS_NONE, MODE_SIGMA_RAW>(p, nblocks, s);
  }
  return e;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  Params p = {};
  p.qbits = a.qbits; p.qmu = a.qmu; p.kbits = a.kbits; p.kmu = a.kmu;
  p.q16 = static_cast<const uint16_t*>(a.q16);
  p.q16_f16 = a.q16_dt == BA_F16;
  p.k16 = static_cast<const uint16_t*>(a.k16);
  p.v16 = static_cast<const uint16_t*>(a.v16);
  p.vq = a.vq; p.vscale = a.vscale;
  p.bias = a.bias; p.bias_bstride = a.bias_bstride;
  p.grid_h = a.grid_h; p.grid_w = a.grid_w; p.n_prefix = a.n_prefix;
  p.gw_magic = a.grid_w >= 2 ? (uint32_t)(((1ull << 32) + (uint64_t)a.grid_w - 1) / (uint64_t)a.grid_w) : 0u;
  p.B = a.B; p.H = a.H; p.N = a.N; p.d = a.d; p.W = (a.d + 31) / 32;
  p.nqb = (a.N + kQB - 1) / kQB;
  p.inv_sqrt_d = (float)(1.0 / sqrt((double)a.d));
  // V tiles by DMA: 16-byte pieces must be 16-byte aligned in global memory
  // (tile starts are (bh*N + 64t)*d bytes from a 16-byte aligned base)
  p.v_dma = (a.d % 16 == 0) || (a.d % 8 == 0 && a.N % 2 == 0);
  p.v_swz_shift = -1;
  if (p.v_dma && (a.d == 32 || a.d == 64 || a.d == 128)) p.v_swz_shift = a.d == 32 ? 2 : a.d == 64 ? 1 : 0;
  p.out = a.out;
  if (a.out_sh > 0x7FFFFFFF || a.out_sn > 0x7FFFFFFF) return hipErrorInvalidValue;
  p.out_sb = a.out_sb; p.out_sh = (int)a.out_sh; p.out_sn = (int)a.out_sn;
  const bool out_vec = a.d % 4 == 0 && a.out_sb % 4 == 0 && a.out_sh % 4 == 0 && a.out_sn % 4 == 0 &&
                       reinterpret_cast<uintptr_t>(a.out) % 8 == 0;
  p.out_mode = (a.out_dt == BA_F16 ? 1 : 0) | (out_vec ? 2 : 0);
  p.mk_vec = (a.N % 4) == 0 && reinterpret_cast<uintptr_t>(a.kmu) % 16 == 0;

  int bias = BIAS_NONE;
  p.bias_f16 = 0;
  p.bias_al4 = 0;
  if (a.bias_kind == BA_BIAS_DENSE) {
    const int per16 = a.bias_dtype == BA_F32 ? 4 : 8;  // elements per 16 bytes
    const bool vec = (a.N % per16 == 0) && (a.bias_bstride % per16 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.bias) % 16 == 0);
    p.bias_f16 = a.bias_dtype == BA_F16;
    const bool base4 = reinterpret_cast<uintptr_t>(a.bias) % 4 == 0;
    p.bias_al4 = (a.bias_dtype == BA_F32 || (a.N % 2 == 0 && a.bias_bstride % 2 == 0 && base4)) ? 1 : base4 ? 2 : 0;
    bias = !vec ? BIAS_DENSE_ANY : (a.bias_dtype == BA_F32 ? BIAS_DENSE_F32 : BIAS_DENSE_F16);
  } else if (a.bias_kind == BA_BIAS_RELPOS) {
    bias = (a.grid_w % 16 == 0 && a.n_prefix == 0) ? BIAS_RELPOS_ROW : BIAS_RELPOS;
  }
  const int64_t nblocks = (int64_t)p.nqb * a.B * a.H;
  if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int ncb = (a.d + 31) / 32;
  if (a.online) {
    switch (ncb) {
      case 1: return launch_bias<1, 1, MODE_ONLINE>(p, bias, (int)nblocks, s);
      case 2: return launch_bias<1, 2, MODE_ONLINE>(p, bias, (int)nblocks, s);
      default: return hipErrorInvalidValue;  // d > 64 (checked by the caller)
    }
  }
  switch (ncb) {
    case 1: return launch_bias<1, 1>(p, bias, (int)nblocks, s);
    case 2: return launch_bias<1, 2>(p, bias, (int)nblocks, s);
    case 3: return launch_bias<2, 3>(p, bias, (int)nblocks, s);
    default: return launch_bias<2, 4>(p, bias, (int)nblocks, s);
  }
}

hipError_t launch_hamming(const uint32_t* qbits, const uint32_t* kbits, int N, int d, int bh_begin, int bh_count,
                          int row_begin, int row_count, int32_t* sigma, hipStream_t s) {
  Params p = {};
  const int W = (d + 31) / 32;
  p.qbits = qbits + (int64_t)bh_begin * N * W;
  p.kbits = kbits + (int64_t)bh_begin * N * W;
  p.B = 1; p.H = bh_count; p.N = N; p.d = d; p.W = W;
  p.inv_sqrt_d = 1.0f;
  p.v_swz_shift = -1;
  p.sigma = sigma;
  p.row0 = row_begin; p.nrows = row_count;
  p.qb0 = row_begin / kQB;
  p.nqb = (row_begin + row_count - 1) / kQB - p.qb0 + 1;
  const int64_t nblocks = (int64_t)p.nqb * bh_count;
  if (nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch ((d + 31) / 32) {
    case 1: return launch_sigma_routes<1, 1>(p, (int)nblocks, s);
    case 2: return launch_sigma_routes<1, 2>(p, (int)nblocks, s);
    case 3: return launch_sigma_routes<2, 3>(p, (int)nblocks, s);
    default: return launch_sigma_routes<2, 4>(p, (int)nblocks, s);
  }
}

}  // namespace binattn
