// probe.hip — microbenchmarks behind the design choices of attention.hip
// (not part of the attention path; built into libbaprobe.so and run by
// `python -m bit_qk_attention_amd.profiling probe`).
//
// Two families, each a kernel of 2048 workgroups x 256 threads (8 waves per
// SIMD on 256 CUs) that loops over register-resident data, timed with HIP
// events over five launches:
//  * issue rates of the vector instructions the softmax of the attention
//    uses (fp32 fma, v_exp_f32, v_cvt_pk_u8_f32, and the per-score mix of
//    pass 2), eight independent chains per lane;
//  * the integer similarity sigma = d - 2 popcount(q xor k) of a 32-key x
//    32-query block at d = 64 (zh technical summary section 2.1) by three
//    routes, each ending with sigma as fp32 in a register and one max per
//    score to consume it: XOR + popcount on the vector ALU (v_bcnt), +-1
//    int8 operands on v_mfma_i32_32x32x32_i8 (two k-steps, then a convert),
//    and +-1 fp4 operands on v_mfma_scale_f32_32x32x64_f8f6f4 (one k-step,
//    fp32 result). The operands change every iteration (one XOR per lane
//    and operand register) so no result is loop-invariant.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBlocks = 2048, kThreads = 256, kChains = 8;

enum {
  P_FMA = 0,        // y = fma(y, a, b)
  P_EXP = 1,        // x = exp2(x)
  P_CVT = 2,        // u = cvt_pk_u8(y + i)   (an add and a convert)
  P_MIX = 3,        // pass-2 mix per score: mul, fma, exp, add, cvt, xor
  P_QK_POPC = 4,    // sigma of 16 keys per lane by xor + popcount
  P_QK_I8 = 5,      // sigma of a 32x32 block by two int8 MFMAs
  P_QK_FP4 = 6,     // sigma of a 32x32 block by one fp4 MFMA
  P_COUNT = 7
};

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int MODE>
__global__ __launch_bounds__(kThreads) void probe_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                          int iters) {
  const int t = blockIdx.x * kThreads + threadIdx.x;  // < kBlocks * kThreads
  const int lane = threadIdx.x & 63;
  const float a = in[0], b = in[1];
  float r = 0.0f;
  if constexpr (MODE <= P_MIX) {
    float x[kChains], y[kChains];
    uint32_t u[kChains];
    for (int c = 0; c < kChains; ++c) {
      x[c] = in[t] * (c + 1) * 1e-3f;
      y[c] = in[t] + c;
      u[c] = (uint32_t)t + c;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        if constexpr (MODE == P_FMA) y[c] = __builtin_fmaf(y[c], a, b);
        if constexpr (MODE == P_EXP) x[c] = __builtin_amdgcn_exp2f(x[c]);
        if constexpr (MODE == P_CVT) u[c] = __builtin_amdgcn_cvt_pk_u8_f32(y[c] + (float)i, c & 3, u[c]);
        if constexpr (MODE == P_MIX) {
          const float s = y[c] * a;
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s, b, a));
          x[c] += e;
          u[c] = __builtin_amdgcn_cvt_pk_u8_f32(e, c & 3, u[c]);
          y[c] = __uint_as_float(__float_as_uint(y[c]) ^ u[c]);
        }
      }
    }
    for (int c = 0; c < kChains; ++c) r += x[c] + y[c] + (float)u[c];
  } else if constexpr (MODE == P_QK_POPC) {
    // lane: one query (two words), 16 keys (two words each)
    uint32_t q0 = (uint32_t)t * 2654435761u, q1 = q0 ^ 0x9E3779B9u;
    uint32_t k0[16], k1[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      k0[j] = (uint32_t)(lane * 16 + j) * 0x85EBCA6Bu;
      k1[j] = k0[j] ^ 0xC2B2AE35u;
    }
    float m = -1e30f;
    for (int i = 0; i < iters; ++i) {
      q0 ^= (uint32_t)i;
      q1 ^= (uint32_t)i << 1;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int pc = __builtin_popcount(q0 ^ k0[j]) + __builtin_popcount(q1 ^ k1[j]);
        m = fmaxf(m, (float)(64 - 2 * pc));
      }
    }
    r = m;
  } else if constexpr (MODE == P_QK_I8) {
    // A: 32 keys x 64 channels of +-1 bytes (two k-steps of 32), B: queries
    v4i ka[2], qb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // bytes 0x01 (+1) or 0xFF (-1), no carry between bytes
        ka[s][w] = (int)(((((uint32_t)(t * 8 + s * 4 + w) * 0x01000193u) & 0x01010101u) * 0xFEu) | 0x01010101u);
        qb[s][w] = (int)(((((uint32_t)(t * 8 + s * 4 + w) * 0x9E3779B1u) & 0x01010101u) * 0xFEu) | 0x01010101u);
      }
    float m = -1e30f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int w = 0; w < 4; ++w) qb[s][w] ^= (i & 1) ? 0xFEFEFEFE : 0;  // +-1 bytes stay +-1 (x ^ 0xFE = -x)
      v16i acc = {};
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[0], qb[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[1], qb[1], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, (float)acc[e]);
    }
    r = m;
  } else {
    // fp4 e2m1 signs: +1 = 0x2, -1 = 0xA; 64 channels in one k-step
    v8i ka = {}, qb = {};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      ka[w] = (int)((((uint32_t)(t * 4 + w) * 0x01000193u) & 0x88888888u) | 0x22222222u);
      qb[w] = (int)((((uint32_t)(t * 4 + w) * 0x9E3779B1u) & 0x88888888u) | 0x22222222u);
    }
    float m = -1e30f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int w = 0; w < 4; ++w) qb[w] ^= (i & 1) ? (int)0x88888888u : 0;  // flip every sign
      v16f acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qb, acc, 4, 4, 0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, acc[e]);
    }
    r = m;
  }
  out[t] = r;
}

template <int MODE>
hipError_t launch(const float* in, float* out, int iters, hipStream_t s) {
  hipLaunchKernelGGL(probe_kernel<MODE>, dim3(kBlocks), dim3(kThreads), 0, s, in, out, iters);
  return hipGetLastError();
}

hipError_t launch_mode(int mode, const float* in, float* out, int iters, hipStream_t s) {
  switch (mode) {
    case P_FMA: return launch<P_FMA>(in, out, iters, s);
    case P_EXP: return launch<P_EXP>(in, out, iters, s);
    case P_CVT: return launch<P_CVT>(in, out, iters, s);
    case P_MIX: return launch<P_MIX>(in, out, iters, s);
    case P_QK_POPC: return launch<P_QK_POPC>(in, out, iters, s);
    case P_QK_I8: return launch<P_QK_I8>(in, out, iters, s);
    default: return launch<P_QK_FP4>(in, out, iters, s);
  }
}

}  // namespace

extern "C" {

// Number of probe modes (see the enum above).
int bap_count(void) { return P_COUNT; }

// Time `mode` for `iters` loop iterations: mean milliseconds per launch over
// five launches after one warm-up launch, on the null stream. Allocates and
// frees its own device buffers. Returns 0, or the HIP error code.
int bap_time(int mode, int iters, float* ms) {
  if (mode < 0 || mode >= P_COUNT || iters < 1 || !ms) return (int)hipErrorInvalidValue;
  float *in = nullptr, *out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const size_t n = (size_t)kBlocks * kThreads;
  hipError_t e = hipMalloc(&in, n * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&out, n * sizeof(float));
  if (e == hipSuccess) e = hipMemset(in, 0, n * sizeof(float));
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = launch_mode(mode, in, out, iters, 0);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipEventRecord(e0, 0);
  for (int r = 0; r < 5 && e == hipSuccess; ++r) e = launch_mode(mode, in, out, iters, 0);
  if (e == hipSuccess) e = hipEventRecord(e1, 0);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float t = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
  *ms = t / 5.0f;
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  if (in) hipFree(in);
  if (out) hipFree(out);
  return (int)e;
}

}  // extern "C"
