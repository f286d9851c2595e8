/* Calls every entry point of include/binattn.h, as a C program would, with
 * accepted and rejected arguments (fake, never dereferenced device
 * addresses; enum arguments outside their enums), linked against the C-ABI
 * layer and host-only launcher stubs, so that a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer checks the validation code. Each accepted
 * call must reach its launcher, each rejected one must return its status
 * before any launch. Exits 0 when all of that holds. Test infrastructure
 * only. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "binattn.h"

extern int ba_stub_calls; /* launches the stubs have seen */

static int fails = 0;
static void expect(const char* what, int got, int want, int launched) {
  static int last = 0;
  const int calls = ba_stub_calls - last;
  last = ba_stub_calls;
  const int ok = got == want && (want == BA_OK ? calls >= 1 : calls == 0) && (!launched || calls >= 1);
  if (!ok) {
    printf("FAIL %s: status %d (want %d), launches %d\n", what, (int)got, (int)want, calls);
    ++fails;
  }
}

static void* A(int i) { return (void*)((uintptr_t)0x7F0000000000ull + (uintptr_t)i * (1ull << 32)); }
#define P(T, i) ((T*)A(i))

static ba_status attn(const ba_bias* b, int N, void* out, ba_dtype odt) {
  return ba_attention_fwd(P(uint32_t, 1), P(float, 2), P(uint32_t, 3), P(float, 4), P(int8_t, 5), P(float, 6), b, 8,
                          16, N, 72, out, odt, NULL);
}

int main(void) {
  const ba_dtype bf = BA_BF16;
  /* pack */
  expect("pack ok", ba_pack_qk(A(0), A(1), bf, 2, 3, 100, 72, P(uint32_t, 2), P(float, 3), P(uint32_t, 4),
                               P(float, 5), NULL), BA_OK, 1);
  expect("pack d=129", ba_pack_qk(A(0), A(1), bf, 2, 3, 100, 129, P(uint32_t, 2), P(float, 3), P(uint32_t, 4),
                                  P(float, 5), NULL), BA_ERR_UNSUPPORTED, 0);
  expect("pack overlap", ba_pack_qk(A(0), A(1), bf, 2, 3, 100, 72, P(uint32_t, 2), P(float, 3), P(uint32_t, 2),
                                    P(float, 5), NULL), BA_ERR_INVALID_ARG, 0);
  expect("pack N max+1", ba_pack_qk(A(0), A(1), bf, 1, 1, BA_MAX_TOKENS + 1, 64, P(uint32_t, 2), P(float, 3),
                                    P(uint32_t, 4), P(float, 5), NULL), BA_ERR_UNSUPPORTED, 0);
  expect("pack huge B*H", ba_pack_qk(A(0), A(1), bf, 1 << 20, 1 << 11, 10, 64, P(uint32_t, 2), P(float, 3),
                                     P(uint32_t, 4), P(float, 5), NULL), BA_ERR_UNSUPPORTED, 0);
  /* quant */
  expect("quant ok", ba_quant_v(A(0), BA_F16, 4, 16, 4096, 64, P(int8_t, 1), P(float, 2), NULL), BA_OK, 1);
  expect("quant alias", ba_quant_v(A(0), BA_F16, 4, 16, 4096, 64, P(int8_t, 0), P(float, 2), NULL),
         BA_ERR_INVALID_ARG, 0);
  expect("quant f32", ba_quant_v(A(0), BA_F32, 4, 16, 4096, 64, P(int8_t, 1), P(float, 2), NULL),
         BA_ERR_UNSUPPORTED, 0);
  /* a value outside the enum, as a C caller may pass it */
  const ba_dtype bad_dt = (ba_dtype)7;
  expect("quant dtype 7", ba_quant_v(A(0), bad_dt, 4, 16, 4096, 64, P(int8_t, 1), P(float, 2), NULL),
         BA_ERR_UNSUPPORTED, 0);
  expect("pack dtype 7", ba_pack_qk(A(0), A(1), bad_dt, 2, 3, 100, 72, P(uint32_t, 2), P(float, 3), P(uint32_t, 4),
                                    P(float, 5), NULL), BA_ERR_UNSUPPORTED, 0);
  /* one-call pre-pass, dense and strided */
  expect("prep ok", ba_pack_qk_quant_v(A(0), A(1), A(2), bf, 8, 16, 1024, 72, P(uint32_t, 3), P(float, 4),
                                       P(uint32_t, 5), P(float, 6), P(int8_t, 7), P(float, 8), NULL), BA_OK, 1);
  expect("prep overlap", ba_pack_qk_quant_v(A(0), A(1), A(2), bf, 8, 16, 1024, 72, P(uint32_t, 3), P(float, 4),
                                            P(uint32_t, 5), P(float, 6), P(int8_t, 7), P(float, 7), NULL),
         BA_ERR_INVALID_ARG, 0);
  const ba_strides qkv = {3 * 4096 * 16 * 64, 64, 3 * 16 * 64};
  expect("prep strided ok", ba_pack_qk_quant_v_strided(A(0), (void*)(P(uint16_t, 0) + 16 * 64), (void*)(P(uint16_t, 0) + 32 * 64),
                                                       &qkv, bf, 2, 16, 4096, 64, P(uint32_t, 3), P(float, 4),
                                                       P(uint32_t, 5), P(float, 6), P(int8_t, 7), P(float, 8), NULL),
         BA_OK, 1);
  ba_strides neg = {-1, 0, 64};
  expect("prep strided negative", ba_pack_qk_quant_v_strided(A(0), A(1), A(2), &neg, bf, 2, 16, 4096, 64,
                                                             P(uint32_t, 3), P(float, 4), P(uint32_t, 5), P(float, 6),
                                                             P(int8_t, 7), P(float, 8), NULL),
         BA_ERR_INVALID_ARG, 0);
  ba_strides big = {(int64_t)1 << 45, 0, 64};
  expect("prep strided span", ba_pack_qk_quant_v_strided(A(0), A(1), A(2), &big, bf, 2, 16, 4096, 64,
                                                         P(uint32_t, 3), P(float, 4), P(uint32_t, 5), P(float, 6),
                                                         P(int8_t, 7), P(float, 8), NULL),
         BA_ERR_INVALID_ARG, 0);
  /* attention: each bias kind, accepted and rejected */
  ba_bias none = {BA_BIAS_NONE, NULL, BA_F32, 0, 0, 0, 0};
  ba_bias dense16 = {BA_BIAS_DENSE, A(7), BA_F16, 0, 0, 0, 0};
  ba_bias dense_pb = {BA_BIAS_DENSE, A(7), BA_F32, 16 * 1024 * 1024, 0, 0, 0};
  ba_bias dense_bad = {BA_BIAS_DENSE, A(7), BA_F32, 100, 0, 0, 0};
  ba_bias rp = {BA_BIAS_RELPOS, A(7), BA_F32, 0, 32, 32, 0};
  ba_bias rp_bad = {BA_BIAS_RELPOS, A(7), BA_F32, 0, 31, 32, 0};
  ba_bias rp_wide = {BA_BIAS_RELPOS, A(7), BA_F32, 0, 4, 257, 0};
  ba_bias kind_bad = {(ba_bias_kind)9, A(7), BA_F32, 0, 0, 0, 0};
  ba_bias rp_small = {BA_BIAS_RELPOS, A(7), BA_F32, 0, 14, 14, 1};
  expect("attn no bias", attn(NULL, 1024, A(9), bf), BA_OK, 1);
  expect("attn kind none", attn(&none, 1024, A(9), bf), BA_OK, 1);
  expect("attn dense f16", attn(&dense16, 1024, A(9), bf), BA_OK, 1);
  expect("attn dense per batch", attn(&dense_pb, 1024, A(9), bf), BA_OK, 1);
  expect("attn dense stride", attn(&dense_bad, 1024, A(9), bf), BA_ERR_INVALID_ARG, 0);
  expect("attn relpos", attn(&rp, 1024, A(9), bf), BA_OK, 1);
  expect("attn relpos grid", attn(&rp_bad, 1024, A(9), bf), BA_ERR_INVALID_ARG, 0);
  expect("attn relpos wide", attn(&rp_wide, 1028, A(9), bf), BA_ERR_UNSUPPORTED, 0);
  expect("attn bias kind", attn(&kind_bad, 1024, A(9), bf), BA_ERR_INVALID_ARG, 0);
  expect("attn out f32", attn(NULL, 1024, A(9), BA_F32), BA_ERR_UNSUPPORTED, 0);
  expect("attn out dtype 7", attn(NULL, 1024, A(9), bad_dt), BA_ERR_UNSUPPORTED, 0);
  expect("attn out aliases vq", attn(NULL, 1024, A(5), bf), BA_ERR_INVALID_ARG, 0);
  expect("attn out misaligned", attn(NULL, 1024, (void*)(P(char, 9) + 2), bf), BA_ERR_INVALID_ARG, 0);
  ba_strides ost = {1024 * 16 * 72, 72, 16 * 72};
  expect("attn strided ok", ba_attention_fwd_strided(P(uint32_t, 1), P(float, 2), P(uint32_t, 3), P(float, 4),
                                                      P(int8_t, 5), P(float, 6), &rp, 8, 16, 1024, 72, A(9), &ost, bf,
                                                      NULL), BA_OK, 1);
  ba_strides alias = {0, 72, 16 * 72};
  expect("attn strided alias", ba_attention_fwd_strided(P(uint32_t, 1), P(float, 2), P(uint32_t, 3), P(float, 4),
                                                        P(int8_t, 5), P(float, 6), NULL, 8, 16, 1024, 72, A(9),
                                                        &alias, bf, NULL), BA_ERR_INVALID_ARG, 0);
  /* the fused forms */
  expect("pack k/v ok", ba_pack_k_quant_v(A(1), A(2), bf, 8, 16, 1024, 72, P(uint32_t, 5), P(float, 6), P(int8_t, 7),
                                          P(float, 8), NULL), BA_OK, 1);
  expect("pack k/v overlap", ba_pack_k_quant_v(A(1), A(2), bf, 8, 16, 1024, 72, P(uint32_t, 5), P(float, 6),
                                               P(int8_t, 5), P(float, 8), NULL), BA_ERR_INVALID_ARG, 0);
  expect("attn q16 ok", ba_attention_fwd_q16(A(0), bf, P(uint32_t, 3), P(float, 4), P(int8_t, 5), P(float, 6),
                                             &dense16, 8, 16, 1024, 72, A(9), bf, NULL), BA_OK, 1);
  expect("attn q16 d=20", ba_attention_fwd_q16(A(0), bf, P(uint32_t, 3), P(float, 4), P(int8_t, 5), P(float, 6),
                                               NULL, 8, 16, 1024, 20, A(9), bf, NULL), BA_ERR_UNSUPPORTED, 0);
  expect("attn q16 out aliases q", ba_attention_fwd_q16(A(0), bf, P(uint32_t, 3), P(float, 4), P(int8_t, 5),
                                                        P(float, 6), NULL, 8, 16, 1024, 72, A(0), bf, NULL),
         BA_ERR_INVALID_ARG, 0);
  expect("attn qkv16 ok", ba_attention_fwd_qkv16(A(0), A(1), A(2), bf, &rp_small, 64, 6, 197, 64, A(9), BA_F16, NULL),
         BA_OK, 1);
  /* (refused by the launcher, before any launch: the stub is consulted once) */
  {
    const int before = ba_stub_calls;
    const ba_status st = ba_attention_fwd_qkv16(A(0), A(1), A(2), bf, NULL, 8, 16, 1024, 72, A(9), bf, NULL);
    if (st != BA_ERR_UNSUPPORTED || ba_stub_calls - before != 1) {
      printf("FAIL attn qkv16 long: status %d\n", (int)st);
      ++fails;
    }
    expect("(resync)", BA_OK, BA_OK, 1);
  }
  expect("attn qkv16 out aliases v", ba_attention_fwd_qkv16(A(0), A(1), A(2), bf, NULL, 8, 16, 256, 72, A(2), bf,
                                                            NULL), BA_ERR_INVALID_ARG, 0);
  expect("attn qkv16 no v", ba_attention_fwd_qkv16(A(0), A(1), NULL, bf, NULL, 8, 16, 256, 72, A(9), bf, NULL),
         BA_ERR_INVALID_ARG, 0);
  /* the similarity window */
  expect("hamming ok", ba_debug_hamming_scores(P(uint32_t, 0), P(uint32_t, 1), 2, 16, 4096, 64, 3, 5, 100, 200,
                                               P(int32_t, 2), NULL), BA_OK, 1);
  expect("hamming window", ba_debug_hamming_scores(P(uint32_t, 0), P(uint32_t, 1), 2, 16, 4096, 64, 30, 5, 100, 200,
                                                   P(int32_t, 2), NULL), BA_ERR_INVALID_ARG, 0);
  expect("hamming alias", ba_debug_hamming_scores(P(uint32_t, 0), P(uint32_t, 1), 2, 16, 4096, 64, 0, 5, 0, 200,
                                                  P(int32_t, 1), NULL), BA_ERR_INVALID_ARG, 0);
  if (ba_packed_words(72) != 3 || ba_packed_words(0) != 0) { puts("FAIL ba_packed_words"); ++fails; }
  for (int s = 0; s < 5; ++s)
    if (!ba_status_string((ba_status)s)) { puts("FAIL ba_status_string"); ++fails; }
  printf("api driver: %d failure(s)\n", fails);
  return fails != 0;
}
