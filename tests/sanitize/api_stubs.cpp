// Host-only stand-ins for the gfx950 launchers (bit_qk_attention_amd/csrc),
// linked with the C-ABI layer (api.hip) in the sanitizer build: each records
// that validation let a call through and launches nothing. Test
// infrastructure only.
#include "common.h"

extern "C" {
int ba_stub_calls = 0;  // launches the stubs have seen
}

namespace binattn {

InView dense_view(int H, int N, int d) {
  InView v;
  v.sn = d;
  v.sh = (int64_t)N * d;
  v.sb = (int64_t)H * v.sh;
  v.H = H;
  v.vec = d % 8 == 0;
  return v;
}
hipError_t launch_pack_qk(const void*, const void*, ba_dtype, const InView&, int, int, int, uint32_t*, float*,
                          uint32_t*, float*, hipStream_t, uint32_t*, int64_t) {
  ++ba_stub_calls;
  return hipSuccess;
}
hipError_t launch_quant_v(const void*, ba_dtype, const InView&, int, int, int, int8_t*, float*, hipStream_t) {
  ++ba_stub_calls;
  return hipSuccess;
}
hipError_t launch_prepass(const void*, const void*, const void*, ba_dtype, const InView&, int, int, int, uint32_t*,
                          float*, uint32_t*, float*, int8_t*, float*, hipStream_t) {
  ++ba_stub_calls;
  return hipSuccess;
}
hipError_t launch_hamming(const uint32_t*, const uint32_t*, int, int, int, int, int, int, int32_t*, hipStream_t) {
  ++ba_stub_calls;
  return hipSuccess;
}
hipError_t launch_attention(const AttnArgs& a, hipStream_t) {
  ++ba_stub_calls;
  // 16-bit K and V outside the resident mode (the real launcher refuses
  // them before any launch)
  if (a.k16 && a.N > 256) return hipErrorNotSupported;
  // the descriptor validation hands over is consistent with the call
  const bool q_ok = a.q16 ? (a.qbits == nullptr && a.qmu == nullptr) : (a.qbits && a.qmu);
  const bool kv_ok = a.k16 ? (a.v16 && !a.kbits && !a.kmu && !a.vq && !a.vscale) : (a.kbits && a.kmu && a.vq && a.vscale);
  return (a.B > 0 && a.H > 0 && a.N > 0 && a.d > 0 && a.out && q_ok && kv_ok) ? hipSuccess : hipErrorInvalidValue;
}

}  // namespace binattn
