"""The C ABI library loads, exports every symbol include/binattn.h declares,
and rejects bad arguments before any HIP call (so these run without a GPU:
every call here is one that validation refuses)."""
import ctypes

import pytest

import bit_qk_attention_amd as ba
from bit_qk_attention_amd import ba_bias, ba_strides

OK, INV, UNS = ba.BA_OK, ba.BA_ERR_INVALID_ARG, ba.BA_ERR_UNSUPPORTED
P = 0x7F0000000000  # fake, 256-byte aligned device addresses (never dereferenced)


def A(i):
    return ctypes.c_void_p(P + i * (1 << 32))


@pytest.fixture(scope="module")
def L():
    return ba.lib()


def test_exports_every_declared_symbol(L):
    names = ba.header_symbols()
    assert set(names) == {"ba_packed_words", "ba_pack_qk", "ba_quant_v", "ba_pack_qk_quant_v",
                          "ba_pack_qk_quant_v_strided", "ba_attention_fwd", "ba_attention_fwd_strided",
                          "ba_attention_fwd_online", "ba_pack_k_quant_v", "ba_attention_fwd_q16",
                          "ba_attention_fwd_qkv16",
                          "ba_debug_hamming_scores", "ba_status_string"}
    for n in names:
        assert hasattr(L, n), n


# The four calls of the hot path, in the form their contract states
# (argument types and order); extension calls may add to, but not alter them.
CONTRACT = {
    "ba_pack_qk": "const void* q, const void* k, ba_dtype dt, int B, int H, int N, int d, uint32_t* qbits, "
                  "float* qmu, uint32_t* kbits, float* kmu, void* stream",
    "ba_quant_v": "const void* v, ba_dtype dt, int B, int H, int N, int d, int8_t* vq, float* vscale, void* stream",
    "ba_attention_fwd": "const uint32_t* qbits, const float* qmu, const uint32_t* kbits, const float* kmu, "
                        "const int8_t* vq, const float* vscale, const ba_bias* bias, int B, int H, int N, int d, "
                        "void* out, ba_dtype out_dt, void* stream",
    "ba_debug_hamming_scores": "const uint32_t* qbits, const uint32_t* kbits, int B, int H, int N, int d, "
                               "int bh_begin, int bh_count, int row_begin, int row_count, int32_t* sigma, "
                               "void* stream",
}


def _prototypes():
    import re
    text = re.sub(r"/\*.*?\*/", "", open(ba.HEADER_PATH).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"ba_status\s+(ba_[a-z0-9_]+)\s*\(([^;]*?)\)\s*;", text):
        out[m.group(1)] = " ".join(m.group(2).split())
    return out


def test_contract_prototypes():
    protos = _prototypes()
    for name, args in CONTRACT.items():
        assert protos.get(name) == args, (name, protos.get(name))
    # every argument of every declared call is a plain C type (no torch or C++ types)
    for name, args in protos.items():
        for a in args.split(","):
            assert a.strip().split()[0] in {"const", "void*", "int", "ba_dtype", "uint32_t*", "float*",
                                            "int8_t*", "int32_t*"}, (name, a)


def test_small_helpers(L):
    assert [L.ba_packed_words(d) for d in (0, 1, 32, 33, 64, 72, 128)] == [0, 1, 1, 2, 2, 3, 4]
    for s in range(4):
        assert isinstance(ba.status_string(s), str)
    assert ba.status_string(99) == "unknown status"


def pack(L, q=A(0), k=A(1), dt=ba.BA_BF16, B=1, H=1, N=8, d=64, qb=A(2), qm=A(3), kb=A(4), km=A(5)):
    return L.ba_pack_qk(q, k, dt, B, H, N, d, qb, qm, kb, km, None)


def test_pack_rejections(L):
    assert pack(L, q=None) == INV
    assert pack(L, km=None) == INV
    assert pack(L, N=0) == INV and pack(L, B=-1) == INV and pack(L, d=0) == INV
    assert pack(L, d=129) == UNS
    assert pack(L, N=ba.BA_MAX_TOKENS + 1) == UNS
    assert pack(L, dt=ba.BA_F32) == UNS and pack(L, dt=7) == UNS
    assert pack(L, q=ctypes.c_void_p(P + 2)) == INV       # not 16-byte aligned
    assert pack(L, qm=ctypes.c_void_p(P + 3 * (1 << 32) + 2)) == INV
    assert pack(L, kb=A(2)) == INV                        # outputs overlap


def quant(L, v=A(0), dt=ba.BA_F16, B=1, H=1, N=8, d=64, vq=A(1), vs=A(2)):
    return L.ba_quant_v(v, dt, B, H, N, d, vq, vs, None)


def test_quant_rejections(L):
    assert quant(L, v=None) == INV and quant(L, vs=None) == INV and quant(L, vq=None) == INV
    assert quant(L, vs=ctypes.c_void_p(P + 2 * (1 << 32) + 2)) == INV  # not 4-byte aligned
    assert quant(L, vs=A(1)) == INV  # outputs overlap
    assert quant(L, H=0) == INV and quant(L, d=200) == UNS and quant(L, dt=ba.BA_F32) == UNS
    assert quant(L, vq=ctypes.c_void_p(P + 1 * (1 << 32) + 8)) == INV
    assert quant(L, vq=A(0)) == INV  # output aliases the input


def prep(L, q=A(0), k=A(1), v=A(2), dt=ba.BA_BF16, B=1, H=1, N=8, d=64, **kw):
    o = dict(qb=A(3), qm=A(4), kb=A(5), km=A(6), vq=A(7), vs=A(8))
    o.update(kw)
    return L.ba_pack_qk_quant_v(q, k, v, dt, B, H, N, d, o["qb"], o["qm"], o["kb"], o["km"], o["vq"], o["vs"],
                                None)


def test_pack_qk_quant_v_rejections(L):
    assert prep(L, v=None) == INV and prep(L, km=None) == INV and prep(L, vs=None) == INV
    assert prep(L, N=0) == INV and prep(L, d=129) == UNS and prep(L, dt=ba.BA_F32) == UNS
    assert prep(L, N=ba.BA_MAX_TOKENS + 1) == UNS
    assert prep(L, v=ctypes.c_void_p(P + 2 * (1 << 32) + 8)) == INV   # not 16-byte aligned
    assert prep(L, vs=ctypes.c_void_p(P + 8 * (1 << 32) + 2)) == INV  # not 4-byte aligned
    assert prep(L, vq=A(3)) == INV    # outputs overlap (vq on qbits)
    assert prep(L, vs=A(2)) == INV    # output aliases the V input
    assert prep(L, qb=A(1)) == INV    # output aliases the K input


def attn(L, bias=None, B=2, H=2, N=16, d=64, out=A(9), out_dt=ba.BA_BF16, fn="ba_attention_fwd", **kw):
    args = dict(qb=A(1), qm=A(2), kb=A(3), km=A(4), vq=A(5), vs=A(6))
    args.update(kw)
    pb = ctypes.byref(bias) if bias is not None else None
    return getattr(L, fn)(args["qb"], args["qm"], args["kb"], args["km"], args["vq"], args["vs"],
                          pb, B, H, N, d, out, out_dt, None)


def test_attention_rejections(L):
    assert attn(L, qb=None) == INV and attn(L, out=None) == INV and attn(L, vs=None) == INV
    assert attn(L, out=A(6)) == INV  # output aliases vscale
    assert attn(L, d=0) == INV and attn(L, d=129) == UNS
    assert attn(L, N=ba.BA_MAX_TOKENS + 1) == UNS
    assert attn(L, out_dt=ba.BA_F32) == UNS and attn(L, out_dt=5) == UNS
    assert attn(L, vs=ctypes.c_void_p(P + 6 * (1 << 32) + 1)) == INV
    assert attn(L, out=A(5)) == INV  # output aliases vq
    # dense bias
    assert attn(L, bias=ba_bias(ba.BA_BIAS_DENSE, None, ba.BA_F32, 0, 0, 0, 0)) == INV
    assert attn(L, bias=ba_bias(ba.BA_BIAS_DENSE, P + 7 * (1 << 32), ba.BA_BF16, 0, 0, 0, 0)) == UNS
    assert attn(L, bias=ba_bias(ba.BA_BIAS_DENSE, P + 7 * (1 << 32), ba.BA_F32, 100, 0, 0, 0)) == INV
    assert attn(L, bias=ba_bias(ba.BA_BIAS_DENSE, P + 9 * (1 << 32) - 64, ba.BA_F32, 0, 0, 0, 0)) == INV
    # relative-position bias
    assert attn(L, bias=ba_bias(ba.BA_BIAS_RELPOS, P + 7 * (1 << 32), ba.BA_F16, 0, 4, 4, 0)) == UNS
    assert attn(L, bias=ba_bias(ba.BA_BIAS_RELPOS, P + 7 * (1 << 32), ba.BA_F32, 0, 3, 5, 0)) == INV
    assert attn(L, bias=ba_bias(ba.BA_BIAS_RELPOS, P + 7 * (1 << 32), ba.BA_F32, 0, 0, 16, 0)) == INV
    assert attn(L, bias=ba_bias(ba.BA_BIAS_RELPOS, P + 7 * (1 << 32), ba.BA_F32, 0, 3, 5, -1)) == INV
    assert attn(L, bias=ba_bias(7, P + 7 * (1 << 32), ba.BA_F32, 0, 0, 0, 0)) == INV
    assert attn(L, N=257 * 4, bias=ba_bias(ba.BA_BIAS_RELPOS, P + 7 * (1 << 32), ba.BA_F32, 0, 4, 257, 0)) == UNS


def test_online_rejections(L):
    """The one-pass form validates as ba_attention_fwd and takes d <= 64 only."""
    f = "ba_attention_fwd_online"
    assert attn(L, qb=None, fn=f) == INV and attn(L, out=A(6), fn=f) == INV
    assert attn(L, d=0, fn=f) == INV and attn(L, d=65, fn=f) == UNS and attn(L, d=129, fn=f) == UNS
    assert attn(L, out_dt=ba.BA_F32, fn=f) == UNS
    assert attn(L, bias=ba_bias(ba.BA_BIAS_RELPOS, P + 7 * (1 << 32), ba.BA_F32, 0, 3, 5, 0), fn=f) == INV


def test_pack_k_quant_v_rejections(L):
    def pkv(k=A(1), v=A(2), dt=ba.BA_BF16, B=1, H=1, N=8, d=64, kb=A(5), km=A(6), vq=A(7), vs=A(8)):
        return L.ba_pack_k_quant_v(k, v, dt, B, H, N, d, kb, km, vq, vs, None)
    assert pkv(k=None) == INV and pkv(v=None) == INV and pkv(km=None) == INV and pkv(vs=None) == INV
    assert pkv(N=0) == INV and pkv(d=129) == UNS and pkv(dt=ba.BA_F32) == UNS
    assert pkv(N=ba.BA_MAX_TOKENS + 1) == UNS
    assert pkv(k=ctypes.c_void_p(P + 1 * (1 << 32) + 8)) == INV   # not 16-byte aligned
    assert pkv(vq=A(5)) == INV    # outputs overlap
    assert pkv(kb=A(1)) == INV    # output aliases the K input


def test_attention_q16_rejections(L):
    def aq(q=A(0), q_dt=ba.BA_BF16, bias=None, B=2, H=2, N=16, d=64, out=A(9), out_dt=ba.BA_BF16, **kw):
        args = dict(kb=A(3), km=A(4), vq=A(5), vs=A(6))
        args.update(kw)
        pb = ctypes.byref(bias) if bias is not None else None
        return L.ba_attention_fwd_q16(q, q_dt, args["kb"], args["km"], args["vq"], args["vs"], pb, B, H, N, d,
                                      out, out_dt, None)
    assert aq(q=None) == INV and aq(kb=None) == INV and aq(out=None) == INV
    assert aq(d=20) == UNS and aq(d=129) == UNS and aq(d=0) == INV    # d % 8 == 0 only
    assert aq(q_dt=ba.BA_F32) == UNS and aq(out_dt=ba.BA_F32) == UNS
    assert aq(q=ctypes.c_void_p(P + 8)) == INV                        # not 16-byte aligned
    assert aq(out=A(0)) == INV                                        # output aliases Q
    assert aq(out=A(5)) == INV                                        # output aliases vq
    assert aq(bias=ba_bias(ba.BA_BIAS_RELPOS, P + 7 * (1 << 32), ba.BA_F32, 0, 3, 5, 0)) == INV


def test_attention_qkv16_rejections(L):
    """Refused before any launch (also the shapes the one-launch form does
    not take: those are decided on the host)."""
    def aqkv(q=A(0), k=A(1), v=A(2), dt=ba.BA_BF16, bias=None, B=2, H=2, N=64, d=64, out=A(9), out_dt=ba.BA_BF16):
        pb = ctypes.byref(bias) if bias is not None else None
        return L.ba_attention_fwd_qkv16(q, k, v, dt, pb, B, H, N, d, out, out_dt, None)
    assert aqkv(q=None) == INV and aqkv(k=None) == INV and aqkv(v=None) == INV and aqkv(out=None) == INV
    assert aqkv(d=20) == UNS and aqkv(d=128) == UNS and aqkv(N=257) == UNS and aqkv(dt=ba.BA_F32) == UNS
    assert aqkv(bias=ba_bias(ba.BA_BIAS_DENSE, P + 7 * (1 << 32), ba.BA_F16, 0, 0, 0, 0)) == UNS
    assert aqkv(N=66, bias=ba_bias(ba.BA_BIAS_DENSE, P + 7 * (1 << 32), ba.BA_F32, 0, 0, 0, 0)) == UNS
    assert aqkv(v=ctypes.c_void_p(P + 2 * (1 << 32) + 8)) == INV     # not 16-byte aligned
    assert aqkv(out=A(1)) == INV                                      # output aliases K
    assert aqkv(bias=ba_bias(ba.BA_BIAS_RELPOS, P + 7 * (1 << 32), ba.BA_F32, 0, 3, 5, 0)) == INV


def test_hamming_rejections(L):
    def ham(qb=A(0), kb=A(1), B=1, H=2, N=10, d=64, bh0=0, nbh=2, r0=0, nr=10, sig=A(2)):
        return L.ba_debug_hamming_scores(qb, kb, B, H, N, d, bh0, nbh, r0, nr, sig, None)
    assert ham(qb=None) == INV and ham(sig=None) == INV
    assert ham(nbh=0) == INV and ham(nr=0) == INV
    assert ham(bh0=1, nbh=2) == INV and ham(r0=5, nr=6) == INV and ham(bh0=-1) == INV
    assert ham(d=129) == UNS
    assert ham(sig=A(0)) == INV


def prep_s(L, st=ba_strides(3 * 8 * 64, 64, 3 * 64), q=A(0), k=None, v=None, dt=ba.BA_BF16, B=1, H=1, N=8, d=64,
           **kw):
    # default: q, k, v are the head slices of one [B, N, 3, H, d] buffer
    k = k or ctypes.c_void_p(P + 2 * H * d)
    v = v or ctypes.c_void_p(P + 4 * H * d)
    o = dict(qb=A(3), qm=A(4), kb=A(5), km=A(6), vq=A(7), vs=A(8))
    o.update(kw)
    pst = ctypes.byref(st) if st is not None else None
    return L.ba_pack_qk_quant_v_strided(q, k, v, pst, dt, B, H, N, d, o["qb"], o["qm"], o["kb"], o["km"],
                                        o["vq"], o["vs"], None)


def test_pack_qk_quant_v_strided_rejections(L):
    assert prep_s(L, st=None) == INV
    assert prep_s(L, st=ba_strides(0, 0, -1)) == INV
    assert prep_s(L, st=ba_strides(1 << 40, 0, 64), B=2) == INV      # span above 2^40 elements
    assert prep_s(L, q=None) == INV and prep_s(L, vs=None) == INV
    assert prep_s(L, q=ctypes.c_void_p(P + 1)) == INV                 # not 2-byte aligned
    assert prep_s(L, N=0) == INV and prep_s(L, d=129) == UNS and prep_s(L, dt=ba.BA_F32) == UNS
    # an output inside the span of the V view: V's last token starts at element 2*C + 7*3*C
    assert prep_s(L, vq=ctypes.c_void_p(P + 2 * (2 * 64 + 7 * 3 * 64) + 16)) == INV
    assert prep_s(L, qm=A(3)) == INV                                  # outputs overlap


def attn_s(L, st=ba_strides(16 * 2 * 64, 64, 2 * 64), B=2, H=2, N=16, d=64, out=A(9), **kw):
    args = dict(qb=A(1), qm=A(2), kb=A(3), km=A(4), vq=A(5), vs=A(6))
    args.update(kw)
    pst = ctypes.byref(st) if st is not None else None
    return L.ba_attention_fwd_strided(args["qb"], args["qm"], args["kb"], args["km"], args["vq"], args["vs"],
                                      None, B, H, N, d, out, pst, ba.BA_BF16, None)


def test_attention_strided_rejections(L):
    assert attn_s(L, st=None) == INV and attn_s(L, out=None) == INV
    assert attn_s(L, st=ba_strides(-1, 64, 128)) == INV
    assert attn_s(L, out=ctypes.c_void_p(P + 9 * (1 << 32) + 1)) == INV  # not 2-byte aligned
    # views that map two elements to one address
    assert attn_s(L, st=ba_strides(0, 64, 128)) == INV                     # batches alias
    assert attn_s(L, st=ba_strides(2048, 32, 128)) == INV                  # heads overlap channels
    assert attn_s(L, st=ba_strides(2048, 64, 0)) == INV                    # tokens alias
    assert attn_s(L, st=ba_strides(2048, 64, 64)) == INV                   # tokens land on the next head
    # the span of the view reaches an input (vscale at A(6))
    assert attn_s(L, out=ctypes.c_void_p(P + 6 * (1 << 32) - 1024)) == INV
    assert attn_s(L, d=129) == UNS
    assert attn_s(L, st=ba_strides(1 << 33, 1 << 32, 64), N=1) == UNS   # head stride above 2^31 - 1


def test_probe_library_loads():
    """The microbenchmark library (profiling.py probe) is built and rejects
    bad arguments before any GPU call."""
    import os
    L = ctypes.CDLL(os.path.join(os.path.dirname(ba.__file__), "libbaprobe.so"))
    from bit_qk_attention_amd.profiling import PROBES
    assert L.bap_count() == len(PROBES)
    L.bap_time.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    ms = ctypes.c_float()
    assert L.bap_time(-1, 10, ctypes.byref(ms)) != 0
    assert L.bap_time(len(PROBES), 10, ctypes.byref(ms)) != 0
    assert L.bap_time(0, 0, ctypes.byref(ms)) != 0
