"""Guard bytes after every output of every call.

Each output tensor is the front of a larger device buffer whose bytes are
all set to a sentinel first; after the call the bytes past the output must
still hold it (no kernel writes past the end it was given), and the guarded
outputs must equal those of the same call on plain tensors, bit for bit.
Shapes cover every kernel family: the fused and the separate pre-passes,
the split V quantiser of long heads, the per-element paths (d % 8 != 0),
the resident and the streaming attention, ragged query and key tiles, the
dense-bias variants, the one-pass form, and a window of the sigma routes.
"""
import numpy as np
import pytest
import torch

import bit_qk_attention_amd as ba
import workloads
from gpu_helpers import dev_bias, to_dev

pytestmark = pytest.mark.gpu
GUARD = 512       # guard bytes after each output
FILL = 0x5A

CASES = [
    # name, B, H, N, d, dtype, bias kind (workload-style), n_prefix/grid for relpos
    ("dense_f32_ragged", 1, 3, 197, 64, workloads.F16, "dense_f32"),
    ("dense_f16_odd_rows", 2, 3, 129, 72, workloads.BF16, "dense_f16"),
    ("long_head_split_quantiser", 1, 2, 6000, 64, workloads.BF16, "none"),
    ("element_paths_d20", 2, 2, 77, 20, workloads.BF16, "none"),
    ("resident_d72", 1, 2, 256, 72, workloads.BF16, "none"),
    ("resident_relpos_d64", 2, 3, 197, 64, workloads.F16, "relpos"),
    ("long_head_parts", 1, 2, 4096, 64, workloads.BF16, "none"),
    ("d100_relpos", 1, 2, 197, 100, workloads.F16, "relpos"),
]


def guarded(shape, dtype):
    """(view of the front of a sentinel-filled buffer, the whole buffer)."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((n + GUARD,), FILL, dtype=torch.uint8, device="cuda")
    return buf[:n].view(dtype).view(shape), buf, n


def tail_intact(buf, n):
    return bool((buf[n:] == FILL).all())


def make_inputs(B, H, N, d, dt, bias):
    kw = dict(B=B, H=H, N=N, d=d, dtype=dt)
    if bias == "none":
        inp = workloads.make("dit_256", bias="none", **kw)
    elif bias == "dense_f32":
        inp = workloads.make("deit_tiny", **kw)
    elif bias == "dense_f16":
        inp = workloads.make("dit_512", outlier_frac=0.0, **kw)
    else:
        inp = workloads.make("deit_small", grid=(14, 14), n_prefix=1, **kw)
    return inp


@pytest.mark.parametrize("name,B,H,N,d,dt,bias", CASES)
def test_outputs_stop_at_their_end(name, B, H, N, d, dt, bias):
    print(f"[guards] {name}: B={B} H={H} N={N} d={d}", flush=True)
    inp = make_inputs(B, H, N, d, dt, bias)
    s = inp.spec
    q, k, v = (to_dev(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    lib_bias, _ = dev_bias(inp)
    W = ba.ba_packed_words(d)
    shapes = {"qbits": ((B, H, N, W), torch.int32), "qmu": ((B, H, N), torch.float32),
              "kbits": ((B, H, N, W), torch.int32), "kmu": ((B, H, N), torch.float32),
              "vq": ((B, H, N, d), torch.int8), "vscale": ((B, H, d), torch.float32)}

    def fresh():
        return {key: guarded(shp, dt_) for key, (shp, dt_) in shapes.items()}

    ref = ba.prepare(q, k, v)
    ref_out = ba.attention(q, k, v, bias=lib_bias)

    # the contract's two pre-pass calls, then the one-call pre-pass
    g = fresh()
    ba.ba_pack_qk(q, k, g["qbits"][0], g["qmu"][0], g["kbits"][0], g["kmu"][0])
    ba.ba_quant_v(v, g["vq"][0], g["vscale"][0])
    g2 = fresh()
    ba.ba_pack_qk_quant_v(q, k, v, *(g2[key][0] for key in ("qbits", "qmu", "kbits", "kmu", "vq", "vscale")))
    torch.cuda.synchronize()
    for gg in (g, g2):
        for key, r in zip(("qbits", "qmu", "kbits", "kmu", "vq", "vscale"), ref):
            t, buf, n = gg[key]
            assert tail_intact(buf, n), f"{key} written past its end"
            assert torch.equal(t, r), key

    # the attention (and, for d <= 64, its one-pass form)
    outs = [ba.ba_attention_fwd] + ([ba.ba_attention_fwd_online] if d <= 64 else [])
    for fn in outs:
        out, buf, n = guarded(tuple(q.shape), q.dtype)
        fn(*(g2[key][0] for key in ("qbits", "qmu", "kbits", "kmu", "vq", "vscale")), lib_bias, out)
        torch.cuda.synchronize()
        assert tail_intact(buf, n), f"{fn.__name__}: output written past its end"
        if fn is ba.ba_attention_fwd:
            assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))

    # the fused forms: K/V pre-pass, attention binarising Q, and (short
    # heads) the whole pass in one launch
    if d % 8 == 0:
        g3 = fresh()
        ba.ba_pack_k_quant_v(k, v, *(g3[key][0] for key in ("kbits", "kmu", "vq", "vscale")))
        out, buf, n = guarded(tuple(q.shape), q.dtype)
        ba.ba_attention_fwd_q16(q, *(g3[key][0] for key in ("kbits", "kmu", "vq", "vscale")), lib_bias, out)
        torch.cuda.synchronize()
        for key, r in zip(("kbits", "kmu", "vq", "vscale"), ref[2:]):
            t, gbuf, gn = g3[key]
            assert tail_intact(gbuf, gn), f"{key} (K/V pre-pass) written past its end"
            assert torch.equal(t, r), key
        for key in ("qbits", "qmu"):
            assert bool((g3[key][1] == FILL).all()), f"{key} touched by the K/V pre-pass"
        assert tail_intact(buf, n), "ba_attention_fwd_q16: output written past its end"
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        out, buf, n = guarded(tuple(q.shape), q.dtype)
        try:
            ba.ba_attention_fwd_qkv16(q, k, v, lib_bias, out)
        except ba.BinAttnError as e:
            assert e.status == ba.BA_ERR_UNSUPPORTED
            torch.cuda.synchronize()
            assert bool((buf == FILL).all()), "a refused one-launch call wrote"
        else:
            torch.cuda.synchronize()
            assert tail_intact(buf, n), "ba_attention_fwd_qkv16: output written past its end"
            assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))

    # a window of the similarity
    bh0, nbh = (1, 1) if B * H > 1 else (0, 1)
    r0, nr = 5, min(40, N - 5)
    sig, buf, n = guarded((nbh, nr, N), torch.int32)
    ba.ba_debug_hamming_scores(g2["qbits"][0], g2["kbits"][0], d, bh0, nbh, r0, nr, sig)
    full = torch.empty((nbh, nr, N), dtype=torch.int32, device="cuda")
    ba.ba_debug_hamming_scores(ref[0], ref[2], d, bh0, nbh, r0, nr, full)
    torch.cuda.synchronize()
    assert tail_intact(buf, n), "sigma written past its end"
    assert torch.equal(sig, full)
    print(f"[guards] {name}: every output stops at its end", flush=True)
