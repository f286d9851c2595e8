"""Strided views through the C ABI.

The pre-pass reads Q, K and V as the head slices of one [B, N, 3, H, d]
projection buffer (rows optionally padded), and the attention writes through
a [B, H, N, d] view of a [B, N, H, d + pad] buffer. Both must give the same
bits as the dense calls on dense copies (which the parity tests pin to the
oracle), and the attention must leave every element outside its view as it
was. One case is also checked against the oracle directly. The cases cover
every pre-pass path: the one-launch pre-pass, the separate packer and
channel-group quantiser (long heads), the per-token packer and element
quantiser (d % 8 != 0, or rows not 16-byte aligned), and the 8-byte and
element-wise output stores.
"""
import numpy as np
import pytest
import torch

import bit_qk_attention_amd as ba
import oracle
from gpu_helpers import to_dev
from workloads import BF16, F16, to_bits

pytestmark = pytest.mark.gpu
TOL = 2e-2
SENTINEL = -7.0

# B, N, H, d, dtype, row pad of the QKV buffer, row pad of the output, bias
CASES = [
    (2, 197, 3, 64, F16, 0, 0, "relpos_prefix"),   # one launch; relative position with a class token
    (2, 129, 3, 72, BF16, 0, 0, "dense_f16"),      # one launch, d = 72; dense fp16 bias
    (8, 1024, 16, 72, BF16, 0, 0, "none"),         # one launch, four chunks per packing thread
    (1, 2000, 2, 64, BF16, 0, 4, "none"),          # separate packer + channel-group quantiser
    (1, 4096, 2, 64, F16, 0, 0, "relpos_grid"),    # 64 x 64 grid, row-run relative position
    (1, 300, 2, 40, F16, 0, 3, "none"),            # five 16-byte pieces per token; element stores
    (2, 77, 3, 20, BF16, 0, 0, "none"),            # d % 8 != 0: per-token packer
    (1, 50, 2, 36, F16, 0, 1, "dense_f32"),        # d = 36
    (3, 64, 1, 128, BF16, 0, 0, "none"),           # d = 128, one head
    (2, 150, 2, 64, F16, 4, 0, "none"),            # rows not 16-byte aligned: element paths at d % 8 == 0
]


def qkv_views(B, N, H, d, dt, pad, seed):
    """q, k, v as [B, H, N, d] views of one [B, N, 3*H*d + pad] buffer."""
    C = H * d
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, N, 3 * C + pad)).astype(np.float32)
    x[:, :, 2 * C + 1] = 0.0   # an all-zero V channel (head 0, channel 1)
    x[:, 5 % N, :C] *= 8.0     # an outlier query row
    buf = to_dev(to_bits(x, dt), dt)
    t = buf[..., :3 * C].view(B, N, 3, H, d)
    return tuple(t[:, :, i].transpose(1, 2) for i in range(3))


def make_bias(kind, B, H, N, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "none":
        return None, None
    if kind in ("dense_f16", "dense_f32"):
        dense = torch.randn(H, N, N, generator=g)
        dense = dense.half() if kind == "dense_f16" else dense
        odt = F16 if kind == "dense_f16" else oracle.F32
        data = dense.numpy().view(np.uint16) if kind == "dense_f16" else dense.numpy()
        return (ba.Bias(ba.BA_BIAS_DENSE, dense.cuda()),
                oracle.Bias(oracle.BIAS_DENSE, data, odt, 0))
    n_prefix = 1 if kind == "relpos_prefix" else 0
    side = int(round((N - n_prefix) ** 0.5))
    assert side * side + n_prefix == N
    table = torch.randn(H, (2 * side - 1) ** 2, generator=g)
    return (ba.Bias(ba.BA_BIAS_RELPOS, table.cuda(), 0, side, side, n_prefix),
            oracle.Bias(oracle.BIAS_RELPOS, table.numpy(), oracle.F32, 0, side, side, n_prefix))


def bits16(t):
    return t.contiguous().view(torch.int16)


@pytest.mark.parametrize("B,N,H,d,dt,pad,opad,bias", CASES)
def test_strided_views_match_dense(B, N, H, d, dt, pad, opad, bias):
    seed = B * 7919 + N * 31 + H * 101 + d
    q, k, v = qkv_views(B, N, H, d, dt, pad, seed)
    assert not q.is_contiguous()
    dense = [x.contiguous() for x in (q, k, v)]
    got = ba.prepare(q, k, v)
    ref = ba.prepare(*dense)
    torch.cuda.synchronize()
    for name, g, r in zip(("qbits", "qmu", "kbits", "kmu", "vq", "vscale"), got, ref):
        assert torch.equal(g, r), name

    lib_bias, _ = make_bias(bias, B, H, N, seed)
    obuf = torch.full((B, N, H, d + opad), SENTINEL, dtype=q.dtype, device="cuda")
    oview = obuf[..., :d].transpose(1, 2)
    ba.attention(q, k, v, bias=lib_bias, out=oview)
    want = ba.attention(*dense, bias=lib_bias)
    torch.cuda.synchronize()
    assert torch.equal(bits16(oview), bits16(want))
    if opad:
        assert bool((obuf[..., d:] == SENTINEL).all())
    print(f"B={B} N={N} H={H} d={d} pad={pad} opad={opad} bias={bias}: bit-equal to the dense calls")


def test_strided_against_oracle():
    B, N, H, d, dt = 2, 129, 3, 72, BF16
    q, k, v = qkv_views(B, N, H, d, dt, 0, 11)
    lib_bias, ora_bias = make_bias("dense_f16", B, H, N, 12)
    obuf = torch.empty((B, N, H, d), dtype=q.dtype, device="cuda")
    ba.attention(q, k, v, bias=lib_bias, out=obuf.transpose(1, 2))
    torch.cuda.synchronize()
    q16, k16, v16 = (bits16(x).cpu().numpy().view(np.uint16) for x in (q, k, v))
    ref = oracle.attention(q16, k16, v16, dt, bias=ora_bias)
    got = obuf.transpose(1, 2).float().cpu().numpy().reshape(B * H, N, d)
    vm = float(np.abs(v.float().cpu().numpy()).max())
    err = np.abs(got - ref.out).max() / vm
    print(f"strided views against the oracle: max|gpu - oracle| / max|V| = {err:.2e}")
    assert err <= TOL


def test_strided_rejects_mismatched_views():
    q, k, v = qkv_views(1, 16, 2, 64, F16, 0, 3)
    with pytest.raises(ValueError):
        ba.prepare(q, k.contiguous(), v)
