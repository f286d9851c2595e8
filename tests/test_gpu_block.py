"""The attention block (QKV projection -> BinaryAttention -> output
projection) against CPU references: the projections against float64 GEMMs of
the same 16-bit operands, the attention on the block's own Q, K, V against the
oracle, the output projection of the oracle's attention against the block's
output. Synthetic weights (no trained model)."""
import numpy as np
import pytest
import torch

import oracle
from bit_qk_attention_amd.block import attention_block
from workloads import BF16, F16

pytestmark = pytest.mark.gpu
TOL = 2e-2


def bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("B,N,H,d,dt", [(1, 300, 2, 64, BF16), (2, 129, 3, 72, F16)])
def test_block_against_references(B, N, H, d, dt):
    tdt = torch.float16 if dt == F16 else torch.bfloat16
    C = H * d
    g = torch.Generator().manual_seed(B * 1000 + N + H + d)
    x = torch.randn(B, N, C, generator=g).to(tdt).cuda()
    w_qkv = (torch.randn(C, 3 * C, generator=g) / C ** 0.5).to(tdt).cuda()
    b_qkv = (0.1 * torch.randn(3 * C, generator=g)).to(tdt).cuda()
    w_out = (torch.randn(C, C, generator=g) / C ** 0.5).to(tdt).cuda()
    b_out = (0.1 * torch.randn(C, generator=g)).to(tdt).cuda()
    keep = {}
    y = attention_block(x, w_qkv, b_qkv, w_out, b_out, H, keep=keep)
    torch.cuda.synchronize()

    # 1. the projection and the head split: q, k, v against a float64 GEMM
    X, Wq, bq = (t.double().cpu().numpy() for t in (x, w_qkv, b_qkv))
    qkv = (X.reshape(B * N, C) @ Wq + bq).reshape(B, N, 3, H, d).transpose(2, 0, 3, 1, 4)
    for i, name in enumerate("qkv"):
        got = keep[name].double().cpu().numpy()
        assert got.shape == (B, H, N, d)
        assert np.abs(got - qkv[i]).max() <= 2e-2 * np.abs(qkv[i]).max()

    # 2. the attention on the block's own q, k, v against the oracle
    q16, k16, v16 = (bits_of(keep[n]) for n in "qkv")
    ref = oracle.attention(q16, k16, v16, dt)
    got_o = keep["o"].float().cpu().numpy().reshape(B * H, N, d)
    vm = float(np.abs(keep["v"].float().cpu().numpy()).max())
    err = np.abs(got_o - ref.out).max() / vm
    print(f"block attention: max|gpu - oracle| / max|V| = {err:.2e}")
    assert err <= TOL

    # 3. the output projection of the oracle's attention against the block output
    O = ref.out.reshape(B, H, N, d).transpose(0, 2, 1, 3).reshape(B * N, C)
    Wo, bo = w_out.double().cpu().numpy(), b_out.double().cpu().numpy()
    want = (O @ Wo + bo).reshape(B, N, C)
    got_y = y.double().cpu().numpy()
    e_y = np.abs(got_y - want).max() / np.abs(want).max()
    print(f"block output: max|gpu - reference| / max|reference| = {e_y:.2e}")
    assert e_y <= TOL
