"""The largest sequence the library accepts (N = BA_MAX_TOKENS = 65536 keys).

- Uniform attention with every quantised V value at +-127: the integer P.V
  sum reaches 255 * 127 * N, the int32 bound the token limit is derived from,
  and the channel sums 127 * N, the 24-bit bound of the epilogue's multiply.
  The output must equal V (a convex combination of identical rows).
- Random Q, K, V with the widest relative-position table (a 256 x 256 grid,
  the largest window the attention stages in LDS): the pre-pass bit-exact
  against the oracle, sampled output rows within the usual bound.
"""
import numpy as np
import pytest
import torch

import bit_qk_attention_amd as ba
import oracle
from gpu_helpers import to_dev
from workloads import BF16, F16, from_bits, to_bits

pytestmark = pytest.mark.gpu
TOL = 2e-2
N = ba.BA_MAX_TOKENS


@pytest.mark.parametrize("d,dt", [(64, BF16), (128, F16)])
def test_max_tokens_uniform_extreme_sums(d, dt):
    print(f"[limits] uniform N={N} d={d}", flush=True)
    q = np.zeros((1, 1, N, d), np.float32)                     # mu_q = 0: every score is 0
    k = np.random.default_rng(d).standard_normal((1, 1, N, d)).astype(np.float32)
    col = np.array([(1 if c % 2 == 0 else -1) * (c + 1) / 8.0 for c in range(d)], np.float32)
    v = np.broadcast_to(col, (1, 1, N, d)).copy()              # every row the same
    qd, kd, vd = (to_dev(to_bits(x, dt), dt) for x in (q, k, v))
    qbits, qmu, kbits, kmu, vq, vscale = ba.prepare(qd, kd, vd)
    out = torch.empty_like(qd)
    ba.ba_attention_fwd(qbits, qmu, kbits, kmu, vq, vscale, None, out)
    torch.cuda.synchronize()
    assert bool((vq.abs() == 127).all())                       # every v8 at the int8 limit
    # the kernel's channel sums reach 127 * N and its P.V sum 255 * 127 * N
    got = out.float().cpu().numpy()
    want = from_bits(to_bits(v, dt), dt)
    err = np.abs(got - want).max() / np.abs(want).max()
    print(f"uniform attention over {N} keys: max|out - v| / max|v| = {err:.2e}")
    assert err <= 1e-2


def test_max_tokens_widest_relpos_table():
    B, H, d, dt, side = 1, 1, 64, BF16, 256
    print(f"[limits] relpos {side}x{side} N={N} d={d}", flush=True)
    rng = np.random.default_rng(65536)
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    q16, k16, v16 = (to_bits(x[i], dt) for i in range(3))
    table = (0.1 * rng.standard_normal((H, (2 * side - 1) ** 2))).astype(np.float32)
    qd, kd, vd = (to_dev(b, dt) for b in (q16, k16, v16))
    bias = ba.Bias(ba.BA_BIAS_RELPOS, torch.from_numpy(table).cuda(), 0, side, side, 0)
    qbits, qmu, kbits, kmu, vq, vscale = ba.prepare(qd, kd, vd)
    out = torch.empty_like(qd)
    ba.ba_attention_fwd(qbits, qmu, kbits, kmu, vq, vscale, bias, out)
    torch.cuda.synchronize()

    qb, qm = oracle.pack(q16, dt)
    ovq, ovs = oracle.quant_v(v16, dt)
    assert np.array_equal(qbits.cpu().numpy().view(np.uint32), qb)
    assert np.array_equal(qmu.cpu().numpy(), qm)
    assert np.array_equal(vq.cpu().numpy(), ovq)
    assert np.array_equal(vscale.cpu().numpy(), ovs)

    ora_bias = oracle.Bias(oracle.BIAS_RELPOS, table, oracle.F32, 0, side, side, 0)
    got = out.float().cpu().numpy().reshape(B * H, N, d)
    vm = float(np.abs(from_bits(v16, dt)).max())
    for r0 in (0, 31 * side + 100, N - 8):
        ref = oracle.attention(q16, k16, v16, dt, bias=ora_bias, bh0=0, nbh=1, row0=r0, nrows=8)
        err = np.abs(got[0, r0:r0 + 8] - ref.out[0]).max() / vm
        print(f"rows {r0}..{r0 + 7}: max|gpu - oracle| / max|V| = {err:.2e}")
        assert err <= TOL
