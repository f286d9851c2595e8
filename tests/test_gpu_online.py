"""The one-pass attention (ba_attention_fwd_online: running row maximum,
keys in blocks of 32) through the C ABI.

Its p8 are quantised against the maximum of the blocks seen so far, so it
follows the plain definition (the oracle) only up to that blocking: the bar
is the method's stated bound, 2e-2 * max|V| against the oracle and against
the unquantised reference. Where the blocking changes nothing, it must agree
with the two-pass ba_attention_fwd to 1 ulp (the float row sums add in
another order): a single key block (N <= 32), and rows whose maximum lies in
the first block (checked with the oracle before the comparison).
"""
import numpy as np
import pytest
import torch

import bit_qk_attention_amd as ba
import oracle
from gpu_helpers import dev_bias, out_bits, to_dev, vmax
from parity import ulp_distance
from workloads import BF16, F16, F32, Inputs, Spec, from_bits, make, to_bits

pytestmark = pytest.mark.gpu
TOL = 2e-2

REDUCED = {
    "deit_tiny": dict(),
    "deit_small": dict(B=2),
    "long_4k": dict(B=1, H=2, N=700),
    "long_4k_rp": dict(B=1, H=2, N=23 * 29, grid=(23, 29)),
    "long_16k": dict(B=1, H=1, N=1100),
    "long_16k_rp": dict(B=1, H=2, N=1 + 16 * 48, grid=(16, 48), n_prefix=1),
}


def _run(inp, lib_bias):
    """(two-pass output, one-pass output) on the device inputs of inp."""
    s = inp.spec
    q, k, v = (to_dev(x, s.dtype) for x in (inp.q, inp.k, inp.v))
    qbits, qmu, kbits, kmu = ba.pack_qk(q, k)
    vq, vscale = ba.quant_v(v)
    two = torch.empty_like(q)
    one = torch.empty_like(q)
    ba.ba_attention_fwd(qbits, qmu, kbits, kmu, vq, vscale, lib_bias, two)
    ba.ba_attention_fwd_online(qbits, qmu, kbits, kmu, vq, vscale, lib_bias, one)
    torch.cuda.synchronize()
    return two, one


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_online_within_bound(name):
    inp = make(name, **REDUCED[name])
    s = inp.spec
    lib_b, ora_b = dev_bias(inp)
    two, one = _run(inp, lib_b)
    ref = oracle.attention(inp.q, inp.k, inp.v, s.dtype, bias=ora_b)
    fp, _ = oracle.attention_fp(inp.q, inp.k, inp.v, s.dtype, bias=ora_b)
    got = from_bits(out_bits(one), s.dtype).reshape(ref.out.shape).astype(np.float64)
    vm = vmax(inp)
    e_or = np.abs(got - ref.out).max() / vm
    e_fp = np.abs(got - fp.reshape(got.shape)).max() / vm
    same = float((out_bits(one) == out_bits(two)).mean())
    print(f"{name}: one-pass max|err|/max|V| vs oracle {e_or:.2e}, vs unquantised {e_fp:.2e}; "
          f"bit-identical to the two-pass output {same:.4f}")
    assert np.isfinite(got).all()
    assert e_or <= TOL and e_fp <= TOL


@pytest.mark.parametrize("N", [1, 17, 32])
def test_online_single_block_matches_two_pass(N):
    inp = make("long_4k", B=1, H=3, N=N)
    two, one = _run(inp, None)
    dist = ulp_distance(out_bits(one), out_bits(two))
    assert dist.max() <= 1, int(dist.max())


@pytest.mark.parametrize("dt", [F16, BF16])
def test_online_max_in_first_block_matches_two_pass(dt):
    """A dense bias of +3 on keys 0..31 puts every row maximum in the first
    block: the running maximum is then the row maximum from the first block
    on, every p8 equals the two-pass one and every fold factor is 1."""
    B, H, N, d = 1, 2, 300, 64
    rng = np.random.default_rng(77)
    shape = (B, H, N, d)
    q, k, v = (to_bits(rng.standard_normal(shape, dtype=np.float32), dt) for _ in range(3))
    bias = (0.1 * rng.standard_normal((H, N, N))).astype(np.float32)
    bias[:, :, :32] += 3.0
    ora_b = oracle.Bias(oracle.BIAS_DENSE, bias, F32, 0)
    ref = oracle.attention(q, k, v, dt, bias=ora_b, want_e255=True)
    # precondition: the key with 255 * p~ = 255 (the row maximum) is in block 0
    assert (ref.e255[..., 32:] < 255.0).all()
    lib_b = ba.Bias(ba.BA_BIAS_DENSE, torch.from_numpy(bias).cuda(), 0)

    two, one = _run(Inputs(Spec("first_block", B, H, N, d, dt, 0), q, k, v), lib_b)
    dist = ulp_distance(out_bits(one), out_bits(two))
    assert dist.max() <= 1, int(dist.max())
    assert (dist == 0).mean() > 0.5
