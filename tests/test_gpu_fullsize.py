"""Full-size workloads in the launch configuration the benchmark times:
sampled output rows against the oracle (the parity bar of tests/parity.py),
sampled Hamming windows bit-exact (every Q.K route of the fused kernel), and
whole-tensor properties (finite, rows are convex combinations of the
dequantised V, so |out| <= max|v8 * scale|)."""
import numpy as np
import pytest
import torch

import bit_qk_attention_amd as ba
import oracle
from gpu_helpers import DeviceRun, out_bits, vmax
from parity import check_output
from workloads import WORKLOADS, make

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_size_sampled(name):
    inp = make(name)
    s = inp.spec
    print(f"[full-size] {name} B={s.B} H={s.H} N={s.N} d={s.d}", flush=True)
    run = DeviceRun(inp)
    out = run.out.float()
    assert torch.isfinite(out).all()
    vq, vs = oracle.quant_v(inp.v, s.dtype)
    deq_max = float((np.abs(vq).max(axis=2).astype(np.float64) * vs).max())
    assert out.abs().max().item() <= deq_max * (1 + 1e-2)
    rng = np.random.default_rng(s.seed)
    BH = s.B * s.H
    qb, _ = oracle.pack(inp.q, s.dtype)
    kb, _ = oracle.pack(inp.k, s.dtype)
    vm = vmax(inp)
    bits = out_bits(run.out).reshape(BH, s.N, s.d)
    vq = vq.reshape(BH, s.N, s.d)
    vs = vs.reshape(BH, s.d)
    for bh in sorted(set([0, BH - 1, int(rng.integers(0, BH))])):
        for r0 in sorted(set([0, s.N - 8, int(rng.integers(0, s.N - 8))])):
            ref = oracle.attention(inp.q, inp.k, inp.v, s.dtype, bias=run.ora_bias,
                                   bh0=bh, nbh=1, row0=r0, nrows=8, want_e255=True)
            check_output(bits[bh:bh + 1, r0:r0 + 8], ref, vq[bh:bh + 1], vs[bh:bh + 1], s.dtype, vm,
                         label=f"{name} head {bh} rows {r0}..{r0 + 7}", loose=TOL)
            sig = torch.empty((1, 8, s.N), dtype=torch.int32, device="cuda")
            ba.ba_debug_hamming_scores(run.qbits, run.kbits, s.d, bh, 1, r0, 8, sig)
            want = oracle.hamming(qb, kb, s.d, bh0=bh, nbh=1, row0=r0, nrows=8)
            assert np.array_equal(sig.cpu().numpy(), want)
