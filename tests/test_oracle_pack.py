"""Pins for the oracle's number formats, sign/scale packing and V quantisation.

Each check compares the oracle with something other than itself: numpy's own
fp16 conversion, bit-level brute force, closed forms of the definitions
(BinaryAttention summaries, gist.science zh technical summary section 2.2
items 1 and 3), invariants and a hand-worked example.
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import BF16, F16, from_bits, to_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_exhaustive(oracle_lib):
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got16 = oracle.decode16(allbits, F16)
    ref16 = allbits.view(np.float16).astype(np.float32)
    fin = np.isfinite(ref16)
    assert np.array_equal(got16[fin].view(np.uint32), ref16[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got16), np.isnan(ref16))
    gotbf = oracle.decode16(allbits, BF16)
    refbf = (allbits.astype(np.uint32) << 16).view(np.float32)
    fin = np.isfinite(refbf)
    assert np.array_equal(gotbf[fin].view(np.uint32), refbf[fin].view(np.uint32))


def test_round16_fp16_matches_numpy(oracle_lib):
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 5, 4000),
                         [0.0, -0.0, 65504.0, 65519.99, 6.1e-5, 5.96e-8, 2.98e-8, 1e-9]])
    # numpy converts double -> half with one round-to-nearest-even
    for x in xs:
        assert oracle.round16(x, F16) == int(np.float16(x).view(np.uint16)), x


def _bf16_brute(x: float) -> int:
    """Nearest bf16 by exhaustive search over the finite bf16 values; ties go
    to the even mantissa."""
    vals = _bf16_brute.vals
    i = np.searchsorted(vals, x)
    cands = [j for j in (i - 1, i) if 0 <= j < len(vals)]
    best = min(cands, key=lambda j: (abs(vals[j] - x), int(_bf16_brute.bits[j]) & 1))
    return int(_bf16_brute.bits[best])


_pos = np.arange(0, 0x7F80, dtype=np.uint32)
_bf16_brute.vals = np.concatenate([-(_pos[::-1] << 16).view(np.float32).astype(np.float64)[:-1],
                                   (_pos << 16).view(np.float32).astype(np.float64)])
_bf16_brute.bits = np.concatenate([(_pos[::-1] | 0x8000)[:-1], _pos]).astype(np.uint16)


def test_round16_bf16_brute_force(oracle_lib):
    rng = np.random.default_rng(8)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    # exact midpoints between neighbours: ties to even
    for b in rng.integers(1, 0x7F00, 200):
        lo = float((np.uint32(b) << 16).view(np.float32))
        hi = float((np.uint32(b + 1) << 16).view(np.float32))
        xs += [(lo + hi) / 2, -(lo + hi) / 2]
    for x in xs:
        got = oracle.round16(x, BF16)
        want = _bf16_brute(x)
        if x == 0.0:
            continue
        assert got == want, (x, hex(got), hex(want))


@pytest.mark.parametrize("d", [1, 5, 31, 32, 33, 64, 72, 96, 128])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_pack_bits_brute_force(oracle_lib, d, dtype):
    rng = np.random.default_rng(100 + d)
    x = rng.standard_normal((3, 17, d)).astype(np.float32)
    x[0, 0, :] = 0.0
    x[0, 1, :] = -0.0
    x[0, 2, ::2] = -0.0
    x[1, 0, :] = 1e-30   # underflows to +0 in fp16; a tiny positive in bf16
    x[1, 1, :] = -1e-30  # -0 in fp16, tiny negative in bf16
    bits16 = to_bits(x, dtype)
    xf = from_bits(bits16, dtype)
    bits, mu = oracle.pack(bits16, dtype)
    W = (d + 31) // 32
    assert bits.shape == (3, 17, W)
    for c in range(32 * W):
        got = (bits[..., c // 32] >> np.uint32(c % 32)) & 1
        want = (xf[..., c] < 0).astype(np.uint32) if c < d else np.zeros_like(got)
        assert np.array_equal(got, want), c
    # mu: the mean absolute value over the channels (fp64 sum of fp16/bf16
    # values is exact, so numpy's pairwise sum gives the same double)
    ref = (np.abs(xf.astype(np.float64)).sum(-1) / d).astype(np.float32)
    assert np.array_equal(mu, ref)


def test_pack_closed_forms(oracle_lib):
    rng = np.random.default_rng(3)
    d = 72
    s = np.where(rng.random((40, d)) < 0.5, -1.0, 1.0).astype(np.float32)
    bits, mu = oracle.pack(to_bits(s, BF16), BF16)
    assert np.all(mu == 1.0)
    # scaling by a positive power of two leaves the bits and scales mu exactly
    x = rng.standard_normal((40, d)).astype(np.float32)
    b1, m1 = oracle.pack(to_bits(x, BF16), BF16)
    b2, m2 = oracle.pack(to_bits(4.0 * x, BF16), BF16)
    assert np.array_equal(b1, b2) and np.array_equal(m2, 4.0 * m1)
    # all-positive input gives all-zero words; pad bits stay zero
    bp, _ = oracle.pack(to_bits(np.abs(x) + 0.5, BF16), BF16)
    assert not bp.any()
    bn, _ = oracle.pack(to_bits(-np.abs(x) - 0.5, BF16), BF16)
    assert np.all(bn[:, :2] == 0xFFFFFFFF) and np.all(bn[:, 2] == 0xFF)


def test_quant_v_invariants(oracle_lib):
    rng = np.random.default_rng(11)
    v = rng.standard_normal((2, 3, 50, 40)).astype(np.float32)
    v[0, 1, :, 7] = 0.0          # all-zero channel
    v[1, 2, :, 3] = -0.0
    bits = to_bits(v, F16)
    vf = from_bits(bits, F16).astype(np.float64)
    vq, vs = oracle.quant_v(bits, F16)
    amax = np.abs(vf).max(axis=2)
    assert np.all(vs[amax == 0] == 0) and np.all(vq[0, 1, :, 7] == 0) and np.all(vq[1, 2, :, 3] == 0)
    nz = amax > 0
    assert np.array_equal(vs[nz], (amax[nz].astype(np.float32) / np.float32(127.0)))
    # the largest |v| of every channel lands on +-127
    arg = np.abs(vf).argmax(axis=2)
    at = np.take_along_axis(vq, arg[:, :, None, :], axis=2)[:, :, 0, :]
    assert np.all(np.abs(at[nz]) == 127)
    assert np.all(np.sign(at[nz]) == np.sign(np.take_along_axis(vf, arg[:, :, None, :], 2)[:, :, 0, :][nz]))
    # rounding to nearest: reconstruction error at most half a step
    err = np.abs(vf - vq.astype(np.float64) * vs[:, :, None, :].astype(np.float64))
    assert np.all(err <= 0.5 * vs[:, :, None, :] * (1 + 1e-5) + 1e-30)
    assert vq.min() >= -127


def test_quant_v_closed_forms(oracle_lib):
    # a constant channel quantises to +-127 in every token; a channel with one
    # non-zero token has +-127 there and 0 elsewhere; all-zero channels give 0
    v = np.zeros((1, 2, 30, 16), np.float32)
    v[0, 0, :, 3] = 2.5
    v[0, 1, :, 5] = -0.75
    v[0, 0, 7, 9] = 1.0
    vq, vs = oracle.quant_v(to_bits(v, F16), F16)
    assert np.all(vq[0, 0, :, 3] == 127) and np.all(vq[0, 1, :, 5] == -127)
    assert vq[0, 0, 7, 9] == 127 and np.count_nonzero(vq) == 2 * 30 + 1
    assert vs[0, 0, 3] == np.float32(2.5) / np.float32(127) and vs[0, 1, 0] == 0.0
    # quantisation is odd-symmetric: negating V negates every code
    rv = np.random.default_rng(12).standard_normal((2, 2, 40, 24)).astype(np.float32)
    pos = oracle.quant_v(to_bits(rv, BF16), BF16)
    neg = oracle.quant_v(to_bits(-rv, BF16), BF16)
    assert np.array_equal(neg[0], -pos[0]) and np.array_equal(neg[1], pos[1]) and np.any(pos[0] != 0)


def test_hand_example_pack_and_quant(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "hand_d4.json")))
    q = np.array(g["q"], np.float32)[None, None]
    k = np.array(g["k"], np.float32)[None, None]
    v = np.array(g["v"], np.float32)[None, None]
    q[0, 0, 1, 0] = -0.0
    qb, qm = oracle.pack(to_bits(q, F16), F16)
    kb, km = oracle.pack(to_bits(k, F16), F16)
    assert qb[0, 0, :, 0].tolist() == g["qbits"] and kb[0, 0, :, 0].tolist() == g["kbits"]
    assert qm[0, 0].tolist() == g["qmu"] and km[0, 0].tolist() == g["kmu"]
    vq, vs = oracle.quant_v(to_bits(v, F16), F16)
    assert vq[0, 0].tolist() == g["vq"]
    want = [np.float32(a) / np.float32(g["vscale_den"]) for a in g["vscale_num"]]
    assert vs[0, 0].tolist() == [float(w) for w in want]
