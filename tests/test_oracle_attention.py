"""Pins for the oracle's Hamming similarity, scores, softmax and quantised
aggregation.

References: BinaryAttention summaries on gist.science — zh technical summary
sections 2.1-2.3, nl Methodologie 1-3, it/fr/pt section 2. The pins are:
brute-force +-1 dot products (numpy matmul) against the XOR/popcount route,
exhaustive sign patterns for d <= 6, a textbook reduction to softmax(S)V
(scipy), closed forms of the quantised path (uniform keys, one-hot bias,
N = 1, identical V rows), invariants (key permutation, per-row bias shift, relpos = dense,
rows of P summing to 1) and hand-worked examples in tests/golden/.
"""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import Bias
from workloads import BF16, F16, F32, from_bits, make, to_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def signs(x):
    """+-1 with sign(0) = +1, as floats."""
    return np.where(x < 0, -1.0, 1.0)


# ---------------------------------------------------------------- Hamming --

@pytest.mark.parametrize("d", [1, 3, 31, 32, 33, 64, 72, 128])
def test_hamming_equals_sign_dot(oracle_lib, d):
    rng = np.random.default_rng(d)
    q = rng.standard_normal((2, 2, 37, d)).astype(np.float32)
    k = rng.standard_normal((2, 2, 37, d)).astype(np.float32)
    q[0, 0, 0, :5] = 0.0
    k[0, 0, 1, :5] = -0.0
    qb16, kb16 = to_bits(q, BF16), to_bits(k, BF16)
    qbits, _ = oracle.pack(qb16, BF16)
    kbits, _ = oracle.pack(kb16, BF16)
    sig = oracle.hamming(qbits, kbits, d)
    sq = signs(from_bits(qb16, BF16)).reshape(4, 37, d)
    sk = signs(from_bits(kb16, BF16)).reshape(4, 37, d)
    want = np.einsum("hid,hjd->hij", sq, sk).astype(np.int32)
    assert np.array_equal(sig, want)


@pytest.mark.parametrize("d", [1, 2, 3, 4, 5, 6])
def test_hamming_exhaustive_small_d(oracle_lib, d):
    pats = np.array(list(itertools.product([1.0, -1.0], repeat=d)), np.float32)  # 2^d x d
    x = pats[None, None]
    bits, mu = oracle.pack(to_bits(x, F16), F16)
    sig = oracle.hamming(bits, bits, d)[0]
    assert np.array_equal(sig, (pats @ pats.T).astype(np.int32))
    assert np.all(mu == 1.0)


def test_hamming_invariants(oracle_lib):
    rng = np.random.default_rng(5)
    d = 72
    q = rng.standard_normal((1, 1, 64, d)).astype(np.float32)
    q[0, 0, :, ::7] = 0.0
    k = rng.standard_normal((1, 1, 64, d)).astype(np.float32)
    qb, _ = oracle.pack(to_bits(q, BF16), BF16)
    kb, _ = oracle.pack(to_bits(k, BF16), BF16)
    s = oracle.hamming(qb, kb, d)[0]
    assert np.all(np.abs(s) <= d) and np.all((s - d) % 2 == 0)
    assert np.all(np.diag(oracle.hamming(qb, qb, d)[0]) == d)
    assert np.array_equal(oracle.hamming(kb, qb, d)[0], s.T)
    nb, _ = oracle.pack(to_bits(-q, BF16), BF16)
    zeros = (q[0, 0] == 0).sum(-1)
    assert np.array_equal(np.diag(oracle.hamming(qb, nb, d)[0]), -d + 2 * zeros)
    # windowed call returns the matching block
    w = oracle.hamming(qb, kb, d, bh0=0, nbh=1, row0=10, nrows=7)
    assert np.array_equal(w[0], s[10:17])


# ------------------------------------------------- scores and softmax (R2) --

def numpy_scores(q16, k16, dtype, d, bias_dense=None):
    qf = from_bits(q16, dtype).astype(np.float64)
    kf = from_bits(k16, dtype).astype(np.float64)
    mq = np.float32(1) * (np.abs(qf).sum(-1) / d).astype(np.float32)
    mk = (np.abs(kf).sum(-1) / d).astype(np.float32)
    S = signs(qf) @ np.swapaxes(signs(kf), -1, -2)
    S = mq.astype(np.float64)[..., :, None] * mk.astype(np.float64)[..., None, :] * S / np.sqrt(d)
    if bias_dense is not None:
        S = S + bias_dense
    return S


def test_textbook_reduction_pm1(oracle_lib):
    """Q, K in {+-1} (so mu = 1), no bias: the unquantised path is exactly
    softmax(Q K^T / sqrt(d)) V."""
    rng = np.random.default_rng(21)
    B, H, N, d = 1, 2, 40, 64
    q = signs(rng.standard_normal((B, H, N, d))).astype(np.float32)
    k = signs(rng.standard_normal((B, H, N, d))).astype(np.float32)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    q16, k16, v16 = to_bits(q, F16), to_bits(k, F16), to_bits(v, F16)
    out, prob = oracle.attention_fp(q16, k16, v16, F16, want_prob=True)
    P = softmax(q.astype(np.float64) @ np.swapaxes(k, -1, -2).astype(np.float64) / np.sqrt(d), axis=-1)
    O = P @ from_bits(v16, F16).astype(np.float64)
    assert np.allclose(out.reshape(O.shape), O, rtol=0, atol=1e-12)
    assert np.allclose(prob.reshape(P.shape), P, rtol=0, atol=1e-14)


@pytest.mark.parametrize("bias", ["none", "dense_f32", "dense_f16"])
def test_fp_reference_matches_numpy(oracle_lib, bias):
    rng = np.random.default_rng(22)
    B, H, N, d = 2, 2, 33, 72
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32) * 1.5
    q16, k16, v16 = (to_bits(t, BF16) for t in x)
    ob = None
    dense = None
    if bias != "none":
        bf = (0.3 * rng.standard_normal((H, N, N))).astype(np.float32)
        if bias == "dense_f16":
            bits = bf.astype(np.float16).view(np.uint16)
            dense = bits.view(np.float16).astype(np.float64)
            ob = Bias(oracle.BIAS_DENSE, bits, oracle.F16, 0)
        else:
            dense = bf.astype(np.float64)
            ob = Bias(oracle.BIAS_DENSE, bf, oracle.F32, 0)
    out, prob = oracle.attention_fp(q16, k16, v16, BF16, bias=ob, want_prob=True)
    S = numpy_scores(q16, k16, BF16, d, None if dense is None else dense[None])
    P = softmax(S, axis=-1)
    O = P @ from_bits(v16, BF16).astype(np.float64)
    assert np.allclose(prob.reshape(P.shape), P, rtol=1e-12, atol=1e-15)
    assert np.allclose(out.reshape(O.shape), O, rtol=1e-11, atol=1e-12)
    assert np.allclose(prob.sum(-1), 1.0, atol=1e-12)  # rows sum to 1 before quantisation


# --------------------------------------------------------- quantised path --

def test_p8_and_acc_from_numpy(oracle_lib):
    """p8 = rne(255 exp(s - max s)) and A = p8 @ v8, recomputed through numpy
    matmul/scipy-free routes from the oracle's own v8 (pinned separately)."""
    rng = np.random.default_rng(23)
    B, H, N, d = 1, 2, 50, 64
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    q16, k16, v16 = (to_bits(t, F16) for t in x)
    r = oracle.attention(q16, k16, v16, F16, want_p8=True)
    S = numpy_scores(q16, k16, F16, d).reshape(B * H, N, N)
    m = S.max(-1, keepdims=True)
    e = 255.0 * np.exp(S - m)
    p8 = np.rint(e)
    near_tie = np.abs(e - np.floor(e) - 0.5) < 1e-9
    assert np.array_equal(r.p8[~near_tie], p8[~near_tie].astype(np.uint8))
    assert np.allclose(r.m, m[..., 0], rtol=0, atol=1e-12)
    # float normaliser (the default): the unquantised row sums from numpy
    assert np.allclose(r.l, np.exp(S - m).sum(-1), rtol=1e-13)
    vq, vs = oracle.quant_v(v16, F16)
    A = r.p8.astype(np.int64) @ vq.reshape(B * H, N, d).astype(np.int64)
    assert np.array_equal(r.acc, A)
    want = A * vs.reshape(B * H, 1, d).astype(np.float64) / (255.0 * np.exp(S - m).sum(-1)[..., None])
    assert np.allclose(r.out, want, rtol=1e-12, atol=0)
    # integer normaliser: the row sums of p8 from numpy, same p8 and A
    ri = oracle.attention(q16, k16, v16, F16, want_p8=True, norm=oracle.NORM_P8)
    assert np.array_equal(ri.p8, r.p8) and np.array_equal(ri.acc, r.acc)
    assert np.array_equal(ri.l * 255.0, r.p8.astype(np.int64).sum(-1).astype(np.float64))
    wanti = A * vs.reshape(B * H, 1, d).astype(np.float64) / r.p8.astype(np.int64).sum(-1, keepdims=True)
    assert np.allclose(ri.out, wanti, rtol=1e-14, atol=0)
    # dequantised output against the unquantised reference: differs only by
    # quantisation error, far below max|V|/50
    fp, _ = oracle.attention_fp(q16, k16, v16, F16)
    vmax = np.abs(from_bits(v16, F16)).max()
    assert np.abs(r.out - fp).max() < 0.02 * vmax
    assert np.abs(r.out - fp).max() > 0  # quantisation is really applied


def test_uniform_keys_closed_form(oracle_lib):
    """All keys identical, no bias: every p~ = 1, p8 = 255, l = N, so
    O_ic = scale_c * sum_j v8_jc / N exactly."""
    rng = np.random.default_rng(24)
    B, H, N, d = 1, 2, 70, 72
    q = rng.standard_normal((B, H, N, d)).astype(np.float32)
    k = np.repeat(rng.standard_normal((B, H, 1, d)).astype(np.float32), N, axis=2)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    q16, k16, v16 = (to_bits(t, BF16) for t in (q, k, v))
    vq, vs = oracle.quant_v(v16, BF16)
    want = vs.reshape(B * H, 1, d).astype(np.float64) * vq.reshape(B * H, N, d).sum(1, keepdims=True) / N
    for norm in (oracle.NORM_P8, oracle.NORM_FLOAT):
        r = oracle.attention(q16, k16, v16, BF16, want_p8=True, norm=norm)
        assert np.all(r.p8 == 255) and np.all(r.l == N)
        assert np.allclose(r.out, np.broadcast_to(want, r.out.shape), rtol=1e-14, atol=0)


def test_constant_v_rows_closed_form(oracle_lib):
    """Every token carries the same V row: with the integer normaliser the
    output is a weighted mean of identical dequantised rows whose weights
    sum to exactly 1, so O_i = v8 * scale exactly for every query, whatever
    Q, K and the bias are. The float normaliser misses this by
    sum_j p8 / (255 * sum_j p~), which is not 1."""
    rng = np.random.default_rng(34)
    B, H, N, d = 1, 2, 90, 64
    q = rng.standard_normal((B, H, N, d)).astype(np.float32)
    k = rng.standard_normal((B, H, N, d)).astype(np.float32)
    v = np.repeat(rng.standard_normal((B, H, 1, d)).astype(np.float32), N, axis=2)
    bias = (0.5 * rng.standard_normal((H, N, N))).astype(np.float32)
    q16, k16, v16 = (to_bits(t, F16) for t in (q, k, v))
    ob = Bias(oracle.BIAS_DENSE, bias, oracle.F32, 0)
    vq, vs = oracle.quant_v(v16, F16)
    row = vq[0, :, :1].astype(np.float64) * vs[0, :, None].astype(np.float64)  # [H,1,d]
    r = oracle.attention(q16, k16, v16, F16, bias=ob, norm=oracle.NORM_P8)
    assert np.array_equal(r.out, np.broadcast_to(row, r.out.shape))
    rf = oracle.attention(q16, k16, v16, F16, bias=ob)
    assert not np.allclose(rf.out, np.broadcast_to(row, rf.out.shape), rtol=1e-6, atol=0)


def test_float_normaliser_meets_the_unquantised_bound(oracle_lib):
    """Why l is the float sum of the unquantised values: with the DiT-512
    workload's 1% x8 outlier tokens, rows are so peaked that many keys have
    p~ < 1/510 (p8 = 0) yet carry a few percent of the mass together.
    The float normaliser keeps that mass in l and stays far inside
    2e-2 * max|V| of the unquantised reference; renormalising over the keys
    that survive quantisation (the integer row sum of p8) inflates the
    dominant keys' weight and leaves the bound."""
    inp = make("dit_512", B=2, H=2, N=333)
    ob = Bias(oracle.BIAS_DENSE, inp.bias_data, inp.bias_dtype, 0)
    fp, _ = oracle.attention_fp(inp.q, inp.k, inp.v, BF16, bias=ob)
    vmax = np.abs(from_bits(inp.v, BF16)).max()
    e_float = np.abs(oracle.attention(inp.q, inp.k, inp.v, BF16, bias=ob).out - fp).max() / vmax
    e_p8 = np.abs(oracle.attention(inp.q, inp.k, inp.v, BF16, bias=ob, norm=oracle.NORM_P8).out - fp).max() / vmax
    print(f"max|quantised - unquantised| / max|V|: float normaliser {e_float:.2e}, integer {e_p8:.2e}")
    assert e_float < 1e-2 < 2e-2 < e_p8


def test_one_hot_bias_closed_form(oracle_lib):
    """A +1e4 bias at one key per row: p8 = 255 there and 0 elsewhere, l = 1,
    so O_i = v8_{j*} * scale."""
    rng = np.random.default_rng(25)
    B, H, N, d = 1, 3, 45, 64
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    q16, k16, v16 = (to_bits(t, F16) for t in x)
    jstar = rng.integers(0, N, size=(H, N))
    bias = np.zeros((H, N, N), np.float32)
    for h in range(H):
        bias[h, np.arange(N), jstar[h]] = 1e4
    r = oracle.attention(q16, k16, v16, F16, bias=Bias(oracle.BIAS_DENSE, bias, oracle.F32, 0),
                         want_p8=True)
    vq, vs = oracle.quant_v(v16, F16)
    for h in range(H):
        assert np.all(r.p8[h].sum(-1) == 255)
        want = vq[0, h][jstar[h]].astype(np.float64) * vs[0, h].astype(np.float64)
        assert np.allclose(r.out[h], want, rtol=1e-12, atol=0)
        assert np.all(r.l[h] == 1.0)


def test_single_token(oracle_lib):
    rng = np.random.default_rng(26)
    x = rng.standard_normal((3, 2, 2, 1, 40)).astype(np.float32)
    q16, k16, v16 = (to_bits(t, BF16) for t in x)
    r = oracle.attention(q16, k16, v16, BF16)
    vq, vs = oracle.quant_v(v16, BF16)
    want = vq.reshape(4, 1, 40) * vs.reshape(4, 1, 40).astype(np.float64)
    assert np.array_equal(r.out, want)


def test_key_permutation_invariance(oracle_lib):
    """Permuting keys, values and bias columns together leaves the integer
    accumulator bit-identical and the output equal up to fp64 rounding."""
    rng = np.random.default_rng(27)
    B, H, N, d = 2, 2, 64, 64
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    bias = (0.1 * rng.standard_normal((H, N, N))).astype(np.float32)
    q16, k16, v16 = (to_bits(t, BF16) for t in x)
    perm = rng.permutation(N)
    r0 = oracle.attention(q16, k16, v16, BF16, bias=Bias(oracle.BIAS_DENSE, bias, oracle.F32, 0))
    r1 = oracle.attention(q16, np.ascontiguousarray(k16[:, :, perm]), np.ascontiguousarray(v16[:, :, perm]),
                          BF16, bias=Bias(oracle.BIAS_DENSE, np.ascontiguousarray(bias[:, :, perm]),
                                          oracle.F32, 0))
    assert np.array_equal(r0.acc, r1.acc)
    assert np.allclose(r0.out, r1.out, rtol=1e-13, atol=1e-15)
    assert np.allclose(r0.l, r1.l, rtol=1e-13)


def test_bias_row_shift_invariance(oracle_lib):
    rng = np.random.default_rng(28)
    B, H, N, d = 1, 2, 48, 64
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    q16, k16, v16 = (to_bits(t, F16) for t in x)
    bias = (0.1 * rng.standard_normal((H, N, N))).astype(np.float64)
    shift = rng.integers(-8, 8, size=(H, N, 1)).astype(np.float64)  # exact in fp32
    b0 = bias.astype(np.float32)
    b1 = (b0.astype(np.float64) + shift).astype(np.float32)
    r0 = oracle.attention(q16, k16, v16, F16, bias=Bias(oracle.BIAS_DENSE, b0, oracle.F32, 0))
    r1 = oracle.attention(q16, k16, v16, F16, bias=Bias(oracle.BIAS_DENSE, b1, oracle.F32, 0))
    # b1 - b0 is the exact per-row shift only where the float32 sum is exact;
    # outputs agree to rounding, accumulators up to rare rounding flips
    assert np.allclose(r0.out, r1.out, rtol=0, atol=1e-3 * np.abs(r0.out).max())
    assert (r0.acc != r1.acc).mean() < 0.05


def relpos_dense(table, gh, gw, npre):
    """Materialise the relative-position table into a dense [H,N,N] bias with
    explicit grid coordinates."""
    H = table.shape[0]
    N = npre + gh * gw
    out = np.zeros((H, N, N), np.float32)
    for i in range(npre, N):
        ri, ci = divmod(i - npre, gw)
        for j in range(npre, N):
            rj, cj = divmod(j - npre, gw)
            out[:, i, j] = table[:, (ri - rj + gh - 1) * (2 * gw - 1) + (ci - cj + gw - 1)]
    return out


def test_relpos_index_hand_example(oracle_lib):
    """Pin the table indexing against the hand-worked index grid: with Q = 0
    (mu = 0) the scores are the bias alone, so log-probabilities recover it."""
    g = json.load(open(os.path.join(GOLDEN, "relpos_2x3.json")))
    gh, gw, npre = g["grid_h"], g["grid_w"], g["n_prefix"]
    N = npre + gh * gw
    T = (2 * gh - 1) * (2 * gw - 1)
    table = (0.01 * np.arange(T) + 0.5).astype(np.float32)[None]  # distinct entries
    zeros = np.zeros((1, 1, N, 8), np.float32)
    v = np.random.default_rng(0).standard_normal((1, 1, N, 8)).astype(np.float32)
    q16 = to_bits(zeros, F16)
    _, prob = oracle.attention_fp(q16, q16, to_bits(v, F16), F16,
                                  bias=Bias(oracle.BIAS_RELPOS, table, oracle.F32, 0, gh, gw, npre),
                                  want_prob=True)
    idx = np.array(g["index"])
    want_b = np.where(idx >= 0, table[0][np.maximum(idx, 0)], 0.0)
    logp = np.log(prob[0])
    got_b = logp - logp[:, :1]  # key 0 is the prefix token with bias 0
    assert np.allclose(got_b, want_b - want_b[:, :1], atol=1e-6)


def test_relpos_equals_dense(oracle_lib):
    inp = make("deit_small", B=2, H=2)
    table = inp.bias_data[:2]
    r0 = oracle.attention(inp.q, inp.k, inp.v, F16,
                          bias=Bias(oracle.BIAS_RELPOS, table, oracle.F32, 0, 14, 14, 1))
    dense = relpos_dense(table, 14, 14, 1)
    r1 = oracle.attention(inp.q, inp.k, inp.v, F16, bias=Bias(oracle.BIAS_DENSE, dense, oracle.F32, 0))
    assert np.array_equal(r0.out, r1.out) and np.array_equal(r0.acc, r1.acc)


def test_batch_stride(oracle_lib):
    """A per-batch dense bias with stride H*N*N equals running each batch
    element with its own shared slice."""
    rng = np.random.default_rng(29)
    B, H, N, d = 3, 2, 20, 32
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    q16, k16, v16 = (to_bits(t, F16) for t in x)
    bias = (0.2 * rng.standard_normal((B, H, N, N))).astype(np.float32)
    r = oracle.attention(q16, k16, v16, F16, bias=Bias(oracle.BIAS_DENSE, bias, oracle.F32, H * N * N))
    for b in range(B):
        rb = oracle.attention(q16[b:b + 1], k16[b:b + 1], v16[b:b + 1], F16,
                              bias=Bias(oracle.BIAS_DENSE, np.ascontiguousarray(bias[b]), oracle.F32, 0))
        assert np.array_equal(r.out[b * H:(b + 1) * H], rb.out)


def test_row_window(oracle_lib):
    inp = make("dit_256", B=1, H=3, N=100)
    full = oracle.attention(inp.q, inp.k, inp.v, BF16)
    part = oracle.attention(inp.q, inp.k, inp.v, BF16, bh0=1, nbh=2, row0=37, nrows=11)
    assert np.array_equal(part.out, full.out[1:3, 37:48])
    assert np.array_equal(part.out_bits, full.out_bits[1:3, 37:48])


def test_output_rounding(oracle_lib):
    """out_bits is the one-step rounding of out to the output format."""
    inp = make("deit_tiny", N=60)
    r = oracle.attention(inp.q, inp.k, inp.v, F16,
                         bias=Bias(oracle.BIAS_DENSE, np.ascontiguousarray(inp.bias_data[:, :60, :60]),
                                   oracle.F32, 0))
    assert np.array_equal(r.out_bits, r.out.astype(np.float16).view(np.uint16))


def test_hand_example_attention(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "hand_d4.json")))
    q = np.array(g["q"], np.float32)[None, None]
    k = np.array(g["k"], np.float32)[None, None]
    v = np.array(g["v"], np.float32)[None, None]
    q16, k16, v16 = (to_bits(t, F16) for t in (q, k, v))
    qb, _ = oracle.pack(q16, F16)
    kb, _ = oracle.pack(k16, F16)
    assert oracle.hamming(qb, kb, 4)[0].tolist() == g["sigma"]
    scale = np.array(g["vscale_num"]) / g["vscale_den"]
    # integer normaliser: 255 l = row sum of p8
    r = oracle.attention(q16, k16, v16, F16, want_p8=True, norm=oracle.NORM_P8)
    assert r.p8[0].tolist() == g["p8"]
    assert r.acc[0].tolist() == g["acc"]
    assert np.allclose(r.m[0], g["m"], rtol=0, atol=1e-15)
    assert (r.l[0] * 255.0).tolist() == g["p8_row_sum"]
    want = np.array(g["acc"]) * scale[None] / np.array(g["p8_row_sum"], np.float64)[:, None]
    assert np.allclose(r.out[0], want, rtol=1e-6)
    # float normaliser (the default): l = sum of the unquantised exp(s - m)
    rf = oracle.attention(q16, k16, v16, F16, want_p8=True)
    assert rf.p8[0].tolist() == g["p8"] and rf.acc[0].tolist() == g["acc"]
    l_hand = np.array([1 + np.exp(-1.96875), 1 + np.exp(-0.046875)])
    assert np.allclose(rf.l[0], l_hand, rtol=1e-15)
    wantf = np.array(g["acc"]) * scale[None] / (255.0 * l_hand[:, None])
    assert np.allclose(rf.out[0], wantf, rtol=1e-6)


def test_rejects_bad_arguments(oracle_lib):
    x = np.zeros((1, 1, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.attention(x, x, x, F32)
    with pytest.raises(ValueError):
        oracle.attention(x, x, x, F16, bias=Bias(oracle.BIAS_RELPOS, np.zeros((1, 9), np.float32),
                                                 oracle.F32, 0, 2, 3, 0))
    with pytest.raises(ValueError):
        oracle.attention(x, x, x, F16, norm=2)


# ---------------------------------------------------- given scales (mu in) --
# mu is an input of the attention step (zh §2.2(1): a learnable scale), so the
# oracle also takes it as given arrays, e.g. one scalar per head.

def test_given_mu_zero_is_uniform_average(oracle_lib):
    """mu = 0 and no bias: every score is 0, every p~ = 1 and p8 = 255, l = N,
    so the output is the plain average of the dequantised V rows."""
    rng = np.random.default_rng(31)
    B, H, N, d = 2, 3, 45, 40
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    q16, k16, v16 = (to_bits(t, BF16) for t in x)
    z = np.zeros((B, H, N), np.float32)
    r = oracle.attention(q16, k16, v16, BF16, qmu=z, kmu=z, want_p8=True)
    assert (r.p8 == 255).all()
    assert np.array_equal(r.l, np.full((B * H, N), float(N)))
    vq, vs = oracle.quant_v(v16, BF16)
    mean = (vq.astype(np.float64).sum(axis=2) * vs.astype(np.float64) / N).reshape(B * H, 1, d)
    assert np.allclose(r.out, np.broadcast_to(mean, r.out.shape), rtol=1e-14, atol=0)
    out_fp, _ = oracle.attention_fp(q16, k16, v16, BF16, qmu=z, kmu=z)
    want_fp = from_bits(v16, BF16).astype(np.float64).mean(axis=2).reshape(B * H, 1, d)
    assert np.allclose(out_fp, np.broadcast_to(want_fp, out_fp.shape), rtol=1e-12, atol=1e-15)


def test_given_mu_matches_scores_from_numpy(oracle_lib):
    """One scalar scale per head (query side c_q, key side c_k): the
    unquantised path is softmax(c_q c_k sign(Q) sign(K)^T / sqrt(d)) V."""
    rng = np.random.default_rng(32)
    B, H, N, d = 1, 3, 37, 72
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    q16, k16, v16 = (to_bits(t, F16) for t in x)
    cq = np.array([0.5, 1.25, 2.0], np.float32)
    ck = np.array([0.75, 1.5, 0.3], np.float32)
    qmu = np.broadcast_to(cq[None, :, None], (B, H, N)).copy()
    kmu = np.broadcast_to(ck[None, :, None], (B, H, N)).copy()
    out, prob = oracle.attention_fp(q16, k16, v16, F16, qmu=qmu, kmu=kmu, want_prob=True)
    qs = signs(from_bits(q16, F16).astype(np.float64))
    ks = signs(from_bits(k16, F16).astype(np.float64))
    S = (cq.astype(np.float64) * ck.astype(np.float64))[None, :, None, None] * (qs @ np.swapaxes(ks, -1, -2)) / np.sqrt(d)
    P = softmax(S, axis=-1)
    O = P @ from_bits(v16, F16).astype(np.float64)
    assert np.allclose(prob.reshape(P.shape), P, rtol=1e-12, atol=1e-15)
    assert np.allclose(out.reshape(O.shape), O, rtol=1e-11, atol=1e-12)


def test_given_mu_invariances(oracle_lib):
    """Passing the per-token scales the oracle computes changes nothing, and
    moving a factor 4 from the key scales to the query scales changes
    nothing either (the products are exact)."""
    rng = np.random.default_rng(33)
    B, H, N, d = 2, 2, 50, 64
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    q16, k16, v16 = (to_bits(t, BF16) for t in x)
    _, qm = oracle.pack(q16, BF16)
    _, km = oracle.pack(k16, BF16)
    r0 = oracle.attention(q16, k16, v16, BF16, want_p8=True)
    r1 = oracle.attention(q16, k16, v16, BF16, qmu=qm, kmu=km, want_p8=True)
    r2 = oracle.attention(q16, k16, v16, BF16, qmu=qm * np.float32(4), kmu=km / np.float32(4), want_p8=True)
    for r in (r1, r2):
        assert np.array_equal(r.p8, r0.p8)
        assert np.array_equal(r.acc, r0.acc)
        assert np.array_equal(r.out_bits, r0.out_bits)
