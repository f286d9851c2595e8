"""Parity of the gfx950 library with the CPU oracle, through the C ABI.

Bar: sign bits, integer Hamming scores (from every Q.K route of the fused
kernel) and int8 V bit-exact; mu and V scales exact; attention outputs
within 1 ulp of the oracle's rounded output in every row without a near-tie
p8, and within the near-tie bound of tests/parity.py elsewhere; all outputs
also within 2e-2 * max|V| of the oracle and of the unquantised reference
(the bound stated for this method's kernel).
"""
import numpy as np
import pytest
import torch

import bit_qk_attention_amd as ba
import oracle
from gpu_helpers import DeviceRun, out_bits, tdtype, to_dev, vmax
from parity import check_output
from workloads import BF16, F16, from_bits, make, to_bits

pytestmark = pytest.mark.gpu
TOL = 2e-2

# reduced versions of every workload: several 64-key tiles and 128-query
# blocks, ragged tails, all bias kinds
REDUCED = {
    "deit_tiny": dict(),
    "deit_small": dict(B=3),
    "dit_256": dict(B=2, H=3),
    "dit_512": dict(B=2, H=2, N=333),
    "long_4k": dict(B=1, H=2, N=700),
    "long_4k_rp": dict(B=1, H=2, N=23 * 29, grid=(23, 29)),
    "long_16k": dict(B=1, H=1, N=1100),
    "long_16k_rp": dict(B=1, H=2, N=1 + 16 * 48, grid=(16, 48), n_prefix=1),
}


def check_out(run, rows=None, label="", out=None, qmu=None, kmu=None):
    """The output of run (or `out`, computed from run's inputs with the given
    scales) against the oracle: the parity bar of tests/parity.py, and
    2e-2 * max|V| against the unquantised reference."""
    inp = run.inp
    s = inp.spec
    out = run.out if out is None else out
    odt = F16 if out.dtype == torch.float16 else BF16
    BH = s.B * s.H
    bh0, nbh, row0, nrows = (0, BH, 0, s.N) if rows is None else rows
    kw = dict(bh0=bh0, nbh=nbh, row0=row0, nrows=nrows, qmu=qmu, kmu=kmu)
    ref = oracle.attention(inp.q, inp.k, inp.v, s.dtype, bias=run.ora_bias, out_dtype=odt, want_e255=True, **kw)
    fp, _ = oracle.attention_fp(inp.q, inp.k, inp.v, s.dtype, bias=run.ora_bias, **kw)
    got_bits = out_bits(out).reshape(BH, s.N, s.d)[bh0:bh0 + nbh, row0:row0 + nrows]
    vq, vs = oracle.quant_v(inp.v, s.dtype)
    vq = vq.reshape(BH, s.N, s.d)[bh0:bh0 + nbh]
    vs = vs.reshape(BH, s.d)[bh0:bh0 + nbh]
    vm = vmax(inp)
    stats = check_output(got_bits, ref, vq, vs, odt, vm, label=label or s.name, loose=TOL)
    e_fp = np.abs(from_bits(got_bits, odt) - fp).max() / vm
    print(f"{label or s.name}: max|gpu-fp|/max|V| = {e_fp:.2e}")
    assert e_fp <= TOL
    return stats


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_prepass_bit_exact(name):
    inp = make(name, **REDUCED[name])
    s = inp.spec
    run = DeviceRun(inp)
    qb, qm = oracle.pack(inp.q, s.dtype)
    kb, km = oracle.pack(inp.k, s.dtype)
    assert np.array_equal(run.qbits.cpu().numpy().view(np.uint32), qb)
    assert np.array_equal(run.kbits.cpu().numpy().view(np.uint32), kb)
    assert np.array_equal(run.qmu.cpu().numpy(), qm)
    assert np.array_equal(run.kmu.cpu().numpy(), km)
    vq, vs = oracle.quant_v(inp.v, s.dtype)
    assert np.array_equal(run.vq.cpu().numpy(), vq)
    assert np.array_equal(run.vscale.cpu().numpy(), vs)


# sigma comes from the fused kernel's own Q.K routes (staged tiles, keys
# straight from global memory, and at 65..96 channels the raw-word route);
# an element on which they disagree would read 0x7FFFFFFF
@pytest.mark.parametrize("name", sorted(REDUCED))
def test_hamming_bit_exact(name):
    inp = make(name, **REDUCED[name])
    s = inp.spec
    run = DeviceRun(inp)
    sig = torch.empty((s.B * s.H, s.N, s.N), dtype=torch.int32, device="cuda")
    ba.ba_debug_hamming_scores(run.qbits, run.kbits, s.d, 0, s.B * s.H, 0, s.N, sig)
    qb, _ = oracle.pack(inp.q, s.dtype)
    kb, _ = oracle.pack(inp.k, s.dtype)
    assert np.array_equal(sig.cpu().numpy(), oracle.hamming(qb, kb, s.d))


# every head dim class (1-4 channel blocks, one or two fp4 k-steps), ragged
# key tiles and 32-key blocks, windows that start and end inside a 128-query
# block
@pytest.mark.parametrize("d", [1, 16, 31, 40, 64, 65, 72, 96, 97, 128])
@pytest.mark.parametrize("N,win", [(333, (0, 333)), (1000, (130, 300)), (64, (63, 1))])
def test_hamming_windows_every_route(d, N, win):
    dt = BF16 if d % 2 == 0 else F16
    rng = np.random.default_rng(d * 1009 + N)
    x = rng.standard_normal((2, 1, 3, N, d)).astype(np.float32)
    x[0, 0, 1, :5] = 0.0  # zero queries: all bits clear
    q16, k16 = to_bits(x[0], dt), to_bits(x[1], dt)
    qb, _ = oracle.pack(q16, dt)
    kb, _ = oracle.pack(k16, dt)
    qd, kd = to_dev(q16, dt), to_dev(k16, dt)
    qbits, _, kbits, _ = ba.pack_qk(qd, kd)
    r0, nr = win
    sig = torch.empty((2, nr, N), dtype=torch.int32, device="cuda")
    ba.ba_debug_hamming_scores(qbits, kbits, d, 1, 2, r0, nr, sig)
    want = oracle.hamming(qb, kb, d, bh0=1, nbh=2, row0=r0, nrows=nr)
    assert np.array_equal(sig.cpu().numpy(), want)


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_attention_parity(name):
    run = DeviceRun(make(name, **REDUCED[name]))
    check_out(run)


@pytest.mark.parametrize("N", [1, 2, 31, 63, 64, 65, 127, 128, 129, 200])
def test_token_counts(N):
    run = DeviceRun(make("long_4k", B=1, H=2, N=N))
    check_out(run, label=f"N={N}")


@pytest.mark.parametrize("d", [1, 5, 16, 31, 32, 33, 48, 63, 64, 65, 72, 80, 96, 100, 127, 128])
def test_head_dims(d):
    dt_name = "deit_tiny" if d % 2 else "dit_256"
    run = DeviceRun(make(dt_name, B=1, H=2, N=150, d=d))
    check_out(run, label=f"d={d}")


def test_output_dtype_other_than_input():
    inp = make("dit_256", B=1, H=2, N=100)
    run = DeviceRun(inp, out_dt=F16)
    check_out(run, label="bf16 in, fp16 out")


def test_zero_queries_give_uniform_attention():
    inp = make("long_4k", B=1, H=1, N=90)
    inp.q[...] = 0  # +0: mu = 0 and every score is 0
    run = DeviceRun(inp)
    vq, vs = oracle.quant_v(inp.v, BF16)
    vq = vq.reshape(90, 64).astype(np.float64)
    vs = vs.reshape(64).astype(np.float64)
    want = vs * vq.sum(0) / 90  # p8 = 255 everywhere
    got = run.out_f32().reshape(90, 64)
    assert np.abs(got - want[None]).max() <= 8e-3 * np.abs(want).max() + 1e-6


def test_uniform_keys_closed_form():
    inp = make("dit_256", B=1, H=2, N=200)
    inp.k[:, :, 1:, :] = inp.k[:, :, :1, :]  # every key identical
    run = DeviceRun(inp)
    vq, vs = oracle.quant_v(inp.v, BF16)
    want = vs.reshape(2, 1, 72).astype(np.float64) * vq.reshape(2, 200, 72).sum(1, keepdims=True) / 200
    got = run.out_f32().reshape(2, 200, 72)
    assert np.abs(got - want).max() <= 8e-3 * np.abs(want).max()


def test_per_batch_dense_bias():
    inp = make("dit_512", B=3, H=2, N=150)
    rng = np.random.default_rng(5)
    per_b = (0.5 * rng.standard_normal((3, 2, 150, 150))).astype(np.float32)
    inp.bias_data = per_b.astype(np.float16).view(np.uint16)
    inp.bias_batch_stride = 2 * 150 * 150
    run = DeviceRun(inp)
    check_out(run, label="per-batch dense fp16 bias")


def test_one_hot_bias():
    inp = make("deit_tiny", N=120)
    jstar = np.random.default_rng(3).integers(0, 120, size=(3, 120))
    bias = np.zeros((3, 120, 120), np.float32)
    for h in range(3):
        bias[h, np.arange(120), jstar[h]] = 1e4
    inp.bias_data = bias
    run = DeviceRun(inp)
    vq, vs = oracle.quant_v(inp.v, F16)
    got = run.out_f32().reshape(3, 120, 64)
    for h in range(3):
        want = vq[0, h][jstar[h]].astype(np.float64) * vs[0, h]
        assert np.abs(got[h] - want).max() <= 1e-3 * np.abs(want).max()


def test_relpos_equals_materialised_dense():
    from test_oracle_attention import relpos_dense
    inp = make("deit_small", B=2, H=6)
    run_rp = DeviceRun(inp)
    dense = relpos_dense(inp.bias_data, 14, 14, 1)
    inp2 = make("deit_small", B=2, H=6)
    inp2.bias_kind, inp2.bias_data, inp2.bias_dtype, inp2.bias_batch_stride = 1, dense, 2, 0
    run_d = DeviceRun(inp2)
    assert torch.equal(run_rp.out, run_d.out)


def test_relpos_grid_rows_equal_materialised_dense():
    """The grid-run relative-position path (no prefix token, grid width a
    multiple of 16: 16 consecutive keys read one reversed table window), at
    the long sequences' real shape (64 x 64 grid, 4096 tokens, d = 64),
    against the same table materialised as a dense fp32 bias."""
    from test_oracle_attention import relpos_dense
    inp = make("long_4k_rp", B=1, H=2)
    run_rp = DeviceRun(inp)
    dense = relpos_dense(inp.bias_data, 64, 64, 0)
    inp2 = make("long_4k_rp", B=1, H=2)
    inp2.bias_kind, inp2.bias_data, inp2.bias_dtype, inp2.bias_batch_stride = 1, dense, 2, 0
    run_d = DeviceRun(inp2)
    assert torch.equal(run_rp.out, run_d.out)
    check_out(run_rp, rows=(0, 2, 2040, 16), label="grid rows, sampled")


def test_deterministic():
    run = DeviceRun(make("dit_512", B=2, H=2, N=300))
    assert torch.equal(run.out, run.rerun())


def test_key_permutation():
    inp = make("long_4k", B=1, H=2, N=257)
    run0 = DeviceRun(inp)
    perm = np.random.default_rng(9).permutation(257)
    inp.k = np.ascontiguousarray(inp.k[:, :, perm])
    inp.v = np.ascontiguousarray(inp.v[:, :, perm])
    run1 = DeviceRun(inp)
    # the same scores per key and integer sums: the same bits
    assert torch.equal(run0.out, run1.out)


# V quantisation over the launch shapes the library chooses between: whole
# rows per block, channel groups of several or one 16-byte piece (with a
# shorter last group), heads at the register-resident row limit, and the
# two-pass column-group kernel beyond it or for d % 8 != 0; many short heads
# share a block (8, 4 and 2 heads per block, the last block part empty)
@pytest.mark.parametrize("B,H,N,d", [
    (1, 1, 1, 8), (2, 3, 5, 72), (1, 2, 1024, 72), (8, 16, 300, 72), (1, 3, 777, 24),
    (1, 1, 16384, 64), (1, 1, 16385, 64), (2, 1, 4096, 128), (1, 2, 50, 20), (3, 1, 2049, 40),
    (5, 103, 77, 64), (3, 97, 200, 72), (1, 131, 250, 128),
    # the register-resident quantiser's last head length (10 rows per thread)
    # and the first one past it
    (1, 4, 1280, 64), (1, 4, 1281, 64), (1, 2, 1130, 72), (1, 2, 1131, 72),
    # heads split over two to four blocks that each take the whole head's
    # maxima (head counts not a multiple of the eight XCDs included), and the
    # two-pass split quantiser past four parts
    (2, 3, 1600, 72), (1, 1, 20000, 128), (2, 16, 4096, 64), (1, 4, 1537, 64), (1, 1, 7000, 16),
    (1, 3, 5120, 64), (1, 1, 5121, 64), (3, 5, 2261, 72), (1, 2, 2560, 128), (1, 1, 2561, 128)])
@pytest.mark.parametrize("dt", [F16, BF16])
def test_quant_v_launch_shapes(B, H, N, d, dt):
    rng = np.random.default_rng(B * 1000003 + H * 1009 + N * 13 + d + dt)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    v[..., 0] *= 30.0          # one wide channel
    if d > 3:
        v[..., 3] = 0.0        # an all-zero channel
    bits = to_bits(v, dt)
    vd = to_dev(bits, dt)
    vq, vs = ba.quant_v(vd)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_v(bits, dt)
    assert np.array_equal(vq.cpu().numpy(), rq)
    assert np.array_equal(vs.cpu().numpy(), rs)


# the one-launch pre-pass (and its K/V-only form) at the head lengths that
# select each V path: heads in registers, heads in two to four parts, the
# split quantiser with the zero fill in the packing launch
@pytest.mark.parametrize("B,H,N,d", [(2, 3, 1130, 72), (2, 3, 1600, 72), (1, 3, 5120, 64), (3, 5, 2261, 72),
                                     (1, 1, 5121, 64), (1, 2, 2560, 128), (2, 16, 4096, 64),
                                     # heads one block holds, in two parts (fewer heads than CUs)
                                     (1, 16, 1024, 72), (2, 8, 700, 64), (1, 3, 566, 72), (1, 2, 565, 72)])
@pytest.mark.parametrize("dt", [F16, BF16])
def test_prepass_launch_shapes(B, H, N, d, dt):
    rng = np.random.default_rng(B * 7919 + H * 101 + N * 7 + d + dt)
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    x[2, ..., 0] *= 30.0
    x[2, ..., 3] = 0.0
    q16, k16, v16 = (to_bits(x[i], dt) for i in range(3))
    qd, kd, vd = (to_dev(b, dt) for b in (q16, k16, v16))
    qb, qm, kb, km, vq, vs = ba.prepare(qd, kd, vd)
    kb2, km2, vq2, vs2 = ba.prepare_kv(kd, vd)
    torch.cuda.synchronize()
    rqb, rqm = oracle.pack(q16, dt)
    rkb, rkm = oracle.pack(k16, dt)
    rvq, rvs = oracle.quant_v(v16, dt)
    assert np.array_equal(qb.cpu().numpy().view(np.uint32), rqb) and np.array_equal(qm.cpu().numpy(), rqm)
    for b_, m_, q_, s_ in ((kb, km, vq, vs), (kb2, km2, vq2, vs2)):
        assert np.array_equal(b_.cpu().numpy().view(np.uint32), rkb) and np.array_equal(m_.cpu().numpy(), rkm)
        assert np.array_equal(q_.cpu().numpy(), rvq) and np.array_equal(s_.cpu().numpy(), rvs)


# every bias kind at head dims that select the smaller kernel instantiations
# (one or two 32-channel blocks, one fp4 k-step)
@pytest.mark.parametrize("name,d", [
    ("dit_512", 16), ("dit_512", 48), ("dit_512", 64),  # N = 333: unaligned rows
    ("long_4k_rp", 32), ("long_16k_rp", 24), ("deit_tiny", 40), ("deit_small", 32)])
def test_bias_kinds_small_head_dims(name, d):
    kw = dict(REDUCED[name])
    kw["d"] = d
    run = DeviceRun(make(name, **kw))
    check_out(run, label=f"{name} d={d}")


# the fp16 dense bias with 16-byte aligned rows (N % 8 == 0), the path the
# DiT layers take: whole 64-key tiles, a ragged last tile of 8 keys, every
# instantiation of the channel blocks, a shared and a per-batch bias
@pytest.mark.parametrize("N,d", [(64, 72), (320, 72), (328, 72), (136, 96), (328, 80), (392, 64),
                                 (200, 48), (256, 16), (8, 72)])
def test_dense_f16_aligned_rows(N, d):
    run = DeviceRun(make("dit_512", B=2, H=2, N=N, d=d))
    check_out(run, label=f"fp16 bias N={N} d={d}")


def test_dense_f16_aligned_rows_per_batch():
    run = DeviceRun(make("dit_512", B=3, H=2, N=264, bias_shared=False))
    assert run.inp.bias_batch_stride == 2 * 264 * 264
    check_out(run, label="per-batch fp16 bias, aligned rows")


# the one-call pre-pass: bit-identical to ba_pack_qk + ba_quant_v, on the
# fused single launch (d % 8 == 0, heads within the register-resident
# quantiser) and on its two-launch fallback (long heads, d % 8 != 0)
@pytest.mark.parametrize("B,H,N,d,dt", [
    (8, 16, 1024, 72, BF16), (2, 3, 333, 72, BF16), (1, 1, 1, 8, F16), (3, 2, 197, 64, F16),
    (1, 2, 2000, 64, BF16), (2, 2, 150, 36, F16), (1, 3, 50, 128, BF16),
    (5, 103, 77, 64, F16), (3, 97, 200, 72, BF16)])
def test_pack_qk_quant_v_one_call(B, H, N, d, dt):
    rng = np.random.default_rng(B * 7919 + H * 104729 + N * 31 + d)
    x = rng.standard_normal((3, B, H, N, d)).astype(np.float32)
    x[2, ..., 1] = 0.0
    q, k, v = (to_dev(to_bits(x[i], dt), dt) for i in range(3))
    got = ba.prepare(q, k, v)
    ref = ba.pack_qk(q, k) + ba.quant_v(v)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    qb, qm = oracle.pack(to_bits(x[0], dt), dt)
    vq, vs = oracle.quant_v(to_bits(x[2], dt), dt)
    assert np.array_equal(got[0].cpu().numpy().view(np.uint32), qb)
    assert np.array_equal(got[1].cpu().numpy(), qm)
    assert np.array_equal(got[4].cpu().numpy(), vq)
    assert np.array_equal(got[5].cpu().numpy(), vs)


# sign bits and scales of the special 16-bit values, on the cooperative
# packer (d % 8 == 0: alone and inside the one-call pre-pass) and the
# per-token one: -0 and +0 give bit 0, -inf bit 1, subnormals and the
# largest finite values of either sign; an infinite input gives mu = inf
@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("d", [64, 72, 20])
def test_pack_special_values(dt, d):
    inf, big = (0x7C00, 0x7BFF) if dt == F16 else (0x7F80, 0x7F7F)
    special = np.array([0x0000, 0x8000, 0x0001, 0x8001, big, 0x8000 | big, 0x3C00, 0xBC00], np.uint16)
    rng = np.random.default_rng(d * 7 + dt)
    x = to_bits(rng.standard_normal((2, 3, 50, d)).astype(np.float32), dt)
    flat = x.reshape(-1)
    pos = rng.choice(flat.size, size=flat.size // 4, replace=False)
    flat[pos] = special[rng.integers(0, special.size, pos.size)]
    x[0, 0, 7, :] = 0x8000                       # a token of -0 only: all bits 0, mu 0
    x[0, 1, 9, 3] = inf | 0x8000                 # -inf: bit 1, mu inf
    x[1, 2, 11, d - 1] = inf                     # +inf: bit 0, mu inf
    q = to_dev(x, dt)
    k = to_dev(x[:, ::-1].copy(), dt)
    qb, qm = oracle.pack(x, dt)
    kb, km = oracle.pack(x[:, ::-1].copy(), dt)
    got = ba.pack_qk(q, k)
    torch.cuda.synchronize()
    assert np.array_equal(got[0].cpu().numpy().view(np.uint32), qb)
    assert np.array_equal(got[1].cpu().numpy(), qm)
    assert np.array_equal(got[2].cpu().numpy().view(np.uint32), kb)
    assert np.array_equal(got[3].cpu().numpy(), km)
    assert np.isinf(qm[0, 1, 9]) and qm[0, 0, 7] == 0.0
    if d % 8 == 0:
        both = ba.prepare(q, k, q)
        torch.cuda.synchronize()
        assert np.array_equal(both[0].cpu().numpy().view(np.uint32), qb)
        assert np.array_equal(both[1].cpu().numpy(), qm)
        assert np.array_equal(both[2].cpu().numpy().view(np.uint32), kb)
        assert np.array_equal(both[3].cpu().numpy(), km)


# scales given as inputs (mu is an input of ba_attention_fwd): one scalar per
# head on each side, the per-token values' head mean, against the oracle
# with the same scales; and mu = 0, where every score is the bias alone or 0
@pytest.mark.parametrize("name", ["dit_512", "long_4k", "deit_small"])
def test_given_mu_per_head(name):
    inp = make(name, **REDUCED[name])
    s = inp.spec
    run = DeviceRun(inp)
    qm = run.qmu.mean(dim=2, keepdim=True).expand_as(run.qmu).contiguous()
    km = (0.5 * run.kmu.mean(dim=2, keepdim=True)).expand_as(run.kmu).contiguous()
    out = torch.empty_like(run.out)
    ba.ba_attention_fwd(run.qbits, qm, run.kbits, km, run.vq, run.vscale, run.lib_bias, out)
    torch.cuda.synchronize()
    check_out(run, out=out, qmu=qm.cpu().numpy(), kmu=km.cpu().numpy(), label=f"{name} per-head mu")


def test_given_mu_zero_no_bias():
    inp = make("dit_256", B=2, H=3, N=200)
    s = inp.spec
    run = DeviceRun(inp)
    z = torch.zeros_like(run.qmu)
    out = torch.empty_like(run.out)
    ba.ba_attention_fwd(run.qbits, z, run.kbits, z, run.vq, run.vscale, None, out)
    torch.cuda.synchronize()
    vq, vs = oracle.quant_v(inp.v, s.dtype)
    mean = vq.astype(np.float64).sum(axis=2) * vs.astype(np.float64) / s.N  # [B,H,d]
    got = out.float().cpu().numpy()
    err = np.abs(got - mean[:, :, None, :]).max() / vmax(inp)
    print(f"mu = 0: max|gpu - mean of dequantised V| / max|V| = {err:.2e}")
    assert err <= 4e-3  # one 16-bit rounding of the output


# a seeded sweep over random shapes, dtypes and bias kinds (every kernel
# instantiation family: 1-4 channel blocks, one or two fp4 k-steps, dense
# fp32 / fp16 / per-batch, relative position with and without prefix tokens,
# grid rows that are and are not multiples of 16)
def _random_case(i):
    rng = np.random.default_rng(4242 + i)
    d = int(rng.integers(1, 129))
    bias = ["none", "dense_f32", "dense_f16", "relpos"][i % 4]
    kw = dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), d=d,
              dtype=[F16, BF16][int(rng.integers(0, 2))], seed=9000 + i, bias=bias)
    if bias == "relpos":
        gh = int(rng.integers(2, 12))
        gw = [16, 32][i % 2] if i % 8 < 4 else int(rng.integers(2, 20))
        pre = int(rng.integers(0, 2))
        kw.update(grid=(gh, gw), n_prefix=pre, N=pre + gh * gw)
    else:
        kw["N"] = int(rng.integers(1, 300))
        if bias.startswith("dense"):
            kw["bias_shared"] = bool(rng.integers(0, 2))
    return kw


@pytest.mark.parametrize("i", range(24))
def test_random_shapes(i):
    kw = _random_case(i)
    run = DeviceRun(make("dit_512", **kw))
    check_out(run, label=f"random case {i}: {kw}")
