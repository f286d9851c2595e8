"""The path with Q packed inside the attention (ba_pack_k_quant_v +
ba_attention_fwd_q16), through the C ABI.

Its kernels repeat the packing arithmetic of ba_pack_qk in the attention's
prologue, so the bar is bit-identity with the two-step path (ba_pack_qk,
ba_quant_v, ba_attention_fwd), which the other GPU tests hold to the oracle;
the reduced workloads are also checked against the oracle directly.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import bit_qk_attention_amd as ba
from gpu_helpers import DeviceRun
from test_gpu_parity import REDUCED, check_out
from workloads import BF16, F16, WORKLOADS, generate, make

pytestmark = pytest.mark.gpu


def q16_run(run, out_dt=None):
    """kbits, kmu, vq, vscale from ba_pack_k_quant_v and the output of
    ba_attention_fwd_q16 for the inputs of a DeviceRun."""
    kbits, kmu, vq, vscale = ba.prepare_kv(run.k, run.v)
    out = torch.empty(run.q.shape, dtype=run.out.dtype if out_dt is None else out_dt, device="cuda")
    ba.ba_attention_fwd_q16(run.q, kbits, kmu, vq, vscale, run.lib_bias, out)
    torch.cuda.synchronize()
    return (kbits, kmu, vq, vscale), out


def assert_same(a, b, what):
    assert a.shape == b.shape and torch.equal(a.view(torch.int16) if a.dtype in (torch.float16, torch.bfloat16)
                                              else a, b.view(torch.int16) if b.dtype in (torch.float16,
                                                                                       torch.bfloat16) else b), what


@pytest.mark.parametrize("name", sorted(REDUCED))
def test_q16_equals_two_step_and_oracle(name):
    inp = make(name, **REDUCED[name])
    run = DeviceRun(inp)
    (kbits, kmu, vq, vscale), out = q16_run(run)
    assert torch.equal(kbits, run.kbits) and torch.equal(kmu.view(torch.int32), run.kmu.view(torch.int32))
    assert torch.equal(vq, run.vq) and torch.equal(vscale.view(torch.int32), run.vscale.view(torch.int32))
    assert_same(out, run.out, name)
    check_out(run, out=out, label=name + " (q16)")


def synth(B, H, N, d, dt, seed, bias="none", grid=(0, 0), n_prefix=0):
    """A small seeded input with the recipe of the workloads (other sizes)."""
    return generate(replace(WORKLOADS["long_4k"], name=f"q16_d{d}_n{N}", B=B, H=H, N=N, d=d, dtype=dt, seed=seed,
                            bias=bias, grid=grid, n_prefix=n_prefix))


def relpos_grid(N):
    """A grid of width 16 (one token when N < 16) and the leading tokens
    left off it."""
    gw = 16 if N >= 16 else 1
    gh = N // gw
    return (gh, gw), N - gh * gw


# every head-dim class the q16 form takes (d % 8 == 0: one to four 32-channel
# blocks, one or two fp4 k-steps), the resident mode (N <= 256) and the
# staged and key-split modes, ragged query blocks and key tiles, every bias
# kind (relative position with and without leading tokens), both input
# types, fp16 output from bf16 input
CASES = []
for i, d in enumerate([8, 16, 24, 40, 64, 72, 96, 128]):
    for j, N in enumerate([1, 65, 200, 333]):
        CASES.append((d, N, ["none", "dense", "relpos", "dense"][(i + j) % 4], (i + j) % 2))
CASES += [(64, 256, "relpos", 0), (64, 320, "relpos", 0), (72, 320, "relpos", 1), (128, 512, "relpos", 0)]


@pytest.mark.parametrize("d,N,kind,alt", CASES)
def test_q16_shapes_bit_equal(d, N, kind, alt):
    dt = F16 if alt else BF16
    kw = {}
    if kind == "dense":
        kw = dict(bias="dense_f16" if alt else "dense_f32")
    elif kind == "relpos":
        grid, npre = relpos_grid(N)
        kw = dict(bias="relpos", grid=grid, n_prefix=npre)
    inp = synth(2, 2, N, d, dt, 7000 + 31 * d + N, **kw)
    out_dt = F16 if (dt == BF16 and N % 2 == 1) else None  # fp16 output from bf16 input
    run = DeviceRun(inp, out_dt=out_dt)
    _, out = q16_run(run)
    assert_same(out, run.out, (d, N, kind, alt))


def test_q16_special_values():
    """Signed zeros, subnormals, the largest finite value and magnitudes far
    apart in one query (float64 sums of |x| that are not exact, so their
    order matters): the signs and scales packed in the prologue equal
    ba_pack_qk's, seen through the output."""
    for dt in (BF16, F16):
        inp = synth(1, 2, 130, 72, dt, 99 + dt)
        q = inp.q
        q[0, 0, 3, :] = 0x8000                       # -0 everywhere
        q[0, 1, 7, :] = 0x8001                       # negative subnormals
        if dt == BF16:
            q[0, 0, 4, 5] = 0x5D80                   # 2^60
            q[0, 0, 4, 6:70] = 0x4080                # 4.0 beside it
        else:
            q[0, 0, 4, :8] = 0x7BFF                  # largest finite
        run = DeviceRun(inp)
        _, out = q16_run(run)
        assert_same(out, run.out, dt)


def test_q16_longest_head_and_per_batch_bias():
    """The token limit (65536 keys, the query blocks' last rows) and a dense
    bias given per batch element: still the two-step path's bits."""
    run = DeviceRun(synth(1, 1, 65536, 64, BF16, 12))
    _, out = q16_run(run)
    assert_same(out, run.out, "N=65536")
    run = DeviceRun(generate(replace(WORKLOADS["dit_512"], name="q16_pb", B=3, H=2, N=264, bias_shared=False)))
    assert run.inp.bias_batch_stride == 2 * 264 * 264
    _, out = q16_run(run)
    assert_same(out, run.out, "per-batch bias")


FULL = ["deit_tiny", "deit_small", "dit_256", "dit_512", "long_4k", "long_4k_rp", "long_16k", "long_16k_rp"]


@pytest.mark.parametrize("name", FULL)
def test_q16_full_size_bit_equal(name):
    """At full size, in the launch configuration bench.py times: the q16
    path's output equals the two-step path's, every element."""
    inp = make(name)
    run = DeviceRun(inp)
    _, out = q16_run(run)
    assert_same(out, run.out, name)


def test_q16_rejects():
    """d % 8 != 0 is unsupported; Q misaligned or overlapping the output is
    an invalid argument (nothing is launched)."""
    run = DeviceRun(synth(1, 1, 64, 20, BF16, 3))
    kbits, kmu, vq, vscale = ba.prepare_kv(run.k, run.v)
    out = torch.empty_like(run.out)
    with pytest.raises(ba.BinAttnError) as e:
        ba.ba_attention_fwd_q16(run.q, kbits, kmu, vq, vscale, None, out)
    assert e.value.status == ba.BA_ERR_UNSUPPORTED
    run = DeviceRun(synth(1, 1, 64, 64, BF16, 3))
    kbits, kmu, vq, vscale = ba.prepare_kv(run.k, run.v)
    with pytest.raises(ba.BinAttnError) as e:
        ba.ba_attention_fwd_q16(run.q, kbits, kmu, vq, vscale, None, run.q)
    assert e.value.status == ba.BA_ERR_INVALID_ARG
    big = torch.zeros(run.q.numel() + 8, dtype=run.q.dtype, device="cuda")
    qmis = big[1:1 + run.q.numel()].view(run.q.shape)
    with pytest.raises(ba.BinAttnError) as e:
        ba.ba_attention_fwd_q16(qmis, kbits, kmu, vq, vscale, None, torch.empty_like(run.out))
    assert e.value.status == ba.BA_ERR_INVALID_ARG


@pytest.mark.parametrize("seed", range(12))
def test_q16_random_shapes(seed):
    """Seeded random shapes, dtypes and biases: the q16 path's output equals
    the two-step path's bit for bit, and a second call gives the same bits."""
    rng = np.random.default_rng(4242 + seed)
    d = int(rng.choice([8, 16, 24, 32, 40, 48, 56, 64, 72, 80, 88, 96, 104, 112, 120, 128]))
    N = int(rng.integers(1, 1500))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    dt = BF16 if rng.random() < 0.5 else F16
    kind = ["none", "dense_f32", "dense_f16", "relpos"][int(rng.integers(0, 4))]
    kw = {}
    if kind.startswith("dense"):
        kw = dict(bias=kind)
    elif kind == "relpos":
        grid, npre = relpos_grid(N)
        kw = dict(bias="relpos", grid=grid, n_prefix=npre)
    print(f"q16 random {seed}: B={B} H={H} N={N} d={d} dt={dt} bias={kind}", flush=True)
    run = DeviceRun(synth(B, H, N, d, dt, 100 + seed, **kw))
    _, out = q16_run(run)
    assert_same(out, run.out, (seed, B, H, N, d, kind))
    _, out2 = q16_run(run)
    assert_same(out2, out, "repeat")
