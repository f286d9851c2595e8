"""The whole forward pass in one launch for short heads
(ba_attention_fwd_qkv16), through the C ABI.

The kernel binarises Q and K and quantises V itself with the arithmetic of
the pre-pass kernels, so the bar is bit-identity with the two-step path
(ba_pack_qk, ba_quant_v, ba_attention_fwd), which the other GPU tests hold
to the oracle; the reduced workloads are also checked against the oracle
directly.
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


def qkv16_out(run, out_dt=None):
    out = torch.empty(run.q.shape, dtype=run.out.dtype if out_dt is None else out_dt, device="cuda")
    ba.ba_attention_fwd_qkv16(run.q, run.k, run.v, run.lib_bias, out)
    torch.cuda.synchronize()
    return out


def same_bits(a, b):
    return a.shape == b.shape and torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", ["deit_small", "dit_256"])
def test_qkv16_reduced_equals_two_step_and_oracle(name):
    run = DeviceRun(make(name, **REDUCED[name]))
    out = qkv16_out(run)
    assert same_bits(out, run.out), name
    check_out(run, out=out, label=name + " (qkv16)")


@pytest.mark.parametrize("name", ["deit_small", "dit_256"])
def test_qkv16_full_size_bit_equal(name):
    run = DeviceRun(make(name))
    assert same_bits(qkv16_out(run), run.out), name


def synth(B, H, N, d, dt, seed, bias="none", grid=(0, 0), n_prefix=0):
    return generate(replace(WORKLOADS["deit_small"], name=f"qkv16_d{d}_n{N}", B=B, H=H, N=N, d=d, dtype=dt,
                            seed=seed, bias=bias, grid=grid, n_prefix=n_prefix, channel_scale=True))


def relpos_grid(N, prefix):
    """A grid of width 16 (narrower for few tokens) after `prefix` leading
    tokens; the tokens past its last full row join the leading ones."""
    gw = 16 if N >= 32 else 4 if N >= 8 else 1
    gh = (N - prefix) // gw
    if gh < 1:
        return (N, 1), 0
    return (gh, gw), N - gh * gw


# every head-dim class of the resident mode (d % 8 == 0, one to three
# 32-channel blocks, one or two fp4 k-steps), one to four key tiles with
# ragged ends, every bias kind it takes (relative position with and without
# leading tokens), both input types, fp16 output from bf16 input
CASES = []
for i, d in enumerate([8, 16, 24, 40, 64, 72, 96]):
    for j, N in enumerate([1, 33, 64, 100, 200, 256]):
        CASES.append((d, N, ["none", "relpos", "dense", "relpos0"][(i + j) % 4], (i + j) % 2))


@pytest.mark.parametrize("d,N,kind,alt", CASES)
def test_qkv16_shapes_bit_equal(d, N, kind, alt):
    dt = F16 if alt else BF16
    kw = {}
    if kind == "dense":
        if N % 4:
            N += 4 - N % 4  # 16-byte fp32 bias rows
        kw = dict(bias="dense_f32")
    elif kind.startswith("relpos"):
        grid, npre = relpos_grid(N, 0 if kind == "relpos0" else 1)
        kw = dict(bias="relpos", grid=grid, n_prefix=npre)
    inp = synth(2, 3, N, d, dt, 9000 + 31 * d + N, **kw)
    out_dt = F16 if (dt == BF16 and N % 2 == 1) else None
    run = DeviceRun(inp, out_dt=out_dt)
    assert same_bits(qkv16_out(run), run.out), (d, N, kind, alt)


def test_qkv16_special_values():
    """Signed zeros, subnormals, the largest finite value, an all-zero V
    channel and key magnitudes far apart (float64 sums of |x| that are not
    exact): signs, scales and int8 V formed inside the kernel equal the
    pre-pass's, seen through the output."""
    for dt in (BF16, F16):
        inp = synth(1, 2, 200, 72, dt, 77 + dt)
        k, v = inp.k, inp.v
        k[0, 0, 3, :] = 0x8000                    # -0 everywhere
        k[0, 1, 7, :] = 0x8001                    # negative subnormals
        v[0, 0, :, 5] = 0x0000                    # an all-zero channel (scale 0)
        v[0, 1, :, 9] = 0x8000                    # an all -0 channel
        if dt == BF16:
            k[0, 0, 4, 5] = 0x5D80                # 2^60 beside 4.0: inexact float64 sums
            k[0, 0, 4, 6:70] = 0x4080
            v[0, 0, 11, 2] = 0x7F7F               # largest finite bf16
        else:
            k[0, 0, 4, :8] = 0x7BFF               # largest finite fp16
            v[0, 1, 13, 0] = 0xFBFF
        run = DeviceRun(inp)
        assert same_bits(qkv16_out(run), run.out), dt


@pytest.mark.parametrize("shape,bias", [((1, 1, 257, 64), "none"), ((1, 1, 128, 128), "none"),
                                         ((1, 1, 128, 20), "none"), ((1, 2, 128, 72), "dense_f16"),
                                         ((1, 2, 197, 64), "dense_f32"), ((1, 2, 144, 40), "relpos_rows")])
def test_qkv16_unsupported(shape, bias):
    """Outside the resident mode the call refuses and enqueues nothing."""
    B, H, N, d = shape
    kw = dict(bias=bias)
    if bias == "relpos_rows":  # grid rows of 16 keys, no leading token, 33..64 channels
        kw = dict(bias="relpos", grid=(N // 16, 16), n_prefix=0)
    run = DeviceRun(synth(B, H, N, d, BF16, 5, **kw))
    out = torch.full_like(run.out, 7.0)
    with pytest.raises(ba.BinAttnError) as e:
        ba.ba_attention_fwd_qkv16(run.q, run.k, run.v, run.lib_bias, out)
    assert e.value.status == ba.BA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_qkv16_rejects_bad_pointers():
    run = DeviceRun(synth(1, 2, 128, 64, BF16, 6))
    out = torch.empty_like(run.out)
    with pytest.raises(ba.BinAttnError) as e:
        ba.ba_attention_fwd_qkv16(run.q, run.k, run.v, None, run.k)   # output over K
    assert e.value.status == ba.BA_ERR_INVALID_ARG
    big = torch.zeros(run.v.numel() + 8, dtype=run.v.dtype, device="cuda")
    vmis = big[1:1 + run.v.numel()].view(run.v.shape)
    with pytest.raises(ba.BinAttnError) as e:
        ba.ba_attention_fwd_qkv16(run.q, run.k, vmis, None, out)      # V not 16-byte aligned
    assert e.value.status == ba.BA_ERR_INVALID_ARG
    assert np.isfinite(run.out.float().cpu().numpy()).all()


@pytest.mark.parametrize("seed", range(12))
def test_qkv16_random_shapes(seed):
    """Seeded random short heads, dtypes and biases the one-launch form
    takes: its output equals the two-step path's bit for bit, and a second
    call gives the same bits."""
    rng = np.random.default_rng(8484 + seed)
    d = int(rng.choice([8, 16, 24, 32, 40, 48, 56, 64, 72, 80, 88, 96]))
    N = int(rng.integers(1, 257))
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    dt = BF16 if rng.random() < 0.5 else F16
    kind = ["none", "dense", "relpos", "relpos0"][int(rng.integers(0, 4))]
    kw = {}
    if kind == "dense":
        N = max(4, N - N % 4)
        kw = dict(bias="dense_f32")
    elif kind.startswith("relpos"):
        grid, npre = relpos_grid(N, 0 if kind == "relpos0" else 1)
        kw = dict(bias="relpos", grid=grid, n_prefix=npre)
    print(f"qkv16 random {seed}: B={B} H={H} N={N} d={d} dt={dt} bias={kind}", flush=True)
    run = DeviceRun(synth(B, H, N, d, dt, 300 + seed, **kw))
    if kind.startswith("relpos") and kw["n_prefix"] == 0 and kw["grid"][1] % 16 == 0 and 32 < d <= 64:
        # grid-run relative position at 33..64 channels: no resident form
        with pytest.raises(ba.BinAttnError) as e:
            qkv16_out(run)
        assert e.value.status == ba.BA_ERR_UNSUPPORTED
        return
    out = qkv16_out(run)
    assert same_bits(out, run.out), (seed, B, H, N, d, kind)
    assert same_bits(qkv16_out(run), out), "repeat"


@pytest.mark.parametrize("dt,bias", [(BF16, "none"), (F16, "dense_f32")])
def test_qkv16_largest_resident_shape(dt, bias):
    """The largest head the one-launch form takes (256 tokens, 96 channels:
    four key tiles, three 32-channel blocks) on a grid of 512 heads, with and
    without a dense fp32 bias: the two-step path's bits."""
    print(f"qkv16 largest: B=32 H=16 N=256 d=96 dt={dt} bias={bias}", flush=True)
    run = DeviceRun(synth(32, 16, 256, 96, dt, 4321 + dt, bias=bias))
    out = qkv16_out(run)
    assert same_bits(out, run.out), (dt, bias)
