"""Benchmark of the BinaryAttention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME | --all | --block]

One step = the whole hot path over one batch of synthetic input already
resident in HBM, on one stream. By default (--form q16, for d % 8 == 0) it is
ba_pack_k_quant_v (sign bits + scales of K, channel-wise int8 V) and
ba_attention_fwd_q16 (the fused attention, binarising Q in its prologue);
--form two-step, and any d % 8 != 0, time ba_pack_qk_quant_v (Q and K packed,
V quantised: the outputs of ba_pack_qk and ba_quant_v) and ba_attention_fwd.
Both forms give the same output bit for bit; the other one is timed beside
the step under "other_form", and for heads of at most 256 tokens the whole
pass in one launch (ba_attention_fwd_qkv16) under "qkv_in_one_launch".
--form qkv16 times that one launch as the step where it applies (q16
elsewhere), with the q16 form beside it.
The headline value is effective attention throughput 4*B*H*N^2*d / t_step
(d the real head dim), for the DiT-XL/2 512px layer (B=8, H=16, N=1024,
d=72, dense fp16 bias shared over the batch); the same figures for the
64x64-token long sequence (B=2, H=16, N=4096, d=64) ride along under
"secondary". Prints one JSON line (rank 0). --block instead times the
attention block around the kernels (QKV projection on the ROCm BLAS,
BinaryAttention, output projection) at the 64x64-token shape.

Before the W warm-up steps, each measurement runs the step back to back for
--device-warmup seconds (0.3 by default): a fresh MI355X runs the first tens
of milliseconds of sustained load at a lower clock, and the timed steps are
meant to show the rate the device holds under sustained load.

roofline: the fused attention kernel, timed alone with HIP events on the
stream it runs on: achieved = effective ops per launch / mean launch time,
against the int8 MFMA dense peak (5.0 POP/s; the effective op count is the
int8 op count of the P.V and +-1 Q.K products at the real d). traffic: HBM
bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (profiles/), scaled
by a copy-kernel calibration, or null if the kernel source changed since.

cpu_baseline: the CPU oracle (plain C, fp64 softmax) on the host cores, on a
bounded sample of the same workload (leading heads, leading query rows, all
keys), scaled to the same effective-ops unit.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, tera-ops/s
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
# Vector ALU issue peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one lane-op
# per lane per cycle (a wave64 instruction takes 4 cycles on a 16-lane SIMD).
VALU_PEAK_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12  # 39.32 tera lane-ops/s


def valu_ops_per_score(s) -> float:
    """Vector issue slots one score element needs at least, whatever the
    tiling: the score's scaling (sigma * mu_k, then one fma into base-2
    units; one more fma with a bias), one exp2 (a transcendental: two issue
    slots), the u8 conversion, the row-sum add, and half a slot for the row
    maximum (a three-input max takes two elements)."""
    return 6.5 + (1.0 if s.bias != "none" else 0.0)
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "bit_qk_attention_amd", "csrc", "attention.hip")


def kernel_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def algorithmic_bytes(s, form: str = "two-step") -> int:
    """HBM bytes one attention launch must move at minimum: packed Q (16-bit
    Q for the q16 form) and packed K (bits + scale), int8 V + channel scales,
    the output, and the bias (a shared dense bias once, not per batch
    element; a relative-position table)."""
    W = (s.d + 31) // 32
    BH, N, d = s.B * s.H, s.N, s.d
    q_bytes = 2 * BH * N * d if form in ("q16", "qkv16") else BH * N * (4 * W + 4)
    if form == "qkv16":  # 16-bit K and V, nothing packed in HBM
        nb = q_bytes + 2 * 2 * BH * N * d + 2 * BH * N * d
    else:
        nb = q_bytes + BH * N * (4 * W + 4) + BH * N * d + 4 * BH * d + 2 * BH * N * d
    if s.bias.startswith("dense"):
        esz = 4 if s.bias == "dense_f32" else 2
        nb += (1 if s.bias_shared else s.B) * s.H * N * N * esz
    elif s.bias == "relpos":
        gh, gw = s.grid
        nb += s.H * (2 * gh - 1) * (2 * gw - 1) * 4
    return nb


def prepass_bytes(s) -> int:
    """HBM bytes the pre-pass (ba_pack_qk_quant_v) must move: Q, K and V read
    once (16-bit), sign words and scales of Q and K, int8 V and the channel
    scales written."""
    W = (s.d + 31) // 32
    BH, N, d = s.B * s.H, s.N, s.d
    return 3 * 2 * BH * N * d + 2 * BH * N * (4 * W + 4) + BH * N * d + 4 * BH * d


def traffic_for(name: str, form: str = "two-step"):
    """Measured HBM bytes per attention launch of the form, if the counters
    were taken on the current kernel source."""
    pre = {"q16": "q16_", "qkv16": "qkv16_"}.get(form, "")
    path = os.path.join(PROFILE_DIR, f"attn_fwd_{pre}{name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, target_s: float = 12.0):
    """Time the oracle on a bounded sample: leading heads and query rows."""
    import oracle
    import numpy as np
    s = inp.spec
    ob = None
    if inp.bias_kind == 1:
        ob = oracle.Bias(oracle.BIAS_DENSE, inp.bias_data, inp.bias_dtype, inp.bias_batch_stride)
    elif inp.bias_kind == 2:
        ob = oracle.Bias(oracle.BIAS_RELPOS, inp.bias_data, oracle.F32, 0, inp.grid_h, inp.grid_w, inp.n_prefix)
    # calibrate on a small slice, then size the sample to ~target_s
    rows = min(s.N, 64)
    t0 = time.perf_counter()
    oracle.attention(inp.q, inp.k, inp.v, s.dtype, bias=ob, bh0=0, nbh=1, row0=0, nrows=rows)
    per_row = (time.perf_counter() - t0) / rows
    total_rows = max(1, int(target_s / max(per_row, 1e-9)))
    nbh = max(1, min(s.B * s.H, total_rows // s.N))
    nrows = s.N if total_rows >= s.N else total_rows
    t0 = time.perf_counter()
    oracle.attention(inp.q, inp.k, inp.v, s.dtype, bias=ob, bh0=0, nbh=nbh, row0=0, nrows=nrows)
    dt = time.perf_counter() - t0
    reps = 1
    if nbh == s.B * s.H and nrows == s.N and dt < target_s / 2:
        # the whole workload is a short sample: repeat it to about target_s
        reps = max(1, int(target_s / max(dt, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.attention(inp.q, inp.k, inp.v, s.dtype, bias=ob, bh0=0, nbh=nbh, row0=0, nrows=nrows)
        dt = time.perf_counter() - t0
    ops = 4.0 * nbh * nrows * s.N * s.d * reps
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS (effective)",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{nbh} head(s) x {nrows} query rows x all {s.N} keys of {s.name}"
                      f"{f' (whole workload, {reps} times)' if reps > 1 else ''} "
                      f"(pack + quantise + attention), {dt:.1f} s"}


class Workload:
    """Device-resident inputs and outputs of one workload."""

    def __init__(self, name: str):
        import numpy as np
        import torch
        import bit_qk_attention_amd as ba
        import workloads
        self.ba, self.torch = ba, torch
        self.inp = inp = workloads.make(name)
        s = self.spec = inp.spec
        tdt = torch.float16 if s.dtype == workloads.F16 else torch.bfloat16

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()

        self.q, self.k, self.v = dev(inp.q), dev(inp.k), dev(inp.v)
        self.bias = None
        if inp.bias_kind == workloads.BIAS_DENSE:
            if inp.bias_dtype == workloads.F32:
                bt = torch.from_numpy(inp.bias_data).cuda()
            else:
                bt = torch.from_numpy(inp.bias_data.view(np.int16)).view(torch.float16).cuda()
            self.bias = ba.Bias(ba.BA_BIAS_DENSE, bt, inp.bias_batch_stride)
        elif inp.bias_kind == workloads.BIAS_RELPOS:
            bt = torch.from_numpy(inp.bias_data).cuda()
            self.bias = ba.Bias(ba.BA_BIAS_RELPOS, bt, 0, inp.grid_h, inp.grid_w, inp.n_prefix)
        B, H, N, d = s.B, s.H, s.N, s.d
        W = ba.ba_packed_words(d)
        self.qbits = torch.empty((B, H, N, W), dtype=torch.int32, device="cuda")
        self.kbits = torch.empty_like(self.qbits)
        self.qmu = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        self.kmu = torch.empty_like(self.qmu)
        self.vq = torch.empty((B, H, N, d), dtype=torch.int8, device="cuda")
        self.vscale = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
        self.out = torch.empty_like(self.q)
        self.stream = torch.cuda.current_stream()

    def step(self):
        self.prepass()
        self.attn()

    def prepass(self):
        self.ba.ba_pack_qk_quant_v(self.q, self.k, self.v, self.qbits, self.qmu, self.kbits, self.kmu,
                                   self.vq, self.vscale, self.stream)

    def prepass_kv(self):
        self.ba.ba_pack_k_quant_v(self.k, self.v, self.kbits, self.kmu, self.vq, self.vscale, self.stream)

    def attn(self):
        self.ba.ba_attention_fwd(self.qbits, self.qmu, self.kbits, self.kmu, self.vq, self.vscale,
                                 self.bias, self.out, self.stream)

    def step_q16(self):
        """The same pass with Q packed inside the attention: ba_pack_k_quant_v
        (K signs and scales, int8 V) and ba_attention_fwd_q16."""
        self.prepass_kv()
        self.attn_q16()

    def attn_q16(self):
        self.ba.ba_attention_fwd_q16(self.q, self.kbits, self.kmu, self.vq, self.vscale, self.bias, self.out,
                                     self.stream)

    def step_qkv16(self):
        """The whole pass in one launch (ba_attention_fwd_qkv16; short heads only)."""
        self.ba.ba_attention_fwd_qkv16(self.q, self.k, self.v, self.bias, self.out, self.stream)

    def attn_online(self):
        self.ba.ba_attention_fwd_online(self.qbits, self.qmu, self.kbits, self.kmu, self.vq, self.vscale,
                                        self.bias, self.out, self.stream)

    def time(self, fn, iters: int, warmup: int) -> float:
        """Mean ms per call of fn over `iters` calls, HIP events on the stream."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(iters):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    def time_cold(self, fn, calls: int = 12) -> float:
        """Median ms of single calls of fn, each after a 512 MB device write
        that evicts L2 and the 256 MB MALL (inputs come from HBM)."""
        torch = self.torch
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        times = []
        for i in range(calls):
            scratch.fill_(i & 0xFF)
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del scratch
        times = sorted(times[2:])
        return times[len(times) // 2]


def device_warmup(fn, seconds: float) -> int:
    """Run fn back to back for `seconds` of wall time (synchronising every ten
    calls). A fresh MI355X runs the first tens of milliseconds of sustained
    load at a lower clock (DiT-512: 87.6 us per step after 5 warm-up steps,
    77.7 us after 1000); this brings it to the clock it holds under sustained
    load before the W warm-up steps and the timed ones. Returns the calls."""
    torch = __import__("torch")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        n += 10
    return n


def step_form(s, form: str) -> str:
    """The form timed for a workload: q16 needs d % 8 == 0."""
    return "q16" if form == "q16" and s.d % 8 == 0 else "two-step"


def qkv16_applies(w) -> bool:
    """Whether ba_attention_fwd_qkv16 takes the workload (one trial call)."""
    try:
        w.step_qkv16()
    except w.ba.BinAttnError as e:
        if e.status != w.ba.BA_ERR_UNSUPPORTED:
            raise
        return False
    return True


def measure(name: str, steps: int, warmup: int, cold: bool = False, device_warmup_s: float = 0.3,
            alt: bool = True, form: str = "q16") -> dict:
    """form: "q16" (ba_pack_k_quant_v + ba_attention_fwd_q16, where d % 8 ==
    0), "two-step" (ba_pack_qk_quant_v + ba_attention_fwd) or "qkv16"
    (ba_attention_fwd_qkv16 alone, where it applies; else q16) is the step
    timed; alt: also time the other form and the one-launch pass."""
    import workloads
    torch = __import__("torch")
    w = Workload(name)
    s = w.spec
    ops = workloads.eff_ops(s)
    if form == "qkv16" and not qkv16_applies(w):
        form = "q16"
    if form != "qkv16":
        form = step_form(s, form)
    step_fn, attn_fn = {"two-step": (w.step, w.attn), "q16": (w.step_q16, w.attn_q16),
                        "qkv16": (w.step_qkv16, w.step_qkv16)}[form]
    dev_warm = device_warmup(step_fn, device_warmup_s)
    # whole step, bracketed by synchronisation on both sides
    for _ in range(warmup):
        step_fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(w.stream)
    for _ in range(steps):
        step_fn()
    e1.record(w.stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    step_ms = e0.elapsed_time(e1) / steps
    # the dominant kernel alone: median (and min) of five runs of back-to-back
    # launches, and the median of single launches with cold caches
    runs = sorted(w.time(attn_fn, iters=max(steps, 20), warmup=3 if i == 0 else 0) for i in range(5))
    attn_ms = runs[2]
    # the pre-pass alone (HBM-bound), same protocol; the one-launch form has none
    pre_ms = None
    if form != "qkv16":
        pre_fn = w.prepass if form == "two-step" else w.prepass_kv
        pre_ms = sorted(w.time(pre_fn, iters=max(steps, 20), warmup=3) for _ in range(3))[1]
    # the other form of the step (where both apply), same protocol, right
    # after the step's own runs (before the cold-cache launches)
    other = None
    if alt and s.d % 8 == 0:
        o_form = "two-step" if form == "q16" else "q16"
        o_step, o_attn = (w.step, w.attn) if o_form == "two-step" else (w.step_q16, w.attn_q16)
        device_warmup(o_step, min(device_warmup_s, 0.1))
        other = {"form": o_form,
                 "step_ms": sorted(w.time(o_step, iters=steps, warmup=warmup) for _ in range(3))[1],
                 "attn_ms": sorted(w.time(o_attn, iters=max(steps, 20), warmup=3) for _ in range(3))[1]}
    # the whole pass in one launch where it applies (heads of at most 256 tokens)
    qkv16_ms = None
    if alt and form != "qkv16" and qkv16_applies(w):
        device_warmup(w.step_qkv16, min(device_warmup_s, 0.1))
        qkv16_ms = sorted(w.time(w.step_qkv16, iters=steps, warmup=warmup) for _ in range(3))[1]
    attn_cold_ms = w.time_cold(attn_fn) if cold else None
    # the one-pass (running maximum) form beside it, d <= 64
    online_ms = None
    if s.d <= 64:
        if form != "two-step":
            w.prepass()  # (the packed queries the one-pass form reads)
        online_ms = sorted(w.time(w.attn_online, iters=max(steps, 20), warmup=3) for _ in range(3))[1]
    step_fn()  # leave the step's output in place
    nbytes = algorithmic_bytes(s, form)
    return {
        "name": name, "spec": s, "form": form, "ops": ops, "step_ms": step_ms, "wall_ms": wall_ms,
        "device_warmup": {"seconds": device_warmup_s, "steps": dev_warm},
        "attn_ms": attn_ms, "attn_min_ms": runs[0], "attn_cold_ms": attn_cold_ms, "online_ms": online_ms,
        "other": other, "pre_ms": pre_ms, "qkv16_ms": qkv16_ms,
        "tops": ops / (step_ms * 1e-3) / 1e12,
        "attn_tops": ops / (attn_ms * 1e-3) / 1e12,
        "attn_gbs": nbytes / (attn_ms * 1e-3) / 1e9, "alg_bytes": nbytes, "inp": w.inp,
        "scores": s.B * s.H * s.N * s.N,
        "valu_tops": s.B * s.H * s.N * s.N * valu_ops_per_score(s) / (attn_ms * 1e-3) / 1e12,
    }


def measure_block(steps: int, warmup: int, B=2, N=4096, H=16, d=64, device_warmup_s: float = 0.3) -> dict:
    """The attention block (QKV projection -> BinaryAttention -> output
    projection) at the 64x64-token shape with synthetic bf16 weights: time per
    block (HIP events, back-to-back blocks), the attention call alone on the
    block's strided views, and on dense copies of them."""
    import torch
    from bit_qk_attention_amd.block import attention_block, split_heads
    import bit_qk_attention_amd as ba
    C = H * d
    g = torch.Generator().manual_seed(1234)
    bf = torch.bfloat16
    x = torch.randn(B, N, C, generator=g).to(bf).cuda()
    w_qkv = (torch.randn(C, 3 * C, generator=g) / C ** 0.5).to(bf).cuda()
    b_qkv = (0.1 * torch.randn(3 * C, generator=g)).to(bf).cuda()
    w_out = (torch.randn(C, C, generator=g) / C ** 0.5).to(bf).cuda()
    b_out = (0.1 * torch.randn(C, generator=g)).to(bf).cuda()
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    device_warmup(lambda: attention_block(x, w_qkv, b_qkv, w_out, b_out, H), device_warmup_s)
    block_ms = timed(lambda: attention_block(x, w_qkv, b_qkv, w_out, b_out, H))
    qkv = torch.addmm(b_qkv, x.view(B * N, C), w_qkv).view(B, N, 3 * C)
    q, k, v = split_heads(qkv, H)  # strided head views of the projection output
    o = torch.empty(B, N, H, d, dtype=bf, device=x.device)
    attn_ms = timed(lambda: ba.attention(q, k, v, out=o.transpose(1, 2)))
    qc, kc, vc = q.contiguous(), k.contiguous(), v.contiguous()
    attn_dense_ms = timed(lambda: ba.attention(qc, kc, vc))
    gemm_ms = timed(lambda: torch.addmm(b_qkv, x.view(B * N, C), w_qkv)) + \
        timed(lambda: torch.addmm(b_out, x.view(B * N, C), w_out))
    return {"B": B, "N": N, "H": H, "d": d, "C": C, "block_ms": block_ms, "attn_ms": attn_ms,
            "attn_dense_inputs_ms": attn_dense_ms,
            "gemm_ms": gemm_ms, "tokens_per_s": B * N / (block_ms * 1e-3),
            "attn_ops": 4.0 * B * H * N * N * d, "gemm_flops": 2.0 * B * N * C * 4 * C}


def prepass_line(r, form: str):
    """The pre-pass launch against the HBM roofline (it moves each input and
    output once and does little arithmetic); None for the one-launch form."""
    if form == "qkv16":
        return None
    s = r["spec"]
    nb = prepass_bytes(s)
    if form != "two-step":  # K and V only
        W = (s.d + 31) // 32
        nb -= 2 * s.B * s.H * s.N * s.d + s.B * s.H * s.N * (4 * W + 4)
    gbs = nb / (r["pre_ms"] * 1e-3) / 1e9
    return {"call": "ba_pack_qk_quant_v" if form == "two-step" else "ba_pack_k_quant_v",
            "ms": round(r["pre_ms"], 5), "bound": "hbm", "alg_bytes": nb, "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "note": "algorithmic bytes (16-bit Q, K, V read; packed and quantised outputs written) / launch "
                    "time (HIP events, back-to-back launches, median of 3 runs)"}


def config_of(s) -> dict:
    bias = {"none": "none", "dense_f32": "dense fp32 [H,N,N]", "dense_f16": "dense fp16 [H,N,N]",
            "relpos": f"relative-position table fp32 [H,{(2 * s.grid[0] - 1) * (2 * s.grid[1] - 1)}]"}[s.bias]
    if s.bias.startswith("dense") and s.bias_shared:
        bias += " shared over batch"
    return {"workload": s.name, "B": s.B, "H": s.H, "N": s.N, "d": s.d,
            "io_dtype": "fp16" if s.dtype == 0 else "bf16", "bias": bias, "about": s.about}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dit_512")
    ap.add_argument("--secondary", default="long_4k")
    ap.add_argument("--all", action="store_true", help="one line per workload (no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--device-warmup", type=float, default=0.3, metavar="SECONDS",
                    help="wall time of back-to-back steps run before the W warm-up steps, so the timed "
                         "steps run at the clock the GPU holds under sustained load (0 to skip)")
    ap.add_argument("--form", choices=["q16", "two-step", "qkv16"], default="q16",
                    help="the step timed: q16 (ba_pack_k_quant_v + ba_attention_fwd_q16: Q binarised inside the "
                         "attention; the default, where d %% 8 == 0), two-step (ba_pack_qk_quant_v + "
                         "ba_attention_fwd) or qkv16 (ba_attention_fwd_qkv16 alone, heads of at most 256 tokens; "
                         "q16 elsewhere)")
    ap.add_argument("--no-alt", action="store_true",
                    help="do not time the other form or the one-launch pass beside the step (the two forms' "
                         "attention launches share one kernel name in a profile)")
    ap.add_argument("--block", action="store_true",
                    help="only the attention block (QKV projection, BinaryAttention, output "
                         "projection) at B=2, N=4096, 16 heads of 64, synthetic bf16 weights")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (read BYTES, write BYTES) five "
                         "times: the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path "
              "(the attention shards by head with no communication)", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes 4n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n}))
        return 0
    if args.block:
        r = measure_block(args.steps, args.warmup, device_warmup_s=args.device_warmup)
        print(json.dumps({
            "metric": "attention block tokens/s (QKV projection + BinaryAttention + output projection)",
            "value": round(r["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(r["block_ms"], 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16 GEMMs, int8 attention",
            "data": "synthetic (seeded N(0,1) activations, N(0,1/C) weights)",
            "config": {"workload": "attention_block_64x64_tokens", "B": r["B"], "N": r["N"], "H": r["H"],
                       "d": r["d"], "C": r["C"]},
            "attn_ms": round(r["attn_ms"], 5), "attn_dense_inputs_ms": round(r["attn_dense_inputs_ms"], 5),
            "gemm_ms": round(r["gemm_ms"], 5), "attn_share": round(r["attn_ms"] / r["block_ms"], 3),
            "gemm_tflops": round(r["gemm_flops"] / (r["gemm_ms"] * 1e-3) / 1e12, 1)}), flush=True)
        return 0
    import workloads
    names = list(workloads.WORKLOADS) if args.all else [args.workload]
    for name in names:
        r = measure(name, args.steps, args.warmup, cold=not args.all, device_warmup_s=args.device_warmup,
                    alt=not args.no_alt, form=args.form)
        s = r["spec"]
        line = {
            "metric": "effective attention TOPS (4*B*H*N^2*d / t_step), step = pack Q/K + quantise V + fused attention",
            "value": round(r["tops"], 3), "unit": "TOPS",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(r["step_ms"], 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "int8",
            "dtype_detail": "Q.K: +-1 signs on fp4 MFMA (exact integer sums); softmax fp32; P.V u8 x int8 -> int32 MFMA",
            "data": "synthetic (seeded N(0,1) activations of the workload's shape)",
            "config": config_of(s),
            "step_form": r["form"],
            "device_warmup": r["device_warmup"],
            "attn_ms": round(r["attn_ms"], 5), "attn_min_ms": round(r["attn_min_ms"], 5),
            "attn_tops": round(r["attn_tops"], 3),
            "roofline": {
                "bound": "alu", "achieved": round(r["valu_tops"], 3), "peak": round(VALU_PEAK_TLANEOPS, 2),
                "unit": "T lane-ops/s", "frac": round(r["valu_tops"] / VALU_PEAK_TLANEOPS, 4),
                "traffic": traffic_for(name, r["form"]),
                "kernel": {"q16": "attn_fwd_kernel (ba_attention_fwd_q16)",
                           "qkv16": "attn_fwd_kernel (ba_attention_fwd_qkv16)"}.get(
                               r["form"], "attn_fwd_kernel (ba_attention_fwd)"),
                "scores_per_launch": r["scores"],
                "lane_ops_per_score": valu_ops_per_score(s),
                "note": "vector-ALU bound: B*H*N^2 scores x the minimum issue slots per score / launch time "
                        "(HIP events on the launch stream; median of 5 runs of back-to-back launches); peak "
                        "256 CUs x 64 lanes x 2.4 GHz; the packing inside the q16 and qkv16 forms is not "
                        "counted as work",
            },
            "int8_mfma": {"achieved": round(r["attn_tops"], 3), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                          "frac": round(r["attn_tops"] / INT8_PEAK_TOPS, 4),
                          "note": "effective ops 4*B*H*N^2*d per launch / launch time"},
            "hbm": {"alg_bytes_per_launch": r["alg_bytes"], "achieved_GBs": round(r["attn_gbs"], 1),
                    "peak_GBs": HBM_PEAK_GBS, "frac": round(r["attn_gbs"] / HBM_PEAK_GBS, 4)},
            "prepass": prepass_line(r, r["form"]),
        }
        if r["attn_cold_ms"] is not None:
            c = r["attn_cold_ms"]
            line["attn_cold"] = {"ms": round(c, 5), "tops": round(r["ops"] / (c * 1e-3) / 1e12, 3),
                                 "hbm_GBs": round(r["alg_bytes"] / (c * 1e-3) / 1e9, 1),
                                 "note": "single launches after a 512 MB write that evicts L2 and the MALL"}
        if r["online_ms"] is not None:
            line["attn_online"] = {"ms": round(r["online_ms"], 5), "vs_two_pass": round(r["online_ms"] / r["attn_ms"], 3),
                                   "note": "ba_attention_fwd_online: one pass over the keys with a running "
                                           "row maximum (same timing protocol)"}
        if r["other"] is not None:
            o = r["other"]
            line["other_form"] = {
                "form": o["form"], "ms_per_step": round(o["step_ms"], 5), "attn_ms": round(o["attn_ms"], 5),
                "value": round(r["ops"] / (o["step_ms"] * 1e-3) / 1e12, 3),
                "note": ("ba_pack_qk_quant_v + ba_attention_fwd" if o["form"] == "two-step" else
                         "ba_pack_k_quant_v + ba_attention_fwd_q16") +
                        " (the same output bit for bit); mean of back-to-back steps, median of 3 runs"}
        if r["qkv16_ms"] is not None:
            line["qkv_in_one_launch"] = {
                "ms_per_step": round(r["qkv16_ms"], 5), "value": round(r["ops"] / (r["qkv16_ms"] * 1e-3) / 1e12, 3),
                "note": "step = ba_attention_fwd_qkv16 alone (Q, K binarised and V quantised inside the "
                        "attention; heads of at most 256 tokens; the same output bit for bit)"}
        if not args.all and args.secondary:
            r2 = measure(args.secondary, args.steps, args.warmup, device_warmup_s=args.device_warmup,
                         alt=not args.no_alt, form=args.form)
            line["secondary"] = {"config": config_of(r2["spec"]), "step_form": r2["form"],
                                 "value": round(r2["tops"], 3),
                                 "ms_per_step": round(r2["step_ms"], 5), "attn_ms": round(r2["attn_ms"], 5),
                                 "attn_online_ms": None if r2["online_ms"] is None else round(r2["online_ms"], 5),
                                 "other_form_ms_per_step": None if r2["other"] is None
                                 else round(r2["other"]["step_ms"], 5),
                                 "attn_tops": round(r2["attn_tops"], 3),
                                 "frac_int8_peak": round(r2["attn_tops"] / INT8_PEAK_TOPS, 4),
                                 "frac_valu_peak": round(r2["valu_tops"] / VALU_PEAK_TLANEOPS, 4)}
        line["cpu_baseline"] = None
        if not args.all and not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline(r["inp"])
        print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
