"""Summaries of rocprofv3 output for the BinaryAttention kernels.

    # per-kernel time table from a --kernel-trace --stats run
    python -m bit_qk_attention_amd.profiling stats <dir>/..._kernel_stats.csv

    # HBM traffic of one kernel from two --pmc runs (FETCH_SIZE, WRITE_SIZE),
    # calibrated against a plain copy of known size profiled the same way
    python -m bit_qk_attention_amd.profiling traffic --kernel attn_fwd \\
        --fetch <a>/..._counter_collection.csv --write <b>/..._counter_collection.csv \\
        --copy-fetch <c>/... --copy-write <d>/... --copy-bytes N --out file.json

    # SQ counter table (two --pmc passes per workload, see profiles/)
    python -m bit_qk_attention_amd.profiling sq <root> <workload> ...

    # instruction issue rates and the three Q.K routes on the GPU
    python -m bit_qk_attention_amd.profiling probe

FETCH_SIZE / WRITE_SIZE are reported in KiB per dispatch. The copy kernel
reads and writes exactly N bytes, so the counter's reading for it gives a
scale factor (N / measured) applied to the kernel's reading.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(_HERE, "csrc", "attention.hip")


def kernel_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        short = name.split("(")[0].replace("void ", "").replace("binattn::", "")
        out.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(out)


def per_dispatch(path: str, kernel: str, counter: str) -> list[float]:
    """Counter value (summed over instances) of each dispatch of `kernel`."""
    acc = collections.defaultdict(float)
    for r in csv.DictReader(open(path)):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            acc[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return [acc[k] for k in sorted(acc)]


def median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2] if xs else float("nan")


def traffic(kernel, fetch, write, copy_fetch, copy_write, copy_bytes, copy_kernel="copy"):
    kf = median(per_dispatch(fetch, kernel, "FETCH_SIZE")) * 1024
    kw = median(per_dispatch(write, kernel, "WRITE_SIZE")) * 1024
    cf = median(per_dispatch(copy_fetch, copy_kernel, "FETCH_SIZE")) * 1024
    cw = median(per_dispatch(copy_write, copy_kernel, "WRITE_SIZE")) * 1024
    f_scale = copy_bytes / cf
    w_scale = copy_bytes / cw
    return {
        "kernel": kernel, "kernel_sha": kernel_sha(),
        "fetch_bytes_raw": kf, "write_bytes_raw": kw,
        "copy_bytes": copy_bytes, "copy_fetch_raw": cf, "copy_write_raw": cw,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "bytes_per_launch": kf * f_scale + kw * w_scale,
    }


# probe modes of libbaprobe.so (csrc/probe.hip): name, loop iterations,
# vector instructions per chain and iteration (rate modes) or None (Q.K modes)
PROBES = [
    ("v_fma_f32", 4096, 1),
    ("v_exp_f32", 2048, 1),
    ("v_add_f32 + v_cvt_pk_u8_f32", 2048, 2),
    ("pass-2 mix: mul, fma, exp, add, cvt, xor", 1024, 6),
    ("sigma by v_xor + v_bcnt (VALU)", 2048, None),
    ("sigma by 2 x v_mfma_i32_32x32x32_i8", 2048, None),
    ("sigma by 1 x v_mfma_scale_f32_32x32x64_f8f6f4 (fp4)", 2048, None),
]


# workload -> (B*H, N): the score count B*H*N^2 of one launch
SQ_SHAPES = {"deit_tiny": (3, 197), "deit_small": (384, 197), "dit_256": (512, 256), "dit_512": (128, 1024),
             "long_4k": (32, 4096), "long_4k_rp": (32, 4096), "long_16k": (32, 16384), "long_16k_rp": (32, 16384)}


def sq_row(workload: str, csv_a: str, csv_b: str, kernel: str = "attn_fwd_kernel") -> tuple[str, dict]:
    """One row of the SQ counter table for the two-pass attention kernel of
    a workload (medians over its dispatches; the one-pass form, MODE 4, is
    left out), from the two counter passes."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for path in (csv_a, csv_b):
        for r in csv.DictReader(open(path)):
            n = r["Kernel_Name"]
            if kernel not in n:
                continue
            inst = n[n.index(kernel):].split(">")[0] + ">"
            if inst.replace(" ", "").split(",")[3] == "4":  # the one-pass extension
                continue
            key = (path, int(r["Dispatch_Id"]))
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
            names[key] = inst
    med = {}
    for c in ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES",
              "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT",
              "SQ_ACTIVE_INST_LDS", "SQ_INSTS_VALU_TRANS_F32", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY"):
        vals = [v[c] for k, v in per.items() if c in v]
        if vals:
            med[c] = median(vals)
    inst = sorted(set(names.values()))
    bh, n = SQ_SHAPES[workload]
    scores = bh * n * n
    T = med["GRBM_GUI_ACTIVE"] / 8  # cycles per XCD
    valu = med["SQ_INSTS_VALU"]
    row = (f"| {workload} | `{', '.join(inst)}` | {T / 2400:.1f} | {64 * valu / scores:.2f} | "
           f"{64 * med['SQ_INSTS_VALU_TRANS_F32'] / scores:.2f} | {4 * valu / (1024 * T):.0%} | "
           f"{4 * (valu + med['SQ_INSTS_VALU_TRANS_F32']) / (1024 * T):.0%} | "
           f"{4 * med['SQ_ACTIVE_INST_VALU'] / (1024 * T):.0%} | {med['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * T):.0%} | "
           f"{4 * med['SQ_WAVE_CYCLES'] / (256 * T):.1f} | {med['SQ_WAIT_INST_ANY'] / med['SQ_WAVE_CYCLES']:.0%} | "
           f"{med['SQ_LDS_BANK_CONFLICT'] / med['SQ_ACTIVE_INST_LDS']:.2f} |")
    return row, med


def sq_table(args) -> str:
    """The SQ counter table: for each workload w, sqa_w/a_counter_collection.csv
    and sqb_w/b_counter_collection.csv under `root`."""
    out = ["| workload | kernel | T (us at 2.4 GHz) | VALU / score | exp / score | VALU issue | with exp | "
           "VALU active | MFMA busy | waves / CU | waiting | LDS conflicts |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    raw = ["| workload | counter | value |", "|---|---|---|"]
    for w in args.workloads:
        row, med = sq_row(w, os.path.join(args.root, f"sqa_{w}", "a_counter_collection.csv"),
                          os.path.join(args.root, f"sqb_{w}", "b_counter_collection.csv"))
        out.append(row)
        raw += [f"| {w} | {c} | {v:.4g} |" for c, v in sorted(med.items())]
    return "\n".join(out) + "\n\nRaw medians:\n\n" + "\n".join(raw)


def probe() -> str:
    """Run every probe mode; a markdown table of the rates."""
    import ctypes
    L = ctypes.CDLL(os.path.join(_HERE, "libbaprobe.so"))
    L.bap_time.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    assert L.bap_count() == len(PROBES)
    waves_per_simd = 2048 * 4 / 1024  # 2048 workgroups of 4 waves on 1024 SIMDs
    out = ["| probe | ms per launch | result |", "|---|---|---|"]
    for mode, (name, iters, ops) in enumerate(PROBES):
        ms = ctypes.c_float()
        rc = L.bap_time(mode, iters, ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"probe {name}: HIP error {rc}")
        if ops is not None:
            per = ms.value * 1e6 / (waves_per_simd * iters * 8 * ops)
            res = f"{per:.2f} ns per wave instruction per SIMD"
        else:
            per = ms.value * 1e6 / (waves_per_simd * iters)
            tops = 2048 * 4 * iters * 1024 * 64 * 2 / (ms.value * 1e-3) / 1e12
            res = f"{per:.1f} ns per 32x32 block per SIMD ({tops:.0f} effective TOPS for the sigma alone)"
        out.append(f"| {name} | {ms.value:.3f} | {res} |")
    return "\n".join(out)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    b = sub.add_parser("traffic")
    b.add_argument("--kernel", required=True)
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--copy-fetch", required=True)
    b.add_argument("--copy-write", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--copy-kernel", default="copy")
    b.add_argument("--out")
    sub.add_parser("probe")
    c = sub.add_parser("sq")
    c.add_argument("root", help="folder holding sqa_<workload>/ and sqb_<workload>/")
    c.add_argument("workloads", nargs="+")
    args = ap.parse_args(argv)
    if args.cmd == "probe":
        print(probe())
        return 0
    if args.cmd == "sq":
        print(sq_table(args))
        return 0
    if args.cmd == "stats":
        print(stats_table(args.csv))
        return 0
    rec = traffic(args.kernel, args.fetch, args.write, args.copy_fetch, args.copy_write,
                  args.copy_bytes, args.copy_kernel)
    text = json.dumps(rec, indent=1)
    if args.out:
        open(args.out, "w").write(text + "\n")
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
