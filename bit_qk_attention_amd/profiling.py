"""Summaries of rocprofv3 output for the BinaryAttention kernels.

    # per-kernel time table from a --kernel-trace --stats run
    python -m bit_qk_attention_amd.profiling stats <dir>/..._kernel_stats.csv

    # HBM traffic of one kernel from two --pmc runs (FETCH_SIZE, WRITE_SIZE),
    # calibrated against a plain copy of known size profiled the same way
    python -m bit_qk_attention_amd.profiling traffic --kernel attn_fwd \\
        --fetch <a>/..._counter_collection.csv --write <b>/..._counter_collection.csv \\
        --copy-fetch <c>/... --copy-write <d>/... --copy-bytes N --out file.json

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
    args = ap.parse_args(argv)
    if args.cmd == "probe":
        print(probe())
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
