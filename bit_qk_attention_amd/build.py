"""Build libbinattn.so (the gfx950 C-ABI library) in-tree with hipcc.

    python -m bit_qk_attention_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libbinattn.so")
PROBE_LIB = os.path.join(HERE, "libbaprobe.so")
SOURCES = ["api.hip", "prepass.hip", "attention.hip"]
# attention.hip: fmaxf without NaN canonicalisation (scores are never NaN;
# masked keys are -inf, which stays honoured)
EXTRA = {"attention.hip": ["-fno-honor-nans"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 VALU ops (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    objs = []
    tmpdir = os.path.join(HERE, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = False
    for cmd, pr in procs:
        out, _ = pr.communicate()
        lines = [l for l in out.splitlines() if "not a recognized feature for this target" not in l]
        if pr.returncode != 0 or (verbose and lines):
            print(" ".join(cmd), file=sys.stderr)
            print("\n".join(lines), file=sys.stderr)
        failed |= pr.returncode != 0
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    # the microbenchmarks behind the kernel's design (not the attention path)
    tmp = PROBE_LIB + ".tmp"
    subprocess.run([HIPCC, *FLAGS, "-shared", os.path.join(CSRC, "probe.hip"), "-o", tmp], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
