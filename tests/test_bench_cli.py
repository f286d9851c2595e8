"""bench.py on the host: the one-GPU refusal and the algorithmic byte counts
of each step form, counted here from the sizes of the arrays one launch
reads and writes (the seeded inputs, the packed and quantised buffers the
library's header defines, the output) rather than from bench.py's formula.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def launch_bytes(inp, form):
    """Bytes one attention launch of the form must move, from the arrays."""
    s = inp.spec
    BH, N, d = s.B * s.H, s.N, s.d
    words = (d + 31) // 32
    packed = np.empty((BH, N, words), np.uint32).nbytes + np.empty((BH, N), np.float32).nbytes  # bits + scale
    int8_v = np.empty((BH, N, d), np.int8).nbytes + np.empty((BH, d), np.float32).nbytes         # codes + scales
    out = inp.q.nbytes  # the output has Q's shape and a 16-bit type
    bias = 0 if inp.bias_data is None else inp.bias_data.nbytes
    if form == "qkv16":
        return inp.q.nbytes + inp.k.nbytes + inp.v.nbytes + out + bias
    q_side = inp.q.nbytes if form == "q16" else packed
    return q_side + packed + int8_v + out + bias


@pytest.mark.parametrize("name", ["deit_small", "dit_256", "dit_512", "long_4k_rp"])
@pytest.mark.parametrize("form", ["two-step", "q16", "qkv16"])
def test_algorithmic_bytes(name, form):
    inp = workloads.make(name)
    assert inp.q.dtype == np.uint16 and inp.q.shape == (inp.spec.B, inp.spec.H, inp.spec.N, inp.spec.d)
    assert bench.algorithmic_bytes(inp.spec, form) == launch_bytes(inp, form)


def test_prepass_bytes():
    inp = workloads.make("dit_512")
    s = inp.spec
    BH, N, d = s.B * s.H, s.N, s.d
    words = (d + 31) // 32
    packed = BH * N * words * 4 + BH * N * 4
    expect = inp.q.nbytes + inp.k.nbytes + inp.v.nbytes + 2 * packed + BH * N * d + BH * d * 4
    assert bench.prepass_bytes(s) == expect
