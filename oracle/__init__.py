"""CPU oracle for the BinaryAttention forward pass (test infrastructure only).

A plain, slow, obviously-correct implementation of what the method computes,
written from the technical summaries of "BinaryAttention: One-Bit
QK-Attention for Vision and Diffusion Transformers" (gist.science pages zh,
nl, it, fr, pt). The arithmetic lives in ``bao_ref.c`` (plain C, OpenMP,
double-precision softmax, host libm ``exp``); this module only marshals numpy
arrays into it.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the GPU library and the GPU
library never imports it.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, brute force on tiny inputs, library routines and invariants; the
quantised output as a whole has no printed worked example on the pages, so
its agreement with the method rests on those pins (see the per-test notes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bao_ref.c")
_LIB = os.path.join(_HERE, "libbao_ref.so")

F16, BF16, F32 = 0, 1, 2
BIAS_NONE, BIAS_DENSE, BIAS_RELPOS = 0, 1, 2
# Row normaliser of the quantised output (see bao_ref.h): the float sum of
# the unquantised probabilities (the library's reading) or the integer row sum
# of the quantised P.
NORM_FLOAT, NORM_P8 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Bias(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("data", ctypes.c_void_p), ("dtype", ctypes.c_int),
                ("batch_stride", ctypes.c_int64), ("grid_h", ctypes.c_int),
                ("grid_w", ctypes.c_int), ("n_prefix", ctypes.c_int)]


@dataclass
class Bias:
    """Bias description mirroring the C struct. ``data`` is a numpy array:
    dense [H,N,N] (or [B,H,N,N] with batch_stride H*N*N) float32/float16 bits,
    relpos [H,(2gh-1)(2gw-1)] float32."""
    kind: int = BIAS_NONE
    data: np.ndarray | None = None
    dtype: int = F32
    batch_stride: int = 0
    grid_h: int = 0
    grid_w: int = 0
    n_prefix: int = 0


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("BAO_REF_LIB")  # a planted-mistake build (tests only)
        if path is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            path = _LIB
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        L.bao_words.argtypes = [I]
        L.bao_decode16.argtypes = [P, I, I64, P]
        L.bao_round16.argtypes = [ctypes.c_double, I]
        L.bao_round16.restype = ctypes.c_uint16
        L.bao_pack.argtypes = [P, I, I64, I, P, P]
        L.bao_quant_v.argtypes = [P, I, I64, I, I, P, P]
        L.bao_hamming.argtypes = [P, P, I, I, I, I, I, I, P]
        L.bao_attention_mu.argtypes = [P, P, P, I, I, I, I, I, ctypes.POINTER(_Bias), P, P, I,
                                       I, I, I, I, I, P, P, P, P, P, P, P]
        L.bao_attention_fp_mu.argtypes = [P, P, P, I, I, I, I, I, ctypes.POINTER(_Bias), P, P,
                                          I, I, I, I, P, P]
        L.bao_num_threads.restype = I
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, "16-bit inputs are passed as raw uint16 bit patterns"
    return x


def words(d: int) -> int:
    return lib().bao_words(d)


def num_threads() -> int:
    return lib().bao_num_threads()


def decode16(x: np.ndarray, dtype: int) -> np.ndarray:
    x = _u16(x)
    out = np.empty(x.shape, np.float32)
    lib().bao_decode16(_ptr(x), dtype, x.size, _ptr(out))
    return out


def round16(x: float, dtype: int) -> int:
    return int(lib().bao_round16(float(x), dtype))


def pack(x: np.ndarray, dtype: int):
    """x: uint16 [..., d] -> (bits uint32 [..., W], mu float32 [...])."""
    x = _u16(x)
    d = x.shape[-1]
    W = words(d)
    ntok = x.size // d
    bits = np.empty(x.shape[:-1] + (W,), np.uint32)
    mu = np.empty(x.shape[:-1], np.float32)
    lib().bao_pack(_ptr(x), dtype, ntok, d, _ptr(bits), _ptr(mu))
    return bits, mu


def quant_v(v: np.ndarray, dtype: int):
    """v: uint16 [B,H,N,d] -> (vq int8 [B,H,N,d], vscale float32 [B,H,d])."""
    v = _u16(v)
    B, H, N, d = v.shape
    vq = np.empty(v.shape, np.int8)
    vs = np.empty((B, H, d), np.float32)
    lib().bao_quant_v(_ptr(v), dtype, B * H, N, d, _ptr(vq), _ptr(vs))
    return vq, vs


def hamming(qbits, kbits, d, bh0=0, nbh=None, row0=0, nrows=None):
    """qbits, kbits: uint32 [B,H,N,W] -> sigma int32 [nbh, nrows, N]."""
    qbits = np.ascontiguousarray(qbits, np.uint32)
    kbits = np.ascontiguousarray(kbits, np.uint32)
    B, H, N, W = qbits.shape
    nbh = B * H - bh0 if nbh is None else nbh
    nrows = N - row0 if nrows is None else nrows
    sig = np.empty((nbh, nrows, N), np.int32)
    lib().bao_hamming(_ptr(qbits), _ptr(kbits), N, d, bh0, nbh, row0, nrows, _ptr(sig))
    return sig


def _cbias(bias: Bias | None):
    if bias is None or bias.kind == BIAS_NONE:
        return _Bias(BIAS_NONE, None, F32, 0, 0, 0, 0), None
    data = np.ascontiguousarray(bias.data)
    if bias.kind == BIAS_DENSE:
        want = np.float32 if bias.dtype == F32 else np.uint16
    else:
        want = np.float32
    assert data.dtype == want, f"bias data must be {want}"
    return _Bias(bias.kind, data.ctypes.data, bias.dtype, bias.batch_stride,
                 bias.grid_h, bias.grid_w, bias.n_prefix), data


@dataclass
class AttnResult:
    out: np.ndarray        # float64 [nbh, nrows, d] before output rounding
    out_bits: np.ndarray   # uint16 [nbh, nrows, d] rounded to the output dtype
    m: np.ndarray          # float64 [nbh, nrows] row max of the scores
    l: np.ndarray          # float64 [nbh, nrows] row normaliser: sum_j exp(s - m) (NORM_FLOAT)
                           # or sum_j p8 / 255 (NORM_P8)
    acc: np.ndarray        # int64 [nbh, nrows, d] integer P.V accumulator
    p8: np.ndarray | None  # uint8 [nbh, nrows, N] quantised probabilities
    e255: np.ndarray | None = None  # float64 [nbh, nrows, N]: 255 * exp(s - m), before rounding


def _mu_arg(mu, shape):
    """A given scale array float32 [B,H,N] (or None: computed per token)."""
    if mu is None:
        return None
    mu = np.ascontiguousarray(mu, dtype=np.float32)
    assert mu.shape == shape[:3], (mu.shape, shape)
    return mu


def attention(q, k, v, dtype, bias: Bias | None = None, bh0=0, nbh=None, row0=0,
              nrows=None, out_dtype=None, want_p8=False, qmu=None, kmu=None,
              norm=NORM_FLOAT, want_e255=False) -> AttnResult:
    """Quantised BinaryAttention forward from raw uint16 Q, K, V [B,H,N,d].

    qmu, kmu: optional given scales float32 [B,H,N] in place of the per-token
    mean |x| (mu is an input of the attention step, e.g. a per-head scalar).
    norm: NORM_FLOAT (l = sum_j exp(s - m)) or NORM_P8 (l = sum_j p8 / 255)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, N, d = q.shape
    qmu, kmu = _mu_arg(qmu, q.shape), _mu_arg(kmu, q.shape)
    assert k.shape == q.shape and v.shape == q.shape
    nbh = B * H - bh0 if nbh is None else nbh
    nrows = N - row0 if nrows is None else nrows
    out_dtype = dtype if out_dtype is None else out_dtype
    out = np.empty((nbh, nrows, d), np.float64)
    bits = np.empty((nbh, nrows, d), np.uint16)
    m = np.empty((nbh, nrows), np.float64)
    l = np.empty((nbh, nrows), np.float64)
    acc = np.empty((nbh, nrows, d), np.int64)
    p8 = np.empty((nbh, nrows, N), np.uint8) if want_p8 else None
    e255 = np.empty((nbh, nrows, N), np.float64) if want_e255 else None
    cb, keep = _cbias(bias)
    rc = lib().bao_attention_mu(_ptr(q), _ptr(k), _ptr(v), dtype, B, H, N, d, ctypes.byref(cb),
                                _ptr(qmu), _ptr(kmu), norm, bh0, nbh, row0, nrows, out_dtype, _ptr(out),
                                _ptr(bits), _ptr(m), _ptr(l), _ptr(p8), _ptr(acc), _ptr(e255))
    del keep
    if rc == -2:
        raise OverflowError("integer P.V accumulator left int32 range")
    if rc != 0:
        raise ValueError(f"bao_attention rejected its arguments (rc={rc})")
    return AttnResult(out, bits, m, l, acc, p8, e255)


def attention_fp(q, k, v, dtype, bias: Bias | None = None, bh0=0, nbh=None, row0=0,
                 nrows=None, want_prob=False, qmu=None, kmu=None):
    """Unquantised reference: (out float64 [nbh,nrows,d], prob or None)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, N, d = q.shape
    qmu, kmu = _mu_arg(qmu, q.shape), _mu_arg(kmu, q.shape)
    nbh = B * H - bh0 if nbh is None else nbh
    nrows = N - row0 if nrows is None else nrows
    out = np.empty((nbh, nrows, d), np.float64)
    prob = np.empty((nbh, nrows, N), np.float64) if want_prob else None
    cb, keep = _cbias(bias)
    rc = lib().bao_attention_fp_mu(_ptr(q), _ptr(k), _ptr(v), dtype, B, H, N, d, ctypes.byref(cb),
                                   _ptr(qmu), _ptr(kmu), bh0, nbh, row0, nrows, _ptr(out), _ptr(prob))
    del keep
    if rc != 0:
        raise ValueError(f"bao_attention_fp rejected its arguments (rc={rc})")
    return out, prob
