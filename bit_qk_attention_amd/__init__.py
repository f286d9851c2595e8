"""Python binding of the MI355X BinaryAttention library (libbinattn.so).

Argument marshalling only: each ``ba_*`` function here has the name of, and
forwards to, the C entry point declared in ``include/binattn.h``; every step
of the computation runs in the gfx950 kernels. Torch is used for device
memory and streams. There is no CPU fallback: if the library is missing or
the device is not a gfx950 GPU, calls raise.

Build the library in-tree with ``python -m bit_qk_attention_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbinattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "binattn.h")

BA_OK, BA_ERR_INVALID_ARG, BA_ERR_UNSUPPORTED, BA_ERR_HIP = 0, 1, 2, 3
BA_F16, BA_BF16, BA_F32 = 0, 1, 2
BA_BIAS_NONE, BA_BIAS_DENSE, BA_BIAS_RELPOS = 0, 1, 2
BA_MAX_TOKENS = 65536


class BinAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


class ba_bias(ctypes.Structure):
    """Mirror of the C struct ba_bias."""
    _fields_ = [("kind", ctypes.c_int), ("data", ctypes.c_void_p), ("dtype", ctypes.c_int),
                ("batch_stride", ctypes.c_int64), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("n_prefix", ctypes.c_int32)]


class ba_strides(ctypes.Structure):
    """Mirror of the C struct ba_strides (element strides of a [B,H,N,d] view)."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbinattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with `python -m bit_qk_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.ba_packed_words.argtypes = [I]
        L.ba_packed_words.restype = I
        L.ba_pack_qk.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P]
        L.ba_pack_qk.restype = I
        L.ba_quant_v.argtypes = [P, I, I, I, I, I, P, P, P]
        L.ba_quant_v.restype = I
        L.ba_pack_qk_quant_v.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P, P, P, P]
        L.ba_pack_qk_quant_v.restype = I
        L.ba_pack_qk_quant_v_strided.argtypes = [P, P, P, ctypes.POINTER(ba_strides), I, I, I, I, I,
                                                 P, P, P, P, P, P, P]
        L.ba_pack_qk_quant_v_strided.restype = I
        L.ba_attention_fwd.argtypes = [P, P, P, P, P, P, ctypes.POINTER(ba_bias), I, I, I, I, P, I, P]
        L.ba_attention_fwd_online.argtypes = [P, P, P, P, P, P, ctypes.POINTER(ba_bias), I, I, I, I, P, I, P]
        L.ba_attention_fwd.restype = I
        L.ba_attention_fwd_strided.argtypes = [P, P, P, P, P, P, ctypes.POINTER(ba_bias), I, I, I, I, P,
                                               ctypes.POINTER(ba_strides), I, P]
        L.ba_attention_fwd_strided.restype = I
        L.ba_pack_k_quant_v.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P]
        L.ba_pack_k_quant_v.restype = I
        L.ba_attention_fwd_q16.argtypes = [P, I, P, P, P, P, ctypes.POINTER(ba_bias), I, I, I, I, P, I, P]
        L.ba_attention_fwd_q16.restype = I
        L.ba_attention_fwd_qkv16.argtypes = [P, P, P, I, ctypes.POINTER(ba_bias), I, I, I, I, P, I, P]
        L.ba_attention_fwd_qkv16.restype = I
        L.ba_debug_hamming_scores.argtypes = [P, P, I, I, I, I, I, I, I, I, P, P]
        L.ba_debug_hamming_scores.restype = I
        L.ba_status_string.argtypes = [I]
        L.ba_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Names of the functions declared in include/binattn.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ba_[a-z0-9_]+)\s*\(", text)))


def status_string(s: int) -> str:
    return lib().ba_status_string(s).decode()


def _check(fn: str, st: int) -> None:
    if st != BA_OK:
        raise BinAttnError(fn, st, status_string(st))


# --------------------------------------------------------------- torch glue --

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    return {torch.float16: BA_F16, torch.bfloat16: BA_BF16, torch.float32: BA_F32}.get(t.dtype, -1)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        torch = _torch()
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _require_gpu(*ts, contiguous=True):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libbinattn takes device tensors only (no CPU path)")
        if contiguous and t is not None and not t.is_contiguous():
            raise ValueError("libbinattn takes contiguous tensors only")


def view_strides(t) -> ba_strides:
    """(batch, head, token) element strides of a [B,H,N,d] view whose channels
    are contiguous."""
    if t.dim() != 4 or (t.shape[-1] > 1 and t.stride(-1) != 1):
        raise ValueError("a [B,H,N,d] view with contiguous channels is required")
    return ba_strides(t.stride(0), t.stride(1), t.stride(2))


@dataclass
class Bias:
    """Bias description (see ba_bias in include/binattn.h).

    DENSE: ``data`` [H,N,N] (shared over the batch, batch_stride 0) or
    [B,H,N,N] (batch_stride H*N*N), float32 or float16.
    RELPOS: ``data`` float32 [H,(2*grid_h-1)*(2*grid_w-1)].
    """
    kind: int = BA_BIAS_NONE
    data: object = None
    batch_stride: int = 0
    grid_h: int = 0
    grid_w: int = 0
    n_prefix: int = 0

    def to_c(self) -> ba_bias:
        if self.kind == BA_BIAS_NONE or self.data is None:
            return ba_bias(BA_BIAS_NONE, None, BA_F32, 0, 0, 0, 0)
        _require_gpu(self.data)
        return ba_bias(self.kind, self.data.data_ptr(), _dt(self.data), self.batch_stride,
                       self.grid_h, self.grid_w, self.n_prefix)


# ------------------------------------------------------------ entry points --

def ba_packed_words(d: int) -> int:
    return lib().ba_packed_words(d)


def ba_pack_qk(q, k, qbits, qmu, kbits, kmu, stream=None) -> None:
    """q, k [B,H,N,d] fp16/bf16 -> qbits/kbits int32 [B,H,N,W], qmu/kmu float32 [B,H,N]."""
    _require_gpu(q, k, qbits, qmu, kbits, kmu)
    B, H, N, d = q.shape
    _check("ba_pack_qk", lib().ba_pack_qk(_ptr(q), _ptr(k), _dt(q), B, H, N, d, _ptr(qbits), _ptr(qmu),
                                          _ptr(kbits), _ptr(kmu), _stream(stream)))


def ba_quant_v(v, vq, vscale, stream=None) -> None:
    """v [B,H,N,d] fp16/bf16 -> vq int8 [B,H,N,d], vscale float32 [B,H,d]."""
    _require_gpu(v, vq, vscale)
    B, H, N, d = v.shape
    _check("ba_quant_v", lib().ba_quant_v(_ptr(v), _dt(v), B, H, N, d, _ptr(vq), _ptr(vscale),
                                          _stream(stream)))


def ba_pack_qk_quant_v(q, k, v, qbits, qmu, kbits, kmu, vq, vscale, stream=None) -> None:
    """ba_pack_qk and ba_quant_v in one call (same outputs, bit for bit)."""
    _require_gpu(q, k, v, qbits, qmu, kbits, kmu, vq, vscale)
    B, H, N, d = q.shape
    _check("ba_pack_qk_quant_v", lib().ba_pack_qk_quant_v(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), B, H, N, d, _ptr(qbits), _ptr(qmu), _ptr(kbits), _ptr(kmu),
        _ptr(vq), _ptr(vscale), _stream(stream)))


def ba_pack_qk_quant_v_strided(q, k, v, qbits, qmu, kbits, kmu, vq, vscale, stream=None) -> None:
    """ba_pack_qk_quant_v reading q, k, v through [B,H,N,d] views with one
    set of strides (e.g. the head slices of a [B,N,3,H,d] projection)."""
    _require_gpu(q, k, v, contiguous=False)
    _require_gpu(qbits, qmu, kbits, kmu, vq, vscale)
    if not (q.shape == k.shape == v.shape and q.stride() == k.stride() == v.stride()):
        raise ValueError("q, k and v must be views of one shape and one set of strides")
    st = view_strides(q)
    B, H, N, d = q.shape
    _check("ba_pack_qk_quant_v_strided", lib().ba_pack_qk_quant_v_strided(
        _ptr(q), _ptr(k), _ptr(v), ctypes.byref(st), _dt(q), B, H, N, d, _ptr(qbits), _ptr(qmu), _ptr(kbits),
        _ptr(kmu), _ptr(vq), _ptr(vscale), _stream(stream)))


def ba_attention_fwd(qbits, qmu, kbits, kmu, vq, vscale, bias, out, stream=None) -> None:
    """Fused forward; out [B,H,N,d] fp16/bf16 defines the shape and output dtype."""
    _require_gpu(qbits, qmu, kbits, kmu, vq, vscale, out)
    B, H, N, d = out.shape
    cb = (bias or Bias()).to_c()
    _check("ba_attention_fwd", lib().ba_attention_fwd(
        _ptr(qbits), _ptr(qmu), _ptr(kbits), _ptr(kmu), _ptr(vq), _ptr(vscale),
        ctypes.byref(cb), B, H, N, d, _ptr(out), _dt(out), _stream(stream)))


def ba_attention_fwd_online(qbits, qmu, kbits, kmu, vq, vscale, bias, out, stream=None) -> None:
    """The one-pass (running row maximum) form of ba_attention_fwd, d <= 64."""
    _require_gpu(qbits, qmu, kbits, kmu, vq, vscale, out)
    B, H, N, d = out.shape
    cb = (bias or Bias()).to_c()
    _check("ba_attention_fwd_online", lib().ba_attention_fwd_online(
        _ptr(qbits), _ptr(qmu), _ptr(kbits), _ptr(kmu), _ptr(vq), _ptr(vscale),
        ctypes.byref(cb), B, H, N, d, _ptr(out), _dt(out), _stream(stream)))


def ba_attention_fwd_strided(qbits, qmu, kbits, kmu, vq, vscale, bias, out, stream=None) -> None:
    """ba_attention_fwd writing through ``out``, any [B,H,N,d] view with
    contiguous channels (e.g. ``o.transpose(1, 2)`` of an o [B,N,H,d])."""
    _require_gpu(qbits, qmu, kbits, kmu, vq, vscale)
    _require_gpu(out, contiguous=False)
    st = view_strides(out)
    B, H, N, d = out.shape
    cb = (bias or Bias()).to_c()
    _check("ba_attention_fwd_strided", lib().ba_attention_fwd_strided(
        _ptr(qbits), _ptr(qmu), _ptr(kbits), _ptr(kmu), _ptr(vq), _ptr(vscale),
        ctypes.byref(cb), B, H, N, d, _ptr(out), ctypes.byref(st), _dt(out), _stream(stream)))


def ba_pack_k_quant_v(k, v, kbits, kmu, vq, vscale, stream=None) -> None:
    """The K and V half of ba_pack_qk_quant_v (Q is left to ba_attention_fwd_q16)."""
    _require_gpu(k, v, kbits, kmu, vq, vscale)
    B, H, N, d = k.shape
    _check("ba_pack_k_quant_v", lib().ba_pack_k_quant_v(
        _ptr(k), _ptr(v), _dt(k), B, H, N, d, _ptr(kbits), _ptr(kmu), _ptr(vq), _ptr(vscale), _stream(stream)))


def ba_attention_fwd_q16(q, kbits, kmu, vq, vscale, bias, out, stream=None) -> None:
    """ba_attention_fwd with q [B,H,N,d] fp16/bf16 packed inside the kernel (d % 8 == 0)."""
    _require_gpu(q, kbits, kmu, vq, vscale, out)
    B, H, N, d = out.shape
    cb = (bias or Bias()).to_c()
    _check("ba_attention_fwd_q16", lib().ba_attention_fwd_q16(
        _ptr(q), _dt(q), _ptr(kbits), _ptr(kmu), _ptr(vq), _ptr(vscale),
        ctypes.byref(cb), B, H, N, d, _ptr(out), _dt(out), _stream(stream)))


def ba_attention_fwd_qkv16(q, k, v, bias, out, stream=None) -> None:
    """The whole forward pass in one launch for short heads (N <= 256, d % 8 == 0,
    d <= 96): q, k, v [B,H,N,d] fp16/bf16, binarised and quantised inside the kernel."""
    _require_gpu(q, k, v, out)
    B, H, N, d = out.shape
    cb = (bias or Bias()).to_c()
    _check("ba_attention_fwd_qkv16", lib().ba_attention_fwd_qkv16(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), ctypes.byref(cb), B, H, N, d, _ptr(out), _dt(out), _stream(stream)))


def ba_debug_hamming_scores(qbits, kbits, d, bh_begin, bh_count, row_begin, row_count, sigma,
                            stream=None) -> None:
    """sigma int32 [bh_count, row_count, N] = d - 2*popcount(q xor k) over a window."""
    _require_gpu(qbits, kbits, sigma)
    B, H, N, _W = qbits.shape
    _check("ba_debug_hamming_scores", lib().ba_debug_hamming_scores(
        _ptr(qbits), _ptr(kbits), B, H, N, d, bh_begin, bh_count, row_begin, row_count,
        _ptr(sigma), _stream(stream)))


# ------------------------------------------------------------- conveniences --

def pack_qk(q, k, stream=None):
    torch = _torch()
    B, H, N, d = q.shape
    W = ba_packed_words(d)
    qbits = torch.empty((B, H, N, W), dtype=torch.int32, device=q.device)
    kbits = torch.empty_like(qbits)
    qmu = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    kmu = torch.empty_like(qmu)
    ba_pack_qk(q, k, qbits, qmu, kbits, kmu, stream)
    return qbits, qmu, kbits, kmu


def quant_v(v, stream=None):
    torch = _torch()
    B, H, N, d = v.shape
    vq = torch.empty((B, H, N, d), dtype=torch.int8, device=v.device)
    vscale = torch.empty((B, H, d), dtype=torch.float32, device=v.device)
    ba_quant_v(v, vq, vscale, stream)
    return vq, vscale


def prepare(q, k, v, stream=None):
    """Packed Q/K and quantised V of one forward pass, from one call. q, k, v
    are contiguous [B,H,N,d], or views sharing one set of strides."""
    torch = _torch()
    B, H, N, d = q.shape
    W = ba_packed_words(d)
    qbits = torch.empty((B, H, N, W), dtype=torch.int32, device=q.device)
    kbits = torch.empty_like(qbits)
    qmu = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    kmu = torch.empty_like(qmu)
    vq = torch.empty((B, H, N, d), dtype=torch.int8, device=v.device)
    vscale = torch.empty((B, H, d), dtype=torch.float32, device=v.device)
    if q.is_contiguous() and k.is_contiguous() and v.is_contiguous():
        ba_pack_qk_quant_v(q, k, v, qbits, qmu, kbits, kmu, vq, vscale, stream)
    else:
        ba_pack_qk_quant_v_strided(q, k, v, qbits, qmu, kbits, kmu, vq, vscale, stream)
    return qbits, qmu, kbits, kmu, vq, vscale


def attention(q, k, v, bias: Bias | None = None, out=None, stream=None):
    """Whole forward pass: pack Q/K and quantise V (one call), fused attention.
    q, k, v and out may be strided [B,H,N,d] views (see prepare and
    ba_attention_fwd_strided)."""
    torch = _torch()
    qbits, qmu, kbits, kmu, vq, vscale = prepare(q, k, v, stream)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if out.is_contiguous():
        ba_attention_fwd(qbits, qmu, kbits, kmu, vq, vscale, bias, out, stream)
    else:
        ba_attention_fwd_strided(qbits, qmu, kbits, kmu, vq, vscale, bias, out, stream)
    return out


def prepare_kv(k, v, stream=None):
    """Packed K and quantised V (ba_pack_k_quant_v), for attention_q16."""
    torch = _torch()
    B, H, N, d = k.shape
    W = ba_packed_words(d)
    kbits = torch.empty((B, H, N, W), dtype=torch.int32, device=k.device)
    kmu = torch.empty((B, H, N), dtype=torch.float32, device=k.device)
    vq = torch.empty((B, H, N, d), dtype=torch.int8, device=v.device)
    vscale = torch.empty((B, H, d), dtype=torch.float32, device=v.device)
    ba_pack_k_quant_v(k, v, kbits, kmu, vq, vscale, stream)
    return kbits, kmu, vq, vscale


def attention_q16(q, k, v, bias: Bias | None = None, out=None, stream=None):
    """Whole forward pass with Q packed inside the attention: ba_pack_k_quant_v,
    then ba_attention_fwd_q16 (contiguous q, k, v, out; d % 8 == 0). The same
    output as attention(), bit for bit."""
    torch = _torch()
    kbits, kmu, vq, vscale = prepare_kv(k, v, stream)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    ba_attention_fwd_q16(q, kbits, kmu, vq, vscale, bias, out, stream)
    return out
