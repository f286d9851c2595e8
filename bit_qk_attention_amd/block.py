"""An attention block around the BinaryAttention kernels: QKV projection,
BinaryAttention, output projection. The pages measure the method end to end
as well as the kernel (zh technical summary section 4, efficiency comparison:
end-to-end throughput at 1024x1024 input; nl Resultaten, speed and
efficiency); this block is the part of a transformer layer that the method
changes, at synthetic weights.

The two projections are plain GEMMs on the ROCm BLAS (``torch.matmul``); the
head split and merge are layout copies. Everything between them — packing Q
and K, quantising V, the fused attention — runs in this library's kernels
through the C ABI.
"""
from __future__ import annotations

from . import Bias, attention


def split_heads(qkv, H: int):
    """[B, N, 3*H*d] -> three contiguous [B, H, N, d] tensors (q, k, v)."""
    B, N, C3 = qkv.shape
    d = C3 // (3 * H)
    t = qkv.view(B, N, 3, H, d).permute(2, 0, 3, 1, 4).contiguous()
    return t[0], t[1], t[2]


def merge_heads(o):
    """[B, H, N, d] -> [B, N, H*d]."""
    B, H, N, d = o.shape
    return o.permute(0, 2, 1, 3).reshape(B, N, H * d)


def attention_block(x, w_qkv, b_qkv, w_out, b_out, H: int, bias: Bias | None = None,
                    stream=None, keep=None):
    """out = merge(BinaryAttention(split(x @ w_qkv + b_qkv))) @ w_out + b_out.

    x [B, N, C] fp16/bf16, w_qkv [C, 3C], b_qkv [3C], w_out [C, C], b_out [C]
    (same dtype). ``keep``, if a dict, receives the intermediate q, k, v and
    attention output (for checking)."""
    import torch
    B, N, C = x.shape
    qkv = torch.addmm(b_qkv, x.view(B * N, C), w_qkv).view(B, N, 3 * C)
    q, k, v = split_heads(qkv, H)
    o = attention(q, k, v, bias=bias, stream=stream)
    if keep is not None:
        keep.update(q=q, k=k, v=v, o=o)
    return torch.addmm(b_out, merge_heads(o).reshape(B * N, C), w_out).view(B, N, C)
