"""An attention block around the BinaryAttention kernels: QKV projection,
BinaryAttention, output projection. The pages measure the method end to end
as well as the kernel (zh technical summary section 4, efficiency comparison:
end-to-end throughput at 1024x1024 input; nl Resultaten, speed and
efficiency); this block is the part of a transformer layer that the method
changes, at synthetic weights.

The two projections are plain GEMMs on the ROCm BLAS (``torch.addmm``).
Between them there is no layout copy: the pre-pass reads Q, K and V as
strided head views of the [B, N, 3, H, d] projection output, and the
attention writes [B, N, H, d], which the output projection reads as
[B*N, C]. Packing Q and K, quantising V and the fused attention run in this
library's kernels through the C ABI.
"""
from __future__ import annotations

from . import Bias, attention


def split_heads(qkv, H: int):
    """[B, N, 3*H*d] -> three [B, H, N, d] views (q, k, v), no copy."""
    B, N, C3 = qkv.shape
    t = qkv.view(B, N, 3, H, C3 // (3 * H))
    return t[:, :, 0].transpose(1, 2), t[:, :, 1].transpose(1, 2), t[:, :, 2].transpose(1, 2)


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
    o = torch.empty(B, N, H, C // H, dtype=x.dtype, device=x.device)
    attention(q, k, v, bias=bias, out=o.transpose(1, 2), stream=stream)
    if keep is not None:
        keep.update(q=q, k=k, v=v, o=o.transpose(1, 2))
    return torch.addmm(b_out, o.view(B * N, C), w_out).view(B, N, C)
