"""Seeded synthetic inputs for the BinaryAttention forward pass.

This module holds no arithmetic of the method: it only draws random numbers
and rounds them to the 16-bit input formats. Both the GPU library's tests and
the CPU oracle are fed from here, so they see identical bit patterns.

The shapes follow the workloads the BinaryAttention pages evaluate on (ViT /
DeiT classifiers at 224px, DiT-XL/2 diffusion transformers at 256px and
512px, and high-resolution long sequences); the value distributions are
synthetic stand-ins for the ImageNet / COCO / ADE20K activations, which are
not used. Recipe per workload (numpy PCG64, ``default_rng(seed)``):

1. Q, K, V ~ N(0, 1) float32 [B,H,N,d], drawn in that order.
2. ``channel_scale``: one U(0.5, 2) draw of shape [H,d] for each of Q, K, V
   (in that order), broadcast over batch and tokens.
3. ``outlier_frac``: per batch element, round(frac*N) token indices without
   replacement; those rows of Q, K and V (all heads) are scaled by 8.
4. Bias: dense [H,N,N] or relative-position table [H,(2gh-1)(2gw-1)], entries
   N(0, 0.1^2), drawn last.
5. Cast to fp16 with numpy's round-to-nearest-even, or to bf16 by
   round-to-nearest-even on the float32 bit pattern.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

F16, BF16, F32 = 0, 1, 2
BIAS_NONE, BIAS_DENSE, BIAS_RELPOS = 0, 1, 2


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, np.float32).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, dtype: int) -> np.ndarray:
    return to_f16_bits(x) if dtype == F16 else to_bf16_bits(x)


def from_bits(b: np.ndarray, dtype: int) -> np.ndarray:
    """16-bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float32)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Spec:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: int
    seed: int
    bias: str = "none"            # none | dense_f32 | dense_f16 | relpos
    bias_shared: bool = True      # dense: one [H,N,N] slice for every batch element
    grid: tuple = (0, 0)          # relpos grid (gh, gw)
    n_prefix: int = 0             # relpos: leading tokens with no grid position
    channel_scale: bool = False
    outlier_frac: float = 0.0
    about: str = ""


# The workloads of the pages' evaluation, as single attention layers.
WORKLOADS = {
    "deit_tiny": Spec("deit_tiny", 1, 3, 197, 64, F16, 1000, bias="dense_f32",
                      bias_shared=True,
                      about="DeiT-Tiny layer at 224px: 196 patches + CLS, 3 heads of 64; dense fp32 bias"),
    "deit_small": Spec("deit_small", 64, 6, 197, 64, F16, 1001, bias="relpos", grid=(14, 14),
                       n_prefix=1, channel_scale=True,
                       about="DeiT-Small layer, batch 64: uneven channel magnitudes; 14x14 relative-position table"),
    "dit_256": Spec("dit_256", 32, 16, 256, 72, BF16, 1002,
                    about="DiT-XL/2 at 256px: 16x16 latent patches, 16 heads of 72; no bias"),
    "dit_512": Spec("dit_512", 8, 16, 1024, 72, BF16, 1003, bias="dense_f16", bias_shared=True,
                    outlier_frac=0.01,
                    about="DiT-XL/2 at 512px: 32x32 patches; 1% outlier tokens x8; dense fp16 bias shared over batch"),
    "long_4k": Spec("long_4k", 2, 16, 4096, 64, BF16, 1005,
                    about="high-resolution ViT-L / DiT long sequence, 64x64 tokens; no bias"),
    "long_4k_rp": Spec("long_4k_rp", 2, 16, 4096, 64, BF16, 1005, bias="relpos", grid=(64, 64),
                       about="as long_4k with a 64x64 relative-position table"),
    "long_16k": Spec("long_16k", 2, 16, 16384, 64, BF16, 1006,
                     about="high-resolution long sequence, 128x128 tokens; no bias"),
    "long_16k_rp": Spec("long_16k_rp", 2, 16, 16384, 64, BF16, 1006, bias="relpos", grid=(128, 128),
                        about="as long_16k with a 128x128 relative-position table"),
}


@dataclass
class Inputs:
    spec: Spec
    q: np.ndarray      # uint16 [B,H,N,d]
    k: np.ndarray
    v: np.ndarray
    bias_kind: int = BIAS_NONE
    bias_data: np.ndarray | None = None   # dense: float32 or uint16(fp16) [H,N,N] / [B,H,N,N]; relpos float32 [H,T]
    bias_dtype: int = F32
    bias_batch_stride: int = 0
    grid_h: int = 0
    grid_w: int = 0
    n_prefix: int = 0
    extra: dict = field(default_factory=dict)


def spec(name: str, **overrides) -> Spec:
    """A workload spec, optionally shrunk (same structure, other sizes)."""
    s = WORKLOADS[name]
    return replace(s, **overrides) if overrides else s


def generate(s: Spec) -> Inputs:
    rng = np.random.default_rng(s.seed)
    shape = (s.B, s.H, s.N, s.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if s.channel_scale:
        for x in (q, k, v):
            sc = rng.uniform(0.5, 2.0, size=(s.H, s.d)).astype(np.float32)
            x *= sc[None, :, None, :]
    if s.outlier_frac > 0.0:
        n_out = int(round(s.outlier_frac * s.N))
        for b in range(s.B):
            idx = rng.choice(s.N, size=n_out, replace=False)
            for x in (q, k, v):
                x[b, :, idx, :] *= np.float32(8.0)
    inp = Inputs(s, to_bits(q, s.dtype), to_bits(k, s.dtype), to_bits(v, s.dtype))
    if s.bias in ("dense_f32", "dense_f16"):
        nb = 1 if s.bias_shared else s.B
        bias = (0.1 * rng.standard_normal((nb, s.H, s.N, s.N), dtype=np.float32)).astype(np.float32)
        if s.bias == "dense_f16":
            inp.bias_data = to_f16_bits(bias)
            inp.bias_dtype = F16
        else:
            inp.bias_data = bias
            inp.bias_dtype = F32
        inp.bias_data = inp.bias_data[0] if s.bias_shared else inp.bias_data
        inp.bias_kind = BIAS_DENSE
        inp.bias_batch_stride = 0 if s.bias_shared else s.H * s.N * s.N
    elif s.bias == "relpos":
        gh, gw = s.grid
        assert s.n_prefix + gh * gw == s.N, "relative-position grid must cover the tokens"
        T = (2 * gh - 1) * (2 * gw - 1)
        inp.bias_data = (0.1 * rng.standard_normal((s.H, T), dtype=np.float32)).astype(np.float32)
        inp.bias_kind = BIAS_RELPOS
        inp.bias_dtype = F32
        inp.grid_h, inp.grid_w, inp.n_prefix = gh, gw, s.n_prefix
    return inp


def make(name: str, **overrides) -> Inputs:
    return generate(spec(name, **overrides))


def eff_ops(s: Spec) -> float:
    """Effective attention operations 4*B*H*N^2*d (real head dim)."""
    return 4.0 * s.B * s.H * s.N * s.N * s.d
