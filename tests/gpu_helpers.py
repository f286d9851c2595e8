"""Shared plumbing for the GPU tests: move seeded workload inputs to the
device, run the library through its C ABI, and describe the same bias to the
oracle. Holds none of the method's arithmetic."""
import numpy as np
import torch

import bit_qk_attention_amd as ba
import oracle
from workloads import BF16, BIAS_DENSE, BIAS_RELPOS, F16, F32, from_bits


def tdtype(dt):
    return torch.float16 if dt == F16 else torch.bfloat16


def to_dev(bits: np.ndarray, dt) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdtype(dt))
    return t.cuda()


def dev_bias(inp):
    """(library Bias, oracle Bias) for a workload's bias."""
    if inp.bias_kind == BIAS_DENSE:
        if inp.bias_dtype == F32:
            t = torch.from_numpy(np.ascontiguousarray(inp.bias_data)).cuda()
        else:
            t = torch.from_numpy(np.ascontiguousarray(inp.bias_data).view(np.int16)).view(torch.float16).cuda()
        lib_b = ba.Bias(ba.BA_BIAS_DENSE, t, batch_stride=inp.bias_batch_stride)
        ora_b = oracle.Bias(oracle.BIAS_DENSE, inp.bias_data, inp.bias_dtype, inp.bias_batch_stride)
        return lib_b, ora_b
    if inp.bias_kind == BIAS_RELPOS:
        t = torch.from_numpy(np.ascontiguousarray(inp.bias_data)).cuda()
        lib_b = ba.Bias(ba.BA_BIAS_RELPOS, t, 0, inp.grid_h, inp.grid_w, inp.n_prefix)
        ora_b = oracle.Bias(oracle.BIAS_RELPOS, inp.bias_data, F32, 0, inp.grid_h, inp.grid_w, inp.n_prefix)
        return lib_b, ora_b
    return None, None


class DeviceRun:
    """All device tensors of one forward pass."""

    def __init__(self, inp, out_dt=None):
        self.inp = inp
        s = inp.spec
        self.q, self.k, self.v = (to_dev(x, s.dtype) for x in (inp.q, inp.k, inp.v))
        self.lib_bias, self.ora_bias = dev_bias(inp)
        self.qbits, self.qmu, self.kbits, self.kmu = ba.pack_qk(self.q, self.k)
        self.vq, self.vscale = ba.quant_v(self.v)
        odt = tdtype(s.dtype if out_dt is None else out_dt)
        self.out = torch.empty(self.q.shape, dtype=odt, device="cuda")
        ba.ba_attention_fwd(self.qbits, self.qmu, self.kbits, self.kmu, self.vq, self.vscale,
                            self.lib_bias, self.out)
        torch.cuda.synchronize()

    def out_f32(self) -> np.ndarray:
        return self.out.float().cpu().numpy()

    def rerun(self):
        out = torch.empty_like(self.out)
        ba.ba_attention_fwd(self.qbits, self.qmu, self.kbits, self.kmu, self.vq, self.vscale,
                            self.lib_bias, out)
        torch.cuda.synchronize()
        return out


def out_bits(out: torch.Tensor) -> np.ndarray:
    """The 16-bit patterns of a device fp16/bf16 tensor, on the host."""
    return out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def vmax(inp) -> float:
    return float(np.abs(from_bits(inp.v, inp.spec.dtype)).max())
