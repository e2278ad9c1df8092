"""Upload of seeded host arrays to device tensors and the weight struct of the
binding: plumbing shared by the tests, smoke() and bench.py (no arithmetic of
the method)."""
from __future__ import annotations

import numpy as np
import torch

from . import api
from . import workload as wl

TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def dev_tensor(a: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    """Host array -> contiguous device tensor in dtype "bf16" or "f32" (rounded
    to nearest even, through float32)."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(device=device).to(TORCH_DTYPE[dtype]).contiguous()


def dev_f32(a: np.ndarray, device="cuda:0") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def block_weights(w: wl.Workload, inp: wl.Inputs, device="cuda:0") -> api.BlockWeights:
    """The weights of a seeded workload as device tensors in its compute dtype
    (theta and the null bias in float32)."""
    return api.BlockWeights(
        w_g=dev_tensor(inp.w_g, w.dtype, device), w_v=dev_tensor(inp.w_v, w.dtype, device),
        w_q=dev_tensor(inp.w_q, w.dtype, device), w_k=dev_tensor(inp.w_k, w.dtype, device),
        w_o=dev_tensor(inp.w_o, w.dtype, device), theta=dev_f32(inp.theta, device),
        n_heads=w.n_heads, head_dim=w.head_dim,
        gain=None if inp.gain is None else dev_tensor(inp.gain, w.dtype, device),
        null_bias=None if inp.null_bias is None else dev_f32(inp.null_bias, device))


def run_workload(w: wl.Workload, inp: wl.Inputs, device="cuda:0", x=None, ws=None, stream=None):
    """All R applications in place on one stream; returns the device output."""
    bw = block_weights(w, inp, device)
    if x is None:
        x = dev_tensor(inp.h, w.io, device)
    shape = api.shape_of(x, bw, w.rope_base, w.rms_eps, w.operand_parts)
    if ws is None:
        n = (api.tango_workspace_size(shape) if w.mode == "tango"
             else api.wango_workspace_size(shape, w.window, w.head_dim, w.chunk))
        assert n > 0
        ws = api.workspace(n, device)
    for _ in range(w.repeats):
        if w.mode == "tango":
            api.tango_block_fwd(x, bw, out=x, ws=ws, rope_base=w.rope_base, rms_eps=w.rms_eps,
                                stream=stream, operand_parts=w.operand_parts)
        else:
            api.wango_block_fwd(x, bw, w.window, w.head_dim, w.chunk, out=x, ws=ws,
                                rope_base=w.rope_base, rms_eps=w.rms_eps, stream=stream,
                                operand_parts=w.operand_parts)
    return x
