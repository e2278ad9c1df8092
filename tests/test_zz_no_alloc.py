"""wango_decode_step_noalloc (scratch in the library's own device array) against
wango_decode_step (scratch in a caller workspace), through the C ABI.

Two no-allocation calls in a row on one GPU, the second with fewer sequences
(and other weights and widths), so it runs on an array that still holds the
first call's contents.  Each is compared with the workspace entry point on the
same inputs and a copy of the same state, built by decoding a few positions
past the window first.  Both calls run the same kernels on the same values in
the same order (the output combine adds its partials in a fixed order), so the
outputs and the advanced states must agree bit for bit -- which meets the 2e-2
bar of the block outputs with nothing to spare.  The output is also checked
against the float64 oracle's rows at that position.
"""
import numpy as np
import pytest
import torch

from cross_token_gated_amd import api
from cross_token_gated_amd import workload as wl
from tests import helpers as H
from tests.gpu_common import TORCH_DTYPE, announce, block_weights, dev_tensor, host

pytestmark = pytest.mark.gpu


def _decode_to(w: wl.Workload, inp: wl.Inputs, steps: int):
    """Decode positions 0 .. steps-1 of every sequence with the workspace entry
    point; return what the next step needs: its shape, weights, position
    vector, input row, and the state after position steps-1."""
    dev = torch.device("cuda:0")
    bw = block_weights(w, inp, dev)
    B, T, d = inp.h.shape
    shape = api.decode_shape(B, 1, bw, TORCH_DTYPE[w.io], d, w.rope_base, w.rms_eps)
    ns = api.wango_decode_state_size(shape, w.window, w.head_dim)
    nw = api.wango_decode_workspace_size(shape, w.window, w.head_dim)
    assert ns > 0 and 0 < nw <= api._lib.NOALLOC_SCRATCH_BYTES
    state = torch.full((ns,), 0x7F, dtype=torch.uint8, device=dev)
    ws = api.workspace(nw, dev)
    rows = dev_tensor(np.ascontiguousarray(np.transpose(inp.h, (1, 0, 2))), w.io, dev)   # [T, B, d]
    for p in range(steps):
        pos = torch.full((B,), p, dtype=torch.int32, device=dev)
        out = torch.empty_like(rows[p])
        api.wango_decode_step(shape, bw, w.window, w.head_dim, pos, rows[p], out, state, ws)
    pos = torch.full((B,), steps, dtype=torch.int32, device=dev)
    return shape, bw, pos, rows[steps].contiguous(), state, ws


CASES = [
    dict(B=48, d_model=256, d_gate=512, n_heads=2, head_dim=64, window=16, steps=21, seed=31),
    dict(B=5, d_model=128, d_gate=256, n_heads=1, head_dim=128, window=8, steps=13, seed=32),
]


def test_noalloc_decode_equals_workspace_call_twice():
    for c in CASES:
        c = dict(c)
        steps = c.pop("steps")
        w = wl.small_workload(mode="wango", dtype="bf16", io_dtype="f32", T=steps + 1, chunk=64, **c)
        inp = wl.make_inputs(w)
        announce(f"noalloc decode B={w.B} d={w.d_model} F={w.d_gate} H={w.n_heads} dh={w.head_dim} "
                 f"W={w.window} at position {steps}")
        shape, bw, pos, x, state, ws = _decode_to(w, inp, steps)
        st_ref, st_new = state.clone(), state.clone()
        out_ref, out_new = torch.full_like(x, float("nan")), torch.full_like(x, float("nan"))
        api.wango_decode_step(shape, bw, w.window, w.head_dim, pos, x, out_ref, st_ref, ws)
        api.wango_decode_step_noalloc(shape, bw, w.window, w.head_dim, pos, x, out_new, st_new)
        torch.cuda.synchronize()
        assert torch.equal(out_new, out_ref), "outputs differ"
        assert torch.equal(st_new, st_ref), "advanced states differ"
        # and both are row `steps` of the block forward over the prefix
        ref = H.oracle_block_rows(inp.h[0], H.oracle_params(inp), H.oracle_config(w), [steps])[0]
        got = host(out_new)[0]
        e = float(np.max(np.abs(got - ref))) / float(np.sqrt(np.mean(ref ** 2)))
        print(f"B={w.B}: identical to the workspace call; sequence 0 against the oracle {e:.3e}")
        assert e < H.tol(w.dtype)
