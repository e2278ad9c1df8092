"""Decode-step parity against the float64 oracle, through the C ABI.

Sequences are decoded token by token from position 0.  At every step the
output must be the block output at that position: row p of the oracle's block
forward over the prefix, which is the definition of a decode step (pinned in
tests/test_decode_oracle.py).  Sequences start at different steps, so the
positions in one call are ragged, and a sequence that has not started is
passed pos = -1 and must come back as a NaN row without its state changing.
The bar is that of the block: max|err|/rms <= 2e-2 for bf16 compute, 1e-4 for
float32.
"""
import numpy as np
import pytest
import torch

import oracle.tango_oracle as O
from cross_token_gated_amd import api
from cross_token_gated_amd import workload as wl
from tests import helpers as H
from tests.gpu_common import TORCH_DTYPE, announce, block_weights, dev_tensor, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from cross_token_gated_amd import _lib
    _lib.load()


def decode_run(w: wl.Workload, inp: wl.Inputs, starts, capacity=None, sample_steps=None):
    """Decode the B sequences of ``inp.h`` (sequence b starting at step
    starts[b]) through w.repeats stacked applications, each with its own state.
    Returns {step: out [B, d] as float64} for every step (or the sampled ones)."""
    dev = torch.device("cuda:0")
    bw = block_weights(w, inp, dev)
    B, T, d = inp.h.shape
    cap = T if capacity is None else capacity
    shape = api.decode_shape(B, cap, bw, TORCH_DTYPE[w.io], d, w.rope_base, w.rms_eps)
    if w.mode == "tango":
        ns, nw = api.tango_decode_state_size(shape), api.tango_decode_workspace_size(shape)
    else:
        ns = api.wango_decode_state_size(shape, w.window, w.head_dim)
        nw = api.wango_decode_workspace_size(shape, w.window, w.head_dim)
    assert ns > 0 and nw > 0
    # state filled with garbage: a sequence starting at 0 must not read it
    states = [torch.full((ns,), 0x7F, dtype=torch.uint8, device=dev) for _ in range(w.repeats)]
    ws = api.workspace(nw, dev)
    hT = dev_tensor(np.ascontiguousarray(np.transpose(inp.h, (1, 0, 2))), w.io, dev)   # [T, B, d]
    steps = T + max(starts)
    pos_all = np.full((steps, B), -1, dtype=np.int32)
    for b, s0 in enumerate(starts):
        pos_all[s0:s0 + T, b] = np.arange(T, dtype=np.int32)
    pos_dev = torch.from_numpy(pos_all).to(dev)
    src = torch.zeros(steps, B, d, dtype=TORCH_DTYPE[w.io], device=dev)
    for b, s0 in enumerate(starts):
        src[s0:s0 + T, b] = hT[:, b]
    outs = {}
    for step in range(steps):
        cur = src[step]
        for r in range(w.repeats):
            nxt = torch.empty_like(cur)
            if w.mode == "tango":
                api.tango_decode_step(shape, bw, pos_dev[step], cur, nxt, states[r], ws)
            else:
                api.wango_decode_step(shape, bw, w.window, w.head_dim, pos_dev[step], cur, nxt,
                                      states[r], ws)
            cur = nxt
        if sample_steps is None or step in sample_steps:
            outs[step] = cur
    torch.cuda.synchronize()
    return {k: host(v) for k, v in outs.items()}, pos_all


def check_against_oracle(w, inp, outs, pos_all, rows_ref):
    """rows_ref[b] = oracle output rows [T, d] of sequence b."""
    B = inp.h.shape[0]
    worst = 0.0
    for b in range(B):
        got, ref = [], []
        for step, o in outs.items():
            p = pos_all[step, b]
            if p < 0:
                assert np.isnan(o[b]).all(), (step, b)
                continue
            got.append(o[b])
            ref.append(rows_ref[b][p])
        e = H.err_ratio(np.stack(got), np.stack(ref))
        worst = max(worst, e)
    print(f"{w.name}: max|err|/rms over all steps = {worst:.3e} (bar {H.tol(w.dtype):.0e})")
    assert worst < H.tol(w.dtype)


CASES = [
    dict(mode="tango", dtype="bf16", io_dtype="bf16", B=3, T=40, d_model=128, d_gate=128, n_heads=2,
         head_dim=32),
    dict(mode="tango", dtype="bf16", io_dtype="f32", B=2, T=150, d_model=256, d_gate=256, n_heads=1,
         head_dim=128),
    dict(mode="tango", dtype="f32", B=2, T=40, d_model=128, d_gate=128, n_heads=2, head_dim=64),
    dict(mode="wango", dtype="bf16", io_dtype="bf16", B=3, T=40, d_model=128, d_gate=128, n_heads=2,
         head_dim=32, window=5),
    dict(mode="wango", dtype="bf16", io_dtype="f32", B=2, T=100, d_model=256, d_gate=512, n_heads=2,
         head_dim=64, window=16),
    dict(mode="wango", dtype="f32", B=2, T=40, d_model=128, d_gate=128, n_heads=1, head_dim=32, window=7),
    dict(mode="wango", dtype="bf16", io_dtype="bf16", B=1, T=30, d_model=128, d_gate=128, n_heads=2,
         head_dim=64, window=1),
]


def _id(c):
    return (f"{c['mode']}-{c['dtype']}-io{c.get('io_dtype', c['dtype'])}-B{c['B']}-T{c['T']}-H{c['n_heads']}"
            f"x{c['head_dim']}-F{c['d_gate']}" + (f"-W{c['window']}" if c['mode'] == 'wango' else ""))


@pytest.mark.parametrize("case", CASES, ids=_id)
@pytest.mark.parametrize("null", [False, True])
def test_decode_steps(case, null):
    w = wl.small_workload(**case, null_bias=(-1.0 if null else None))
    inp = wl.make_inputs(w)
    starts = [3 * b for b in range(w.B)]
    announce(f"decode {_id(case)} null={null}")
    outs, pos_all = decode_run(w, inp, starts)
    p, cfg = H.oracle_params(inp), H.oracle_config(w)
    ref = [O.block_sequence(np.asarray(inp.h[b], np.float64), p, cfg) for b in range(w.B)]
    check_against_oracle(w, inp, outs, pos_all, ref)


@pytest.mark.parametrize("mode", ["tango", "wango"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_stack(mode, dtype):
    """Three stacked applications, each with its own state; the stream between
    them is stored in the I/O dtype (float32, as in the shipped workloads; a
    bf16 stream rounded between and after tiny layers already spends most of
    the bf16 bar on storage alone, and the single-layer cases cover it)."""
    w = wl.small_workload(mode=mode, dtype=dtype, io_dtype="f32", B=2, T=30, d_model=128, d_gate=128,
                          n_heads=2, head_dim=32, window=4, repeats=3)
    inp = wl.make_inputs(w)
    announce(f"decode stack {mode} {dtype}")
    outs, pos_all = decode_run(w, inp, [0, 2])
    ref = [O.block_stack(np.asarray(inp.h[b:b + 1], np.float64), H.oracle_params(inp), H.oracle_config(w),
                         repeats=3, io_dtype="f32")[0] for b in range(w.B)]
    check_against_oracle(w, inp, outs, pos_all, ref)


def test_tango_position_past_capacity_is_skipped():
    """pos >= capacity: NaN row, no write into the cache (the next valid steps
    still match the oracle)."""
    w = wl.small_workload(mode="tango", dtype="bf16", io_dtype="bf16", B=2, T=12, d_model=128, d_gate=128,
                          n_heads=1, head_dim=64)
    inp = wl.make_inputs(w)
    dev = torch.device("cuda:0")
    bw = block_weights(w, inp, dev)
    shape = api.decode_shape(2, 12, bw, torch.bfloat16, 128)
    st = torch.zeros(api.tango_decode_state_size(shape), dtype=torch.uint8, device=dev)
    ws = api.workspace(api.tango_decode_workspace_size(shape), dev)
    x = dev_tensor(inp.h[:, 0], "bf16")
    out = torch.empty_like(x)
    announce("decode tango pos past capacity")
    api.tango_decode_step(shape, bw, torch.tensor([0, 12], dtype=torch.int32, device=dev), x, out, st, ws)
    o = host(out)
    assert np.isfinite(o[0]).all() and np.isnan(o[1]).all()
    assert not torch.any(st.view(torch.bfloat16).float().isnan())


@pytest.mark.parametrize("mode", ["tango", "wango"])
def test_decode_workload_geometry(mode):
    """The decode workloads' widths (d = 512, F = 2048; TANGO one head of 128,
    WANGO two heads of 64 with window 256) over 300 positions: past the window
    and across the cache chunks of 128."""
    name = "tango_decode_bf16_b16_p8192_r4" if mode == "tango" else "wango_decode_bf16_b64_p8192_w256"
    w = wl.DECODE_WORKLOADS[name].scaled(B=3, T=300, repeats=1)
    inp = wl.make_inputs(w)
    announce(f"decode geometry {name} B=3 T=300")
    outs, pos_all = decode_run(w, inp, [0, 1, 5])
    p, cfg = H.oracle_params(inp), H.oracle_config(w)
    ref = [O.block_sequence(np.asarray(inp.h[b], np.float64), p, cfg) for b in range(w.B)]
    check_against_oracle(w, inp, outs, pos_all, ref)


@pytest.mark.parametrize("mode", ["tango", "wango"])
def test_decode_workload_full_position(mode):
    """The decode workloads at their full position: 4 sequences decoded from
    position 0 to 8192 (the timed position of the bench), outputs sampled at
    chunk and window edges and at 8192, against oracle rows of the forward."""
    name = "tango_decode_bf16_b16_p8192_r4" if mode == "tango" else "wango_decode_bf16_b64_p8192_w256"
    w = wl.DECODE_WORKLOADS[name].scaled(B=4, repeats=1)
    inp = wl.make_inputs(w)
    rows = [0, 127, 128, 255, 256, 257, 4095, 8191, 8192]
    announce(f"decode full position {name} B=4 T={w.T}")
    outs, pos_all = decode_run(w, inp, [0, 0, 0, 0], sample_steps=set(rows))
    p, cfg = H.oracle_params(inp), H.oracle_config(w)
    ref = {b: dict(zip(rows, H.oracle_block_rows(inp.h[b], p, cfg, rows))) for b in range(w.B)}
    check_against_oracle(w, inp, outs, pos_all, ref)
