"""Scratch independence at full size (GPU, through the C ABI).

Every entry point that takes a workspace is run twice on the same inputs, at
the full size of its workload, once with the workspace filled with 0x00 bytes
and once with 0xFF (NaN in bf16 and float32): the outputs must be bitwise
equal.  A kernel that reads scratch it has not written in the same call fails
here at any size, also where the parity tests' shapes are too small to reach
the faulty index range (the WANGO backward once skipped the window products
of every row tile past the eighth, which only sequences longer than 1,024
positions show).  The parity of these outputs against the oracle is the
business of the other GPU tests.
"""
import math

import pytest
import torch

from cross_token_gated_amd import api
from cross_token_gated_amd import layouts as lay
from cross_token_gated_amd import workload as wl
from tests.gpu_common import announce, block_weights, dev_tensor

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _twice(name, nbytes, run):
    """run(ws) -> list of output tensors; compares the two fills bitwise."""
    got = []
    for fill in (0x00, 0xFF):
        announce(f"scratch {name} fill {fill:#04x}")
        ws = api.workspace(nbytes, DEV)
        ws.fill_(fill)
        got.append([t.clone() for t in run(ws)])
        torch.cuda.synchronize()
        del ws
    for i, (a, b) in enumerate(zip(*got)):
        assert torch.equal(_bits(a), _bits(b)), f"{name}: output {i} depends on the workspace contents"
        assert not torch.isnan(b.float()).any(), f"{name}: output {i} holds NaN"


BLOCKS = ["tango_f32_t256", "tango_bf16_b8_t2048", "tango_bf16_t8192_r4", "wango_bf16_t8192_w256",
          "wango_bf16_b2_t65536_w512_r8", "tango_pages_t8192_r4", "wango_pages_t8192_w64_r4"]


@pytest.mark.parametrize("name", BLOCKS)
def test_block_scratch_independent(name):
    w = {**wl.WORKLOADS, **wl.PAGES_WORKLOADS}[name]
    inp = wl.make_inputs(w)
    b = block_weights(w, inp, DEV)
    x = dev_tensor(inp.h, w.io, DEV)
    shape = api.shape_of(x, b, w.rope_base, w.rms_eps, w.operand_parts)
    if w.mode == "tango":
        n = api.tango_workspace_size(shape)
        _twice(name, n, lambda ws: [api.tango_block_fwd(x, b, ws=ws, rope_base=w.rope_base, rms_eps=w.rms_eps, operand_parts=w.operand_parts)])
    else:
        n = api.wango_workspace_size(shape, w.window, w.head_dim, w.chunk)
        _twice(name, n, lambda ws: [api.wango_block_fwd(x, b, w.window, w.head_dim, w.chunk, ws=ws,
                                                        rope_base=w.rope_base, rms_eps=w.rms_eps, operand_parts=w.operand_parts)])


def test_stack_scratch_independent():
    for name, sw in wl.STACK_WORKLOADS.items():
        inps = wl.make_stack_inputs(sw)
        sets = [block_weights(sw.set_workload(k), inps[k], DEV) for k in range(len(sw.widths))]
        w = sw.base
        x = dev_tensor(inps[0].h, w.io, DEV)
        shapes = [api.shape_of(x, s, w.rope_base, w.rms_eps, w.operand_parts) for s in sets]
        _twice(name, api.tango_stack_workspace_size(shapes),
               lambda ws: [api.tango_stack_fwd(x, sets, sw.schedule, ws=ws, rope_base=w.rope_base,
                                               rms_eps=w.rms_eps, operand_parts=w.operand_parts)])


@pytest.mark.parametrize("mode", ["tango", "wango"])
def test_backward_scratch_independent(mode):
    c = wl.BACKWARD_SHAPE if mode == "tango" else wl.WANGO_BACKWARD_SHAPE
    T, F, Hh, dh = c["T"], c["F"], c["H"], c["dh"]
    Tp = lay.padded_len(T)
    q, k, g, dg_in = wl.aggregate_inputs(T, F, Hh, dh, c["seed"])
    bf = torch.bfloat16
    qd = torch.from_numpy(lay.pad_rows(q.reshape(1, T, Hh * dh), Tp).reshape(Tp, Hh * dh)).to(DEV).to(bf)
    kd = torch.from_numpy(lay.pad_rows(k.reshape(1, T, Hh * dh), Tp).reshape(Tp, Hh * dh)).to(DEV).to(bf)
    gp = torch.from_numpy(lay.pack_gates(lay.pad_rows(g[None], Tp)).reshape(-1)).to(DEV).to(bf)
    dgbar = torch.from_numpy(lay.pad_rows(dg_in[None], Tp).reshape(Tp, F)).to(DEV).to(bf)
    theta = torch.full((Hh,), math.log(10.0), dtype=torch.float32, device=DEV)
    nullb = torch.full((Hh,), -0.5, dtype=torch.float32, device=DEV)
    shape = api.make_shape(1, T, 512, F, Hh, dh, bf)
    gbar = torch.empty((Tp, F), dtype=bf, device=DEV)
    den = torch.empty((Tp, Hh), dtype=torch.float32, device=DEV)
    dq = torch.empty((Tp, Hh * dh), dtype=torch.float32, device=DEV)
    dk = torch.empty_like(dq)
    dg = torch.empty((Tp, F), dtype=bf, device=DEV)
    dth = torch.empty((Hh,), dtype=torch.float32, device=DEV)
    dnl = torch.empty_like(dth)
    announce(f"scratch {mode} backward: forward that saves the denominators")
    if mode == "tango":
        wsf = api.workspace(api.tango_workspace_size(shape), DEV)
        api.tango_aggregate_fwd_train(shape, theta, nullb, qd, kd, gp, gbar, den, wsf)
        n = api.tango_aggregate_bwd_workspace_size(shape)

        def bwd(ws):
            api.tango_aggregate_bwd(shape, theta, nullb, qd, kd, gp, gbar, den, dgbar, dq, dk, dg, dth, dnl, ws)
            return [dq, dk, dg[:T], dth, dnl]
    else:
        W, C = c["window"], c["chunk"]
        wsf = api.workspace(api.wango_aggregate_fwd_train_workspace_size(shape, W, C), DEV)
        api.wango_aggregate_fwd_train(shape, W, C, theta, nullb, qd, kd, gp, gbar, den, wsf)
        n = api.wango_aggregate_bwd_workspace_size(shape, W, C)

        def bwd(ws):
            api.wango_aggregate_bwd(shape, W, C, theta, nullb, qd, kd, gp, gbar, den, dgbar, dq, dk, dg, dth, dnl,
                                    ws)
            return [dq, dk, dg[:T], dth, dnl]
    _twice(f"{mode} backward T={T}", n, bwd)


def test_concurrent_streams_share_nothing():
    """The block calls keep no state between calls: a TANGO and a WANGO block
    at T = 8192 enqueued alternately on two streams (each with its own
    workspace and output, so that their kernels can overlap) give bitwise the
    outputs of the same calls run one after the other."""
    cases = []
    for name in ("tango_bf16_t8192_r4", "wango_bf16_t8192_w256"):
        w = wl.WORKLOADS[name]
        inp = wl.make_inputs(w)
        b = block_weights(w, inp, DEV)
        x = dev_tensor(inp.h, w.io, DEV)
        shape = api.shape_of(x, b, w.rope_base, w.rms_eps, w.operand_parts)
        if w.mode == "tango":
            ws = api.workspace(api.tango_workspace_size(shape), DEV)
            fn = (lambda x, b, w, ws: lambda out, s: api.tango_block_fwd(
                x, b, out=out, ws=ws, rope_base=w.rope_base, rms_eps=w.rms_eps, operand_parts=w.operand_parts, stream=s))(x, b, w, ws)
        else:
            ws = api.workspace(api.wango_workspace_size(shape, w.window, w.head_dim, w.chunk), DEV)
            fn = (lambda x, b, w, ws: lambda out, s: api.wango_block_fwd(
                x, b, w.window, w.head_dim, w.chunk, out=out, ws=ws, rope_base=w.rope_base, rms_eps=w.rms_eps, operand_parts=w.operand_parts,
                stream=s))(x, b, w, ws)
        cases.append((name, x, fn))
    announce("scratch: the two blocks one after the other")
    ref = []
    for name, x, fn in cases:
        out = torch.empty_like(x)
        fn(out, torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref.append(out)
    announce("scratch: the two blocks interleaved on two streams")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(x) for _ in range(3)] for _, x, _ in cases]
    torch.cuda.synchronize()
    for r in range(3):
        for k, (name, x, fn) in enumerate(cases):
            fn(outs[k][r], streams[k])
    torch.cuda.synchronize()
    for k, (name, x, fn) in enumerate(cases):
        for r in range(3):
            assert torch.equal(_bits(outs[k][r]), _bits(ref[k])), f"{name}, launch {r} on its own stream"
