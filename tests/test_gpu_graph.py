"""HIP graph capture of the block and decode calls (GPU, through the C ABI).

The library enqueues only kernels on the caller's stream: its scratch lives in
the caller's workspace and is cleared by kernels (never by a memset or a
copy), and a call allocates nothing and never synchronises.  A call can then
be captured into a HIP graph and replayed, which is how a serving loop or a
training step removes the host's launch cost.  Each case runs the calls
eagerly, captures the same calls on the same buffers, and replays the graph
three times with eager work (refilling the outputs with NaN) and a
synchronisation between the replays; every replay must give bitwise the eager
result.  The decode cases advance their positions inside the graph, so each
replay is the next step of the eager sequence.
"""
import numpy as np
import pytest
import torch

from cross_token_gated_amd import api
from cross_token_gated_amd import workload as wl
from tests.gpu_common import TORCH_DTYPE, announce, block_weights, dev_tensor

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 3


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _capture(fn) -> torch.cuda.CUDAGraph:
    # one run on a side stream first, as graph capture expects; the library's
    # one-time set-up has already happened in the eager calls
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["tango_bf16_t8192_r4", "wango_bf16_t8192_w256", "tango_f32_t256"])
def test_block_graph_replays(name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    b = block_weights(w, inp, DEV)
    x = dev_tensor(inp.h, w.io, DEV)
    shape = api.shape_of(x, b, w.rope_base, w.rms_eps, w.operand_parts)
    if w.mode == "tango":
        ws = api.workspace(api.tango_workspace_size(shape), DEV)

        def call(out):
            api.tango_block_fwd(x, b, out=out, ws=ws, rope_base=w.rope_base, rms_eps=w.rms_eps, operand_parts=w.operand_parts)
    else:
        ws = api.workspace(api.wango_workspace_size(shape, w.window, w.head_dim, w.chunk), DEV)

        def call(out):
            api.wango_block_fwd(x, b, w.window, w.head_dim, w.chunk, out=out, ws=ws, rope_base=w.rope_base,
                                rms_eps=w.rms_eps, operand_parts=w.operand_parts)
    announce(f"graph {name}: eager call")
    ref = torch.empty_like(x)
    call(ref)
    torch.cuda.synchronize()
    y = torch.full_like(x, float("nan"))
    announce(f"graph {name}: capture")
    g = _capture(lambda: call(y))
    for r in range(REPLAYS):
        y.fill_(float("nan"))
        ws.fill_(0xFF)                 # eager work between replays; the scratch is rewritten
        torch.cuda.synchronize()
        announce(f"graph {name}: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(ref)), f"{name}: replay {r} differs from the eager call"


@pytest.mark.parametrize("mode", ["tango", "wango"])
def test_decode_graph_replays(mode):
    """Three decode steps from position 0 of four sequences: eager, then one
    captured step (with the position increment) replayed three times from the
    same initial state."""
    w = wl.small_workload(mode=mode, B=4, T=16, d_model=128, d_gate=256, n_heads=2, head_dim=64,
                          window=8, chunk=8)
    inp = wl.make_inputs(w)
    bw = block_weights(w, inp, DEV)
    B, d = w.B, w.d_model
    shape = api.decode_shape(B, 16, bw, TORCH_DTYPE[w.io], d, w.rope_base, w.rms_eps)
    if mode == "tango":
        ns, nw = api.tango_decode_state_size(shape), api.tango_decode_workspace_size(shape)

        def step(pos, x, out, st, ws):
            api.tango_decode_step(shape, bw, pos, x, out, st, ws)
    else:
        ns = api.wango_decode_state_size(shape, w.window, w.head_dim)
        nw = api.wango_decode_workspace_size(shape, w.window, w.head_dim)

        def step(pos, x, out, st, ws):
            api.wango_decode_step(shape, bw, w.window, w.head_dim, pos, x, out, st, ws)
    xs = [dev_tensor(np.ascontiguousarray(inp.h[:, t]), w.io, DEV) for t in range(REPLAYS)]
    ws = api.workspace(nw, DEV)

    announce(f"graph decode {mode}: eager steps")
    st = torch.full((ns,), 0x7F, dtype=torch.uint8, device=DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    ref = []
    for t in range(REPLAYS):
        out = torch.empty_like(xs[0])
        step(pos, xs[t], out, st, ws)
        pos += 1
        ref.append(out)
    torch.cuda.synchronize()
    ref_state = st.clone()

    # the graph reads the token from a static buffer the host refills
    x_in = torch.empty_like(xs[0])
    y = torch.full_like(xs[0], float("nan"))
    st_g = torch.full((ns,), 0x7F, dtype=torch.uint8, device=DEV)
    pos_g = torch.zeros(B, dtype=torch.int32, device=DEV)

    def one():
        step(pos_g, x_in, y, st_g, ws)
        pos_g.add_(1)

    # the side-stream run before capture takes a step of its own: start over
    x_in.copy_(xs[0])
    announce(f"graph decode {mode}: capture")
    g = _capture(one)
    st_g.fill_(0x7F)
    pos_g.zero_()
    for t in range(REPLAYS):
        x_in.copy_(xs[t])
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"graph decode {mode}: replay {t}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(ref[t])), f"decode {mode}: replay {t} differs from eager step {t}"
    assert torch.equal(st_g, ref_state), f"decode {mode}: state after the replays differs"
