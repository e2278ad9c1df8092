"""Stage-by-stage parity of the HIP kernels against the float64 oracle.

Every stage gets the oracle's own intermediate values (rounded to the I/O
dtype) as input, so each kernel is checked on its own: projections, TANGO
aggregation, output projection, WANGO running sums, WANGO band + combine.
Sizes span several tiles with ragged tails; both storage dtypes are covered.
"""
import math

import numpy as np
import pytest
import torch

import oracle.tango_oracle as O
from cross_token_gated_amd import api
from cross_token_gated_amd import workload as wl
from tests import helpers as H
from tests.gpu_common import announce, block_weights, dev_f32, dev_tensor, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from cross_token_gated_amd import _lib
    _lib.load()   # fails loudly if the library is missing


def _q(a, dtype):
    return wl.quantize(np.asarray(a, dtype=np.float64), dtype).astype(np.float64)


def _stage_inputs(w, inp):
    """Oracle projections of every sequence, rounded to the I/O dtype."""
    p, cfg = H.oracle_params(inp), H.oracle_config(w)
    parts = [O.project(np.asarray(inp.h[b], dtype=np.float64), p, cfg) for b in range(w.B)]
    g = np.stack([_q(x["g"], w.dtype) for x in parts])
    v = np.stack([_q(x["v"], w.dtype) for x in parts])
    qh = np.stack([_q(x["qh"], w.dtype) for x in parts])   # [B, T, H, dh]
    kh = np.stack([_q(x["kh"], w.dtype) for x in parts])
    return parts, g, v, qh, kh


def _upload_intermediates(w, g, v, qh, kh):
    Tp = H.padded_len(w.T)
    HD = w.n_heads * w.head_dim
    gp = dev_tensor(H.pack_gates(H.pad_rows(g, Tp)), w.dtype)
    vd = dev_tensor(H.pad_rows(v, Tp), "f32")   # v is float32 for both dtypes
    qd = dev_tensor(H.pad_rows(qh.reshape(w.B, w.T, HD), Tp), w.dtype)
    kd = dev_tensor(H.pad_rows(kh.reshape(w.B, w.T, HD), Tp), w.dtype)
    return gp, vd, qd, kd


PROJ_CASES = [
    dict(dtype="bf16", B=1, T=200, d_model=128, d_gate=256, n_heads=1, head_dim=128),
    dict(dtype="bf16", B=2, T=77, d_model=256, d_gate=384, n_heads=2, head_dim=64),
    dict(dtype="bf16", B=1, T=130, d_model=128, d_gate=256, n_heads=4, head_dim=32),
    dict(dtype="f32", B=1, T=150, d_model=256, d_gate=256, n_heads=1, head_dim=128),
    dict(dtype="f32", B=2, T=64, d_model=128, d_gate=128, n_heads=2, head_dim=64),
]


@pytest.mark.parametrize("case", PROJ_CASES, ids=lambda c: f"{c['dtype']}-B{c['B']}-T{c['T']}-H{c['n_heads']}")
@pytest.mark.parametrize("with_gain", [False, True])
@pytest.mark.parametrize("op_parts", [1, 2])
def test_stage_proj(case, with_gain, op_parts):
    if op_parts == 2 and case["dtype"] != "bf16":
        pytest.skip("two operand parts exist for bf16 only")
    w = wl.small_workload(operand_parts=op_parts, **case)
    gain = (1.0 + 0.3 * np.random.default_rng(3).standard_normal(w.d_model)) if with_gain else None
    inp = wl.make_inputs(w, gain=gain)
    parts, *_ = _stage_inputs(w, inp)
    bw = block_weights(w, inp)
    x = dev_tensor(inp.h, w.dtype)
    shape = api.shape_of(x, bw, w.rope_base, w.rms_eps, w.operand_parts)
    Tp, HD, F = H.padded_len(w.T), w.n_heads * w.head_dim, w.d_gate
    M = w.B * Tp
    dt = x.dtype
    gp = torch.full((M * F,), float("nan"), dtype=dt, device="cuda:0")
    v = torch.full((M, F), float("nan"), dtype=api.v_dtype(shape), device="cuda:0")
    qh = torch.full((M, HD), float("nan"), dtype=dt, device="cuda:0")
    kh = torch.full((M, HD), float("nan"), dtype=dt, device="cuda:0")
    ws = api.workspace(api.tango_proj_workspace_size(shape), "cuda:0")
    ws.fill_(0xFF)   # scratch contents must not matter
    announce(f"stage_proj {case} gain={with_gain} op_parts={op_parts}")
    api.tango_stage_proj(shape, bw, x, gp, v, qh, kh, ws=ws)
    torch.cuda.synchronize()
    g_got = H.unpad_rows(H.unpack_gates(host(gp), M, F), w.B, w.T)
    v_got = H.unpad_rows(host(v), w.B, w.T)
    q_got = H.unpad_rows(host(qh), w.B, w.T)
    k_got = H.unpad_rows(host(kh), w.B, w.T)
    # padded rows are zeros
    assert np.all(host(v).reshape(w.B, Tp, F)[:, w.T:] == 0)
    assert np.all(host(kh).reshape(w.B, Tp, HD)[:, w.T:] == 0)
    g_ref = np.stack([p["g"] for p in parts])
    v_ref = np.stack([p["v"] for p in parts])
    q_ref = np.stack([p["qh"].reshape(w.T, HD) for p in parts])
    k_ref = np.stack([p["kh"].reshape(w.T, HD) for p in parts])
    H.check_stage(g_got, g_ref, w.dtype, "g")
    # v is stored in float32 for both dtypes: what remains is the float32
    # accumulation and the operand: in float32 and with two bf16 parts (h * gain
    # as hi + lo, about 2^-16 relative) 1e-4 on the rms and 1e-3 on the largest
    # entries; with one part the operand's bf16 rounding (2^-9 relative) sets
    # the error, as for the bf16-stored outputs
    rv, mv = H.rms_ratio(v_got, v_ref), H.err_ratio(v_got, v_ref)
    print(f"v: rms ratio {rv:.2e}, max ratio {mv:.2e}")
    if w.dtype == "bf16" and op_parts == 1:
        H.check_stage(v_got, v_ref, w.dtype, "v")
    else:
        assert rv <= 1e-4 and mv <= 1e-3
    H.check_stage(q_got, q_ref, w.dtype, "q")
    H.check_stage(k_got, k_ref, w.dtype, "k")


AGG_CASES = [
    dict(dtype="bf16", B=1, T=1000, d_model=128, d_gate=256, n_heads=1, head_dim=128),
    dict(dtype="bf16", B=1, T=1, d_model=128, d_gate=128, n_heads=1, head_dim=64),
    dict(dtype="bf16", B=1, T=65, d_model=128, d_gate=2048, n_heads=1, head_dim=128),
    dict(dtype="bf16", B=2, T=300, d_model=128, d_gate=512, n_heads=2, head_dim=64),
    dict(dtype="bf16", B=1, T=257, d_model=128, d_gate=256, n_heads=4, head_dim=32),
    dict(dtype="bf16", B=64, T=200, d_model=128, d_gate=256, n_heads=4, head_dim=32),  # pair mode
    # wider shapes: two heads of 64 at B = 8; an odd tile count (a middle tile of its own)
    # at B = 16; four heads of 32 at a gate width of 4096
    dict(dtype="bf16", B=8, T=1000, d_model=128, d_gate=2048, n_heads=2, head_dim=64),
    dict(dtype="bf16", B=16, T=1100, d_model=128, d_gate=1024, n_heads=1, head_dim=128),
    dict(dtype="bf16", B=6, T=700, d_model=128, d_gate=4096, n_heads=4, head_dim=32),
    # heads of 704, 320 and 1152 columns take waves of 48 columns: the first
    # two end inside a wave (its last block past the head is dropped) and
    # leave the wave after it without columns; 1152 fills three chunks
    dict(dtype="bf16", B=1, T=1000, d_model=128, d_gate=704, n_heads=1, head_dim=128),
    dict(dtype="bf16", B=2, T=300, d_model=128, d_gate=640, n_heads=2, head_dim=64),
    dict(dtype="bf16", B=1, T=520, d_model=128, d_gate=2304, n_heads=2, head_dim=64),
    dict(dtype="f32", B=1, T=333, d_model=128, d_gate=256, n_heads=1, head_dim=128),
    dict(dtype="f32", B=2, T=64, d_model=128, d_gate=128, n_heads=2, head_dim=64),
]


def _agg_ref(w, inp, qh, kh, g, null):
    tau = O.temperature(np.asarray(inp.theta, dtype=np.float64))
    nb = None if null is None else np.asarray(null, dtype=np.float64)
    return np.stack([O.aggregate_direct(qh[b], kh[b], g[b], tau, nb, w.mode, w.window)
                     for b in range(w.B)])


@pytest.mark.parametrize("case", AGG_CASES, ids=lambda c: f"{c['dtype']}-B{c['B']}-T{c['T']}-F{c['d_gate']}-H{c['n_heads']}")
@pytest.mark.parametrize("null", [False, True])
def test_stage_tango_aggregate(case, null):
    w = wl.small_workload(**case)
    nbias = np.linspace(-1.0, 0.5, w.n_heads).astype(np.float32) if null else None
    theta = np.linspace(math.log(10.0), math.log(30.0), w.n_heads).astype(np.float32)  # last clips at 20
    inp = wl.make_inputs(w)
    inp.theta = theta
    inp.null_bias = nbias
    _, g, v, qh, kh = _stage_inputs(w, inp)
    gp, _, qd, kd = _upload_intermediates(w, g, v, qh, kh)
    Tp, F = H.padded_len(w.T), w.d_gate
    shape = api.make_shape(w.B, w.T, w.d_model, F, w.n_heads, w.head_dim, qd.dtype)
    ws = api.workspace(api.tango_workspace_size(shape), "cuda:0")
    ws.fill_(0xFF)
    gbar = torch.full((w.B * Tp, F), float("nan"), dtype=qd.dtype, device="cuda:0")
    announce(f"stage_tango_aggregate {case} null={null}")
    api.tango_stage_aggregate(shape, dev_f32(theta), None if nbias is None else dev_f32(nbias),
                              qd, kd, gp, gbar, ws)
    torch.cuda.synchronize()
    got = H.unpad_rows(host(gbar), w.B, w.T)
    ref = _agg_ref(w, inp, qh, kh, g, nbias)
    H.check_stage(got, ref, w.dtype, "gbar")
    # a second call on the same workspace (counters reset) gives identical bits
    gbar2 = torch.empty_like(gbar)
    api.tango_stage_aggregate(shape, dev_f32(theta), None if nbias is None else dev_f32(nbias),
                              qd, kd, gp, gbar2, ws)
    torch.cuda.synchronize()
    assert torch.equal(gbar[: w.B * Tp].view(w.B, Tp, F)[:, : w.T], gbar2.view(w.B, Tp, F)[:, : w.T])


OUT_CASES = [
    dict(dtype="bf16", B=1, T=200, d_model=256, d_gate=256, n_heads=1, head_dim=128),
    dict(dtype="bf16", B=3, T=50, d_model=128, d_gate=512, n_heads=2, head_dim=64),
    dict(dtype="f32", B=1, T=150, d_model=128, d_gate=256, n_heads=1, head_dim=128),
]


@pytest.mark.parametrize("case", OUT_CASES, ids=lambda c: f"{c['dtype']}-B{c['B']}-T{c['T']}")
@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("op_parts", [1, 2])
def test_stage_out(case, inplace, op_parts):
    if op_parts == 2 and case["dtype"] != "bf16":
        pytest.skip("two operand parts exist for bf16 only")
    w = wl.small_workload(operand_parts=op_parts, **case)
    inp = wl.make_inputs(w)
    rng = np.random.default_rng(5)
    gbar = _q(rng.uniform(-0.3, 1.0, (w.B, w.T, w.d_gate)), w.dtype)
    v = _q(rng.standard_normal((w.B, w.T, w.d_gate)), w.dtype)
    Tp = H.padded_len(w.T)
    x = dev_tensor(inp.h, w.dtype)
    out = x if inplace else torch.empty_like(x)
    shape = api.make_shape(w.B, w.T, w.d_model, w.d_gate, w.n_heads, w.head_dim, x.dtype,
                           operand_parts=op_parts)
    announce(f"stage_out {case} inplace={inplace} op_parts={op_parts}")
    api.tango_stage_out(shape, dev_tensor(inp.w_o, w.dtype), x, dev_tensor(H.pad_rows(gbar, Tp), w.dtype),
                        dev_tensor(H.pad_rows(v, Tp), "bf16" if api.v_dtype(shape) == torch.bfloat16 else "f32"),
                        out)
    torch.cuda.synchronize()
    ref = np.asarray(inp.h, np.float64) + (gbar * v) @ np.asarray(inp.w_o, np.float64).T
    assert H.err_ratio(host(out), ref) < H.tol(w.dtype)
    # the update alone: exact up to float32 accumulation in float32; in bf16 its
    # error is set by rounding h+ (|h| >> |update|) to bf16, about 2^-9 |h+|
    delta_ref = ref - np.asarray(inp.h, np.float64)
    delta_got = host(out) - np.asarray(inp.h, np.float64)
    if w.dtype == "f32":
        H.check_stage(delta_got, delta_ref, w.dtype, "update")
    else:
        # rms of rounding h+ to bf16 (uniform, 2^-9 relative) seen on the update,
        # plus the rounding of the gated product operand (2^-9 relative)
        u = 2.0 ** -9 / math.sqrt(3.0)
        rms_d = math.sqrt(float(np.mean(delta_ref ** 2)))
        bar = 2.0 * u * (math.sqrt(float(np.mean(ref ** 2))) / rms_d + 1.0)
        r = H.rms_ratio(delta_got, delta_ref)
        print(f"update: rms ratio {r:.2e} (bar {bar:.2e})")
        assert r <= bar


SCAN_CASES = [
    dict(dtype="bf16", B=1, T=1000, d_model=128, d_gate=256, n_heads=1, head_dim=128, window=128, chunk=128),
    dict(dtype="bf16", B=1, T=700, d_model=128, d_gate=512, n_heads=2, head_dim=64, window=128, chunk=64),
    dict(dtype="bf16", B=2, T=333, d_model=128, d_gate=256, n_heads=1, head_dim=32, window=64, chunk=64),
    dict(dtype="bf16", B=1, T=100, d_model=128, d_gate=256, n_heads=1, head_dim=64, window=256, chunk=128),
    dict(dtype="bf16", B=1, T=3000, d_model=128, d_gate=1024, n_heads=2, head_dim=64, window=256, chunk=128),
    dict(dtype="f32", B=1, T=400, d_model=128, d_gate=128, n_heads=1, head_dim=64, window=128, chunk=128),
]


def _scan_ids(c):
    return f"{c['dtype']}-B{c['B']}-T{c['T']}-H{c['n_heads']}-dh{c['head_dim']}-W{c['window']}-C{c['chunk']}"


def _phi_inputs(w, inp, qh, kh):
    """Oracle features phi(sqrt(tau) q), phi(sqrt(tau) k) of the stored unit
    vectors, rounded to the dtype, in the layouts of include/tango.h."""
    tau = O.temperature(np.asarray(inp.theta, np.float64))
    st = np.sqrt(tau)[None, None, :, None]
    fq = _q(O.phi(st * qh, w.head_dim), w.dtype)          # [B, T, H, dh]
    fk = _q(O.phi(st * kh, w.head_dim), w.dtype)
    Tp, HD = H.padded_len(w.T), w.n_heads * w.head_dim
    fq_d = dev_tensor(H.permute_features(H.pad_rows(fq.reshape(w.B, w.T, HD), Tp)), w.dtype)
    fk_d = dev_tensor(H.pack_gates(H.pad_rows(fk.reshape(w.B, w.T, HD), Tp)), w.dtype)
    return fq, fk, fq_d, fk_d


@pytest.mark.parametrize("case", SCAN_CASES[:3] + SCAN_CASES[5:], ids=_scan_ids)
@pytest.mark.parametrize("op_parts", [1, 2])
def test_stage_wango_proj(case, op_parts):
    if op_parts == 2 and case["dtype"] != "bf16":
        pytest.skip("two operand parts exist for bf16 only")
    w = wl.small_workload(mode="wango", operand_parts=op_parts, **case)
    inp = wl.make_inputs(w)
    parts, *_ = _stage_inputs(w, inp)
    bw = block_weights(w, inp)
    x = dev_tensor(inp.h, w.dtype)
    shape = api.shape_of(x, bw, w.rope_base, w.rms_eps, w.operand_parts)
    Tp, HD, F = H.padded_len(w.T), w.n_heads * w.head_dim, w.d_gate
    M = w.B * Tp
    dt = x.dtype
    bufs = dict(gp=torch.full((M * F,), float("nan"), dtype=dt, device="cuda:0"),
                v=torch.full((M, F), float("nan"), dtype=api.v_dtype(shape), device="cuda:0"),
                qh=torch.full((M, HD), float("nan"), dtype=dt, device="cuda:0"),
                kh=torch.full((M, HD), float("nan"), dtype=dt, device="cuda:0"),
                fq=torch.full((M, HD), float("nan"), dtype=dt, device="cuda:0"),
                fk=torch.full((M * HD,), float("nan"), dtype=dt, device="cuda:0"))
    announce(f"stage_wango_proj {case} op_parts={op_parts}")
    api.wango_stage_proj(shape, bw, x, bufs["gp"], bufs["v"], bufs["qh"], bufs["kh"], bufs["fq"], bufs["fk"])
    torch.cuda.synchronize()
    tau = O.temperature(np.asarray(inp.theta, np.float64))
    st = np.sqrt(tau)[None, :, None]
    fq_ref = np.stack([O.phi(st * p["qh"], w.head_dim).reshape(w.T, HD) for p in parts])
    fk_ref = np.stack([O.phi(st * p["kh"], w.head_dim).reshape(w.T, HD) for p in parts])
    fq_got = H.unpad_rows(H.unpermute_features(host(bufs["fq"])), w.B, w.T)
    fk_got = H.unpad_rows(H.unpack_gates(host(bufs["fk"]), M, HD), w.B, w.T)
    H.check_stage(fq_got, fq_ref, w.dtype, "phi_q")
    H.check_stage(fk_got, fk_ref, w.dtype, "phi_k")
    g_got = H.unpad_rows(H.unpack_gates(host(bufs["gp"]), M, F), w.B, w.T)
    H.check_stage(g_got, np.stack([p["g"] for p in parts]), w.dtype, "g")


@pytest.mark.parametrize("case", SCAN_CASES, ids=_scan_ids)
def test_stage_wango_scan(case):
    w = wl.small_workload(mode="wango", **case)
    inp = wl.make_inputs(w)
    _, g, v, qh, kh = _stage_inputs(w, inp)
    gp, _, qd, kd = _upload_intermediates(w, g, v, qh, kh)
    _, _, fq_d, fk_d = _phi_inputs(w, inp, qh, kh)
    Tp, F, Hh = H.padded_len(w.T), w.d_gate, w.n_heads
    M = w.B * Tp
    shape = api.make_shape(w.B, w.T, w.d_model, F, Hh, w.head_dim, qd.dtype)
    ws = api.workspace(api.wango_workspace_size(shape, w.window, w.head_dim, w.chunk), "cuda:0")
    n_old = torch.full((M * F,), float("nan"), dtype=torch.float32, device="cuda:0")
    z_old = torch.full((M, Hh), float("nan"), dtype=torch.float32, device="cuda:0")
    announce(f"stage_wango_scan {case}")
    api.wango_stage_scan(shape, w.window, w.chunk, fq_d, fk_d, gp, n_old, z_old, ws)
    torch.cuda.synchronize()
    n_got = H.unpad_rows(H.unblock_nold(host(n_old), M, F), w.B, w.T)
    z_got = H.unpad_rows(host(z_old), w.B, w.T)
    tau = O.temperature(np.asarray(inp.theta, np.float64))
    # the state read-out at chunk boundaries: the first term of the oracle's
    # blocked running sums with blocks of `chunk` positions
    refs = [O.wango_old_blocked(qh[b], kh[b], g[b], tau, w.window, block=w.chunk, split=True)
            for b in range(w.B)]
    n_ref = np.stack([r[0] for r in refs])
    z_ref = np.stack([r[1] for r in refs])
    lim = min(w.T, w.window + w.chunk)   # destinations before this read an empty state
    assert np.all(n_got[:, :lim] == 0) and np.all(z_got[:, :lim] == 0)
    if w.T <= lim:
        return
    H.check_stage(n_got, n_ref, w.dtype, "n_old")
    H.check_stage(z_got, z_ref, w.dtype, "z_old")


BAND_CASES = [
    dict(dtype="bf16", B=1, T=1000, d_model=128, d_gate=256, n_heads=1, head_dim=128, window=128, chunk=128),
    dict(dtype="bf16", B=2, T=333, d_model=128, d_gate=512, n_heads=2, head_dim=64, window=64, chunk=64),
    dict(dtype="bf16", B=1, T=700, d_model=128, d_gate=512, n_heads=2, head_dim=64, window=192, chunk=64),
    dict(dtype="bf16", B=1, T=200, d_model=128, d_gate=256, n_heads=4, head_dim=32, window=512, chunk=128),
    # waves of 48 columns: a head of 704 ends inside a wave; two heads of 384
    dict(dtype="bf16", B=1, T=700, d_model=128, d_gate=704, n_heads=1, head_dim=128, window=192, chunk=64),
    dict(dtype="bf16", B=2, T=333, d_model=128, d_gate=768, n_heads=2, head_dim=64, window=128, chunk=64),
    dict(dtype="f32", B=1, T=300, d_model=128, d_gate=128, n_heads=1, head_dim=64, window=128, chunk=64),
    dict(dtype="f32", B=1, T=400, d_model=128, d_gate=128, n_heads=1, head_dim=64, window=128, chunk=128),
]


@pytest.mark.parametrize("case", BAND_CASES, ids=_scan_ids)
@pytest.mark.parametrize("null", [False, True])
def test_stage_wango_band(case, null):
    w = wl.small_workload(mode="wango", **case)
    inp = wl.make_inputs(w)
    nbias = np.linspace(-2.0, 0.0, w.n_heads).astype(np.float32) if null else None
    inp.null_bias = nbias
    _, g, v, qh, kh = _stage_inputs(w, inp)
    gp, _, qd, kd = _upload_intermediates(w, g, v, qh, kh)
    Tp, F, Hh = H.padded_len(w.T), w.d_gate, w.n_heads
    M = w.B * Tp
    tau = O.temperature(np.asarray(inp.theta, np.float64))
    refs = [O.wango_old_blocked(qh[b], kh[b], g[b], tau, w.window, block=w.chunk, split=True)
            for b in range(w.B)]
    n_old = np.stack([r[0] for r in refs]).astype(np.float32)
    z_old = np.stack([r[1] for r in refs]).astype(np.float32)
    nd = dev_f32(H.block_nold(H.pad_rows(n_old, Tp)))
    zd = dev_f32(H.pad_rows(z_old, Tp))
    shape = api.make_shape(w.B, w.T, w.d_model, F, Hh, w.head_dim, qd.dtype)
    gbar = torch.full((M, F), float("nan"), dtype=qd.dtype, device="cuda:0")
    announce(f"stage_wango_band {case} null={null}")
    api.wango_stage_band(shape, dev_f32(inp.theta), None if nbias is None else dev_f32(nbias),
                         w.window, w.chunk, qd, kd, gp, nd, zd, gbar)
    torch.cuda.synchronize()
    got = H.unpad_rows(host(gbar), w.B, w.T)
    ref = _agg_ref(w, inp, qh, kh, g, nbias)
    H.check_stage(got, ref, w.dtype, "gbar")
