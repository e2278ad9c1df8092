"""Parity of the WANGO aggregation backward pass (GPU, through the C ABI).

The library's gradients of sum(dgbar * gbar) are compared with the float64
oracle ``oracle.backward_oracle.wango_aggregate_backward`` (pinned by central
differences of the forward oracle) on the same bf16 inputs.  The GPU side runs
``wango_aggregate_fwd_train`` (the scan and band that also store the
denominators), then ``wango_aggregate_bwd``.  Cases cover windows of one to
five 128-row tiles, windows at or past the sequence end (no older sources),
one to three heads, d_h 32 / 64 / 128, prefix chunks 64 and 128, sequences of
up to 33 row tiles, and the null gate.

Bars as for the TANGO backward (tests/test_gpu_backward.py, derived there from
the bf16 storage of u, the gates, gbar, the weights and ds; here the older
pairs also go through bf16 features and bf16 prefix states, each one more
2^-9 rounding of a value): rms(err)/rms(ref) <= 1e-2 and max|err|/rms(ref) <=
0.3 for dq, dk, dg; dtheta within 1e-2 of sum_i |q_i . dq_i| (oracle values);
dnull within 5e-2 of the largest head's value.
"""
import math

import numpy as np
import pytest
import torch

import oracle.backward_oracle as BW
import oracle.tango_oracle as O
from cross_token_gated_amd import api
from tests import helpers as H
from tests.gpu_common import announce, dev_f32, dev_tensor, host

pytestmark = pytest.mark.gpu

BARS = (1e-2, 0.3)
THETA_BAR = 1e-2
SCALAR_BAR = 5e-2

CASES = [
    dict(B=1, T=300, H=1, dh=128, Fh=256, W=64, C=64),
    dict(B=2, T=257, H=2, dh=64, Fh=320, W=128, C=64),
    dict(B=1, T=700, H=1, dh=32, Fh=128, W=256, C=128),
    dict(B=1, T=1000, H=2, dh=64, Fh=192, W=512, C=128),
    dict(B=1, T=200, H=1, dh=64, Fh=128, W=256, C=128),   # window past the end: no older sources
    dict(B=1, T=300, H=3, dh=32, Fh=128, W=128, C=64),    # odd head count: rows of 96 q/k columns
    dict(B=1, T=200, H=16, dh=32, Fh=1780, W=64, C=64),   # the pages' geometry: heads padded to 1792
    # more than eight 128-row tiles: every row tile's near tiles are summed
    # (row tiles past the eighth once lost their window terms of dq and dk)
    dict(B=1, T=2500, H=2, dh=64, Fh=128, W=256, C=128),
    dict(B=1, T=1900, H=1, dh=32, Fh=128, W=512, C=64),
    # 33 row tiles: the tile-sum prefix and suffix run in two batches of tiles
    dict(B=1, T=4200, H=1, dh=32, Fh=64, W=128, C=64),
]


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _inputs(case, seed):
    rng = np.random.default_rng(seed)
    B, T, Hh, dh, Fh = case["B"], case["T"], case["H"], case["dh"], case["Fh"]
    q = rng.standard_normal((B, T, Hh, dh))
    k = rng.standard_normal((B, T, Hh, dh))
    q = _bf16(q / np.linalg.norm(q, axis=-1, keepdims=True))
    k = _bf16(k / np.linalg.norm(k, axis=-1, keepdims=True))
    g = _bf16(rng.standard_normal((B, T, Hh * Fh)))
    dgbar = _bf16(rng.standard_normal((B, T, Hh * Fh)))
    theta = np.linspace(math.log(5.0), math.log(15.0), Hh).astype(np.float32)
    nb = np.linspace(-1.0, 0.5, Hh).astype(np.float32)
    return q, k, g, dgbar, theta, nb


def _check(got, ref, what):
    r, m = H.rms_ratio(got, ref), H.err_ratio(got, ref)
    print(f"{what}: rms ratio {r:.2e} (bar {BARS[0]:.0e}), max ratio {m:.2e} (bar {BARS[1]:.0e})")
    assert r <= BARS[0] and m <= BARS[1], (what, r, m)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{B}-T{T}-H{H}-dh{dh}-Fh{Fh}-W{W}-C{C}".format(**c))
@pytest.mark.parametrize("null", [False, True])
def test_wango_aggregate_backward(case, null):
    B, T, Hh, dh, Fh, W, C = (case[x] for x in ("B", "T", "H", "dh", "Fh", "W", "C"))
    F, HD, Tp = Hh * Fh, Hh * dh, H.padded_len(T)
    M = B * Tp
    q, k, g, dgbar, theta, nb = _inputs(case, 23 + T + W)
    nb = nb if null else None
    shape = api.make_shape(B, T, 128, F, Hh, dh, torch.bfloat16)
    qd = dev_tensor(H.pad_rows(q.reshape(B, T, HD), Tp), "bf16")
    kd = dev_tensor(H.pad_rows(k.reshape(B, T, HD), Tp), "bf16")
    gp = dev_tensor(H.pack_gates(H.pad_heads(H.pad_rows(g, Tp), Hh, H.head_pad(Fh, True))).reshape(-1), "bf16")
    th = dev_f32(theta)
    nbd = None if nb is None else dev_f32(nb)
    dg_rows = H.pad_rows(dgbar, Tp).reshape(B, Tp, F)
    dg_rows[:, T:] = 7.0   # padded rows of the incoming gradient must be ignored
    dgd = dev_tensor(dg_rows.reshape(M, F), "bf16")
    gbar = torch.full((M, F), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    den = torch.full((M, Hh), float("nan"), dtype=torch.float32, device="cuda:0")
    wsf = api.workspace(api.wango_aggregate_fwd_train_workspace_size(shape, W, C), "cuda:0")
    announce(f"wango_aggregate_backward {case} null={null}")
    api.wango_aggregate_fwd_train(shape, W, C, th, nbd, qd, kd, gp, gbar, den, wsf)
    dq = torch.full((M, HD), float("nan"), dtype=torch.float32, device="cuda:0")
    dk = torch.full((M, HD), float("nan"), dtype=torch.float32, device="cuda:0")
    dgo = torch.full((M, F), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    dth = torch.full((Hh,), float("nan"), dtype=torch.float32, device="cuda:0")
    dnl = None if nb is None else torch.full((Hh,), float("nan"), dtype=torch.float32, device="cuda:0")
    wsb = api.workspace(api.wango_aggregate_bwd_workspace_size(shape, W, C), "cuda:0")
    wsb.fill_(0xFF)   # scratch contents must not matter
    api.wango_aggregate_bwd(shape, W, C, th, nbd, qd, kd, gp, gbar, den, dgd, dq, dk, dgo, dth, dnl, wsb)
    torch.cuda.synchronize()

    # the forward that the backward builds on
    gb_ref = np.stack([O.aggregate_direct(q[b], k[b], g[b], O.temperature(theta), nb, "wango", W)
                       for b in range(B)])
    _check(H.unpad_rows(host(gbar), B, T), gb_ref, "gbar")
    refs = [BW.wango_aggregate_backward(q[b], k[b], g[b], theta, nb, dgbar[b], W) for b in range(B)]
    dq_ref = np.stack([r[0].reshape(T, HD) for r in refs])
    dk_ref = np.stack([r[1].reshape(T, HD) for r in refs])
    dg_ref = np.stack([r[2] for r in refs])
    _check(H.unpad_rows(host(dgo), B, T), dg_ref, "dg")
    _check(H.unpad_rows(host(dq), B, T), dq_ref, "dq")
    _check(H.unpad_rows(host(dk), B, T), dk_ref, "dk")
    assert np.all(host(dq).reshape(B, Tp, HD)[:, T:] == 0)
    assert np.all(host(dk).reshape(B, Tp, HD)[:, T:] == 0)
    dth_ref = sum(r[3] for r in refs)
    scale = np.abs(np.einsum("bthe,bthe->bth", q, dq_ref.reshape(B, T, Hh, dh))).sum(axis=(0, 1))
    err = np.abs(host(dth) - dth_ref)
    print("dtheta", host(dth), dth_ref, "error / scale", err / scale)
    assert np.all(err <= THETA_BAR * scale), (err, scale)
    if nb is not None:
        dnl_ref = sum(r[4] for r in refs)
        print("dnull", host(dnl), dnl_ref)
        np.testing.assert_allclose(host(dnl), dnl_ref, rtol=SCALAR_BAR, atol=SCALAR_BAR * np.abs(dnl_ref).max())
    # the saved denominators (window, older prefix and null terms), in e^{-tau} units
    tau = O.temperature(theta)
    rows = slice(0, T)
    den_ref = np.stack([np.stack([O.pair_weights(q[b], k[b], tau, a, rows, "wango", W).sum(axis=1)
                                  + O.null_weight(nb, a, rows) for a in range(Hh)], axis=1)
                        for b in range(B)]) * np.exp(-tau)
    np.testing.assert_allclose(H.unpad_rows(host(den), B, T), den_ref, rtol=1e-2)


def test_wango_backward_rejects_unsupported():
    shape = api.make_shape(1, 256, 128, 256, 1, 64, torch.bfloat16)
    assert api.wango_aggregate_bwd_workspace_size(shape, 1024, 128) == 0   # window past 897
    assert api.wango_aggregate_bwd_workspace_size(shape, 96, 64) == 0      # chunk does not divide
    f32 = api.make_shape(1, 256, 128, 256, 1, 64, torch.float32)
    assert api.wango_aggregate_bwd_workspace_size(f32, 128, 64) == 0
