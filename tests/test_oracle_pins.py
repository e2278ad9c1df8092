"""Pins of the CPU oracle against facts fixed outside it.

Each check ties the oracle to something other than its own code: a library
routine computing the same special case (torch's scaled-dot-product attention,
rms_norm, silu), closed forms, invariants the equations imply, brute-force
loops on tiny inputs, and the counts the pages print (Tables 1 and 5, §6.1 of
"TANGO: Token-Aggregated Nonlinear Gating Operators for Natural and Formal
Language Modeling").  A mutation test at the end plants plausible mistakes in
the oracle and checks that some pin fails for each.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.tango_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_params(rng, d, F, H, dh, null=False, gain=False, theta=math.log(10.0)):
    return O.BlockParams(
        w_g=rng.standard_normal((F, d)) / math.sqrt(d),
        w_v=rng.standard_normal((F, d)) / math.sqrt(d),
        w_q=rng.standard_normal((H * dh, d)) / math.sqrt(d),
        w_k=rng.standard_normal((H * dh, d)) / math.sqrt(d),
        w_o=rng.standard_normal((d, F)) / math.sqrt(F),
        theta=np.full(H, theta) + 0.1 * np.arange(H),
        gain=(1.0 + 0.2 * rng.standard_normal(d)) if gain else None,
        null_bias=(rng.standard_normal(H) - 1.0) if null else None,
    )


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("mode,window", [("tango", 0), ("wango", 1), ("wango", 2), ("wango", 3)])
@pytest.mark.parametrize("null", [False, True])
@pytest.mark.parametrize("rope_base", [10000.0, 0.0])
@pytest.mark.parametrize("H", [1, 2])
def test_brute_force_equals_vectorized(mode, window, null, rope_base, H):
    rng = np.random.default_rng(11 + H + int(null) + window)
    d, dh, F, T = 8, 4, 6 * H, 6
    p = rand_params(rng, d, F, H, dh, null=null, gain=True)
    cfg = O.BlockConfig(n_heads=H, head_dim=dh, mode=mode, window=window, rope_base=rope_base)
    h = rng.standard_normal((T, d))
    out_b, gbar_b = O.brute_block(h, p, cfg)
    out_v, parts = O.block_sequence(h, p, cfg, return_parts=True)
    assert rel(parts["gbar"], gbar_b) < 1e-12
    assert rel(out_v, out_b) < 1e-12
    if mode == "wango":
        out_s = O.block_sequence(h, p, cfg, form="scan")
        assert rel(out_s, out_b) < 1e-12


# ------------------------------------------------ library special cases (SDPA)

def _sdpa_gbar(qh, kh, g, tau, null_bias):
    T, H, dh = qh.shape
    fh = g.shape[1] // H
    out = np.empty_like(g)
    for a in range(H):
        q = torch.from_numpy(np.ascontiguousarray(qh[:, a]))[None]
        k = torch.from_numpy(np.ascontiguousarray(kh[:, a]))[None]
        v = torch.from_numpy(np.ascontiguousarray(g[:, a * fh:(a + 1) * fh]))[None]
        if null_bias is None:
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                                 scale=float(tau[a]))
        else:
            # the null gate as one extra key of zeros with a zero value and the
            # additive logit b_a + log(i + 1)
            k = torch.cat([k, torch.zeros(1, 1, dh, dtype=k.dtype)], dim=1)
            v = torch.cat([v, torch.zeros(1, 1, fh, dtype=v.dtype)], dim=1)
            mask = torch.full((T, T + 1), float("-inf"), dtype=torch.float64)
            mask[:, :T] = torch.triu(torch.full((T, T), float("-inf"), dtype=torch.float64), 1)
            mask[:, T] = float(null_bias[a]) + torch.log(torch.arange(1, T + 1, dtype=torch.float64))
            o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask[None],
                                                                 scale=float(tau[a]))
        out[:, a * fh:(a + 1) * fh] = o[0].numpy()
    return out


@pytest.mark.parametrize("null", [False, True])
@pytest.mark.parametrize("H", [1, 2, 4])
def test_tango_aggregation_equals_sdpa(null, H):
    rng = np.random.default_rng(5 + H)
    T, dh, fh = 150, 16, 24
    qh = O.unit_normalize(rng.standard_normal((T, H, dh)))
    kh = O.unit_normalize(rng.standard_normal((T, H, dh)))
    g = rng.standard_normal((T, H * fh))
    tau = O.temperature(np.linspace(1.0, 3.5, H))
    nb = rng.standard_normal(H) if null else None
    ours = O.aggregate_direct(qh, kh, g, tau, nb, "tango", 0, row_block=37)
    ref = _sdpa_gbar(qh, kh, g, tau, nb)
    assert rel(ours, ref) < 1e-12


def test_rmsnorm_and_silu_equal_torch():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((17, 64)) * 3.0
    gain = rng.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (64,), torch.from_numpy(gain),
                                       eps=1e-6).numpy()
    assert rel(O.rms_norm(h, gain, 1e-6), ref) < 1e-14
    a = rng.standard_normal(1000) * 10
    assert rel(O.silu(a), torch.nn.functional.silu(torch.from_numpy(a)).numpy()) < 1e-14


# ---------------------------------------------------------------- closed forms

def test_phi_closed_form():
    dh = 16
    s = math.sqrt(dh)
    assert O.phi(np.array([0.0]), dh)[0] == pytest.approx((1 + 1e-4) / s, rel=1e-15)
    for u in (0.5, 3.0, 17.25):
        assert O.phi(np.array([u]), dh)[0] == pytest.approx((u + 1 + 1e-4) / s, rel=1e-15)
    for u in (-0.5, -3.0, -40.0):
        assert O.phi(np.array([u]), dh)[0] == pytest.approx((math.exp(u) + 1e-4) / s, rel=1e-13)
    assert np.all(O.phi(np.linspace(-50, 50, 1001), dh) > 0)


def test_temperature_clip():
    th = np.array([-1.0, 0.0, math.log(10.0), math.log(20.0), 5.0, 100.0])
    tau = O.temperature(th)
    np.testing.assert_allclose(tau[:3], [math.exp(-1.0), 1.0, 10.0], rtol=1e-15)
    np.testing.assert_allclose(tau[3:], 20.0, rtol=1e-15)


def test_single_token_closed_form():
    rng = np.random.default_rng(1)
    d, F, H, dh = 16, 12, 2, 4
    p = rand_params(rng, d, F, H, dh, gain=True)
    cfg = O.BlockConfig(n_heads=H, head_dim=dh)
    h = rng.standard_normal((1, d))
    x = h * p.gain / np.sqrt(np.mean(h * h) + 1e-6)
    a = x @ p.w_g.T
    g = a / (1 + np.exp(-a))
    expect = h + (g * (x @ p.w_v.T)) @ p.w_o.T
    for mode in ("tango", "wango"):
        cfg.mode, cfg.window = mode, 1
        assert rel(O.block_sequence(h, p, cfg), expect) < 1e-13


def test_two_token_closed_form():
    rng = np.random.default_rng(2)
    T, H, dh, fh = 2, 1, 8, 5
    qh = O.unit_normalize(rng.standard_normal((T, H, dh)))
    kh = O.unit_normalize(rng.standard_normal((T, H, dh)))
    g = rng.standard_normal((T, fh))
    tau = np.array([7.0])
    gbar = O.aggregate_direct(qh, kh, g, tau, None, "tango", 0)
    e10 = math.exp(7.0 * float(qh[1, 0] @ kh[0, 0]))
    e11 = math.exp(7.0 * float(qh[1, 0] @ kh[1, 0]))
    np.testing.assert_allclose(gbar[0], g[0], rtol=1e-14)
    np.testing.assert_allclose(gbar[1], (e10 * g[0] + e11 * g[1]) / (e10 + e11), rtol=1e-13)


# ------------------------------------------------------------------ invariants

def _qkg(rng, T=64, H=2, dh=8, fh=6):
    qh = O.unit_normalize(rng.standard_normal((T, H, dh)))
    kh = O.unit_normalize(rng.standard_normal((T, H, dh)))
    g = rng.standard_normal((T, H * fh))
    return qh, kh, g


@pytest.mark.parametrize("mode,window", [("tango", 0), ("wango", 5)])
def test_weights_sum_to_one(mode, window):
    rng = np.random.default_rng(4)
    qh, kh, _ = _qkg(rng)
    tau = np.array([10.0, 3.0])
    for nb in (None, np.array([-0.5, 1.0])):
        for a in range(2):
            alpha, anull = O.normalized_weights(qh, kh, tau, nb, mode, window, a)
            np.testing.assert_allclose(alpha.sum(axis=1) + anull, 1.0, rtol=1e-14)
            assert np.all(alpha >= 0)
            assert np.all(np.triu(alpha, 1) == 0)
            if nb is None:
                np.testing.assert_array_equal(anull, 0.0)


@pytest.mark.parametrize("mode,window", [("tango", 0), ("wango", 3)])
def test_position_zero_returns_own_gate(mode, window):
    rng = np.random.default_rng(6)
    qh, kh, g = _qkg(rng)
    gbar = O.aggregate_direct(qh, kh, g, np.array([10.0, 20.0]), None, mode, window)
    np.testing.assert_allclose(gbar[0], g[0], rtol=1e-14)


@pytest.mark.parametrize("mode,window", [("tango", 0), ("wango", 4)])
def test_identical_gates_aggregate_to_that_gate(mode, window):
    rng = np.random.default_rng(8)
    qh, kh, _ = _qkg(rng)
    c = rng.standard_normal(12)
    g = np.tile(c, (64, 1))
    gbar = O.aggregate_direct(qh, kh, g, np.array([10.0, 5.0]), None, mode, window)
    np.testing.assert_allclose(gbar, g, rtol=1e-13, atol=1e-14)
    nb = np.array([0.3, -2.0])
    gbar_n = O.aggregate_direct(qh, kh, g, np.array([10.0, 5.0]), nb, mode, window)
    assert np.all(np.abs(gbar_n) <= np.abs(g) + 1e-14)


def test_null_share_independent_of_prefix_length():
    # every logit equal -> null coefficient e^b / (e^l + e^b) at every i
    T, H, dh = 40, 1, 4
    qh = np.zeros((T, H, dh)); qh[..., 0] = 1.0
    kh = qh.copy()
    tau, b = np.array([10.0]), np.array([0.7])
    alpha, anull = O.normalized_weights(qh, kh, tau, b, "tango", 0, 0)
    expect = math.exp(0.7) / (math.exp(10.0) + math.exp(0.7))
    np.testing.assert_allclose(anull, expect, rtol=1e-13)


def test_wango_with_window_covering_prefix_is_tango():
    rng = np.random.default_rng(9)
    d, F, H, dh, T = 32, 16, 2, 8, 50
    p = rand_params(rng, d, F, H, dh, null=True)
    h = rng.standard_normal((T, d))
    t = O.block_sequence(h, p, O.BlockConfig(n_heads=H, head_dim=dh, mode="tango"))
    for W in (T, T + 7):
        w = O.block_sequence(h, p, O.BlockConfig(n_heads=H, head_dim=dh, mode="wango", window=W))
        np.testing.assert_array_equal(w, t)
        ws = O.block_sequence(h, p, O.BlockConfig(n_heads=H, head_dim=dh, mode="wango", window=W),
                              form="scan")
        assert rel(ws, t) < 1e-13


def test_wango_window_one_uses_exp_only_on_self():
    rng = np.random.default_rng(10)
    qh, kh, _ = _qkg(rng, T=20, H=1)
    tau = np.array([10.0])
    alpha_num = O.pair_weights(qh, kh, tau, 0, slice(0, 20), "wango", 1)
    for i in range(20):
        assert alpha_num[i, i] == pytest.approx(math.exp(10.0 * float(qh[i, 0] @ kh[i, 0])),
                                                rel=1e-14)
        fq = O.phi(math.sqrt(10.0) * qh[i, 0], 8)
        for j in range(i):
            assert alpha_num[i, j] == pytest.approx(float(fq @ O.phi(math.sqrt(10.0) * kh[j, 0], 8)),
                                                    rel=1e-13)


@pytest.mark.parametrize("W,block", [(1, 64), (5, 3), (16, 16), (33, 64), (7, 1)])
def test_running_sums_equal_pairwise_old_weights(W, block):
    rng = np.random.default_rng(12 + W)
    T, H, dh, fh = 90, 2, 8, 5
    qh, kh, g = _qkg(rng, T=T, H=H, dh=dh, fh=fh)
    tau = np.array([10.0, 2.0])
    n_run, z_run = O.wango_old_running(qh, kh, g, tau, W)
    n_blk, z_blk = O.wango_old_blocked(qh, kh, g, tau, W, block)
    # explicit pairwise phi(q).phi(k) weighting over the older prefix
    n_pw = np.zeros_like(n_run); z_pw = np.zeros_like(z_run)
    for a in range(H):
        fq = O.phi(math.sqrt(tau[a]) * qh[:, a], dh)
        fk = O.phi(math.sqrt(tau[a]) * kh[:, a], dh)
        for i in range(T):
            for j in range(0, i - W + 1):
                w = float(fq[i] @ fk[j])
                n_pw[i, a * fh:(a + 1) * fh] += w * g[j, a * fh:(a + 1) * fh]
                z_pw[i, a] += w
    assert rel(n_run, n_pw) < 1e-12 and rel(z_run, z_pw) < 1e-12
    assert rel(n_blk, n_pw) < 1e-12 and rel(z_blk, z_pw) < 1e-12


def _phi_scalar(u, dh):
    """The feature map of eq. 8 with the readings of the oracle's header, one
    value at a time: ELU with alpha 1, plus 1 + 1e-4, floored at 1e-4, over
    sqrt(d_h)."""
    elu = u if u > 0 else math.exp(u) - 1.0
    return max(elu + 1.0 + 1e-4, 1e-4) / math.sqrt(dh)


@pytest.mark.parametrize("W, block", [(1, 2), (3, 4), (4, 4), (8, 2), (5, 8), (17, 4)])
def test_blocked_split_halves_equal_cut_pairwise(W, block):
    """Each half of wango_old_blocked(split=True) on its own, against pure-Python
    pairwise loops: for a destination i >= W, with c_i = block * floor((i - W) /
    block), the state half holds the older sources j < c_i (the running sums of
    eq. 10 read at the block boundary) and the in-block half the sources
    c_i <= j <= i - W; both are zero for i < W.  (Their sum, the whole older
    prefix, is pinned by test_running_sums_equal_pairwise_old_weights.)"""
    rng = np.random.default_rng(40 + 3 * W + block)
    T, H, dh, fh = 29, 2, 4, 3
    qh, kh, g = _qkg(rng, T=T, H=H, dh=dh, fh=fh)
    tau = np.array([10.0, 3.0])
    n_st, z_st, n_in, z_in = O.wango_old_blocked(qh, kh, g, tau, W, block, split=True)
    e_st, ez_st = np.zeros((T, H * fh)), np.zeros((T, H))
    e_in, ez_in = np.zeros((T, H * fh)), np.zeros((T, H))
    for a in range(H):
        st = math.sqrt(tau[a])
        for i in range(W, T):
            c = block * ((i - W) // block)
            for j in range(0, i - W + 1):
                w = sum(_phi_scalar(st * qh[i, a, e], dh) * _phi_scalar(st * kh[j, a, e], dh)
                        for e in range(dh))
                tn, tz = (e_st, ez_st) if j < c else (e_in, ez_in)
                for f in range(fh):
                    tn[i, a * fh + f] += w * g[j, a * fh + f]
                tz[i, a] += w
    assert rel(n_st, e_st) < 1e-12 and rel(z_st, ez_st) < 1e-12
    assert rel(n_in, e_in) < 1e-12 and rel(z_in, ez_in) < 1e-12


def test_wango_scan_form_equals_direct_form():
    rng = np.random.default_rng(13)
    d, F, H, dh, T = 32, 24, 2, 8, 300
    p = rand_params(rng, d, F, H, dh, null=True)
    cfg = O.BlockConfig(n_heads=H, head_dim=dh, mode="wango", window=40)
    h = rng.standard_normal((T, d))
    assert rel(O.block_sequence(h, p, cfg, form="scan"), O.block_sequence(h, p, cfg)) < 1e-12


def test_query_key_scale_invariance():
    rng = np.random.default_rng(14)
    d, F, H, dh, T = 32, 16, 2, 8, 30
    p = rand_params(rng, d, F, H, dh)
    cfg = O.BlockConfig(n_heads=H, head_dim=dh, mode="wango", window=6)
    h = rng.standard_normal((T, d))
    base = O.block_sequence(h, p, cfg)
    p2 = O.BlockParams(**{**p.__dict__, "w_q": 3.5 * p.w_q, "w_k": 0.25 * p.w_k})
    assert rel(O.block_sequence(h, p2, cfg), base) < 1e-12


def test_update_linear_in_wo_and_wv():
    rng = np.random.default_rng(15)
    d, F, H, dh, T = 32, 16, 2, 8, 30
    p = rand_params(rng, d, F, H, dh)
    cfg = O.BlockConfig(n_heads=H, head_dim=dh)
    h = rng.standard_normal((T, d))
    delta = O.block_sequence(h, p, cfg) - h
    p2 = O.BlockParams(**{**p.__dict__, "w_o": 2.0 * p.w_o})
    p3 = O.BlockParams(**{**p.__dict__, "w_v": -3.0 * p.w_v})
    assert rel(O.block_sequence(h, p2, cfg) - h, 2.0 * delta) < 1e-12
    assert rel(O.block_sequence(h, p3, cfg) - h, -3.0 * delta) < 1e-12


@pytest.mark.parametrize("mode,window", [("tango", 0), ("wango", 4)])
def test_causality(mode, window):
    rng = np.random.default_rng(16)
    d, F, H, dh, T = 32, 16, 2, 8, 40
    p = rand_params(rng, d, F, H, dh, null=True)
    cfg = O.BlockConfig(n_heads=H, head_dim=dh, mode=mode, window=window)
    h = rng.standard_normal((T, d))
    base = O.block_sequence(h, p, cfg)
    h2 = h.copy(); h2[25] += 1.0
    pert = O.block_sequence(h2, p, cfg)
    np.testing.assert_array_equal(pert[:25], base[:25])
    assert np.max(np.abs(pert[25:] - base[25:])) > 1e-6


# ------------------------------------------------------------------------ RoPE

def test_rope_is_a_rotation_with_relative_logits():
    rng = np.random.default_rng(17)
    T, H, dh = 50, 2, 16
    u = rng.standard_normal((T, H, dh))
    r = O.rope(u, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(r[0], u[0])
    np.testing.assert_array_equal(O.rope(u, 0.0), u)
    # constant rows: the rotated q.k depends only on i - j (Toeplitz)
    q = np.tile(rng.standard_normal((1, 1, dh)), (T, 1, 1))
    k = np.tile(rng.standard_normal((1, 1, dh)), (T, 1, 1))
    L = O.rope(q, 10000.0)[:, 0] @ O.rope(k, 10000.0)[:, 0].T
    for off in range(-5, 6):
        dg = np.diagonal(L, off)
        np.testing.assert_allclose(dg, dg[0], rtol=1e-10, atol=1e-12)


# ------------------------------------------------- stacking and I/O rounding

def test_stack_rounds_between_applications():
    rng = np.random.default_rng(18)
    d, F, H, dh, T = 32, 16, 1, 8, 20
    p = rand_params(rng, d, F, H, dh)
    cfg = O.BlockConfig(n_heads=H, head_dim=dh)
    h = rng.standard_normal((2, T, d))
    two = O.block_stack(h, p, cfg, repeats=2, io_dtype="bf16")
    one = O.block_stack(h, p, cfg, repeats=1)
    mid = O.round_to_dtype(one, "bf16")
    np.testing.assert_array_equal(two, O.block_stack(mid, p, cfg, repeats=1))
    # bf16 rounding: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    np.testing.assert_array_equal(O.round_to_dtype(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8]), "bf16"),
                                  [1.0, 1 + 2 ** -6])


# ------------------------------------------------- the pages' printed counts

def test_counts_reproduce_tables():
    gold = json.load(open(os.path.join(GOLDEN, "paper_counts.json")))
    g = gold["geometry"]
    assert O.block_param_count(g["d"], g["F"], g["H"], g["dh"]) == gold["nonembedding_params"]["value"]
    for mode in ("tango", "wango"):
        m = O.forward_macs(g["T_fineweb"], g["d"], g["F"], g["H"], g["dh"], g["vocab_gpt2"],
                           g["repeats"], mode, g["window"])
        assert abs(m - gold["macs_fineweb"][mode]) <= gold["macs_fineweb"]["abs_tol"]
        m = O.forward_macs(g["T_dmmath"], g["d"], g["F"], g["H"], g["dh"], g["vocab_dmmath"],
                           g["repeats"], mode, g["window"])
        assert abs(m - gold["macs_dmmath"][mode]) <= gold["macs_dmmath"]["abs_tol"]
