"""Pins of the decode-step oracle.

The recurrent decode state (running sums of [TANGO] §2.2 eq. 10 plus the last W
keys and gates for WANGO; every key and gate for TANGO) is checked against the
definition of a decode step, the last row of the block forward over the prefix
("TANGO: Token-Aggregated Nonlinear Gating Operators ...", §2.1 eq. 5: no source
lies after its destination), and against eq. 10 written out as a sum; the size
of the WANGO state is checked to stay constant (§6.1).
"""
import math

import numpy as np
import pytest

import oracle.decode_oracle as D
import oracle.tango_oracle as O
from tests.test_oracle_pins import rand_params, rel


def _setup(mode, window, null, rope_base, H, T=14, d=16, dh=8, fh=6, seed=0):
    rng = np.random.default_rng(seed)
    p = rand_params(rng, d, H * fh, H, dh, null=null, gain=True)
    cfg = O.BlockConfig(n_heads=H, head_dim=dh, mode=mode, window=window, rope_base=rope_base)
    h = rng.standard_normal((T, d))
    return p, cfg, h


@pytest.mark.parametrize("mode,window", [("tango", 0), ("wango", 1), ("wango", 3), ("wango", 20)])
@pytest.mark.parametrize("null", [False, True])
@pytest.mark.parametrize("rope_base", [10000.0, 0.0])
@pytest.mark.parametrize("H", [1, 2])
def test_decode_steps_equal_forward_rows(mode, window, null, rope_base, H):
    p, cfg, h = _setup(mode, window, null, rope_base, H)
    full = O.block_sequence(h, p, cfg)
    st = D.DecodeState(p, cfg)
    for i in range(h.shape[0]):
        out = st.step(h[i])
        assert rel(out, full[i]) < 1e-11, (i, rel(out, full[i]))
        assert rel(out, D.decode_reference(h[:i + 1], p, cfg)) < 1e-11


@pytest.mark.parametrize("window", [1, 4])
def test_wango_state_is_eq10_sum(window):
    p, cfg, h = _setup("wango", window, False, 10000.0, 2, T=12)
    parts = O.project(h, p, cfg)
    tau = O.temperature(p.theta)
    st = D.DecodeState(p, cfg)
    for i in range(h.shape[0]):
        st.step(h[i])
        S, z = D.wango_state_definition(parts["kh"], parts["g"], tau, window, i, cfg.head_dim)
        assert np.max(np.abs(st.S - S)) < 1e-12 and np.max(np.abs(st.z - z)) < 1e-12
        assert len(st.keys) == min(i + 1, window)


def test_wango_state_size_constant_and_tango_grows():
    W = 3
    p, cfg, h = _setup("wango", W, True, 10000.0, 2, T=12)
    st = D.DecodeState(p, cfg)
    sizes = []
    for i in range(h.shape[0]):
        st.step(h[i])
        sizes.append(st.size())
    assert len(set(sizes[W - 1:])) == 1          # constant once the window is full
    p, cfg, h = _setup("tango", 0, True, 10000.0, 2, T=6)
    st = D.DecodeState(p, cfg)
    grow = []
    for i in range(h.shape[0]):
        st.step(h[i])
        grow.append(st.size())
    assert all(b > a for a, b in zip(grow, grow[1:]))


def test_decode_matches_forward_at_distant_position():
    """RoPE at an explicit position: a decode at position P of a sequence whose
    first rows are known equals the forward row; checked at P = 40 with W = 8."""
    p, cfg, h = _setup("wango", 8, False, 10000.0, 1, T=41)
    full = O.block_sequence(h, p, cfg)
    st = D.DecodeState(p, cfg)
    for i in range(h.shape[0]):
        out = st.step(h[i])
    assert rel(out, full[-1]) < 1e-11


@pytest.mark.parametrize("mode,window", [("tango", 0), ("wango", 2)])
def test_decode_stack_equals_forward_stack(mode, window):
    p, cfg, h = _setup(mode, window, False, 10000.0, 2, T=8)
    full = O.block_stack(h[None], p, cfg, repeats=3, io_dtype="bf16")[0]
    stk = D.DecodeStack(p, cfg, repeats=3, io_dtype="bf16")
    for i in range(h.shape[0]):
        out = stk.step(h[i])
        assert rel(out, full[i]) < 1e-11


def test_pin_sees_a_late_fold():
    """A state that folds the leaving token one step late (window W + 1 in the
    recurrence while the forward uses W) must fail the forward-row pin."""
    p, cfg, h = _setup("wango", 3, False, 10000.0, 2)
    full = O.block_sequence(h, p, cfg)
    late = O.BlockConfig(n_heads=cfg.n_heads, head_dim=cfg.head_dim, mode="wango", window=4,
                         rope_base=cfg.rope_base)
    st = D.DecodeState(p, late)
    worst = max(rel(st.step(h[i]), full[i]) for i in range(h.shape[0]))
    assert worst > 1e-6
