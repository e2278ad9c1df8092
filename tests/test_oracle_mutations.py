"""Plants plausible mistakes in the oracle (on the CPU) and checks that the pins
catch every one: a dropped term, a wrong sign or index, a transposed operand."""
import math

import numpy as np
import pytest

import oracle.tango_oracle as O
import tests.test_oracle_pins as P
import tests.test_stack_oracle as SP


def _pins():
    """The pin checks, called directly; each returns normally or raises."""
    return [
        lambda: P.test_brute_force_equals_vectorized("tango", 0, True, 10000.0, 2),
        lambda: P.test_brute_force_equals_vectorized("wango", 2, True, 10000.0, 2),
        lambda: P.test_tango_aggregation_equals_sdpa(True, 2),
        lambda: P.test_tango_aggregation_equals_sdpa(False, 1),
        P.test_rmsnorm_and_silu_equal_torch,
        P.test_phi_closed_form,
        P.test_temperature_clip,
        P.test_single_token_closed_form,
        P.test_two_token_closed_form,
        lambda: P.test_running_sums_equal_pairwise_old_weights(5, 3),
        lambda: P.test_blocked_split_halves_equal_cut_pairwise(5, 8),
        P.test_wango_scan_form_equals_direct_form,
        P.test_rope_is_a_rotation_with_relative_logits,
        P.test_counts_reproduce_tables,
        lambda: SP.test_stack_sets_equal_brute_force_composition(True),
    ]


def _phi_no_eps(u, dh):
    return (O.elu(u) + 1.0) / math.sqrt(dh)


def _elu_alpha2(u):
    return np.where(u > 0, u, 2.0 * np.expm1(np.minimum(u, 0.0)))


def _null_unscaled(null_bias, head, rows):
    n = np.arange(rows.start, rows.stop, dtype=np.float64)
    if null_bias is None:
        return np.zeros_like(n)
    return np.full_like(n, math.exp(float(null_bias[head])))


def _rope_wrong_sign(u, base, positions=None):
    if base == 0:
        return u.copy()
    t, _, dh = u.shape
    inv = base ** (-2.0 * np.arange(dh // 2) / dh)
    pos = np.arange(t) if positions is None else np.asarray(positions, dtype=np.float64)
    ang = pos[:, None] * inv[None]
    c, s = np.cos(ang)[:, None], np.sin(ang)[:, None]
    out = np.empty_like(u)
    out[..., 0::2] = u[..., 0::2] * c + u[..., 1::2] * s
    out[..., 1::2] = -u[..., 0::2] * s + u[..., 1::2] * c
    return out


_orig_pair = O.pair_weights


def _window_off_by_one(qh, kh, tau, head, rows, mode, window):
    return _orig_pair(qh, kh, tau, head, rows, mode, window + 1 if mode == "wango" else window)


def _transposed_logits(qh, kh, tau, head, rows, mode, window):
    m = _orig_pair(qh, kh, tau, head, slice(0, kh.shape[0]), mode, window)
    return np.tril(m.T)[rows]


def _rms_sum(h, gain, eps):
    h = np.asarray(h, dtype=np.float64)
    x = h / np.sqrt(np.sum(h * h, axis=-1, keepdims=True) + eps)
    return x if gain is None else x * gain


def _tau_unclipped(theta):
    return np.exp(np.asarray(theta, dtype=np.float64))


_orig_blocked = O.wango_old_blocked


def _blocked_shifted(qh, kh, g, tau, window, block=64, split=False):
    return _orig_blocked(qh, kh, g, tau, window - 1 if window > 1 else window, block, split)


def _blocked_split_all_in_state(qh, kh, g, tau, window, block=64, split=False):
    """The whole older prefix attributed to the state read-out: the sum of the
    two halves is unchanged, only the split is wrong."""
    n, z, ni, zi = _orig_blocked(qh, kh, g, tau, window, block, split=True)
    if split:
        return n + ni, z + zi, np.zeros_like(ni), np.zeros_like(zi)
    return n + ni, z + zi


def _counts_no_scan(T, d, F, H, dh, vocab, repeats, mode, window=0):
    linear = T * (2 * d * F + 2 * d * H * dh + F * d)
    pairs = T * T * (H * dh + F) if mode == "tango" else T * 3 * window * (H * dh + F)
    return repeats * (linear + pairs) + T * d * vocab


_orig_stack_sets = O.block_stack_sets


def _stack_sets_one_late(h, sets, cfg, schedule, io_dtype="bf16"):
    return _orig_stack_sets(h, sets, cfg, (schedule[0],) + tuple(schedule[:-1]), io_dtype)


MUTATIONS = {
    "phi drops epsilon": ("phi", lambda u, dh: _phi_no_eps(u, dh)),
    "ELU alpha 2": ("elu", _elu_alpha2),
    "null weight not scaled by n_i": ("null_weight", _null_unscaled),
    "RoPE rotates the wrong way": ("rope", _rope_wrong_sign),
    "window one too wide": ("pair_weights", _window_off_by_one),
    "transposed logits": ("pair_weights", _transposed_logits),
    "RMSNorm uses sum for mean": ("rms_norm", _rms_sum),
    "temperature not clipped": ("temperature", _tau_unclipped),
    "blocked running sums one step late": ("wango_old_blocked", _blocked_shifted),
    "block split puts the in-block sources in the state": ("wango_old_blocked", _blocked_split_all_in_state),
    "MAC count drops the running-sum term": ("forward_macs", _counts_no_scan),
    "stack applies each set one application late": ("block_stack_sets", _stack_sets_one_late),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin caught: {name}"


def test_backward_pins_catch_a_wrong_feature_derivative(monkeypatch):
    """A planted mistake in the WANGO backward (the feature map's derivative
    taken as exp(x) on both sides of 0) fails the central-difference pin."""
    import oracle.backward_oracle as BW
    import tests.test_backward_oracle as BP
    monkeypatch.setattr(BW, "phi_prime", lambda x, dh: np.exp(np.minimum(x, 30.0)) / math.sqrt(dh))
    with pytest.raises(AssertionError):
        BP.test_wango_backward_equals_central_differences(False, 9, 2, 4, 5, 2)
