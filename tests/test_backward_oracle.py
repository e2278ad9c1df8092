"""Pins of the backward oracle (CPU only).

The backward formulas are the derivatives of the TANGO aggregation ("TANGO:
Token-Aggregated Nonlinear Gating Operators ...", §2.1 eqs. 4-5, §2.2 eq. 6).
The pages print no gradient, so they are pinned against central differences of
the forward oracle (itself pinned by the forward tests), and the denominators
against a pure-Python loop over the definition.
"""
import math

import numpy as np
import pytest

import oracle.backward_oracle as BW
import oracle.tango_oracle as O


def _inputs(seed, T, H, dh, fh, theta_scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dh))
    k = rng.standard_normal((T, H, dh))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = rng.standard_normal((T, H * fh))
    theta = rng.uniform(0.5, 2.5, size=H) * theta_scale
    nb = rng.standard_normal(H) * 0.5
    dgbar = rng.standard_normal((T, H * fh))
    return q, k, g, theta, nb, dgbar


def _loss(q, k, g, theta, nb, dgbar):
    tau = O.temperature(theta)
    gbar = O.aggregate_direct(q, k, g, tau, nb, "tango", 0)
    return float((dgbar * gbar).sum())


def _central(f, x, idx, eps=1e-6):
    xp = x.copy()
    xm = x.copy()
    xp[idx] += eps
    xm[idx] -= eps
    return (f(xp) - f(xm)) / (2 * eps)


@pytest.mark.parametrize("null", [False, True])
@pytest.mark.parametrize("T,H,dh,fh", [(1, 1, 4, 3), (6, 2, 4, 5), (9, 1, 8, 4)])
def test_backward_equals_central_differences(null, T, H, dh, fh):
    q, k, g, theta, nb, dgbar = _inputs(7 + T + H, T, H, dh, fh)
    nb = nb if null else None
    dq, dk, dg, dtheta, dnull = BW.tango_aggregate_backward(q, k, g, theta, nb, dgbar)
    rng = np.random.default_rng(3)
    for _ in range(12):   # sampled coordinates of every input
        i = tuple(int(rng.integers(0, s)) for s in q.shape)
        assert dq[i] == pytest.approx(_central(lambda x: _loss(x, k, g, theta, nb, dgbar), q, i), rel=1e-6, abs=1e-8)
        i = tuple(int(rng.integers(0, s)) for s in k.shape)
        assert dk[i] == pytest.approx(_central(lambda x: _loss(q, x, g, theta, nb, dgbar), k, i), rel=1e-6, abs=1e-8)
        i = tuple(int(rng.integers(0, s)) for s in g.shape)
        assert dg[i] == pytest.approx(_central(lambda x: _loss(q, k, x, theta, nb, dgbar), g, i), rel=1e-6, abs=1e-8)
    for a in range(H):
        assert dtheta[a] == pytest.approx(_central(lambda x: _loss(q, k, g, x, nb, dgbar), theta, a),
                                          rel=1e-6, abs=1e-8)
        if null:
            assert dnull[a] == pytest.approx(_central(lambda x: _loss(q, k, g, theta, x, dgbar), nb, a),
                                             rel=1e-6, abs=1e-8)
    if not null:
        assert dnull is None


def test_clipped_temperature_has_no_theta_gradient():
    q, k, g, theta, nb, dgbar = _inputs(5, 5, 1, 4, 3)
    theta = np.array([math.log(20.0) + 0.3])   # tau clipped at 20
    _, _, _, dtheta, _ = BW.tango_aggregate_backward(q, k, g, theta, None, dgbar)
    assert dtheta[0] == 0.0
    assert _central(lambda x: _loss(q, k, g, x, None, dgbar), theta, 0) == pytest.approx(0.0, abs=1e-9)


def test_single_token_closed_form():
    # T = 1: gbar_0 = m g_0 / (m + c), so dg_0 = m / (m + c) dgbar_0 and the
    # score gradient is tau m c / (m + c)^2 * dgbar_0 . g_0.
    q, k, g, theta, nb, dgbar = _inputs(11, 1, 1, 4, 6)
    dq, dk, dg, _, _ = BW.tango_aggregate_backward(q, k, g, theta, nb, dgbar)
    tau = float(O.temperature(theta)[0])
    s = float(q[0, 0] @ k[0, 0])
    m = math.exp(tau * s)
    c = math.exp(float(nb[0]))
    np.testing.assert_allclose(dg[0], m / (m + c) * dgbar[0], rtol=1e-12)
    ds = tau * m * c / (m + c) ** 2 * float(dgbar[0] @ g[0])
    np.testing.assert_allclose(dq[0, 0], ds * k[0, 0], rtol=1e-10)
    np.testing.assert_allclose(dk[0, 0], ds * q[0, 0], rtol=1e-10)


def test_denominators_equal_loop_definition():
    q, k, _, theta, nb, _ = _inputs(13, 5, 2, 4, 3)
    den = BW.aggregate_denominators(q, k, theta, nb)
    tau = O.temperature(theta)
    for a in range(2):
        for i in range(5):
            ref = sum(math.exp(tau[a] * sum(q[i, a, e] * k[j, a, e] for e in range(4))) for j in range(i + 1))
            ref += (i + 1) * math.exp(nb[a])
            assert den[i, a] == pytest.approx(ref, rel=1e-13)


def _wloss(q, k, g, theta, nb, dgbar, window):
    tau = O.temperature(theta)
    gbar = O.aggregate_direct(q, k, g, tau, nb, "wango", window)
    return float((dgbar * gbar).sum())


@pytest.mark.parametrize("null", [False, True])
@pytest.mark.parametrize("T,H,dh,fh,window", [(6, 1, 4, 3, 1), (9, 2, 4, 5, 2), (12, 1, 8, 4, 4), (5, 1, 4, 3, 9)])
def test_wango_backward_equals_central_differences(null, T, H, dh, fh, window):
    q, k, g, theta, nb, dgbar = _inputs(17 + T + window, T, H, dh, fh)
    nb = nb if null else None
    dq, dk, dg, dtheta, dnull = BW.wango_aggregate_backward(q, k, g, theta, nb, dgbar, window)
    rng = np.random.default_rng(4)
    f = lambda **kw: _wloss(kw.get("q", q), kw.get("k", k), kw.get("g", g), kw.get("theta", theta),  # noqa: E731
                            kw.get("nb", nb), dgbar, window)
    for _ in range(12):
        i = tuple(int(rng.integers(0, s)) for s in q.shape)
        assert dq[i] == pytest.approx(_central(lambda x: f(q=x), q, i), rel=1e-6, abs=1e-8)
        i = tuple(int(rng.integers(0, s)) for s in k.shape)
        assert dk[i] == pytest.approx(_central(lambda x: f(k=x), k, i), rel=1e-6, abs=1e-8)
        i = tuple(int(rng.integers(0, s)) for s in g.shape)
        assert dg[i] == pytest.approx(_central(lambda x: f(g=x), g, i), rel=1e-6, abs=1e-8)
    for a in range(H):
        assert dtheta[a] == pytest.approx(_central(lambda x: f(theta=x), theta, a), rel=1e-6, abs=1e-8)
        if null:
            assert dnull[a] == pytest.approx(_central(lambda x: f(nb=x), nb, a), rel=1e-6, abs=1e-8)


def test_wango_backward_with_a_window_over_everything_is_tango():
    # W >= T: every source is in the window, so WANGO is TANGO
    q, k, g, theta, nb, dgbar = _inputs(29, 7, 2, 4, 3)
    a = BW.wango_aggregate_backward(q, k, g, theta, nb, dgbar, 7)
    b = BW.tango_aggregate_backward(q, k, g, theta, nb, dgbar)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


def test_phi_prime_is_the_derivative_of_phi():
    x = np.linspace(-3.0, 3.0, 41) + 1e-3   # away from the kink at 0
    num = (O.phi(x + 1e-6, 16) - O.phi(x - 1e-6, 16)) / 2e-6
    np.testing.assert_allclose(BW.phi_prime(x, 16), num, rtol=1e-7, atol=1e-10)
