"""Plain float64 CPU oracle of the TANGO aggregation backward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the HIP library
never calls it and shares no code with it.

What it differentiates: the TANGO aggregation of "TANGO: Token-Aggregated
Nonlinear Gating Operators ..." §2.1 eqs. 4-5 and §2.2 eq. 6, per head a,

    gbar_i = sum_{j<=i} m_ij g_j / (sum_{j<=i} m_ij + c_i),
    m_ij = exp(tau s_ij),  s_ij = q_i . k_j,  c_i = n_i exp(b),  n_i = i + 1,
    tau = exp(min(theta, log 20)),

with q and k taken as free inputs (the unit vectors the forward feeds in; the
normalisation and RoPE before them are ordinary chain-rule steps of the
projections).  The pages train this block (§3, training recipe) but print no
gradient; the formulas below are the plain derivatives of the expression above,
written out for a linear loss L = sum(dgbar * gbar):

    u_i     = dgbar_i / den_i                 (den_i = sum_j m_ij + c_i)
    delta_i = -u_i . gbar_i                   (dL/dden_i)
    dg_j    = sum_{i>=j} m_ij u_i
    dm_ij   = u_i . g_j + delta_i             (j <= i)
    ds_ij   = tau m_ij dm_ij                  (dL/ds_ij)
    dq_i    = sum_j ds_ij k_j,   dk_j = sum_i ds_ij q_i
    dtau    = sum_ij dm_ij m_ij s_ij = sum_ij ds_ij s_ij / tau
    dtheta  = tau dtau  when theta < log 20, else 0
    db      = sum_i delta_i c_i

For WANGO (§2.2 eqs. 7-10) the weight of an older source j <= i - W is
p_i . a_j with p = phi(sqrt(tau) q), a = phi(sqrt(tau) k) (eq. 8), and the
window sources keep exp(tau s_ij).  With the same u, delta and dm_ij = u_i . g_j
+ delta_i over every visible pair:

    ds_ij  = tau m_ij dm_ij          (window pairs)
    dP_ij  = dm_ij                   (older pairs: dL/d(p_i . a_j))
    dp_i   = sum_j dP_ij a_j,   da_j = sum_i dP_ij p_i
    dq_i   = sum_j ds_ij k_j + sqrt(tau) phi'(sqrt(tau) q_i) * dp_i   (and dk alike)
    dtau  += sum_i dp_i . (phi'(sqrt(tau) q_i) * q_i) / (2 sqrt(tau))  (and the keys' term)

They are pinned against central differences of the forward oracle
(``tango_oracle.aggregate_direct``), not against themselves.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .tango_oracle import LOG_TAU_MAX, phi, temperature


def tango_aggregate_backward(qh: np.ndarray, kh: np.ndarray, g: np.ndarray, theta: np.ndarray,
                             null_bias: Optional[np.ndarray], dgbar: np.ndarray):
    """Gradients of sum(dgbar * gbar) for the TANGO aggregation.

    qh, kh: [T, H, d_h]; g, dgbar: [T, F] with F/H columns per head; theta [H];
    null_bias [H] or None.  Returns (dq [T,H,d_h], dk [T,H,d_h], dg [T,F],
    dtheta [H], dnull [H] or None), all float64."""
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    dgbar = np.asarray(dgbar, dtype=np.float64)
    t_len, H, _ = qh.shape
    F = g.shape[1]
    fh = F // H
    tau = temperature(theta)
    dq = np.zeros_like(qh)
    dk = np.zeros_like(kh)
    dg = np.zeros_like(g)
    dtheta = np.zeros(H)
    dnull = np.zeros(H) if null_bias is not None else None
    causal = np.arange(t_len)[None, :] <= np.arange(t_len)[:, None]
    n_i = np.arange(t_len, dtype=np.float64) + 1.0
    for a in range(H):
        qa, ka = qh[:, a, :], kh[:, a, :]
        ga = g[:, a * fh:(a + 1) * fh]
        dga = dgbar[:, a * fh:(a + 1) * fh]
        s = qa @ ka.T
        m = np.where(causal, np.exp(tau[a] * s), 0.0)
        c = n_i * math.exp(float(null_bias[a])) if null_bias is not None else np.zeros(t_len)
        den = m.sum(axis=1) + c
        gbar = (m @ ga) / den[:, None]
        u = dga / den[:, None]
        delta = -(u * gbar).sum(axis=1)
        dg[:, a * fh:(a + 1) * fh] = m.T @ u
        dm = np.where(causal, u @ ga.T + delta[:, None], 0.0)
        ds = tau[a] * m * dm
        dq[:, a, :] = ds @ ka
        dk[:, a, :] = ds.T @ qa
        dtau = float((ds * s).sum()) / tau[a]
        dtheta[a] = tau[a] * dtau if float(theta[a]) < LOG_TAU_MAX else 0.0
        if dnull is not None:
            dnull[a] = float((delta * c).sum())
    return dq, dk, dg, dtheta, dnull


def aggregate_denominators(qh: np.ndarray, kh: np.ndarray, theta: np.ndarray,
                           null_bias: Optional[np.ndarray]) -> np.ndarray:
    """den_i of every head, [T, H] float64: sum_{j<=i} exp(tau q_i.k_j) + n_i exp(b)
    ([TANGO] §2.1 eq. 5, the denominator of the TANGO ratio)."""
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    t_len, H, _ = qh.shape
    tau = temperature(theta)
    causal = np.arange(t_len)[None, :] <= np.arange(t_len)[:, None]
    n_i = np.arange(t_len, dtype=np.float64) + 1.0
    out = np.empty((t_len, H))
    for a in range(H):
        m = np.where(causal, np.exp(tau[a] * (qh[:, a, :] @ kh[:, a, :].T)), 0.0)
        c = n_i * math.exp(float(null_bias[a])) if null_bias is not None else 0.0
        out[:, a] = m.sum(axis=1) + c
    return out


def phi_prime(x: np.ndarray, head_dim: int) -> np.ndarray:
    """Derivative of the feature map phi of [TANGO] §2.2 eq. 8: ELU' / sqrt(d_h),
    i.e. 1 / sqrt(d_h) for x > 0 and exp(x) / sqrt(d_h) otherwise (the floor at
    eps of eq. 8 is never the active branch, since ELU + 1 > 0)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0))) / math.sqrt(head_dim)


def wango_aggregate_backward(qh: np.ndarray, kh: np.ndarray, g: np.ndarray, theta: np.ndarray,
                             null_bias: Optional[np.ndarray], dgbar: np.ndarray, window: int):
    """Gradients of sum(dgbar * gbar) for the WANGO aggregation ([TANGO] §2.2
    eqs. 7-10: window weights exp(tau s) over L_i = {i-W+1 .. i}, older sources
    weighted by phi(sqrt(tau) q_i) . phi(sqrt(tau) k_j), one joint normalisation
    with the null term).  Arguments and results as tango_aggregate_backward."""
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    dgbar = np.asarray(dgbar, dtype=np.float64)
    t_len, H, dh = qh.shape
    F = g.shape[1]
    fh = F // H
    tau = temperature(theta)
    dq = np.zeros_like(qh)
    dk = np.zeros_like(kh)
    dg = np.zeros_like(g)
    dtheta = np.zeros(H)
    dnull = np.zeros(H) if null_bias is not None else None
    ii = np.arange(t_len)[:, None]
    jj = np.arange(t_len)[None, :]
    causal = jj <= ii
    band = causal & (jj >= ii - window + 1)
    older = jj <= ii - window
    n_i = np.arange(t_len, dtype=np.float64) + 1.0
    for a in range(H):
        qa, ka = qh[:, a, :], kh[:, a, :]
        ga = g[:, a * fh:(a + 1) * fh]
        dga = dgbar[:, a * fh:(a + 1) * fh]
        st = math.sqrt(tau[a])
        p, ak = phi(st * qa, dh), phi(st * ka, dh)
        s = qa @ ka.T
        m_band = np.where(band, np.exp(tau[a] * s), 0.0)
        m_old = np.where(older, p @ ak.T, 0.0)
        m = m_band + m_old
        c = n_i * math.exp(float(null_bias[a])) if null_bias is not None else np.zeros(t_len)
        den = m.sum(axis=1) + c
        gbar = (m @ ga) / den[:, None]
        u = dga / den[:, None]
        delta = -(u * gbar).sum(axis=1)
        dg[:, a * fh:(a + 1) * fh] = m.T @ u
        dm = np.where(causal, u @ ga.T + delta[:, None], 0.0)
        ds = tau[a] * m_band * dm
        dP = np.where(older, dm, 0.0)
        dp, da = dP @ ak, dP.T @ p
        fq, fk = phi_prime(st * qa, dh), phi_prime(st * ka, dh)
        dq[:, a, :] = ds @ ka + st * fq * dp
        dk[:, a, :] = ds.T @ qa + st * fk * da
        dtau = float((ds * s).sum()) / tau[a] + \
            (float((dp * fq * qa).sum()) + float((da * fk * ka).sum())) / (2.0 * st)
        dtheta[a] = tau[a] * dtau if float(theta[a]) < LOG_TAU_MAX else 0.0
        if dnull is not None:
            dnull[a] = float((delta * c).sum())
    return dq, dk, dg, dtheta, dnull
