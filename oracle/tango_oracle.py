"""Plain float64 CPU oracle of the TANGO / WANGO gated-aggregation block forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never calls it and shares no code with
it; the two meet only in the seeded input generator, which holds none of the
method's arithmetic.

Source of every formula: "TANGO: Token-Aggregated Nonlinear Gating Operators for
Natural and Formal Language Modeling" (arXiv 2608.22117 v1), cited below as
[TANGO] with its section and equation numbers:

* §2.1, eq. 2   gate g_i = SiLU(W_g x_i) and features v_i = W_v x_i, with
                x_i = RMSNorm(h_i)
* §2.1, eq. 3   residual update h+_i = h_i + W_o(gbar_i * v_i)
* §2.1          H heads; gate split into F/H-wide pieces; per-head query/key of
                width d_h; RoPE, then unit-length normalisation of q and k
* §2.1, eq. 4   logit l_ija = tau_a q_ia . k_ja,  tau_a = exp(min(theta_a, log 20))
* §2.1, eq. 5   normalised aggregation with the null gate of weight n_i exp(b_a)
* §2.2, eq. 6   TANGO full-prefix weights m = exp(l)
* §2.2, eq. 7   WANGO trailing window L_i and older prefix G_i
* §2.2, eq. 8   positive feature map phi(u) = max(ELU(u) + 1 + eps, eps)/sqrt(d_h)
* §2.2, eq. 9   older-source weight phi(sqrt(tau) q)^T phi(sqrt(tau) k)
* §2.2, eq. 10  running sums S = sum phi(sqrt(tau) k) g^T and z = sum phi(sqrt(tau) k),
                updated as tokens leave the window; prefix sums in blocks of 64
* §2.3, eq. 11  one block applied R times with shared weights

Readings taken where the text leaves a step open (each is also listed in the
design notes of the repository):

* RMSNorm: x = gain * h / sqrt(mean(h^2) + eps) with eps = 1e-6; gain = 1 when
  not given.
* Heads: q/k columns and gate columns are split into contiguous per-head blocks.
* RoPE: interleaved pairs (u_2c, u_2c+1) rotated by angle i * base^(-2c/d_h),
  0-based position i restarting in every batch row, base 10000; base 0 = off.
  (The pairing and base are not stated in the text: parity unpinned for them.)
* Unit normalisation: u / max(||u||, 1e-12).
* ELU uses alpha = 1.
* n_i = i + 1 (0-based) in both modes; older WANGO sources count toward n_i.
* Masking is causal per batch row, no document resets.
* Between stacked applications the residual stream is rounded to the I/O dtype
  (round to nearest even), as it is stored there between calls.

No max subtraction is used: q and k have unit norm so |l| <= tau <= 20 and
exp(l) is far from float64 overflow.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

PHI_EPS = 1e-4           # [TANGO] §2.2, eq. 8
LOG_TAU_MAX = math.log(20.0)   # [TANGO] §2.1, eq. 4
NORM_FLOOR = 1e-12       # reading: guard for a zero-length q or k
DEFAULT_RMS_EPS = 1e-6   # reading: RMSNorm epsilon


@dataclass
class BlockParams:
    """Weights of one block, float64, row-major as in the equations.

    w_g, w_v: [F, d]; w_q, w_k: [H*d_h, d]; w_o: [d, F]; gain: [d] or None;
    theta: [H] (temperature logits); null_bias: [H] or None (null gate off).
    """
    w_g: np.ndarray
    w_v: np.ndarray
    w_q: np.ndarray
    w_k: np.ndarray
    w_o: np.ndarray
    theta: np.ndarray
    gain: Optional[np.ndarray] = None
    null_bias: Optional[np.ndarray] = None


@dataclass
class BlockConfig:
    """Shape and mode of one block application."""
    n_heads: int
    head_dim: int
    mode: str = "tango"          # "tango" or "wango"
    window: int = 0              # WANGO window W (counts the destination itself)
    rope_base: float = 10000.0   # 0 disables RoPE
    rms_eps: float = DEFAULT_RMS_EPS
    extra: dict = field(default_factory=dict)


# --------------------------------------------------------------------------
# Elementwise pieces
# --------------------------------------------------------------------------

def rms_norm(h: np.ndarray, gain: Optional[np.ndarray], eps: float) -> np.ndarray:
    """x = gain * h / sqrt(mean(h^2) + eps) over the last axis ([TANGO] §2.1)."""
    h = np.asarray(h, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    x = h * r
    if gain is not None:
        x = x * np.asarray(gain, dtype=np.float64)
    return x


def silu(a: np.ndarray) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a) ([TANGO] §2.1, eq. 2)."""
    return a / (1.0 + np.exp(-a))


def elu(u: np.ndarray) -> np.ndarray:
    """ELU with alpha = 1: u for u > 0, exp(u) - 1 otherwise."""
    return np.where(u > 0, u, np.expm1(np.minimum(u, 0.0)))


def phi(u: np.ndarray, head_dim: int) -> np.ndarray:
    """Positive feature map of [TANGO] §2.2, eq. 8, applied elementwise."""
    return np.maximum(elu(u) + 1.0 + PHI_EPS, PHI_EPS) / math.sqrt(head_dim)


def temperature(theta: np.ndarray) -> np.ndarray:
    """tau_a = exp(min(theta_a, log 20)) ([TANGO] §2.1, eq. 4)."""
    return np.exp(np.minimum(np.asarray(theta, dtype=np.float64), LOG_TAU_MAX))


def rope(u: np.ndarray, base: float, positions: Optional[np.ndarray] = None) -> np.ndarray:
    """Rotary position embedding on u [T, H, d_h] ([TANGO] §2.1, applied before
    unit normalisation).  Reading: interleaved pairs (2c, 2c+1), angle
    i * base^(-2c/d_h) at 0-based position i (row t sits at position t unless
    ``positions`` gives the position of every row).  base == 0 returns u unchanged."""
    if base == 0:
        return u.copy()
    t_len, _, dh = u.shape
    pos = np.arange(t_len, dtype=np.float64) if positions is None else \
        np.asarray(positions, dtype=np.float64)
    c = np.arange(dh // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * c / dh)                      # [d_h/2]
    ang = pos[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    u0 = u[..., 0::2]
    u1 = u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = u0 * cos - u1 * sin
    out[..., 1::2] = u0 * sin + u1 * cos
    return out


def unit_normalize(u: np.ndarray) -> np.ndarray:
    """u / max(||u||, 1e-12) over the last axis ([TANGO] §2.1: q and k are
    normalised to unit length)."""
    n = np.sqrt(np.sum(u * u, axis=-1, keepdims=True))
    return u / np.maximum(n, NORM_FLOOR)


# --------------------------------------------------------------------------
# Projections of one sequence
# --------------------------------------------------------------------------

def project(h: np.ndarray, p: BlockParams, cfg: BlockConfig,
            positions: Optional[np.ndarray] = None) -> dict:
    """One sequence h [T, d] -> x, g, v [T, F], unit q, k [T, H, d_h]
    ([TANGO] §2.1, eq. 2 and the head paragraph that follows eq. 3).  Row t
    sits at position t unless ``positions`` says otherwise (only RoPE sees it)."""
    t_len = h.shape[0]
    H, dh = cfg.n_heads, cfg.head_dim
    x = rms_norm(h, p.gain, cfg.rms_eps)
    a = x @ p.w_g.T
    g = silu(a)
    v = x @ p.w_v.T
    q = (x @ p.w_q.T).reshape(t_len, H, dh)
    k = (x @ p.w_k.T).reshape(t_len, H, dh)
    q = unit_normalize(rope(q, cfg.rope_base, positions))
    k = unit_normalize(rope(k, cfg.rope_base, positions))
    return {"x": x, "a": a, "g": g, "v": v, "qh": q, "kh": k}


# --------------------------------------------------------------------------
# Aggregation: pairwise (direct) form
# --------------------------------------------------------------------------

def pair_weights(qh: np.ndarray, kh: np.ndarray, tau: np.ndarray, head: int,
                 rows: slice, mode: str, window: int) -> np.ndarray:
    """Unnormalised source weights m_ija for destinations ``rows`` of one head,
    all sources 0..T-1 (zero where j > i).

    TANGO: exp(l_ija) for every j <= i ([TANGO] §2.2, eq. 6).
    WANGO: exp(l_ija) for j in the window L_i, and phi(sqrt(tau) q)^T phi(sqrt(tau) k)
    for j in the older prefix G_i ([TANGO] §2.2, eqs. 7 and 9)."""
    t_len, _, dh = kh.shape
    i_idx = np.arange(rows.start, rows.stop)[:, None]
    j_idx = np.arange(t_len)[None, :]
    qa = qh[rows, head, :]
    ka = kh[:, head, :]
    ta = tau[head]
    m = np.exp(ta * (qa @ ka.T))
    causal = j_idx <= i_idx
    if mode == "tango":
        return np.where(causal, m, 0.0)
    if mode != "wango":
        raise ValueError(f"unknown mode {mode!r}")
    in_window = causal & (j_idx >= i_idx - window + 1)
    older = j_idx <= i_idx - window          # G_i = {j : 0 <= j < i - W + 1}
    st = math.sqrt(ta)
    m_old = phi(st * qa, dh) @ phi(st * ka, dh).T
    return np.where(in_window, m, np.where(older, m_old, 0.0))


def null_weight(null_bias: Optional[np.ndarray], head: int, rows: slice) -> np.ndarray:
    """n_i exp(b_a) with n_i = i + 1 visible sources ([TANGO] §2.1, eq. 5);
    zero when the null gate is off."""
    n_i = np.arange(rows.start, rows.stop, dtype=np.float64) + 1.0
    if null_bias is None:
        return np.zeros_like(n_i)
    return n_i * math.exp(float(null_bias[head]))


def aggregate_direct(qh: np.ndarray, kh: np.ndarray, g: np.ndarray, tau: np.ndarray,
                     null_bias: Optional[np.ndarray], mode: str, window: int,
                     row_block: int = 512) -> np.ndarray:
    """gbar [T, F] from the pairwise weights, one head at a time, in blocks of
    destination rows ([TANGO] §2.1, eq. 5)."""
    t_len, H, _ = qh.shape
    F = g.shape[1]
    fh = F // H
    gbar = np.empty((t_len, F), dtype=np.float64)
    for a in range(H):
        ga = g[:, a * fh:(a + 1) * fh]
        for r0 in range(0, t_len, row_block):
            rows = slice(r0, min(t_len, r0 + row_block))
            m = pair_weights(qh, kh, tau, a, rows, mode, window)
            num = m @ ga
            den = m.sum(axis=1) + null_weight(null_bias, a, rows)
            gbar[rows, a * fh:(a + 1) * fh] = num / den[:, None]
    return gbar


def normalized_weights(qh, kh, tau, null_bias, mode, window, head):
    """Normalised coefficients alpha_ija (all destinations, one head) and the
    null coefficient, for the invariant checks ([TANGO] §2.1, eq. 5)."""
    t_len = qh.shape[0]
    rows = slice(0, t_len)
    m = pair_weights(qh, kh, tau, head, rows, mode, window)
    nw = null_weight(null_bias, head, rows)
    den = m.sum(axis=1) + nw
    return m / den[:, None], nw / den


# --------------------------------------------------------------------------
# WANGO older prefix: running sums ([TANGO] §2.2, eq. 10)
# --------------------------------------------------------------------------

def wango_old_running(qh, kh, g, tau, window):
    """Older-prefix numerator N_old [T, F] and denominator Z_old [T, H] with the
    running sums of eq. 10 advanced one token at a time: before destination i
    is read, the token i - W (the one that left the window) is added to S and z.
    Slow; for small T."""
    t_len, H, dh = qh.shape
    F = g.shape[1]
    fh = F // H
    n_old = np.zeros((t_len, F))
    z_old = np.zeros((t_len, H))
    for a in range(H):
        st = math.sqrt(tau[a])
        fq = phi(st * qh[:, a, :], dh)
        fk = phi(st * kh[:, a, :], dh)
        ga = g[:, a * fh:(a + 1) * fh]
        S = np.zeros((dh, fh))
        z = np.zeros(dh)
        for i in range(t_len):
            j = i - window
            if j >= 0:
                S += np.outer(fk[j], ga[j])
                z += fk[j]
            n_old[i, a * fh:(a + 1) * fh] = fq[i] @ S
            z_old[i, a] = fq[i] @ z
    return n_old, z_old


def wango_old_blocked(qh, kh, g, tau, window, block=64, split=False):
    """Same quantities as :func:`wango_old_running`, with the prefix sums taken
    in blocks of ``block`` source positions (the text uses blocks of 64): the
    state S, z holds every source before the block; within the block, a source
    j is visible to destination i exactly when j <= i - W.

    With split=True the two terms are returned apart: (n_state, z_state) read
    out of the state at the block boundary, and (n_intra, z_intra) from the
    sources of the block itself; their sums are the two returned otherwise."""
    t_len, H, dh = qh.shape
    F = g.shape[1]
    fh = F // H
    n_old = np.zeros((t_len, F))
    z_old = np.zeros((t_len, H))
    n_in = np.zeros((t_len, F))
    z_in = np.zeros((t_len, H))
    for a in range(H):
        st = math.sqrt(tau[a])
        fq = phi(st * qh[:, a, :], dh)
        fk = phi(st * kh[:, a, :], dh)
        ga = g[:, a * fh:(a + 1) * fh]
        S = np.zeros((dh, fh))
        z = np.zeros(dh)
        for s0 in range(0, t_len, block):
            s1 = min(t_len, s0 + block)
            d0, d1 = s0 + window, min(t_len, s1 + window)
            if d0 < t_len:
                # destinations whose boundary i - W falls inside this source block
                sel = (np.arange(s0, s1)[None, :] <= np.arange(d0, d1)[:, None] - window)
                w = np.where(sel, fq[d0:d1] @ fk[s0:s1].T, 0.0)
                n_old[d0:d1, a * fh:(a + 1) * fh] = fq[d0:d1] @ S
                z_old[d0:d1, a] = fq[d0:d1] @ z
                n_in[d0:d1, a * fh:(a + 1) * fh] = w @ ga[s0:s1]
                z_in[d0:d1, a] = w.sum(axis=1)
            S += fk[s0:s1].T @ ga[s0:s1]
            z += fk[s0:s1].sum(axis=0)
    if split:
        return n_old, z_old, n_in, z_in
    return n_old + n_in, z_old + z_in


def wango_band(qh, kh, g, tau, window):
    """Window-only numerator and denominator (exp weights over L_i), as [T, F]
    and [T, H] ([TANGO] §2.2, eqs. 6-7 restricted to the window)."""
    t_len, H, _ = qh.shape
    F = g.shape[1]
    fh = F // H
    num = np.zeros((t_len, F))
    den = np.zeros((t_len, H))
    for a in range(H):
        ga = g[:, a * fh:(a + 1) * fh]
        for i0 in range(0, t_len, 256):
            i1 = min(t_len, i0 + 256)
            j0 = max(0, i0 - window + 1)
            ii = np.arange(i0, i1)[:, None]
            jj = np.arange(j0, i1)[None, :]
            m = np.exp(tau[a] * (qh[i0:i1, a] @ kh[j0:i1, a].T))
            m = np.where((jj <= ii) & (jj >= ii - window + 1), m, 0.0)
            num[i0:i1, a * fh:(a + 1) * fh] = m @ ga[j0:i1]
            den[i0:i1, a] = m.sum(axis=1)
    return num, den


def aggregate_wango_scan(qh, kh, g, tau, null_bias, window, block=64):
    """WANGO gbar via the window band plus the blocked running sums; the window,
    older and null terms share one numerator and one denominator
    ([TANGO] §2.2, the joint-normalisation paragraph)."""
    t_len, H, _ = qh.shape
    F = g.shape[1]
    fh = F // H
    num, den = wango_band(qh, kh, g, tau, window)
    n_old, z_old = wango_old_blocked(qh, kh, g, tau, window, block)
    gbar = np.empty((t_len, F))
    rows = slice(0, t_len)
    for a in range(H):
        d = den[:, a] + z_old[:, a] + null_weight(null_bias, a, rows)
        gbar[:, a * fh:(a + 1) * fh] = (num[:, a * fh:(a + 1) * fh]
                                        + n_old[:, a * fh:(a + 1) * fh]) / d[:, None]
    return gbar


# --------------------------------------------------------------------------
# Block and stack
# --------------------------------------------------------------------------

def block_sequence(h: np.ndarray, p: BlockParams, cfg: BlockConfig,
                   form: str = "direct", return_parts: bool = False):
    """One block on one sequence h [T, d] ([TANGO] §2.1, eqs. 2-5 and 3).

    form = "direct" uses the pairwise weights; form = "scan" (WANGO only) uses
    the window band plus the running sums of eq. 10."""
    parts = project(h, p, cfg)
    tau = temperature(p.theta)
    if form == "direct" or cfg.mode == "tango":
        gbar = aggregate_direct(parts["qh"], parts["kh"], parts["g"], tau,
                                p.null_bias, cfg.mode, cfg.window)
    elif form == "scan":
        gbar = aggregate_wango_scan(parts["qh"], parts["kh"], parts["g"], tau,
                                    p.null_bias, cfg.window)
    else:
        raise ValueError(form)
    out = h + (gbar * parts["v"]) @ p.w_o.T
    if return_parts:
        parts["gbar"] = gbar
        parts["tau"] = tau
        return out, parts
    return out


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the I/O dtype and back: "f32" via float32 (round
    to nearest even); "bf16" via float32 and then bfloat16 (round to nearest
    even, done by torch's CPU conversion)."""
    a32 = np.asarray(a, dtype=np.float32)
    if dtype == "f32":
        return a32.astype(np.float64)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(a32)).to(torch.bfloat16) \
            .to(torch.float64).numpy()
    raise ValueError(dtype)


def block_stack(h: np.ndarray, p: BlockParams, cfg: BlockConfig, repeats: int = 1,
                io_dtype: str = "bf16", form: str = "direct") -> np.ndarray:
    """h [B, T, d] -> output after ``repeats`` applications of one shared block
    ([TANGO] §2.3, eq. 11).  Between applications the stream is rounded to the
    I/O dtype; the last output is returned unrounded in float64."""
    cur = np.asarray(h, dtype=np.float64)
    for r in range(repeats):
        nxt = np.stack([block_sequence(cur[b], p, cfg, form=form)
                        for b in range(cur.shape[0])])
        cur = nxt if r == repeats - 1 else round_to_dtype(nxt, io_dtype)
    return cur


def block_stack_sets(h: np.ndarray, sets: list, cfg: BlockConfig, schedule,
                     io_dtype: str = "bf16") -> np.ndarray:
    """h [B, T, d] -> output of a stack whose application r uses parameter set
    ``sets[schedule[r]]`` (the three-set model of "TANGO: Treating Tokens as
    Operators", abstract and Table 2, gives the first, the middle and the last
    applications their own gated-projection set).  Each application is one
    block of [TANGO] §2.1; the stream is rounded to the I/O dtype between
    applications as in :func:`block_stack`."""
    cur = np.asarray(h, dtype=np.float64)
    n = len(schedule)
    for r, k in enumerate(schedule):
        p = sets[k]
        nxt = np.stack([block_sequence(cur[b], p, cfg) for b in range(cur.shape[0])])
        cur = nxt if r == n - 1 else round_to_dtype(nxt, io_dtype)
    return cur


# --------------------------------------------------------------------------
# Brute force: pure-Python loops over the sums of eq. 5, for tiny sizes
# --------------------------------------------------------------------------

def brute_block(h, p: BlockParams, cfg: BlockConfig):
    """One block on one tiny sequence with explicit Python loops: every sum of
    [TANGO] eqs. 2-5 and 6-9 written out term by term.  Returns (out, gbar)."""
    h = [[float(v) for v in row] for row in np.asarray(h)]
    t_len, d = len(h), len(h[0])
    H, dh = cfg.n_heads, cfg.head_dim
    F = p.w_g.shape[0]
    fh = F // H
    Wg, Wv, Wq, Wk, Wo = (np.asarray(w).tolist() for w in
                          (p.w_g, p.w_v, p.w_q, p.w_k, p.w_o))
    gain = [1.0] * d if p.gain is None else [float(v) for v in p.gain]

    def matvec(Wm, x):
        return [sum(Wm[r][c] * x[c] for c in range(len(x))) for r in range(len(Wm))]

    xs, gs, vs, qs, ks = [], [], [], [], []
    for i in range(t_len):
        ms = sum(v * v for v in h[i]) / d
        r = 1.0 / math.sqrt(ms + cfg.rms_eps)
        x = [gain[c] * h[i][c] * r for c in range(d)]
        a = matvec(Wg, x)
        gs.append([ai / (1.0 + math.exp(-ai)) for ai in a])
        vs.append(matvec(Wv, x))
        qv, kv = matvec(Wq, x), matvec(Wk, x)
        qh_i, kh_i = [], []
        for a_ in range(H):
            for vec, dst in ((qv, qh_i), (kv, kh_i)):
                u = vec[a_ * dh:(a_ + 1) * dh]
                if cfg.rope_base != 0:
                    rot = []
                    for c in range(dh // 2):
                        ang = i * cfg.rope_base ** (-2.0 * c / dh)
                        u0, u1 = u[2 * c], u[2 * c + 1]
                        rot += [u0 * math.cos(ang) - u1 * math.sin(ang),
                                u0 * math.sin(ang) + u1 * math.cos(ang)]
                    u = rot
                nrm = max(math.sqrt(sum(e * e for e in u)), NORM_FLOOR)
                dst.append([e / nrm for e in u])
        xs.append(x)
        qs.append(qh_i)
        ks.append(kh_i)

    def phi_s(u):
        out = []
        for e in u:
            el = e if e > 0 else math.exp(e) - 1.0
            out.append(max(el + 1.0 + PHI_EPS, PHI_EPS) / math.sqrt(dh))
        return out

    gbar = [[0.0] * F for _ in range(t_len)]
    for i in range(t_len):
        for a_ in range(H):
            tau = math.exp(min(float(p.theta[a_]), LOG_TAU_MAX))
            num = [0.0] * fh
            den = 0.0
            for j in range(i + 1):
                if cfg.mode == "tango" or j >= i - cfg.window + 1:
                    m = math.exp(tau * sum(qs[i][a_][e] * ks[j][a_][e] for e in range(dh)))
                else:
                    fq = phi_s([math.sqrt(tau) * e for e in qs[i][a_]])
                    fk = phi_s([math.sqrt(tau) * e for e in ks[j][a_]])
                    m = sum(fq[e] * fk[e] for e in range(dh))
                den += m
                for f in range(fh):
                    num[f] += m * gs[j][a_ * fh + f]
            if p.null_bias is not None:
                den += (i + 1) * math.exp(float(p.null_bias[a_]))
            for f in range(fh):
                gbar[i][a_ * fh + f] = num[f] / den
    out = []
    for i in range(t_len):
        u = [gbar[i][f] * vs[i][f] for f in range(F)]
        upd = matvec(Wo, u)
        out.append([h[i][c] + upd[c] for c in range(d)])
    return np.array(out), np.array(gbar)


# --------------------------------------------------------------------------
# The pages' analytical counts (used to pin the parameter list)
# --------------------------------------------------------------------------

def block_param_count(d: int, F: int, H: int, dh: int, vocab_final_norm: bool = True) -> int:
    """Nonembedding parameters of one TANGO/WANGO model ([TANGO] §2 and Table 1):
    bias-free W_g, W_v [F, d], W_q, W_k [H d_h, d], W_o [d, F]; one RMSNorm gain
    in the block and one final RMSNorm gain; theta and b per head."""
    n = 2 * F * d + 2 * H * dh * d + d * F + d + 2 * H
    if vocab_final_norm:
        n += d
    return n


def forward_macs(T: int, d: int, F: int, H: int, dh: int, vocab: int, repeats: int,
                 mode: str, window: int = 0) -> int:
    """Analytical forward MACs of one sequence as counted in [TANGO] §3
    (Parameter and operation counts) and Table 5: linear projections, pair
    computations over the full T x T grid (TANGO) or 3W pairs per token plus the
    running-sum update and readout (WANGO), and the output vocabulary projection;
    normalisation, masking, feature maps and elementwise work are excluded."""
    linear = T * (2 * d * F + 2 * d * H * dh + F * d)
    if mode == "tango":
        pairs = T * T * (H * dh + F)
    else:
        pairs = T * 3 * window * (H * dh + F) + T * 2 * dh * F
    return repeats * (linear + pairs) + T * d * vocab
