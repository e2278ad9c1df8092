"""Test helpers: intermediate-layout packers, oracle drivers, error metric.

Layouts follow include/tango.h: rows padded per sequence to a multiple of 128;
gates in the source-packed layout [M/32][4][F][8]; the WANGO older-prefix
numerator in 16x16 blocks [M/16][F/16][64][4].
"""
from __future__ import annotations

import math

import numpy as np

import oracle.tango_oracle as O
from cross_token_gated_amd import workload as wl

ROW_PAD = 128


def padded_len(T: int) -> int:
    return (T + ROW_PAD - 1) // ROW_PAD * ROW_PAD


def pad_rows(a: np.ndarray, Tp: int) -> np.ndarray:
    """[B, T, X] -> [B*Tp, X] with zero rows appended to every sequence."""
    B, T, X = a.shape
    out = np.zeros((B, Tp, X), dtype=a.dtype)
    out[:, :T] = a
    return out.reshape(B * Tp, X)


def unpad_rows(a: np.ndarray, B: int, T: int) -> np.ndarray:
    return a.reshape(B, -1, a.shape[-1])[:, :T]


_PERM = np.array([[4 * g + s if s < 4 else 16 + 4 * g + (s - 4) for s in range(8)]
                  for g in range(4)])


def head_pad(fh: int, wango: bool) -> int:
    """The padded head width Fhp of the gate layouts (include/tango.h): fh when it
    is a multiple of 64; else WANGO rounds up to 64, TANGO to 512 when that is at
    most 1.2 fh, else to 64."""
    if fh % 64 == 0:
        return fh
    p512 = (fh + 511) // 512 * 512
    if not wango and 5 * p512 <= 6 * fh:
        return p512
    return (fh + 63) // 64 * 64


def pad_heads(g_rows: np.ndarray, n_heads: int, fhp: int) -> np.ndarray:
    """[M, H*Fh] -> [M, H*Fhp]: head a's column c moved to a*Fhp + c, pad columns zero."""
    M, F = g_rows.shape
    fh = F // n_heads
    out = np.zeros((M, n_heads, fhp), dtype=g_rows.dtype)
    out[:, :, :fh] = g_rows.reshape(M, n_heads, fh)
    return out.reshape(M, n_heads * fhp)


def pack_gates(g_rows: np.ndarray) -> np.ndarray:
    """[M, F] (M % 32 == 0) -> packed [M/32, 4, F, 8]."""
    M, F = g_rows.shape
    blk = g_rows.reshape(M // 32, 32, F)
    sel = blk[:, _PERM.reshape(-1), :].reshape(M // 32, 4, 8, F)
    return np.ascontiguousarray(sel.transpose(0, 1, 3, 2))


def unpack_gates(gp: np.ndarray, M: int, F: int) -> np.ndarray:
    sel = gp.reshape(M // 32, 4, F, 8).transpose(0, 1, 3, 2).reshape(M // 32, 32, F)
    out = np.empty((M // 32, 32, F), dtype=gp.dtype)
    out[:, _PERM.reshape(-1), :] = sel
    return out.reshape(M, F)


def permute_features(a: np.ndarray) -> np.ndarray:
    """[..., D] (D % 32 == 0) -> the permuted feature order of include/tango.h:
    position 8g + s of each group of 32 holds feature perm(g, s)."""
    D = a.shape[-1]
    src = np.concatenate([32 * c + _PERM.reshape(-1) for c in range(D // 32)])
    return np.ascontiguousarray(a[..., src])


def unpermute_features(a: np.ndarray) -> np.ndarray:
    D = a.shape[-1]
    src = np.concatenate([32 * c + _PERM.reshape(-1) for c in range(D // 32)])
    out = np.empty_like(a)
    out[..., src] = a
    return out


def unblock_nold(nb: np.ndarray, M: int, F: int) -> np.ndarray:
    """[M/16, F/16, 64, 4] -> [M, F]: lane l holds row l%16, columns 4(l/16)+r."""
    a = nb.reshape(M // 16, F // 16, 4, 16, 4)        # ib, fb, lg, li, r
    return np.ascontiguousarray(a.transpose(0, 3, 1, 2, 4)).reshape(M, F)


def block_nold(n: np.ndarray) -> np.ndarray:
    M, F = n.shape
    a = n.reshape(M // 16, 16, F // 16, 4, 4)          # ib, li, fb, lg, r
    return np.ascontiguousarray(a.transpose(0, 2, 3, 1, 4)).reshape(M // 16, F // 16, 64, 4)


def err_ratio(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / rms(ref): the parity metric of the block outputs."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def rms_ratio(got: np.ndarray, ref: np.ndarray) -> float:
    """rms(got - ref) / rms(ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return math.sqrt(float(np.mean((got - ref) ** 2)) / max(float(np.mean(ref * ref)), 1e-300))


# Stage outputs (gates, features, unit q/k, gbar) are stored in the I/O dtype.
# In bf16 the rounding alone is up to 2^-9 of each value, whose largest
# entries reach 10-25 times the rms, and the aggregation also rounds its
# weights to bf16: so the stage bars are rms(err)/rms(ref) <= 4e-3 (pure
# rounding gives about 1e-3) and max|err|/rms(ref) <= 6e-2.  Float32 stages
# keep the block bar of 1e-4 on both.
STAGE_BARS = {"bf16": (4e-3, 6e-2), "f32": (1e-4, 1e-4)}


def check_stage(got, ref, dtype: str, what: str = "") -> None:
    r, m = rms_ratio(got, ref), err_ratio(got, ref)
    br, bm = STAGE_BARS[dtype]
    print(f"{what}: rms ratio {r:.2e} (bar {br:.0e}), max ratio {m:.2e} (bar {bm:.0e})")
    assert r <= br and m <= bm, (what, r, m)


def tol(dtype: str) -> float:
    """Tolerance on max|err|/rms of a block output: 2e-2 for bf16 compute,
    1e-4 for float32."""
    return 2e-2 if dtype == "bf16" else 1e-4


def oracle_params(inp: wl.Inputs) -> O.BlockParams:
    f = lambda a: None if a is None else np.asarray(a, dtype=np.float64)  # noqa: E731
    return O.BlockParams(w_g=f(inp.w_g), w_v=f(inp.w_v), w_q=f(inp.w_q), w_k=f(inp.w_k),
                         w_o=f(inp.w_o), theta=f(inp.theta), gain=f(inp.gain),
                         null_bias=f(inp.null_bias))


def oracle_config(w: wl.Workload) -> O.BlockConfig:
    return O.BlockConfig(n_heads=w.n_heads, head_dim=w.head_dim, mode=w.mode, window=w.window,
                         rope_base=w.rope_base, rms_eps=w.rms_eps)


def oracle_stack(w: wl.Workload, inp: wl.Inputs, form: str = "direct") -> np.ndarray:
    return O.block_stack(np.asarray(inp.h, dtype=np.float64), oracle_params(inp), oracle_config(w),
                         repeats=w.repeats, io_dtype=w.io, form=form)


def oracle_block_rows(h_seq: np.ndarray, p: O.BlockParams, cfg: O.BlockConfig, rows) -> np.ndarray:
    """Rows ``rows`` of one block application over one sequence h_seq [T, d],
    composed from the oracle's own pieces (projections of every position, the
    pairwise weights of just those destination rows, the null term): for long
    sequences where the whole forward would take minutes."""
    h_seq = np.asarray(h_seq, dtype=np.float64)
    parts = O.project(h_seq, p, cfg)
    tau = O.temperature(p.theta)
    H = cfg.n_heads
    fh = parts["g"].shape[1] // H
    out = []
    for i in rows:
        gbar = np.empty(parts["g"].shape[1])
        for a in range(H):
            sl = slice(int(i), int(i) + 1)
            m = O.pair_weights(parts["qh"], parts["kh"], tau, a, sl, cfg.mode, cfg.window)[0]
            num = m @ parts["g"][:, a * fh:(a + 1) * fh]
            den = m.sum() + O.null_weight(p.null_bias, a, sl)[0]
            gbar[a * fh:(a + 1) * fh] = num / den
        out.append(h_seq[i] + p.w_o @ (gbar * parts["v"][i]))
    return np.stack(out)
