"""Test helpers: oracle drivers, error metrics and bars; the layout packers of
cross_token_gated_amd.layouts re-exported under their old names."""
from __future__ import annotations

import math

import numpy as np

import oracle.tango_oracle as O
from cross_token_gated_amd import workload as wl

# the layout packers live in the package (no oracle there); re-exported here
from cross_token_gated_amd.layouts import (ROW_PAD, block_nold, head_pad, pack_gates,  # noqa: E402,F401
                                           pad_heads, pad_rows, padded_len, permute_features,
                                           unblock_nold, unpack_gates, unpad_rows, unpermute_features)


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


def bf16_ulp(a) -> np.ndarray:
    """Spacing of the bfloat16 values at |a| (8 significant bits): 2^(e - 7) for
    |a| in [2^e, 2^(e+1)).  It bounds the gap between the two bfloat16
    neighbours of any value in that binade."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def oracle_streams(h, apply_one, n_apps: int, io: str) -> list:
    """The oracle's residual stream after each application, as the stacked
    oracle computes it: rounded to the I/O dtype after applications 1 .. n-1
    (the stored stream), unrounded after the last.  apply_one(r, cur) is one
    application of the oracle (rounding nothing)."""
    cur = np.asarray(h, dtype=np.float64)
    out = []
    for r in range(n_apps):
        nxt = apply_one(r, cur)
        cur = nxt if r == n_apps - 1 else O.round_to_dtype(nxt, io)
        out.append(cur)
    return out


def workload_streams(w: wl.Workload, inp: wl.Inputs) -> list:
    p, cfg = oracle_params(inp), oracle_config(w)
    return oracle_streams(inp.h, lambda r, cur: O.block_stack(cur, p, cfg, repeats=1, io_dtype=w.io),
                          w.repeats, w.io)


def flip_aware_error(got: np.ndarray, streams: list) -> dict:
    """Errors of a stacked output whose residual stream was stored in bfloat16
    between applications, against the oracle's streams (oracle_streams).

    Both sides round the stream after every application but the last.  Where
    the GPU's pre-rounding value and the oracle's lie on either side of a
    rounding boundary the two stored values differ by one bfloat16 spacing,
    whatever the size of the difference that put them there, and the residual
    path ([TANGO] §2.3 eq. 11: h is carried unchanged into the next output)
    passes that spacing to the final output at the same element.  Its effect
    through the block itself (one element of one row's RMSNorm input) is
    smaller by about the weights' scale, so it is covered by the kernel bar.
    Each element is therefore allowed one spacing of the oracle's stored value
    per stored stream, and what exceeds that must stay inside the plain bar:
      "max": max|got - ref| / rms(ref) (no allowance),
      "flip": max(|got - ref| - sum_r spacing(stream_r)) / rms(ref),
      "rms": rms(got - ref) / rms(ref) (flips are rare, so this stays small),
      "n_over": elements over 2e-2 rms without the allowance."""
    ref = streams[-1]
    got = np.asarray(got, dtype=np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    err = np.abs(got - ref)
    allow = np.zeros_like(ref)
    for s in streams[:-1]:
        allow += bf16_ulp(s)
    return {"max": float(err.max()) / rms,
            "flip": float(np.max(err - allow)) / rms,
            "rms": rms_ratio(got, ref),
            "n_over": int(np.count_nonzero(err > 2e-2 * rms))}


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
