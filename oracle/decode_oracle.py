"""Float64 CPU oracle of one autoregressive decode step of the TANGO / WANGO block.

TEST INFRASTRUCTURE ONLY, like ``tango_oracle`` whose pieces it uses: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.

A decode step takes, for every sequence, the block input h_p at its next
position p and the state left by positions 0..p-1, and returns the block output
at p.  Sources never lie after their destination ([TANGO] §2.1, eq. 5 sums over
j <= i), so that output is exactly row p of the block applied to the prefix
h_0..h_p: :func:`decode_reference` computes it that way, and it is the
definition every other form here is checked against.

:class:`DecodeState` keeps what the pages say inference needs: for WANGO the
running sums S and z of [TANGO] §2.2 eq. 10, to which the token leaving the
trailing window is added when the position advances (same paragraph), plus the
keys and gates of the last W tokens -- a state whose size does not grow with
the position ([TANGO] §6.1, last sentences of the first paragraph on WANGO).
TANGO has no such form: its state is every key and gate so far.
"""
from __future__ import annotations

import math
from typing import List, Optional

import numpy as np

from . import tango_oracle as O


def decode_reference(history: np.ndarray, p: O.BlockParams, cfg: O.BlockConfig) -> np.ndarray:
    """Output at the last position of ``history`` [p + 1, d]: row p of the block
    applied to the whole prefix (the definition of a decode step)."""
    return O.block_sequence(np.asarray(history, dtype=np.float64), p, cfg)[-1]


def decode_stack_reference(history: np.ndarray, p: O.BlockParams, cfg: O.BlockConfig,
                           repeats: int, io_dtype: str) -> np.ndarray:
    """Last row of ``repeats`` stacked applications ([TANGO] §2.3, eq. 11) of the
    prefix ``history`` [p + 1, d], rounded between applications as the forward."""
    return O.block_stack(np.asarray(history, dtype=np.float64)[None], p, cfg, repeats,
                         io_dtype)[0, -1]


class DecodeState:
    """Per-sequence decode state of one block, advanced one token at a time.

    TANGO: the unit keys k_j [H, d_h] and gates g_j [F] of every position so far.
    WANGO: S [H, d_h, F/H] and z [H, d_h] over the sources that have left the
    window, and the keys and gates of the last W positions."""

    def __init__(self, p: O.BlockParams, cfg: O.BlockConfig):
        self.p, self.cfg = p, cfg
        self.pos = 0
        self.tau = O.temperature(p.theta)
        H, dh = cfg.n_heads, cfg.head_dim
        F = p.w_g.shape[0]
        self.fh = F // H
        self.keys: List[np.ndarray] = []      # TANGO: all; WANGO: the window only
        self.gates: List[np.ndarray] = []
        self.first = 0                        # position of keys[0]
        if cfg.mode == "wango":
            self.S = np.zeros((H, dh, self.fh))
            self.z = np.zeros((H, dh))

    def size(self) -> int:
        """Number of float64 values held (for the constant-size check)."""
        n = sum(k.size for k in self.keys) + sum(g.size for g in self.gates)
        if self.cfg.mode == "wango":
            n += self.S.size + self.z.size
        return n

    def step(self, h_row: np.ndarray) -> np.ndarray:
        """Block output at position self.pos for input row h_row [d]; advances."""
        cfg, p = self.cfg, self.p
        H, dh, fh = cfg.n_heads, cfg.head_dim, self.fh
        i = self.pos
        parts = O.project(np.asarray(h_row, dtype=np.float64)[None], p, cfg,
                          positions=np.array([i]))
        q, k, g, v = parts["qh"][0], parts["kh"][0], parts["g"][0], parts["v"][0]
        if cfg.mode == "wango" and i - cfg.window >= 0:
            # the token i - W leaves the window: add it to S and z (eq. 10)
            j = i - cfg.window
            kj, gj = self.keys[j - self.first], self.gates[j - self.first]
            for a in range(H):
                fk = O.phi(math.sqrt(self.tau[a]) * kj[a], dh)
                self.S[a] += np.outer(fk, gj[a * fh:(a + 1) * fh])
                self.z[a] += fk
            self.keys.pop(0)
            self.gates.pop(0)
            self.first += 1
        self.keys.append(k)
        self.gates.append(g)
        gbar = np.empty_like(g)
        K = np.stack(self.keys)                # [n, H, d_h], positions first .. i
        G = np.stack(self.gates)               # [n, F]
        for a in range(H):
            m = np.exp(self.tau[a] * (K[:, a, :] @ q[a]))      # exp weights (eq. 6 / window of eq. 7)
            num = m @ G[:, a * fh:(a + 1) * fh]
            den = m.sum()
            if cfg.mode == "wango":
                fq = O.phi(math.sqrt(self.tau[a]) * q[a], dh)  # older prefix (eq. 9 via eq. 10)
                num = num + fq @ self.S[a]
                den = den + fq @ self.z[a]
            if p.null_bias is not None:                       # null gate, n_i = i + 1 (eq. 5)
                den = den + (i + 1) * math.exp(float(p.null_bias[a]))
            gbar[a * fh:(a + 1) * fh] = num / den
        self.pos += 1
        return np.asarray(h_row, dtype=np.float64) + p.w_o @ (gbar * v)


class DecodeStack:
    """``repeats`` stacked applications of one block, each with its own state;
    the stream is rounded to the I/O dtype between applications (as the
    forward stack)."""

    def __init__(self, p: O.BlockParams, cfg: O.BlockConfig, repeats: int, io_dtype: str):
        self.layers = [DecodeState(p, cfg) for _ in range(repeats)]
        self.io_dtype = io_dtype

    def step(self, h_row: np.ndarray) -> np.ndarray:
        cur = np.asarray(h_row, dtype=np.float64)
        for r, layer in enumerate(self.layers):
            cur = layer.step(cur)
            if r < len(self.layers) - 1:
                cur = O.round_to_dtype(cur, self.io_dtype)
        return cur


def wango_state_definition(keys: np.ndarray, gates: np.ndarray, tau: np.ndarray, window: int,
                           pos: int, head_dim: int):
    """S and z held after the step at position ``pos``, from their definition
    (eq. 10): sums over the sources j <= pos - W of phi(sqrt(tau) k_j) g_j^T and
    phi(sqrt(tau) k_j).  keys [T, H, d_h], gates [T, F] of the whole sequence."""
    H = keys.shape[1]
    fh = gates.shape[1] // H
    S = np.zeros((H, head_dim, fh))
    z = np.zeros((H, head_dim))
    for a in range(H):
        for j in range(0, pos - window + 1):
            fk = O.phi(math.sqrt(tau[a]) * keys[j, a], head_dim)
            S[a] += np.outer(fk, gates[j, a * fh:(a + 1) * fh])
            z[a] += fk
    return S, z
