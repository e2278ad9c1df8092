"""Workload shapes and seeded synthetic inputs for the TANGO / WANGO block.

This module holds no arithmetic of the method: it names the five workload
shapes and draws the seeded inputs that both the HIP path and the CPU checker
consume.  Inputs are drawn in float64 with numpy's PCG64 generator in the order
h, W_g, W_v, W_q, W_k, W_o, scaled to N(0, 1) activations and N(0, 1/fan_in)
weights, and rounded once to the I/O dtype (float64 -> float32 -> bfloat16,
round to nearest even).  Both sides use the same rounded values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One block workload.  ``mode`` is "tango" (full prefix) or "wango"
    (window + running sums).  ``repeats`` is the number of shared-weight
    applications.  ``dtype`` is the dtype of the weights and of every
    intermediate activation ("f32" or "bf16"); accumulation is always float32.
    ``io_dtype`` is the dtype of the residual stream x/out between
    applications; the bf16 workloads carry it in float32.  The input values
    are rounded to ``dtype`` in either case.  ``operand_parts`` is the number
    of bf16 parts in which the float32 activation operand of the projection
    and output GEMMs enters the MFMA: 1 is the plain bf16 compute; the long
    stacks (eight shared-weight applications) take 2, without which their
    first positions' rounding compounds past the 2e-2 bar."""
    name: str
    mode: str
    dtype: str
    B: int
    T: int
    d_model: int
    d_gate: int
    n_heads: int
    head_dim: int
    window: int = 0
    chunk: int = 0
    repeats: int = 1
    seed: int = 0
    theta: float = math.log(10.0)      # cosine-similarity scale 10
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    null_bias: Optional[float] = None  # None: null gate off
    io_dtype: str = ""                 # dtype of the residual stream x/out ("" = dtype)
    operand_parts: int = 1             # bf16 parts of the GEMMs' activation operand

    @property
    def io(self) -> str:
        return self.io_dtype or self.dtype

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: TANGO fp32 T=256; TANGO bf16 B=8 T=2048; TANGO bf16 T=8192
# applied 4 times; WANGO bf16 T=8192 window 256 (two heads of 64); WANGO bf16
# B=2 T=65536 window 512 applied 8 times.
WORKLOADS = {
    "tango_f32_t256": Workload("tango_f32_t256", "tango", "f32", 1, 256, 512, 1024, 1, 128,
                               seed=0),
    "tango_bf16_b8_t2048": Workload("tango_bf16_b8_t2048", "tango", "bf16", 8, 2048, 512, 2048,
                                    1, 128, seed=1, io_dtype="f32"),
    "tango_bf16_t8192_r4": Workload("tango_bf16_t8192_r4", "tango", "bf16", 1, 8192, 512, 2048,
                                    1, 128, repeats=4, seed=2, io_dtype="f32"),
    "wango_bf16_t8192_w256": Workload("wango_bf16_t8192_w256", "wango", "bf16", 1, 8192, 512,
                                      2048, 2, 64, window=256, chunk=128, seed=3,
                                      io_dtype="f32"),
    "wango_bf16_b2_t65536_w512_r8": Workload("wango_bf16_b2_t65536_w512_r8", "wango", "bf16", 2,
                                             65536, 512, 2048, 1, 128, window=512, chunk=128,
                                             repeats=8, seed=4, io_dtype="f32", operand_parts=2),
}
WORKLOAD_ORDER = list(WORKLOADS)

# The pages' own geometry ([TANGO] §2.3 and Table 5: d = 512, H = 16 heads
# of 32, gate width F = 28,480 so F/H = 1,780, window and prefix-sum block 64,
# one block applied 4 times) at the 8,192-token context of the FineWeb-Edu runs.
PAGES_WORKLOADS = {
    "tango_pages_t8192_r4": Workload("tango_pages_t8192_r4", "tango", "bf16", 1, 8192, 512, 28480, 16,
                                     32, repeats=4, seed=8, io_dtype="f32"),
    "wango_pages_t8192_w64_r4": Workload("wango_pages_t8192_w64_r4", "wango", "bf16", 1, 8192, 512,
                                         28480, 16, 32, window=64, chunk=64, repeats=4, seed=9,
                                         io_dtype="f32"),
}

# Decode workloads: one new token per sequence at position 8192 -- the state
# holds the 8192 earlier positions -- in the geometry of the T = 8192 workloads
# above (TANGO: one head of 128, stacked 4 times, each application with its own
# state; WANGO: two heads of 64, window 256).  B is the number of sequences
# decoded together; T - 1 is the position of the timed step.
DECODE_WORKLOADS = {
    "tango_decode_bf16_b16_p8192_r4": Workload("tango_decode_bf16_b16_p8192_r4", "tango", "bf16", 16,
                                               8193, 512, 2048, 1, 128, repeats=4, seed=5,
                                               io_dtype="f32"),
    "wango_decode_bf16_b64_p8192_w256": Workload("wango_decode_bf16_b64_p8192_w256", "wango", "bf16",
                                                 64, 8193, 512, 2048, 2, 64, window=256, seed=6,
                                                 io_dtype="f32"),
}


def three_set_schedule(n_apps: int) -> tuple:
    """Set index of each application in the three-set model of "TANGO: Treating
    Tokens as Operators" (abstract; Table 2): set 0 for the first application,
    set 2 for the last and set 1 for every one between (one application uses
    set 0 alone; two use sets 0 and 2)."""
    if n_apps < 1:
        raise ValueError("n_apps must be >= 1")
    if n_apps == 1:
        return (0,)
    return (0,) + (1,) * (n_apps - 2) + (2,)


@dataclass(frozen=True)
class StackWorkload:
    """A TANGO stack with several gated-projection sets: ``base`` gives the
    shared sizes (its d_gate is unused), ``widths`` the gate width F of each
    set and ``schedule`` the set of each application."""
    name: str
    base: Workload
    widths: tuple
    schedule: tuple

    def set_workload(self, k: int) -> Workload:
        return replace(self.base, d_gate=self.widths[k], repeats=1)

    @property
    def tokens(self) -> int:
        return self.base.tokens


# The three-set model at the T = 8192 TANGO geometry above, stacked 8 deep as in
# the later revision's Table 2 (depth 8): three gated-projection sets whose
# widths add up to the one-set model's F = 2048 (the sets hold the same number
# of W_g / W_v / W_o parameters as the one-set block; widths are multiples of 64).
STACK_WORKLOADS = {
    "tango_3set_bf16_t8192_r8": StackWorkload(
        "tango_3set_bf16_t8192_r8",
        Workload("tango_3set_bf16_t8192_r8", "tango", "bf16", 1, 8192, 512, 704, 1, 128, seed=10,
                 io_dtype="f32", operand_parts=2),
        (704, 640, 704), three_set_schedule(8)),
}


def make_stack_inputs(sw: StackWorkload, seed: Optional[int] = None) -> list:
    """Inputs of every set of a stack workload, as a list of Inputs.  Drawn in
    the order h, W_q, W_k, then W_g, W_v, W_o of set 0, 1, ...; every set shares
    h, W_q, W_k, theta and the null bias (the same arrays), and has its own
    W_g, W_v [F_k, d] and W_o [d, F_k] (scales as in make_inputs)."""
    w = sw.base
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    d, hd = w.d_model, w.n_heads * w.head_dim
    q = lambda a: quantize(a, w.dtype)  # noqa: E731
    h = q(rng.standard_normal((w.B, w.T, d)))
    w_q = q(rng.standard_normal((hd, d)) / math.sqrt(d))
    w_k = q(rng.standard_normal((hd, d)) / math.sqrt(d))
    theta = np.full(w.n_heads, w.theta, dtype=np.float32)
    nb = None if w.null_bias is None else np.full(w.n_heads, w.null_bias, dtype=np.float32)
    out = []
    for F in sw.widths:
        w_g = q(rng.standard_normal((F, d)) / math.sqrt(d))
        w_v = q(rng.standard_normal((F, d)) / math.sqrt(d))
        w_o = q(rng.standard_normal((d, F)) / math.sqrt(F))
        out.append(Inputs(h, w_g, w_v, w_q, w_k, w_o, None, theta, nb))
    return out


# The aggregation backward at the T = 8192 bench shape: one head of 128,
# F = 2048, bf16.
BACKWARD_SHAPE = dict(T=8192, F=2048, H=1, dh=128, seed=5)
# The WANGO aggregation backward at the T = 8192 WANGO bench shape: two heads
# of 64, F = 2048, window 256, prefix chunk 128.
WANGO_BACKWARD_SHAPE = dict(T=8192, F=2048, H=2, dh=64, window=256, chunk=128, seed=6)


def aggregate_inputs(T: int, F: int, H: int, dh: int, seed: int):
    """Seeded inputs of the aggregation alone, as float32 arrays that bfloat16
    holds exactly: unit query and key vectors q, k [T, H, d_h] (Gaussian
    directions), gates g [T, F] and an incoming gradient dgbar [T, F], both
    N(0, 1).  Drawn with PCG64 in the order q, k, g, dgbar."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((T, H, dh))
    k = rng.standard_normal((T, H, dh))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = rng.standard_normal((T, F))
    dgbar = rng.standard_normal((T, F))
    return round_bf16(q), round_bf16(k), round_bf16(g), round_bf16(dgbar)


def round_f32(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 (round to nearest even)."""
    return np.asarray(a, dtype=np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bfloat16 (round to nearest even at each step),
    returned as float32 values that bfloat16 represents exactly."""
    a32 = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(a32)
    if nan.any():
        out = np.where(nan, np.float32(np.nan), out)
    return out


def quantize(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return round_f32(a)
    if dtype == "bf16":
        return round_bf16(a)
    raise ValueError(dtype)


@dataclass
class Inputs:
    """Seeded inputs as float32 arrays whose values the I/O dtype holds exactly."""
    h: np.ndarray      # [B, T, d]
    w_g: np.ndarray    # [F, d]
    w_v: np.ndarray    # [F, d]
    w_q: np.ndarray    # [H*d_h, d]
    w_k: np.ndarray    # [H*d_h, d]
    w_o: np.ndarray    # [d, F]
    gain: Optional[np.ndarray]       # [d] float32 or None (= 1)
    theta: np.ndarray                # [H] float32
    null_bias: Optional[np.ndarray]  # [H] float32 or None (null gate off)


def make_inputs(w: Workload, seed: Optional[int] = None, gain: Optional[np.ndarray] = None,
                h_override: Optional[np.ndarray] = None) -> Inputs:
    """Draw the inputs of workload ``w`` (seed defaults to the workload's)."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    d, F, hd = w.d_model, w.d_gate, w.n_heads * w.head_dim
    h = rng.standard_normal((w.B, w.T, d))
    w_g = rng.standard_normal((F, d)) / math.sqrt(d)
    w_v = rng.standard_normal((F, d)) / math.sqrt(d)
    w_q = rng.standard_normal((hd, d)) / math.sqrt(d)
    w_k = rng.standard_normal((hd, d)) / math.sqrt(d)
    w_o = rng.standard_normal((d, F)) / math.sqrt(F)
    if h_override is not None:
        h = h_override
    q = lambda a: quantize(a, w.dtype)  # noqa: E731
    theta = np.full(w.n_heads, w.theta, dtype=np.float32)
    nb = None if w.null_bias is None else np.full(w.n_heads, w.null_bias, dtype=np.float32)
    gq = None if gain is None else q(gain)
    return Inputs(q(h), q(w_g), q(w_v), q(w_q), q(w_k), q(w_o), gq, theta, nb)


def small_workload(mode: str = "tango", dtype: str = "bf16", B: int = 1, T: int = 200,
                   d_model: int = 128, d_gate: int = 256, n_heads: int = 1, head_dim: int = 64,
                   window: int = 64, chunk: int = 64, repeats: int = 1, seed: int = 7,
                   **kw) -> Workload:
    """A small workload of the same structure, for tests the checker finishes fast."""
    return Workload(f"small_{mode}", mode, dtype, B, T, d_model, d_gate, n_heads, head_dim,
                    window=window if mode == "wango" else 0,
                    chunk=chunk if mode == "wango" else 0, repeats=repeats, seed=seed, **kw)
