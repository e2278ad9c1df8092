"""Writes the expected outputs of the long WANGO workload for the GPU parity test.

    python tests/golden/make_wango_t65536_golden.py

Workload: WANGO block, bf16 compute with a float32 residual stream, B = 2,
T = 65536, d = 512, F = 2048, one head of width 128, window 512, applied 8 times with shared weights, seeded inputs (seed 4).  The float64
CPU oracle computes all 8 applications over both sequences (the window band
plus the blocked running sums of the older prefix, as the oracle states them),
which takes minutes, so this script stores a sample: 64 output rows of each
sequence (the first rows, rows around the window edge, the last rows and
seeded random rows) together with the root mean square of the whole output.
Only the oracle and the seeded input generator are called.
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle.tango_oracle as O  # noqa: E402
from cross_token_gated_amd import workload as wl  # noqa: E402

NAME = "wango_bf16_b2_t65536_w512_r8"
OUT = os.path.join(HERE, "wango_t65536_samples.npz")


def sample_rows(T: int, W: int, seed: int = 123, n: int = 64) -> np.ndarray:
    fixed = [0, 1, 2, 63, 64, W - 2, W - 1, W, W + 1, 2 * W, 4095, 4096, T // 2, T - 129,
             T - 128, T - 2, T - 1]
    rng = np.random.default_rng(seed)
    extra = rng.choice(np.setdiff1d(np.arange(T), fixed), size=n - len(fixed), replace=False)
    return np.sort(np.concatenate([fixed, extra])).astype(np.int64)


def main():
    w = wl.WORKLOADS[NAME]
    inp = wl.make_inputs(w)
    p = O.BlockParams(w_g=inp.w_g.astype(np.float64), w_v=inp.w_v.astype(np.float64),
                      w_q=inp.w_q.astype(np.float64), w_k=inp.w_k.astype(np.float64),
                      w_o=inp.w_o.astype(np.float64), theta=inp.theta.astype(np.float64))
    cfg = O.BlockConfig(n_heads=w.n_heads, head_dim=w.head_dim, mode="wango", window=w.window,
                        rope_base=w.rope_base, rms_eps=w.rms_eps)
    t0 = time.time()
    out = O.block_stack(inp.h.astype(np.float64), p, cfg, repeats=w.repeats, io_dtype=w.io,
                        form="scan")
    rows = sample_rows(w.T, w.window)
    np.savez_compressed(OUT, rows=rows, expected=out[:, rows, :].astype(np.float64),
                        rms=np.sqrt(np.mean(out * out)), workload=NAME)
    print(f"wrote {OUT} in {time.time() - t0:.0f} s; rms {np.sqrt(np.mean(out * out)):.6f}")


if __name__ == "__main__":
    main()
