"""Writes the expected outputs of the pages-geometry workloads at T = 8192 for
the GPU parity test.

    python tests/golden/make_pages_geometry_golden.py

Workloads: one application of the TANGO block and of the WANGO block (window
and prefix-sum block 64) with d = 512, 16 heads of 32 and gate width 28,480,
bf16 compute, a float32 residual stream, seeded inputs (the workloads
tango_pages_t8192_r4 / wango_pages_t8192_w64_r4 with one application).  The
float64 oracle projects all 8,192 positions and computes 48 destination rows
(fixed rows at block and window edges plus seeded random rows) from its own
pairwise weights; the error is measured against the rms of those rows.  Only
the oracle and the seeded input generator are called.
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
from tests import helpers as H  # noqa: E402

OUT = os.path.join(HERE, "pages_geometry_t8192_samples.npz")


def sample_rows(T: int, seed: int = 321, n: int = 48) -> np.ndarray:
    fixed = [0, 1, 31, 32, 63, 64, 65, 127, 128, 129, 1023, 4096, T - 65, T - 64, T - 2, T - 1]
    rng = np.random.default_rng(seed)
    extra = rng.choice(np.setdiff1d(np.arange(T), fixed), size=n - len(fixed), replace=False)
    return np.sort(np.concatenate([fixed, extra])).astype(np.int64)


def main():
    out = {}
    rows = sample_rows(8192)
    for name in ("tango_pages_t8192_r4", "wango_pages_t8192_w64_r4"):
        w = wl.PAGES_WORKLOADS[name].scaled(repeats=1)
        inp = wl.make_inputs(w)
        p, cfg = H.oracle_params(inp), H.oracle_config(w)
        t0 = time.time()
        h = np.asarray(inp.h[0], dtype=np.float64)
        exp = H.oracle_block_rows(h, p, cfg, rows)
        out[f"{w.mode}_expected"] = exp
        out[f"{w.mode}_rms"] = np.sqrt(np.mean(exp * exp))
        print(f"{name}: {time.time() - t0:.0f} s")
    np.savez_compressed(OUT, rows=rows, **out)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
