"""Shared pieces of the GPU tests: the case announcement, and the device
plumbing of cross_token_gated_amd.device re-exported under its old names."""
from __future__ import annotations

import sys

from cross_token_gated_amd.device import (TORCH_DTYPE, block_weights, dev_f32,  # noqa: F401
                                          dev_tensor, host, run_workload)


def announce(msg: str) -> None:
    """Print the case name before a GPU step, so a failing run names it."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)
