"""CPU float64 oracle of the TANGO / WANGO block forward.

Test infrastructure only: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.
"""
from .tango_oracle import *  # noqa: F401,F403
from .tango_oracle import (BlockConfig, BlockParams, block_sequence, block_stack,  # noqa: F401
                           brute_block, aggregate_direct, aggregate_wango_scan,
                           wango_old_running, wango_old_blocked, wango_band,
                           project, temperature, phi, rope, unit_normalize,
                           normalized_weights, round_to_dtype, block_param_count,
                           forward_macs, rms_norm, silu)
