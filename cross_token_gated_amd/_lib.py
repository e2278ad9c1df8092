"""ctypes view of libtango.so (include/tango.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtango.so")

TANGO_F32 = 0
TANGO_BF16 = 1

STATUS = {
    0: "TANGO_OK", -1: "TANGO_ERR_NULL", -2: "TANGO_ERR_SHAPE", -3: "TANGO_ERR_DTYPE",
    -4: "TANGO_ERR_ALIGN", -5: "TANGO_ERR_UNSUPPORTED", -6: "TANGO_ERR_WORKSPACE",
    -7: "TANGO_ERR_ALIAS", -8: "TANGO_ERR_HIP",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

# Every symbol include/tango.h declares.
EXPORTS = [
    "tango_workspace_size", "tango_block_fwd", "wango_workspace_size", "wango_block_fwd",
    "tango_status_string", "tango_last_error", "tango_version",
    "tango_proj_workspace_size", "tango_stage_proj", "wango_stage_proj", "tango_stage_aggregate", "tango_stage_out",
    "wango_stage_scan", "wango_stage_band",
    "tango_decode_state_size", "tango_decode_workspace_size", "tango_decode_step",
    "wango_decode_state_size", "wango_decode_workspace_size", "wango_decode_step",
    "tango_aggregate_fwd_train", "tango_aggregate_bwd_workspace_size", "tango_aggregate_bwd",
    "tango_stack_workspace_size", "tango_stack_fwd",
    "wango_aggregate_fwd_train_workspace_size", "wango_aggregate_fwd_train",
    "wango_aggregate_bwd_workspace_size", "wango_aggregate_bwd",
    "wango_decode_step_noalloc",
]

NOALLOC_SCRATCH_BYTES = 16 << 20   # TANGO_NOALLOC_SCRATCH_BYTES


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_gate", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("operand_parts", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("w_g", ctypes.c_void_p), ("w_v", ctypes.c_void_p), ("w_q", ctypes.c_void_p),
                ("w_k", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("rms_gain", ctypes.c_void_p),
                ("theta", ctypes.c_void_p), ("null_bias", ctypes.c_void_p)]


class TangoError(RuntimeError):
    def __init__(self, code: int, detail: str):
        super().__init__(f"{STATUS.get(code, code)}: {detail}")
        self.code = code
        self.name = STATUS.get(code, str(code))


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtango.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m cross_token_gated_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    S, W = ctypes.POINTER(Shape), ctypes.POINTER(Weights)
    sig = {
        "tango_workspace_size": (sz, [S]),
        "tango_block_fwd": (ctypes.c_int, [S, W, vp, vp, vp, sz, vp]),
        "wango_workspace_size": (sz, [S, i32, i32, i32]),
        "wango_block_fwd": (ctypes.c_int, [S, W, i32, i32, i32, vp, vp, vp, sz, vp]),
        "tango_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "tango_last_error": (ctypes.c_char_p, []),
        "tango_version": (ctypes.c_int, []),
        "tango_proj_workspace_size": (sz, [S]),
        "tango_stage_proj": (ctypes.c_int, [S, W, vp, vp, vp, vp, vp, vp, sz, vp]),
        "wango_stage_proj": (ctypes.c_int, [S, W, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "tango_stage_aggregate": (ctypes.c_int, [S, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "tango_stage_out": (ctypes.c_int, [S, vp, vp, vp, vp, vp, vp]),
        "wango_stage_scan": (ctypes.c_int, [S, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "wango_stage_band": (ctypes.c_int, [S, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp]),
        "tango_decode_state_size": (sz, [S]),
        "tango_decode_workspace_size": (sz, [S]),
        "tango_decode_step": (ctypes.c_int, [S, W, vp, vp, vp, vp, sz, vp, sz, vp]),
        "wango_decode_state_size": (sz, [S, i32, i32]),
        "wango_decode_workspace_size": (sz, [S, i32, i32]),
        "wango_decode_step": (ctypes.c_int, [S, W, i32, i32, vp, vp, vp, vp, sz, vp, sz, vp]),
        "wango_decode_step_noalloc": (ctypes.c_int, [S, W, i32, i32, vp, vp, vp, vp, sz, vp]),
        "tango_aggregate_fwd_train": (ctypes.c_int, [S, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "tango_aggregate_bwd_workspace_size": (sz, [S]),
        "tango_stack_workspace_size": (sz, [S, i32]),
        "tango_stack_fwd": (ctypes.c_int, [S, W, i32, vp, i32, vp, vp, vp, sz, vp]),
        "wango_aggregate_fwd_train_workspace_size": (sz, [S, i32, i32]),
        "wango_aggregate_fwd_train": (ctypes.c_int, [S, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "wango_aggregate_bwd_workspace_size": (sz, [S, i32, i32]),
        "wango_aggregate_bwd": (ctypes.c_int, [S, i32, i32] + [vp] * 14 + [sz, vp]),
        "tango_aggregate_bwd": (ctypes.c_int, [S, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                               vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(code: int) -> None:
    if code != 0:
        raise TangoError(code, load().tango_last_error().decode())
