"""Python binding of libtango.so with the C ABI's names.

Argument marshalling only: tensors are torch tensors on the GPU (torch owns
the device memory and the stream); every step of the block runs in the HIP
kernels of libtango.so.  There is no fallback path: if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import Shape, Weights, check, load

ROW_PAD = 128   # intermediate rows are padded per sequence to a multiple of this


def padded_len(T: int) -> int:
    return (T + ROW_PAD - 1) // ROW_PAD * ROW_PAD


_DTYPES = {torch.float32: _lib.TANGO_F32, torch.bfloat16: _lib.TANGO_BF16}


@dataclass
class BlockWeights:
    """Device tensors of one block ([F, d] gate/value, [H*d_h, d] query/key,
    [d, F] output, optional [d] RMSNorm gain, [H] float32 temperature logits
    theta and optional [H] float32 null-gate biases)."""
    w_g: torch.Tensor
    w_v: torch.Tensor
    w_q: torch.Tensor
    w_k: torch.Tensor
    w_o: torch.Tensor
    theta: torch.Tensor
    n_heads: int
    head_dim: int
    gain: Optional[torch.Tensor] = None
    null_bias: Optional[torch.Tensor] = None

    def c_struct(self) -> Weights:
        p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        return Weights(p(self.w_g), p(self.w_v), p(self.w_q), p(self.w_k), p(self.w_o),
                       p(self.gain), p(self.theta), p(self.null_bias))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_shape(B: int, T: int, d: int, F: int, H: int, dh: int, dtype: torch.dtype,
               rope_base: float = 10000.0, rms_eps: float = 1e-6,
               io_dtype: Optional[torch.dtype] = None) -> Shape:
    """dtype: weights and intermediate activations; io_dtype: x and out
    (defaults to dtype)."""
    io_dtype = dtype if io_dtype is None else io_dtype
    for t in (dtype, io_dtype):
        if t not in _DTYPES:
            raise TypeError(f"unsupported dtype {t}")
    return Shape(B, T, d, F, H, dh, _DTYPES[dtype], _DTYPES[io_dtype], rope_base, rms_eps)


def shape_of(x: torch.Tensor, w: BlockWeights, rope_base: float = 10000.0,
             rms_eps: float = 1e-6) -> Shape:
    """Shape of a call: compute dtype from the weights, I/O dtype from x."""
    B, T, d = x.shape
    return make_shape(B, T, d, w.w_g.shape[0], w.n_heads, w.head_dim, w.w_g.dtype, rope_base,
                      rms_eps, io_dtype=x.dtype)


def tango_workspace_size(shape: Shape) -> int:
    """Bytes of workspace tango_block_fwd needs (0 for an invalid shape)."""
    return int(load().tango_workspace_size(ctypes.byref(shape)))


def wango_workspace_size(shape: Shape, window: int, phi_dim: int, chunk: int) -> int:
    """Bytes of workspace wango_block_fwd needs (0 for invalid arguments)."""
    return int(load().wango_workspace_size(ctypes.byref(shape), window, phi_dim, chunk))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A byte tensor usable as a workspace (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def tango_block_fwd(x: torch.Tensor, w: BlockWeights, out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, rope_base: float = 10000.0,
                    rms_eps: float = 1e-6, stream=None) -> torch.Tensor:
    """One TANGO block: returns out[B, T, d] (out may be x for in place)."""
    shape = shape_of(x, w, rope_base, rms_eps)
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = workspace(tango_workspace_size(shape), x.device)
    cw = w.c_struct()
    check(load().tango_block_fwd(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(out),
                                 _ptr(ws), ws.numel(), _stream(stream)))
    return out


def tango_stack_workspace_size(shapes) -> int:
    """Bytes of workspace tango_stack_fwd needs for these per-set shapes (the largest block's)."""
    arr = (Shape * len(shapes))(*shapes)
    return int(load().tango_stack_workspace_size(arr, len(shapes)))


def tango_stack_fwd(x: torch.Tensor, sets, schedule, out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, rope_base: float = 10000.0,
                    rms_eps: float = 1e-6, stream=None) -> torch.Tensor:
    """TANGO blocks with several parameter sets: application r uses
    ``sets[schedule[r]]`` (a list of BlockWeights).  Returns out[B, T, d]
    (out may be x for in place)."""
    shapes = [shape_of(x, w, rope_base, rms_eps) for w in sets]
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = workspace(tango_stack_workspace_size(shapes), x.device)
    sh = (Shape * len(shapes))(*shapes)
    cw = (Weights * len(sets))(*[w.c_struct() for w in sets])
    sched = (ctypes.c_int32 * len(schedule))(*[int(k) for k in schedule])
    check(load().tango_stack_fwd(sh, cw, len(sets), sched, len(schedule), _ptr(x), _ptr(out), _ptr(ws),
                                 ws.numel(), _stream(stream)))
    return out


def wango_block_fwd(x: torch.Tensor, w: BlockWeights, window: int, phi_dim: int, chunk: int,
                    out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                    rope_base: float = 10000.0, rms_eps: float = 1e-6, stream=None) -> torch.Tensor:
    """One WANGO block: returns out[B, T, d] (out may be x for in place)."""
    shape = shape_of(x, w, rope_base, rms_eps)
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = workspace(wango_workspace_size(shape, window, phi_dim, chunk), x.device)
    cw = w.c_struct()
    check(load().wango_block_fwd(ctypes.byref(shape), ctypes.byref(cw), window, phi_dim, chunk,
                                 _ptr(x), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


# ---- stage entry points ---------------------------------------------------------

def tango_proj_workspace_size(shape: Shape) -> int:
    """Bytes of scratch the projection stages need (the prepared input rows)."""
    return int(load().tango_proj_workspace_size(ctypes.byref(shape)))


def tango_stage_proj(shape: Shape, w: BlockWeights, x, gp, v, qh, kh, ws=None, stream=None) -> None:
    """KP stage: gates (packed), v, unit q and k from x (include/tango.h layouts)."""
    cw = w.c_struct()
    if ws is None:
        ws = workspace(tango_proj_workspace_size(shape), x.device)
    check(load().tango_stage_proj(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(gp),
                                  _ptr(v), _ptr(qh), _ptr(kh), _ptr(ws), ws.numel(), _stream(stream)))


def wango_stage_proj(shape: Shape, w: BlockWeights, x, gp, v, qh, kh, fq, fk, ws=None,
                     stream=None) -> None:
    """KP stage for WANGO: as tango_stage_proj plus the feature maps fq, fk."""
    cw = w.c_struct()
    if ws is None:
        ws = workspace(tango_proj_workspace_size(shape), x.device)
    check(load().wango_stage_proj(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(gp),
                                  _ptr(v), _ptr(qh), _ptr(kh), _ptr(fq), _ptr(fk), _ptr(ws),
                                  ws.numel(), _stream(stream)))


def tango_stage_aggregate(shape: Shape, theta, null_bias, qh, kh, gp, gbar, ws, stream=None) -> None:
    """KA stage: gbar from q, k and the packed gates."""
    check(load().tango_stage_aggregate(ctypes.byref(shape), _ptr(theta), _ptr(null_bias), _ptr(qh),
                                       _ptr(kh), _ptr(gp), _ptr(gbar), _ptr(ws), ws.numel(),
                                       _stream(stream)))


def tango_aggregate_fwd_train(shape: Shape, theta, null_bias, qh, kh, gp, gbar, den, ws,
                              stream=None) -> None:
    """tango_stage_aggregate that also writes den [B, Tp, H] float32 for the backward pass."""
    check(load().tango_aggregate_fwd_train(ctypes.byref(shape), _ptr(theta), _ptr(null_bias), _ptr(qh),
                                           _ptr(kh), _ptr(gp), _ptr(gbar), _ptr(den), _ptr(ws), ws.numel(),
                                           _stream(stream)))


def tango_aggregate_bwd_workspace_size(shape: Shape) -> int:
    """Bytes of workspace tango_aggregate_bwd needs (0 unless bf16 and valid)."""
    return int(load().tango_aggregate_bwd_workspace_size(ctypes.byref(shape)))


def tango_aggregate_bwd(shape: Shape, theta, null_bias, qh, kh, gp, gbar, den, dgbar, dq, dk, dg, dtheta,
                        dnull, ws, stream=None) -> None:
    """Gradients of sum(dgbar * gbar) of the TANGO aggregation (see include/tango.h)."""
    check(load().tango_aggregate_bwd(ctypes.byref(shape), _ptr(theta), _ptr(null_bias), _ptr(qh), _ptr(kh),
                                     _ptr(gp), _ptr(gbar), _ptr(den), _ptr(dgbar), _ptr(dq), _ptr(dk),
                                     _ptr(dg), _ptr(dtheta), _ptr(dnull), _ptr(ws), ws.numel(),
                                     _stream(stream)))


def wango_aggregate_fwd_train_workspace_size(shape: Shape, window: int, chunk: int) -> int:
    """Bytes of workspace wango_aggregate_fwd_train needs (0 for invalid arguments)."""
    return int(load().wango_aggregate_fwd_train_workspace_size(ctypes.byref(shape), window, chunk))


def wango_aggregate_fwd_train(shape: Shape, window: int, chunk: int, theta, null_bias, qh, kh, gp, gbar, den,
                              ws, stream=None) -> None:
    """WANGO aggregation (scan + band) from unit q, k and packed gates into gbar,
    also storing the denominators den [B*Tp, H] for wango_aggregate_bwd."""
    check(load().wango_aggregate_fwd_train(ctypes.byref(shape), window, chunk, _ptr(theta), _ptr(null_bias),
                                           _ptr(qh), _ptr(kh), _ptr(gp), _ptr(gbar), _ptr(den), _ptr(ws),
                                           ws.numel(), _stream(stream)))


def wango_aggregate_bwd_workspace_size(shape: Shape, window: int, chunk: int) -> int:
    """Bytes of workspace wango_aggregate_bwd needs (0 for invalid arguments)."""
    return int(load().wango_aggregate_bwd_workspace_size(ctypes.byref(shape), window, chunk))


def wango_aggregate_bwd(shape: Shape, window: int, chunk: int, theta, null_bias, qh, kh, gp, gbar, den, dgbar,
                        dq, dk, dg, dtheta, dnull, ws, stream=None) -> None:
    """Gradients of sum(dgbar * gbar) for the WANGO aggregation: dq, dk (float32),
    dg (bf16), dtheta and dnull (float32, dnull None with null_bias None)."""
    check(load().wango_aggregate_bwd(ctypes.byref(shape), window, chunk, _ptr(theta), _ptr(null_bias), _ptr(qh),
                                     _ptr(kh), _ptr(gp), _ptr(gbar), _ptr(den), _ptr(dgbar), _ptr(dq), _ptr(dk),
                                     _ptr(dg), _ptr(dtheta), _ptr(dnull), _ptr(ws), ws.numel(), _stream(stream)))


def tango_stage_out(shape: Shape, w_o, x, gbar, v, out, stream=None) -> None:
    """KO stage: out = x + (gbar * v) W_o^T."""
    check(load().tango_stage_out(ctypes.byref(shape), _ptr(w_o), _ptr(x), _ptr(gbar), _ptr(v),
                                 _ptr(out), _stream(stream)))


def wango_stage_scan(shape: Shape, window: int, chunk: int, fq, fk, gp, n_old, z_old, ws,
                     stream=None) -> None:
    """KS stage: the older-prefix read-outs n_old, z_old."""
    check(load().wango_stage_scan(ctypes.byref(shape), window, chunk, _ptr(fq), _ptr(fk), _ptr(gp),
                                  _ptr(n_old), _ptr(z_old), _ptr(ws), ws.numel(), _stream(stream)))


def wango_stage_band(shape: Shape, theta, null_bias, window: int, chunk: int, qh, kh, gp, n_old,
                     z_old, gbar, stream=None) -> None:
    """KB stage: the window band combined with n_old, z_old into gbar."""
    check(load().wango_stage_band(ctypes.byref(shape), _ptr(theta), _ptr(null_bias), window, chunk,
                                  _ptr(qh), _ptr(kh), _ptr(gp), _ptr(n_old), _ptr(z_old),
                                  _ptr(gbar), _stream(stream)))


# ---- autoregressive decode ---------------------------------------------------------

def decode_shape(B: int, capacity: int, w: BlockWeights, io_dtype: torch.dtype, d: int,
                 rope_base: float = 10000.0, rms_eps: float = 1e-6) -> Shape:
    """Shape of a decode call: B sequences; capacity = TANGO cache positions
    (WANGO: any value >= 1)."""
    return make_shape(B, capacity, d, w.w_g.shape[0], w.n_heads, w.head_dim, w.w_g.dtype, rope_base,
                      rms_eps, io_dtype=io_dtype)


def tango_decode_state_size(shape: Shape) -> int:
    """Bytes of the TANGO decode state (key and gate cache) for shape."""
    return int(load().tango_decode_state_size(ctypes.byref(shape)))


def tango_decode_workspace_size(shape: Shape) -> int:
    """Bytes of scratch one TANGO decode step needs."""
    return int(load().tango_decode_workspace_size(ctypes.byref(shape)))


def wango_decode_state_size(shape: Shape, window: int, phi_dim: int) -> int:
    """Bytes of the WANGO decode state (running sums and window ring)."""
    return int(load().wango_decode_state_size(ctypes.byref(shape), window, phi_dim))


def wango_decode_workspace_size(shape: Shape, window: int, phi_dim: int) -> int:
    """Bytes of scratch one WANGO decode step needs."""
    return int(load().wango_decode_workspace_size(ctypes.byref(shape), window, phi_dim))


def tango_decode_step(shape: Shape, w: BlockWeights, pos: torch.Tensor, x: torch.Tensor, out: torch.Tensor,
                      state: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    """One TANGO decode step: out[B, d] at positions pos[B] (int32, device)."""
    cw = w.c_struct()
    check(load().tango_decode_step(ctypes.byref(shape), ctypes.byref(cw), _ptr(pos), _ptr(x), _ptr(out),
                                   _ptr(state), state.numel(), _ptr(ws), ws.numel(), _stream(stream)))


def wango_decode_step(shape: Shape, w: BlockWeights, window: int, phi_dim: int, pos: torch.Tensor,
                      x: torch.Tensor, out: torch.Tensor, state: torch.Tensor, ws: torch.Tensor,
                      stream=None) -> None:
    """One WANGO decode step: out[B, d] at positions pos[B] (int32, device)."""
    cw = w.c_struct()
    check(load().wango_decode_step(ctypes.byref(shape), ctypes.byref(cw), window, phi_dim, _ptr(pos),
                                   _ptr(x), _ptr(out), _ptr(state), state.numel(), _ptr(ws), ws.numel(),
                                   _stream(stream)))
