"""Python binding of libtango.so with the C ABI's names.

Argument marshalling only: tensors are torch tensors on the GPU (torch owns
the device memory and the stream); every step of the block runs in the HIP
kernels of libtango.so.  There is no fallback path: if the library is not
built, every call raises.

The C side sees raw device pointers and cannot tell a host tensor, a strided
view or a tensor of the wrong dtype from a good one, so every call here checks
each tensor first (on x's GPU, contiguous, the dtype and the shape or minimum
size the header states) and raises TypeError or ValueError before anything is
launched.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import Shape, Weights, check, load
from .layouts import ROW_PAD, head_pad, padded_len  # noqa: F401  (re-exported)

_DTYPES = {torch.float32: _lib.TANGO_F32, torch.bfloat16: _lib.TANGO_BF16}
_TORCH = {v: k for k, v in _DTYPES.items()}


def check_tensor(t, name: str, *, device: Optional[torch.device] = None, dtype=None, shape=None,
                 min_numel: Optional[int] = None, optional: bool = False) -> None:
    """Raise unless `t` can be handed to the library as `name`: a torch tensor on
    `device` (any GPU when None), contiguous, of `dtype` (one dtype or a tuple),
    of exactly `shape` and of at least `min_numel` elements.  None is accepted
    only when `optional`."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if device is None:
        if t.device.type != "cuda":
            raise ValueError(f"{name} is on {t.device}: the library reads and writes GPU memory only")
    elif t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's tensors are on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} is not contiguous (the library takes dense row-major buffers)")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(map(str, allowed))}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, at least {min_numel} are needed")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _check_ws(ws, device, need: Optional[int] = None, name: str = "workspace") -> None:
    check_tensor(ws, name, device=device)
    if need is not None and _nbytes(ws) < need:
        raise ValueError(f"{name} holds {_nbytes(ws)} bytes, the call needs {need}")


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

    def check(self, d_model: int, device: torch.device) -> None:
        """Raise unless the tensors match include/tango.h: w_g, w_v [F, d],
        w_q, w_k [H*d_h, d], w_o [d, F] and the gain [d] in one compute dtype
        (float32 or bfloat16), theta and the null bias [H] float32, all on
        `device` and contiguous."""
        check_tensor(self.w_g, "w_g", device=device, dtype=tuple(_DTYPES))
        F, dt, hd, H = self.w_g.shape[0], self.w_g.dtype, self.n_heads * self.head_dim, self.n_heads
        check_tensor(self.w_g, "w_g", device=device, shape=(F, d_model))
        check_tensor(self.w_v, "w_v", device=device, dtype=dt, shape=(F, d_model))
        check_tensor(self.w_q, "w_q", device=device, dtype=dt, shape=(hd, d_model))
        check_tensor(self.w_k, "w_k", device=device, dtype=dt, shape=(hd, d_model))
        check_tensor(self.w_o, "w_o", device=device, dtype=dt, shape=(d_model, F))
        check_tensor(self.gain, "gain", device=device, dtype=dt, shape=(d_model,), optional=True)
        check_tensor(self.theta, "theta", device=device, dtype=torch.float32, shape=(H,))
        check_tensor(self.null_bias, "null_bias", device=device, dtype=torch.float32, shape=(H,),
                     optional=True)

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
               io_dtype: Optional[torch.dtype] = None, operand_parts: int = 1) -> Shape:
    """dtype: weights and intermediate activations; io_dtype: x and out
    (defaults to dtype); operand_parts: 1 or 2 bf16 parts of the GEMMs'
    activation operand (2 only with bfloat16)."""
    io_dtype = dtype if io_dtype is None else io_dtype
    for t in (dtype, io_dtype):
        if t not in _DTYPES:
            raise TypeError(f"unsupported dtype {t}")
    if operand_parts not in (1, 2) or (operand_parts == 2 and dtype != torch.bfloat16):
        raise ValueError(f"operand_parts {operand_parts}: need 1, or 2 with bfloat16")
    return Shape(B, T, d, F, H, dh, _DTYPES[dtype], _DTYPES[io_dtype], rope_base, rms_eps, operand_parts)


def v_dtype(shape: Shape) -> torch.dtype:
    """dtype of the projection's v buffer: bfloat16 with bf16 compute and one
    operand part, else float32."""
    return torch.bfloat16 if shape.dtype == _DTYPES[torch.bfloat16] and shape.operand_parts <= 1 \
        else torch.float32


def shape_of(x: torch.Tensor, w: BlockWeights, rope_base: float = 10000.0,
             rms_eps: float = 1e-6, operand_parts: int = 1) -> Shape:
    """Shape of a call: compute dtype from the weights, I/O dtype from x.
    Checks x ([B, T, d] on a GPU, float32 or bfloat16) and the weights first."""
    check_tensor(x, "x", dtype=tuple(_DTYPES))
    if x.dim() != 3:
        raise ValueError(f"x has shape {tuple(x.shape)}, expected [B, T, d_model]")
    w.check(x.shape[2], x.device)
    B, T, d = x.shape
    return make_shape(B, T, d, w.w_g.shape[0], w.n_heads, w.head_dim, w.w_g.dtype, rope_base,
                      rms_eps, io_dtype=x.dtype, operand_parts=operand_parts)


class _Sizes:
    """Element counts of the intermediate layouts of include/tango.h for a shape
    (rows padded per sequence to a multiple of 128, gate heads padded)."""

    def __init__(self, shape: Shape, wango: bool):
        self.M = shape.batch * padded_len(shape.seq_len)
        self.F = shape.d_gate
        self.H = shape.n_heads
        self.HD = shape.n_heads * shape.head_dim
        self.Fp = shape.n_heads * head_pad(shape.d_gate // max(shape.n_heads, 1), wango)
        self.x = shape.batch * shape.seq_len * shape.d_model
        self.dt = _TORCH[shape.dtype]
        self.io = _TORCH[shape.io_dtype]


def _check_io(x, out, device, shape: Shape) -> None:
    z = _Sizes(shape, False)
    want = (shape.batch, shape.seq_len, shape.d_model)
    check_tensor(x, "x", device=device, dtype=z.io, shape=want)
    check_tensor(out, "out", device=device, dtype=z.io, shape=want)


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
                    rms_eps: float = 1e-6, stream=None, operand_parts: int = 1) -> torch.Tensor:
    """One TANGO block: returns out[B, T, d] (out may be x for in place)."""
    shape = shape_of(x, w, rope_base, rms_eps, operand_parts)
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = workspace(tango_workspace_size(shape), x.device)
    _check_io(x, out, x.device, shape)
    _check_ws(ws, x.device)
    cw = w.c_struct()
    check(load().tango_block_fwd(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(out),
                                 _ptr(ws), _nbytes(ws), _stream(stream)))
    return out


def tango_stack_workspace_size(shapes) -> int:
    """Bytes of workspace tango_stack_fwd needs for these per-set shapes (the largest block's)."""
    arr = (Shape * len(shapes))(*shapes)
    return int(load().tango_stack_workspace_size(arr, len(shapes)))


def tango_stack_fwd(x: torch.Tensor, sets, schedule, out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, rope_base: float = 10000.0,
                    rms_eps: float = 1e-6, stream=None, operand_parts: int = 1) -> torch.Tensor:
    """TANGO blocks with several parameter sets: application r uses
    ``sets[schedule[r]]`` (a list of BlockWeights).  Returns out[B, T, d]
    (out may be x for in place)."""
    shapes = [shape_of(x, w, rope_base, rms_eps, operand_parts) for w in sets]
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = workspace(tango_stack_workspace_size(shapes), x.device)
    _check_io(x, out, x.device, shapes[0])
    _check_ws(ws, x.device)
    sh = (Shape * len(shapes))(*shapes)
    cw = (Weights * len(sets))(*[w.c_struct() for w in sets])
    sched = (ctypes.c_int32 * len(schedule))(*[int(k) for k in schedule])
    check(load().tango_stack_fwd(sh, cw, len(sets), sched, len(schedule), _ptr(x), _ptr(out), _ptr(ws),
                                 _nbytes(ws), _stream(stream)))
    return out


def wango_block_fwd(x: torch.Tensor, w: BlockWeights, window: int, phi_dim: int, chunk: int,
                    out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                    rope_base: float = 10000.0, rms_eps: float = 1e-6, stream=None,
                    operand_parts: int = 1) -> torch.Tensor:
    """One WANGO block: returns out[B, T, d] (out may be x for in place)."""
    shape = shape_of(x, w, rope_base, rms_eps, operand_parts)
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = workspace(wango_workspace_size(shape, window, phi_dim, chunk), x.device)
    _check_io(x, out, x.device, shape)
    _check_ws(ws, x.device)
    cw = w.c_struct()
    check(load().wango_block_fwd(ctypes.byref(shape), ctypes.byref(cw), window, phi_dim, chunk,
                                 _ptr(x), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)))
    return out


# ---- stage entry points ---------------------------------------------------------
#
# The layout buffers are checked for device, contiguity, dtype and a minimum
# element count (they may be flat or larger than needed).

def tango_proj_workspace_size(shape: Shape) -> int:
    """Bytes of scratch the projection stages need (the prepared input rows)."""
    return int(load().tango_proj_workspace_size(ctypes.byref(shape)))


def _check_proj(shape: Shape, w: BlockWeights, x, gp, v, qh, kh, wango: bool):
    check_tensor(x, "x")
    dev = x.device
    z = _Sizes(shape, wango)
    check_tensor(x, "x", device=dev, dtype=z.io, min_numel=z.x)
    w.check(shape.d_model, dev)
    check_tensor(gp, "gp", device=dev, dtype=z.dt, min_numel=z.M * z.Fp)
    check_tensor(v, "v", device=dev, dtype=v_dtype(shape), min_numel=z.M * z.F)
    check_tensor(qh, "qh", device=dev, dtype=z.dt, min_numel=z.M * z.HD)
    check_tensor(kh, "kh", device=dev, dtype=z.dt, min_numel=z.M * z.HD)
    return dev, z


def tango_stage_proj(shape: Shape, w: BlockWeights, x, gp, v, qh, kh, ws=None, stream=None) -> None:
    """KP stage: gates (packed), v, unit q and k from x (include/tango.h layouts)."""
    dev, _ = _check_proj(shape, w, x, gp, v, qh, kh, False)
    if ws is None:
        ws = workspace(tango_proj_workspace_size(shape), dev)
    _check_ws(ws, dev)
    cw = w.c_struct()
    check(load().tango_stage_proj(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(gp),
                                  _ptr(v), _ptr(qh), _ptr(kh), _ptr(ws), _nbytes(ws), _stream(stream)))


def wango_stage_proj(shape: Shape, w: BlockWeights, x, gp, v, qh, kh, fq, fk, ws=None,
                     stream=None) -> None:
    """KP stage for WANGO: as tango_stage_proj plus the feature maps fq, fk."""
    dev, z = _check_proj(shape, w, x, gp, v, qh, kh, True)
    check_tensor(fq, "fq", device=dev, dtype=z.dt, min_numel=z.M * z.HD)
    check_tensor(fk, "fk", device=dev, dtype=z.dt, min_numel=z.M * z.HD)
    if ws is None:
        ws = workspace(tango_proj_workspace_size(shape), dev)
    _check_ws(ws, dev)
    cw = w.c_struct()
    check(load().wango_stage_proj(ctypes.byref(shape), ctypes.byref(cw), _ptr(x), _ptr(gp),
                                  _ptr(v), _ptr(qh), _ptr(kh), _ptr(fq), _ptr(fk), _ptr(ws),
                                  _nbytes(ws), _stream(stream)))


def _check_agg_in(shape: Shape, theta, null_bias, qh, kh, gp, wango: bool):
    check_tensor(qh, "qh")
    dev = qh.device
    z = _Sizes(shape, wango)
    check_tensor(theta, "theta", device=dev, dtype=torch.float32, shape=(z.H,))
    check_tensor(null_bias, "null_bias", device=dev, dtype=torch.float32, shape=(z.H,), optional=True)
    check_tensor(qh, "qh", device=dev, dtype=z.dt, min_numel=z.M * z.HD)
    check_tensor(kh, "kh", device=dev, dtype=z.dt, min_numel=z.M * z.HD)
    check_tensor(gp, "gp", device=dev, dtype=z.dt, min_numel=z.M * z.Fp)
    return dev, z


def tango_stage_aggregate(shape: Shape, theta, null_bias, qh, kh, gp, gbar, ws, stream=None) -> None:
    """KA stage: gbar from q, k and the packed gates."""
    dev, z = _check_agg_in(shape, theta, null_bias, qh, kh, gp, False)
    check_tensor(gbar, "gbar", device=dev, dtype=z.dt, min_numel=z.M * z.F)
    _check_ws(ws, dev)
    check(load().tango_stage_aggregate(ctypes.byref(shape), _ptr(theta), _ptr(null_bias), _ptr(qh),
                                       _ptr(kh), _ptr(gp), _ptr(gbar), _ptr(ws), _nbytes(ws),
                                       _stream(stream)))


def tango_aggregate_fwd_train(shape: Shape, theta, null_bias, qh, kh, gp, gbar, den, ws,
                              stream=None) -> None:
    """tango_stage_aggregate that also writes den [B, Tp, H] float32 for the backward pass."""
    dev, z = _check_agg_in(shape, theta, null_bias, qh, kh, gp, False)
    check_tensor(gbar, "gbar", device=dev, dtype=z.dt, min_numel=z.M * z.F)
    check_tensor(den, "den", device=dev, dtype=torch.float32, min_numel=z.M * z.H)
    _check_ws(ws, dev)
    check(load().tango_aggregate_fwd_train(ctypes.byref(shape), _ptr(theta), _ptr(null_bias), _ptr(qh),
                                           _ptr(kh), _ptr(gp), _ptr(gbar), _ptr(den), _ptr(ws), _nbytes(ws),
                                           _stream(stream)))


def tango_aggregate_bwd_workspace_size(shape: Shape) -> int:
    """Bytes of workspace tango_aggregate_bwd needs (0 unless bf16 and valid)."""
    return int(load().tango_aggregate_bwd_workspace_size(ctypes.byref(shape)))


def _check_bwd(shape: Shape, theta, null_bias, qh, kh, gp, gbar, den, dgbar, dq, dk, dg, dtheta, dnull,
               ws, wango: bool):
    dev, z = _check_agg_in(shape, theta, null_bias, qh, kh, gp, wango)
    check_tensor(gbar, "gbar", device=dev, dtype=z.dt, min_numel=z.M * z.F)
    check_tensor(den, "den", device=dev, dtype=torch.float32, min_numel=z.M * z.H)
    check_tensor(dgbar, "dgbar", device=dev, dtype=z.dt, min_numel=z.M * z.F)
    check_tensor(dq, "dq", device=dev, dtype=torch.float32, min_numel=z.M * z.HD)
    check_tensor(dk, "dk", device=dev, dtype=torch.float32, min_numel=z.M * z.HD)
    check_tensor(dg, "dg", device=dev, dtype=z.dt, min_numel=z.M * z.F)
    check_tensor(dtheta, "dtheta", device=dev, dtype=torch.float32, min_numel=z.H)
    check_tensor(dnull, "dnull", device=dev, dtype=torch.float32, min_numel=z.H, optional=True)
    _check_ws(ws, dev)


def tango_aggregate_bwd(shape: Shape, theta, null_bias, qh, kh, gp, gbar, den, dgbar, dq, dk, dg, dtheta,
                        dnull, ws, stream=None) -> None:
    """Gradients of sum(dgbar * gbar) of the TANGO aggregation (see include/tango.h)."""
    _check_bwd(shape, theta, null_bias, qh, kh, gp, gbar, den, dgbar, dq, dk, dg, dtheta, dnull, ws, False)
    check(load().tango_aggregate_bwd(ctypes.byref(shape), _ptr(theta), _ptr(null_bias), _ptr(qh), _ptr(kh),
                                     _ptr(gp), _ptr(gbar), _ptr(den), _ptr(dgbar), _ptr(dq), _ptr(dk),
                                     _ptr(dg), _ptr(dtheta), _ptr(dnull), _ptr(ws), _nbytes(ws),
                                     _stream(stream)))


def wango_aggregate_fwd_train_workspace_size(shape: Shape, window: int, chunk: int) -> int:
    """Bytes of workspace wango_aggregate_fwd_train needs (0 for invalid arguments)."""
    return int(load().wango_aggregate_fwd_train_workspace_size(ctypes.byref(shape), window, chunk))


def wango_aggregate_fwd_train(shape: Shape, window: int, chunk: int, theta, null_bias, qh, kh, gp, gbar, den,
                              ws, stream=None) -> None:
    """WANGO aggregation (scan + band) from unit q, k and packed gates into gbar,
    also storing the denominators den [B*Tp, H] for wango_aggregate_bwd."""
    dev, z = _check_agg_in(shape, theta, null_bias, qh, kh, gp, True)
    check_tensor(gbar, "gbar", device=dev, dtype=z.dt, min_numel=z.M * z.F)
    check_tensor(den, "den", device=dev, dtype=torch.float32, min_numel=z.M * z.H)
    _check_ws(ws, dev)
    check(load().wango_aggregate_fwd_train(ctypes.byref(shape), window, chunk, _ptr(theta), _ptr(null_bias),
                                           _ptr(qh), _ptr(kh), _ptr(gp), _ptr(gbar), _ptr(den), _ptr(ws),
                                           _nbytes(ws), _stream(stream)))


def wango_aggregate_bwd_workspace_size(shape: Shape, window: int, chunk: int) -> int:
    """Bytes of workspace wango_aggregate_bwd needs (0 for invalid arguments)."""
    return int(load().wango_aggregate_bwd_workspace_size(ctypes.byref(shape), window, chunk))


def wango_aggregate_bwd(shape: Shape, window: int, chunk: int, theta, null_bias, qh, kh, gp, gbar, den, dgbar,
                        dq, dk, dg, dtheta, dnull, ws, stream=None) -> None:
    """Gradients of sum(dgbar * gbar) for the WANGO aggregation: dq, dk (float32),
    dg (bf16), dtheta and dnull (float32, dnull None with null_bias None)."""
    _check_bwd(shape, theta, null_bias, qh, kh, gp, gbar, den, dgbar, dq, dk, dg, dtheta, dnull, ws, True)
    check(load().wango_aggregate_bwd(ctypes.byref(shape), window, chunk, _ptr(theta), _ptr(null_bias), _ptr(qh),
                                     _ptr(kh), _ptr(gp), _ptr(gbar), _ptr(den), _ptr(dgbar), _ptr(dq), _ptr(dk),
                                     _ptr(dg), _ptr(dtheta), _ptr(dnull), _ptr(ws), _nbytes(ws), _stream(stream)))


def tango_stage_out(shape: Shape, w_o, x, gbar, v, out, stream=None) -> None:
    """KO stage: out = x + (gbar * v) W_o^T."""
    check_tensor(x, "x")
    dev = x.device
    z = _Sizes(shape, False)
    check_tensor(x, "x", device=dev, dtype=z.io, min_numel=z.x)
    check_tensor(out, "out", device=dev, dtype=z.io, min_numel=z.x)
    check_tensor(w_o, "w_o", device=dev, dtype=z.dt, shape=(shape.d_model, shape.d_gate))
    check_tensor(gbar, "gbar", device=dev, dtype=z.dt, min_numel=z.M * z.F)
    check_tensor(v, "v", device=dev, dtype=v_dtype(shape), min_numel=z.M * z.F)
    check(load().tango_stage_out(ctypes.byref(shape), _ptr(w_o), _ptr(x), _ptr(gbar), _ptr(v),
                                 _ptr(out), _stream(stream)))


def wango_stage_scan(shape: Shape, window: int, chunk: int, fq, fk, gp, n_old, z_old, ws,
                     stream=None) -> None:
    """KS stage: the older-prefix read-outs n_old, z_old."""
    check_tensor(fq, "fq")
    dev = fq.device
    z = _Sizes(shape, True)
    check_tensor(fq, "fq", device=dev, dtype=z.dt, min_numel=z.M * z.HD)
    check_tensor(fk, "fk", device=dev, dtype=z.dt, min_numel=z.M * z.HD)
    check_tensor(gp, "gp", device=dev, dtype=z.dt, min_numel=z.M * z.Fp)
    check_tensor(n_old, "n_old", device=dev, dtype=torch.float32, min_numel=z.M * z.Fp)
    check_tensor(z_old, "z_old", device=dev, dtype=torch.float32, min_numel=z.M * z.H)
    _check_ws(ws, dev)
    check(load().wango_stage_scan(ctypes.byref(shape), window, chunk, _ptr(fq), _ptr(fk), _ptr(gp),
                                  _ptr(n_old), _ptr(z_old), _ptr(ws), _nbytes(ws), _stream(stream)))


def wango_stage_band(shape: Shape, theta, null_bias, window: int, chunk: int, qh, kh, gp, n_old,
                     z_old, gbar, stream=None) -> None:
    """KB stage: the window band combined with n_old, z_old into gbar."""
    dev, z = _check_agg_in(shape, theta, null_bias, qh, kh, gp, True)
    check_tensor(n_old, "n_old", device=dev, dtype=torch.float32, min_numel=z.M * z.Fp)
    check_tensor(z_old, "z_old", device=dev, dtype=torch.float32, min_numel=z.M * z.H)
    check_tensor(gbar, "gbar", device=dev, dtype=z.dt, min_numel=z.M * z.F)
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


def _check_decode(shape: Shape, w: BlockWeights, pos, x, out, state, ws=None) -> None:
    check_tensor(x, "x")
    dev = x.device
    io = _TORCH[shape.io_dtype]
    want = (shape.batch, shape.d_model)
    check_tensor(x, "x", device=dev, dtype=io, shape=want)
    check_tensor(out, "out", device=dev, dtype=io, shape=want)
    check_tensor(pos, "pos", device=dev, dtype=torch.int32, shape=(shape.batch,))
    w.check(shape.d_model, dev)
    _check_ws(state, dev, name="state")
    if ws is not None:
        _check_ws(ws, dev)


def tango_decode_step(shape: Shape, w: BlockWeights, pos: torch.Tensor, x: torch.Tensor, out: torch.Tensor,
                      state: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    """One TANGO decode step: out[B, d] at positions pos[B] (int32, device)."""
    _check_decode(shape, w, pos, x, out, state, ws)
    cw = w.c_struct()
    check(load().tango_decode_step(ctypes.byref(shape), ctypes.byref(cw), _ptr(pos), _ptr(x), _ptr(out),
                                   _ptr(state), _nbytes(state), _ptr(ws), _nbytes(ws), _stream(stream)))


def wango_decode_step(shape: Shape, w: BlockWeights, window: int, phi_dim: int, pos: torch.Tensor,
                      x: torch.Tensor, out: torch.Tensor, state: torch.Tensor, ws: torch.Tensor,
                      stream=None) -> None:
    """One WANGO decode step: out[B, d] at positions pos[B] (int32, device)."""
    _check_decode(shape, w, pos, x, out, state, ws)
    cw = w.c_struct()
    check(load().wango_decode_step(ctypes.byref(shape), ctypes.byref(cw), window, phi_dim, _ptr(pos),
                                   _ptr(x), _ptr(out), _ptr(state), _nbytes(state), _ptr(ws), _nbytes(ws),
                                   _stream(stream)))


def wango_decode_step_noalloc(shape: Shape, w: BlockWeights, window: int, phi_dim: int, pos: torch.Tensor,
                              x: torch.Tensor, out: torch.Tensor, state: torch.Tensor, stream=None) -> None:
    """wango_decode_step with the library's own scratch array (no workspace and
    no allocation; see include/tango.h for its size limit and sharing rules)."""
    _check_decode(shape, w, pos, x, out, state)
    cw = w.c_struct()
    check(load().wango_decode_step_noalloc(ctypes.byref(shape), ctypes.byref(cw), window, phi_dim, _ptr(pos),
                                           _ptr(x), _ptr(out), _ptr(state), _nbytes(state), _stream(stream)))
