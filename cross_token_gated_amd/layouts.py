"""Host-side (numpy) packers of the library's intermediate layouts, for callers
that hand the stage and backward entry points their own tensors.

They hold no arithmetic of the method, only index shuffles.  The layouts are
the ones include/tango.h documents: rows padded per sequence to a multiple of
128; gates in the source-packed layout [M/32][4][F][8]; the WANGO older-prefix
numerator in 16x16 blocks [M/16][F/16][64][4]; gate heads padded to the widths
of head_pad.
"""
from __future__ import annotations

import numpy as np

ROW_PAD = 128


def padded_len(T: int) -> int:
    return (T + ROW_PAD - 1) // ROW_PAD * ROW_PAD


def pad_rows(a: np.ndarray, Tp: int) -> np.ndarray:
    """[B, T, X] -> [B*Tp, X] with zero rows appended to every sequence."""
    B, T, X = a.shape
    out = np.zeros((B, Tp, X), dtype=a.dtype)
    out[:, :T] = a
    return out.reshape(B * Tp, X)


def unpad_rows(a: np.ndarray, B: int, T: int) -> np.ndarray:
    return a.reshape(B, -1, a.shape[-1])[:, :T]


# slot s of k group g in a packed block of 32 rows holds row _PERM[g, s]: the
# row order of two stacked 16x16 MFMA accumulator blocks
_PERM = np.array([[4 * g + s if s < 4 else 16 + 4 * g + (s - 4) for s in range(8)]
                  for g in range(4)])


def head_pad(fh: int, wango: bool) -> int:
    """The padded head width Fhp of the gate layouts: fh when it is a multiple
    of 64; else WANGO rounds up to 64, TANGO to 512 when that is at most 1.2 fh,
    else to 64."""
    if fh % 64 == 0:
        return fh
    p512 = (fh + 511) // 512 * 512
    if not wango and 5 * p512 <= 6 * fh:
        return p512
    return (fh + 63) // 64 * 64


def pad_heads(g_rows: np.ndarray, n_heads: int, fhp: int) -> np.ndarray:
    """[M, H*Fh] -> [M, H*Fhp]: head a's column c moved to a*Fhp + c, pad columns zero."""
    M, F = g_rows.shape
    fh = F // n_heads
    out = np.zeros((M, n_heads, fhp), dtype=g_rows.dtype)
    out[:, :, :fh] = g_rows.reshape(M, n_heads, fh)
    return out.reshape(M, n_heads * fhp)


def pack_gates(g_rows: np.ndarray) -> np.ndarray:
    """[M, F] (M % 32 == 0) -> packed [M/32, 4, F, 8]."""
    M, F = g_rows.shape
    blk = g_rows.reshape(M // 32, 32, F)
    sel = blk[:, _PERM.reshape(-1), :].reshape(M // 32, 4, 8, F)
    return np.ascontiguousarray(sel.transpose(0, 1, 3, 2))


def unpack_gates(gp: np.ndarray, M: int, F: int) -> np.ndarray:
    sel = gp.reshape(M // 32, 4, F, 8).transpose(0, 1, 3, 2).reshape(M // 32, 32, F)
    out = np.empty((M // 32, 32, F), dtype=gp.dtype)
    out[:, _PERM.reshape(-1), :] = sel
    return out.reshape(M, F)


def permute_features(a: np.ndarray) -> np.ndarray:
    """[..., D] (D % 32 == 0) -> the permuted feature order: position 8g + s of
    each group of 32 holds feature _PERM[g, s]."""
    D = a.shape[-1]
    src = np.concatenate([32 * c + _PERM.reshape(-1) for c in range(D // 32)])
    return np.ascontiguousarray(a[..., src])


def unpermute_features(a: np.ndarray) -> np.ndarray:
    D = a.shape[-1]
    src = np.concatenate([32 * c + _PERM.reshape(-1) for c in range(D // 32)])
    out = np.empty_like(a)
    out[..., src] = a
    return out


def unblock_nold(nb: np.ndarray, M: int, F: int) -> np.ndarray:
    """[M/16, F/16, 64, 4] -> [M, F]: lane l holds row l%16, columns 4(l/16)+r."""
    a = nb.reshape(M // 16, F // 16, 4, 16, 4)        # ib, fb, lg, li, r
    return np.ascontiguousarray(a.transpose(0, 3, 1, 2, 4)).reshape(M, F)


def block_nold(n: np.ndarray) -> np.ndarray:
    M, F = n.shape
    a = n.reshape(M // 16, 16, F // 16, 4, 4)          # ib, li, fb, lg, r
    return np.ascontiguousarray(a.transpose(0, 2, 3, 1, 4)).reshape(M // 16, F // 16, 64, 4)
