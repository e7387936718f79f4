"""TEST INFRASTRUCTURE ONLY: Python entry to the fp64 C recurrence oracle.

The arithmetic lives in ssd_recurrence.c (per-token update of the Mamba-2
layer's fixed-size hidden state; aiproviderindex page, "Mamba-2 offers a
different scaling path").  This wrapper only
selects heads, upcasts inputs exactly to fp64 and marshals pointers.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.POINTER
        d, i64 = ctypes.c_double, ctypes.c_int64
        lib.ssd_oracle_recurrence.restype = ctypes.c_int
        lib.ssd_oracle_recurrence.argtypes = [
            i64, P(i64), P(i64), i64, i64, i64, i64, i64,
            P(d), P(d), P(d), P(d), P(i64), P(d), P(d), P(d), P(d),
            d, d, P(d), P(d), ctypes.c_int]
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def to_f64(a) -> Optional[np.ndarray]:
    """Exact upcast of a CPU torch tensor (fp32/bf16/fp64) or array to fp64."""
    if a is None:
        return None
    if hasattr(a, "detach"):          # torch tensor
        import torch
        t = a.detach().cpu()
        if t.dtype in (torch.bfloat16, torch.float16):
            t = t.to(torch.float32)
        return np.ascontiguousarray(t.numpy().astype(np.float64))
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, ct=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ct))


def seq_ranges(batch: int, seqlen: int, cu_seqlens=None):
    """(starts, lens) of the sequences on the flattened (batch*seqlen) axis."""
    if cu_seqlens is None:
        starts = np.arange(batch, dtype=np.int64) * seqlen
        lens = np.full(batch, seqlen, dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                        dtype=np.int64)
        starts = np.ascontiguousarray(cu[:-1])
        lens = np.ascontiguousarray(cu[1:] - cu[:-1])
    return starts, lens


def ssd_recurrence(x, dt, dt_bias, A, B, C, D, init=None, cu_seqlens=None,
                   heads: Optional[Sequence[int]] = None, dt_min: float = 0.0,
                   dt_max: float = math.inf, nthreads: int = 0):
    """Run the fp64 recurrence.

    x (b, T, H, P), dt (b, T, H), dt_bias (H) or None, A (H), B/C (b, T, G, N),
    D (H) or None, init (nseq, H, P, N) or None, cu_seqlens (nseq+1) or None.
    heads: subset of heads to compute (default all).
    Returns y (b, T, Hs, P) and final (nseq, Hs, P, N), fp64, for the heads
    in the given order.
    """
    b, T, H, P = (int(s) for s in x.shape)
    G, N = int(B.shape[2]), int(B.shape[3])
    if heads is None:
        heads = list(range(H))
    heads = [int(h) for h in heads]
    Hs = len(heads)
    hidx = np.asarray(heads, dtype=np.int64)
    grp = np.ascontiguousarray(hidx // (H // G), dtype=np.int64)

    def sel(a, axis):
        if a is None:
            return None
        if hasattr(a, "index_select"):
            import torch
            return a.index_select(axis, torch.as_tensor(hidx))
        return np.take(np.asarray(a), hidx, axis=axis)

    xs = to_f64(sel(x, 2)).reshape(b * T, Hs, P)
    dts = to_f64(sel(dt, 2)).reshape(b * T, Hs)
    dtb = to_f64(sel(dt_bias, 0)) if dt_bias is not None else None
    As = to_f64(sel(A, 0))
    Ds = to_f64(sel(D, 0)) if D is not None else None
    Bf = to_f64(B).reshape(b * T, G, N)
    Cf = to_f64(C).reshape(b * T, G, N)
    starts, lens = seq_ranges(b, T, cu_seqlens)
    nseq = len(starts)
    ini = to_f64(sel(init, 1)) if init is not None else None
    y = np.zeros((b * T, Hs, P), dtype=np.float64)
    fin = np.zeros((nseq, Hs, P, N), dtype=np.float64)
    i64 = ctypes.c_int64
    rc = _load().ssd_oracle_recurrence(
        nseq, _ptr(starts, i64), _ptr(lens, i64), b * T, Hs, P, N, G,
        _ptr(xs), _ptr(dts), _ptr(dtb), _ptr(As), _ptr(grp, i64),
        _ptr(Bf), _ptr(Cf), _ptr(Ds), _ptr(ini), float(dt_min), float(dt_max),
        _ptr(y), _ptr(fin), int(nthreads))
    if rc != 0:
        raise ValueError("oracle recurrence rejected its arguments")
    return y.reshape(b, T, Hs, P), fin
