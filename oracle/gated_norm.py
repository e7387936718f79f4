"""TEST INFRASTRUCTURE ONLY: the gated RMS norm that follows the SSD in a
Mamba-2 layer, fp64, CPU.

The pages name this step only through its backward kernel, _layer_norm_bwd,
the layer's largest single share of time, memory-bound (clova.ai page,
table "Share of compute time by kernel", and the case study "The highway got
wider..." / "How we fixed it"); they never write the norm out.  The reading
used here is the plain gated RMS norm of the Mamba-2 layer: the SSD output y
is gated by silu(z) and normalised over groups of consecutive channels,

    g_c   = y_c * silu(z_c),            silu(z) = z / (1 + exp(-z))
    r     = 1 / sqrt(mean_{c in group} g_c^2 + eps)
    out_c = g_c * r * w_c

for every token (row) and every group of `group_size` consecutive channels
of the flattened (head, headdim) channel axis.  The backward, for an output
gradient dout, follows from it by the chain rule:

    u_c   = g_c * r,   du_c = dout_c * w_c
    dw_c  = sum over tokens of dout_c * u_c
    dg_c  = r * (du_c - u_c * mean_{c' in group}(du_c' * u_c'))
    dy_c  = dg_c * silu(z_c)
    dz_c  = dg_c * y_c * sigma(z_c) * (1 + z_c * (1 - sigma(z_c)))

Plain numpy, one group at a time.  Pinned in tests/test_oracle_norm.py
against a hand-derived fixture, torch's rms_norm, scale invariance and
central finite differences of the forward.
"""
from __future__ import annotations

import numpy as np

from .recurrence import to_f64


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def gated_rmsnorm_fwd(y, z, w, eps: float, group_size: int):
    """y, z: (tokens, channels); w: (channels).  Returns (out, rstd) with
    rstd of shape (tokens, channels // group_size), all fp64."""
    y, z, w = to_f64(y), to_f64(z), to_f64(w)
    T, Cn = y.shape
    if Cn % group_size:
        raise ValueError("group_size must divide the channel count")
    ng = Cn // group_size
    out = np.zeros((T, Cn))
    rstd = np.zeros((T, ng))
    for k in range(ng):
        sl = slice(k * group_size, (k + 1) * group_size)
        g = y[:, sl] * (z[:, sl] * _sigmoid(z[:, sl]))
        r = 1.0 / np.sqrt(np.mean(g * g, axis=1) + eps)
        out[:, sl] = g * r[:, None] * w[None, sl]
        rstd[:, k] = r
    return out, rstd


def gated_rmsnorm_bwd(y, z, w, eps: float, group_size: int, dout):
    """Gradients (dy, dz, dw) of sum(out * dout), fp64."""
    y, z, w, dout = to_f64(y), to_f64(z), to_f64(w), to_f64(dout)
    T, Cn = y.shape
    ng = Cn // group_size
    dy = np.zeros((T, Cn))
    dz = np.zeros((T, Cn))
    dw = np.zeros(Cn)
    for k in range(ng):
        sl = slice(k * group_size, (k + 1) * group_size)
        sg = _sigmoid(z[:, sl])
        gate = z[:, sl] * sg
        g = y[:, sl] * gate
        r = 1.0 / np.sqrt(np.mean(g * g, axis=1) + eps)
        u = g * r[:, None]
        du = dout[:, sl] * w[None, sl]
        dw[sl] = np.sum(dout[:, sl] * u, axis=0)
        proj = np.mean(du * u, axis=1)
        dg = r[:, None] * (du - u * proj[:, None])
        dy[:, sl] = dg * gate
        dz[:, sl] = dg * y[:, sl] * sg * (1.0 + z[:, sl] * (1.0 - sg))
    return dy, dz, dw
