"""TEST INFRASTRUCTURE ONLY: gradients of the SSD forward, fp64, CPU.

The pages list the layer's backward kernels next to the forward ones
(clova.ai page, table "Share of compute time by kernel": _chunk_scan_bwd_dx,
_chunk_state_bwd_db, _state_passing_bwd and the others).  What they compute
is fixed by the forward: the gradients of a scalar loss

    loss = sum(y * dy) + sum(final * dfinal)

with respect to every input (x, dt, dt_bias, A, B, C, D, initial states).
Here that definition is taken literally: reverse-mode differentiation
(torch.autograd, float64, CPU) of the forward written out in one of two
forms, independent of the chunked GPU algorithm:

  "dual"        per (sequence, head), the quadratic masked form
                Y = (M o (C B^T)) (diag(delta) X) + diag(exp(Lam)) C h0^T + D X
                with Lam = cumsum(delta A) and M[t,u] = exp(Lam_t - Lam_u)
                for u <= t (the linear-attention view; clova.ai page,
                section "Why optimize Mamba-2? Long context and hybrid
                architectures");
  "recurrence"  token by token, h_t = exp(delta_t A) h_{t-1} + delta_t
                x_t B_t^T, y_t = C_t h_t + D x_t (tiny inputs only).

delta = clamp(softplus(dt + dt_bias), dt_min, dt_max), softplus written as
log(1 + e^u) via logaddexp; the clamp passes the gradient where
dt_min <= softplus <= dt_max (torch.clamp's rule).

Pinned by tests against central finite differences of the C recurrence
(oracle/ssd_recurrence.c, separate code) and against closed forms.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from .recurrence import seq_ranges, to_f64

NAMES = ("x", "dt", "dt_bias", "A", "B", "C", "D", "init")


def _t(a):
    return None if a is None else torch.from_numpy(to_f64(a)).requires_grad_(True)


def _delta(dt_raw, bias, dt_min, dt_max):
    sp = torch.logaddexp(torch.zeros_like(dt_raw), dt_raw + bias)
    return torch.clamp(sp, min=dt_min, max=dt_max if math.isfinite(dt_max) else None)


def _forward_dual(X, DT, bias, Av, Bm, Cm, Dv, h0, starts, lens, G, dt_min, dt_max):
    """y (tokens, H, P) and final (nseq, H, P, N) as differentiable tensors."""
    H, P = X.shape[1], X.shape[2]
    N = Bm.shape[2]
    hpg = H // G
    ys = [[None] * H for _ in starts]
    fins = []
    for s, (t0, n) in enumerate(zip(starts, lens)):
        t0, n = int(t0), int(n)
        sl = slice(t0, t0 + n)
        fs = []
        for h in range(H):
            g = h // hpg
            d = _delta(DT[sl, h], bias[h], dt_min, dt_max)
            lam = torch.cumsum(d * Av[h], 0)
            causal = torch.tril(torch.ones((n, n), dtype=torch.bool))
            diff = torch.where(causal, lam[:, None] - lam[None, :],
                               torch.full((n, n), -math.inf, dtype=torch.float64))
            Mk = torch.exp(diff)
            Cs, Bs, Xs = Cm[sl, g, :], Bm[sl, g, :], X[sl, h, :]
            yy = (Mk * (Cs @ Bs.T)) @ (d[:, None] * Xs)
            if Dv is not None:
                yy = yy + Dv[h] * Xs
            if n > 0:
                ff = ((torch.exp(lam[-1] - lam) * d)[:, None] * Xs).T @ Bs
            else:
                ff = torch.zeros((P, N), dtype=torch.float64)
            if h0 is not None:
                H0 = h0[s, h]
                if n > 0:
                    yy = yy + torch.exp(lam)[:, None] * (Cs @ H0.T)
                    ff = ff + torch.exp(lam[-1]) * H0
                else:
                    ff = ff + H0
            ys[s][h] = yy
            fs.append(ff)
        fins.append(torch.stack(fs))
    y = torch.cat([torch.stack(row, dim=1) for row in ys], dim=0) if starts.size else \
        torch.zeros((0, H, P), dtype=torch.float64)
    return y, torch.stack(fins)


def _forward_recurrence(X, DT, bias, Av, Bm, Cm, Dv, h0, starts, lens, G, dt_min, dt_max):
    H, P = X.shape[1], X.shape[2]
    N = Bm.shape[2]
    hpg = H // G
    rows, fins = [], []
    for s, (t0, n) in enumerate(zip(starts, lens)):
        t0, n = int(t0), int(n)
        fs = []
        per_head = []
        for h in range(H):
            g = h // hpg
            st = h0[s, h] if h0 is not None else torch.zeros((P, N), dtype=torch.float64)
            out = []
            for t in range(t0, t0 + n):
                d = _delta(DT[t, h], bias[h], dt_min, dt_max)
                st = torch.exp(d * Av[h]) * st + d * torch.outer(X[t, h], Bm[t, g])
                yt = st @ Cm[t, g]
                if Dv is not None:
                    yt = yt + Dv[h] * X[t, h]
                out.append(yt)
            per_head.append(torch.stack(out) if out else torch.zeros((0, P), dtype=torch.float64))
            fs.append(st)
        rows.append(torch.stack(per_head, dim=1))
        fins.append(torch.stack(fs))
    y = torch.cat(rows, dim=0) if rows else torch.zeros((0, H, P), dtype=torch.float64)
    return y, torch.stack(fins)


def ssd_grads(x, dt, dt_bias, A, B, C, D, dy, dfinal=None, init=None, cu_seqlens=None,
              dt_min: float = 0.0, dt_max: float = math.inf, form: str = "dual") -> dict:
    """Gradients of sum(y * dy) + sum(final * dfinal), fp64 numpy arrays.

    Shapes as the forward: x (b, T, H, P), dt (b, T, H), dt_bias (H) or None,
    A (H), B/C (b, T, G, N), D (H) or None, init (nseq, H, P, N) or None,
    cu_seqlens (nseq + 1) or None; dy like x, dfinal like the final states
    (or None: zero).  Returns {name: gradient} for x, dt, dt_bias, A, B, C, D
    and init (None where the input was None).
    """
    b, T, H, P = (int(v) for v in x.shape)
    G, N = int(B.shape[2]), int(B.shape[3])
    ins = {"x": _t(x), "dt": _t(dt), "dt_bias": _t(dt_bias), "A": _t(A), "B": _t(B),
           "C": _t(C), "D": _t(D), "init": _t(init)}
    X = ins["x"].reshape(b * T, H, P)
    DT = ins["dt"].reshape(b * T, H)
    bias = ins["dt_bias"] if ins["dt_bias"] is not None else torch.zeros(H, dtype=torch.float64)
    Bm = ins["B"].reshape(b * T, G, N)
    Cm = ins["C"].reshape(b * T, G, N)
    starts, lens = seq_ranges(b, T, cu_seqlens)
    fwd = _forward_dual if form == "dual" else _forward_recurrence
    y, fin = fwd(X, DT, bias, ins["A"], Bm, Cm, ins["D"], ins["init"], starts, lens, G,
                 dt_min, dt_max)
    gy = torch.from_numpy(to_f64(dy)).reshape(b * T, H, P)
    if cu_seqlens is not None:
        # tokens outside every sequence contribute nothing
        covered = torch.zeros(b * T, dtype=torch.bool)
        for t0, n in zip(starts, lens):
            covered[int(t0):int(t0 + n)] = True
        gy = gy[covered]
    loss = (y * gy).sum()
    if dfinal is not None:
        loss = loss + (fin * torch.from_numpy(to_f64(dfinal))).sum()
    leaves = [v for v in ins.values() if v is not None]
    grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    out, k = {}, 0
    for name in NAMES:
        if ins[name] is None:
            out[name] = None
            continue
        g = grads[k]
        k += 1
        out[name] = np.zeros(ins[name].shape) if g is None else g.detach().numpy()
    return out
