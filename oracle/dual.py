"""TEST INFRASTRUCTURE ONLY: the quadratic (dual, masked-attention) form of
the SSD forward, fp64 numpy, for tiny inputs.

The same layer written as one masked matrix product per (sequence, head):
the linear-attention view of Mamba-2 that the clova.ai page contrasts with
self-attention (section "Why optimize Mamba-2? Long context and hybrid
architectures", Figure 1 and the complexity table).  With the within-sequence
cumulative log-decay  Lam_t = sum_{k<=t} delta_k * A  and the causal decay
mask  M[t,u] = exp(Lam_t - Lam_u)  for u <= t (zero above the diagonal):

  Y     = (M o (C B^T)) (diag(delta) X) + diag(exp(Lam)) (C h0^T) + D X
  final = sum_u exp(Lam_last - Lam_u) delta_u x_u (x) B_u + exp(Lam_last) h0

It is written independently of the C recurrence (different softplus
routine, matrix form instead of a token loop) so that the two pin each other.
"""
from __future__ import annotations

import math

import numpy as np

from .recurrence import to_f64, seq_ranges


def _delta(dt_raw: np.ndarray, bias: float, dt_min: float, dt_max: float) -> np.ndarray:
    # softplus via the library's log(exp(0) + exp(u))
    return np.clip(np.logaddexp(0.0, dt_raw + bias), dt_min, dt_max)


def ssd_dual(x, dt, dt_bias, A, B, C, D, init=None, cu_seqlens=None,
             dt_min: float = 0.0, dt_max: float = math.inf):
    """Returns y (b, T, H, P) and final (nseq, H, P, N) in fp64."""
    X = to_f64(x)
    b, T, H, P = X.shape
    Bm, Cm = to_f64(B), to_f64(C)
    G, N = Bm.shape[2], Bm.shape[3]
    X = X.reshape(b * T, H, P)
    Bm, Cm = Bm.reshape(b * T, G, N), Cm.reshape(b * T, G, N)
    DT = to_f64(dt).reshape(b * T, H)
    bias = to_f64(dt_bias) if dt_bias is not None else np.zeros(H)
    Av = to_f64(A)
    Dv = to_f64(D) if D is not None else np.zeros(H)
    h0 = to_f64(init)
    starts, lens = seq_ranges(b, T, cu_seqlens)
    y = np.zeros((b * T, H, P))
    fin = np.zeros((len(starts), H, P, N))
    hpg = H // G
    for s, (t0, n) in enumerate(zip(starts, lens)):
        sl = slice(int(t0), int(t0 + n))
        for h in range(H):
            g = h // hpg
            d = _delta(DT[sl, h], bias[h], dt_min, dt_max)          # (n,)
            lam = np.cumsum(d * Av[h])                               # (n,)
            diff = lam[:, None] - lam[None, :]
            causal = np.tril(np.ones((n, n), dtype=bool))
            Mk = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
            Cs, Bs, Xs = Cm[sl, g, :], Bm[sl, g, :], X[sl, h, :]
            yy = (Mk * (Cs @ Bs.T)) @ (d[:, None] * Xs) + Dv[h] * Xs
            ff = ((np.exp(lam[-1] - lam) * d)[:, None] * Xs).T @ Bs if n > 0 else np.zeros((P, N))
            if h0 is not None:
                H0 = h0[s, h]                                        # (P, N)
                yy = yy + np.exp(lam)[:, None] * (Cs @ H0.T)
                ff = ff + (math.exp(lam[-1]) if n > 0 else 1.0) * H0
            y[sl, h, :] = yy
            fin[s, h] = ff
    return y.reshape(b, T, H, P), fin
