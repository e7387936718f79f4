"""TEST INFRASTRUCTURE ONLY: the SSD chunked scan written out stage by stage
in fp64 numpy, returning every intermediate.

The stages are the ones the pages name for the Mamba-2 forward: the
chunk-wise cumulative sum of the discretised step (aiproviderindex.com,
"Mamba-2 offers a different scaling path": chunk_cumsum), the per-chunk
state (clova.ai, table "Share of compute time by kernel": _chunk_state_fwd),
the inter-chunk state passing (_state_passing_fwd; "state propagation") and
the output construction (_chunk_scan_fwd; compute_out).  The pages give no
formulas; the stage contents below are the plain split of the recurrence at
chunk boundaries.  In exact arithmetic the result equals the recurrence for
every chunk size; the tests check that for L in {1, 3, 16, 64, T}.

Chunks never straddle a sequence: sequence s (a batch row, or a cu_seqlens
segment) owns ceil(len_s / L) chunks starting at its first token, so only its
last chunk can be short.  Per logical chunk c with clen valid tokens:

  delta[c,h,l]   softplus(dt + dt_bias) clamped; 0 for l >= clen
  dAcs[c,h,l]    sum_{k<=l} delta[c,h,k] * A[h]    (flat for l >= clen)
  CB[c,g,l,s]    sum_n C[l,g,n] B[s,g,n]            (l, s < clen)
  S[c,h,p,n]     sum_l exp(dAcs[last] - dAcs[l]) delta[l] x[l,h,p] B[l,g,n]
  Hin[c,h]       state entering chunk c: init of its sequence for the first
                 chunk, else exp(dAcs[c-1,last]) Hin[c-1] + S[c-1]
  y[l,h,p]       sum_{s<=l} CB[l,s] exp(dAcs[l]-dAcs[s]) delta[s] x[s,h,p]
                 + exp(dAcs[l]) sum_n C[l,g,n] Hin[c,h,p,n] + D[h] x[l,h,p]
  final[s,h]     exp(dAcs[last chunk, last]) Hin[last] + S[last]
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np

from .recurrence import to_f64, seq_ranges


def chunk_list(starts, lens, L: int) -> List[Tuple[int, int, int, int]]:
    """[(sequence, first token, valid length, index within sequence)]."""
    out = []
    for s, (t0, n) in enumerate(zip(starts, lens)):
        k = 0
        while k * L < n:
            out.append((s, int(t0 + k * L), int(min(L, n - k * L)), k))
            k += 1
    return out


def ssd_chunked(x, dt, dt_bias, A, B, C, D, chunk_size: int, init=None,
                cu_seqlens=None, dt_min: float = 0.0, dt_max: float = math.inf):
    """Returns a dict with y (b,T,H,P), final (nseq,H,P,N) and the
    intermediates delta, dAcs (nc,H,L), CB (nc,G,L,L), S, Hin (nc,H,P,N)
    and the chunk list."""
    L = int(chunk_size)
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
    chunks = chunk_list(starts, lens, L)
    nc = len(chunks)
    hpg = H // G
    gidx = np.arange(H) // hpg

    delta = np.zeros((nc, H, L))
    dAcs = np.zeros((nc, H, L))
    CB = np.zeros((nc, G, L, L))
    S = np.zeros((nc, H, P, N))
    Hin = np.zeros((nc, H, P, N))
    y = np.zeros((b * T, H, P))
    fin = np.zeros((len(starts), H, P, N))

    # stage 1: discretised step and its chunk-local inclusive cumulative sum
    for c, (s, t0, n, k) in enumerate(chunks):
        u = DT[t0:t0 + n, :] + bias[None, :]                         # (n, H)
        sp = np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))
        delta[c, :, :n] = np.clip(sp, dt_min, dt_max).T
        dAcs[c] = np.cumsum(delta[c] * Av[:, None], axis=1)
    # stage 2: C B^T inside each chunk
    for c, (s, t0, n, k) in enumerate(chunks):
        for g in range(G):
            CB[c, g, :n, :n] = Cm[t0:t0 + n, g, :] @ Bm[t0:t0 + n, g, :].T
    # stage 3: chunk states from a zero start
    for c, (s, t0, n, k) in enumerate(chunks):
        for h in range(H):
            w = np.exp(dAcs[c, h, n - 1] - dAcs[c, h, :n]) * delta[c, h, :n]   # (n,)
            S[c, h] = (w[:, None] * X[t0:t0 + n, h, :]).T @ Bm[t0:t0 + n, gidx[h], :]
    # stage 4: pass states along each sequence's chunks
    for s_id in range(len(starts)):
        state = h0[s_id].copy() if h0 is not None else np.zeros((H, P, N))
        for c, (s, t0, n, k) in enumerate(chunks):
            if s != s_id:
                continue
            Hin[c] = state
            state = np.exp(dAcs[c, :, n - 1])[:, None, None] * state + S[c]
        fin[s_id] = state
    # stage 5: outputs
    for c, (s, t0, n, k) in enumerate(chunks):
        causal = np.tril(np.ones((n, n), dtype=bool))
        for h in range(H):
            g = gidx[h]
            a = dAcs[c, h, :n]
            decay = np.where(causal, np.exp(np.where(causal, a[:, None] - a[None, :], 0.0)), 0.0)
            Mm = CB[c, g, :n, :n] * decay * delta[c, h, None, :n]
            xs = X[t0:t0 + n, h, :]
            yy = Mm @ xs
            yy += np.exp(a)[:, None] * (Cm[t0:t0 + n, g, :] @ Hin[c, h].T)
            yy += Dv[h] * xs
            y[t0:t0 + n, h, :] = yy
    return dict(y=y.reshape(b, T, H, P), final=fin, delta=delta, dAcs=dAcs,
                CB=CB, S=S, Hin=Hin, chunks=chunks)
