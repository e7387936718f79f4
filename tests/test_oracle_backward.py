"""Pins of the fp64 gradient oracle (oracle/backward.py), CPU only.

The oracle differentiates the forward by torch.autograd.  It is pinned to
things other than itself:
  - central finite differences of the C recurrence (oracle/ssd_recurrence.c,
    separate code with its own softplus), for every element of every input,
    on tiny problems (rows, packed sequences, an active clamp);
  - the two forms it can differentiate (quadratic and token loop) agreeing;
  - closed forms: with every step zero (dt_raw = -1e4, softplus exactly 0)
    the layer is y_t = C_t h0 + D x_t and final = h0, so dinit = sum_t
    dy_t C_t^T + dfinal, dx = D dy, dC_t = dy_t h0, and dB, dA, ddt vanish;
    dD = sum dy * x for any input.
"""
import math

import numpy as np
import pytest
import torch

from oracle.backward import NAMES, ssd_grads
from oracle.recurrence import ssd_recurrence


def _inputs(b, T, H, P, N, G, seed, nseq=0, init=True, dt_shift=-1.0):
    g = np.random.default_rng(seed)
    nst = nseq if nseq else b
    d = dict(
        x=g.standard_normal((b, T, H, P)),
        dt=g.standard_normal((b, T, H)) + dt_shift,
        dt_bias=g.uniform(-0.5, 0.5, H),
        A=-np.exp(g.uniform(0.0, math.log(4.0), H)),
        B=g.standard_normal((b, T, G, N)),
        C=g.standard_normal((b, T, G, N)),
        D=g.standard_normal(H),
        init=g.standard_normal((nst, H, P, N)) * 0.5 if init else None,
    )
    dy = g.standard_normal((b, T, H, P))
    dfin = g.standard_normal((nst, H, P, N))
    return d, dy, dfin


def _loss_c(d, dy, dfin, cu, dt_min, dt_max):
    y, fin = ssd_recurrence(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"],
                            init=d["init"], cu_seqlens=cu, dt_min=dt_min, dt_max=dt_max)
    return float((y * dy).sum() + (fin * dfin).sum())


def _fd_check(d, dy, dfin, cu=None, dt_min=0.0, dt_max=math.inf, eps=1e-6):
    got = ssd_grads(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"], dy, dfin,
                    init=d["init"], cu_seqlens=cu, dt_min=dt_min, dt_max=dt_max)
    for name in NAMES:
        if d[name] is None:
            assert got[name] is None
            continue
        arr = d[name]
        fd = np.zeros_like(arr)
        flat = arr.reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + eps
            lp = _loss_c(d, dy, dfin, cu, dt_min, dt_max)
            flat[i] = keep - eps
            lm = _loss_c(d, dy, dfin, cu, dt_min, dt_max)
            flat[i] = keep
            fd.reshape(-1)[i] = (lp - lm) / (2 * eps)
        scale = np.abs(fd).max() + 1.0
        err = np.abs(got[name] - fd).max()
        assert err <= 2e-6 * scale, (name, err, scale)


def test_finite_differences_rows():
    d, dy, dfin = _inputs(2, 7, 2, 3, 2, 1, seed=0)
    _fd_check(d, dy, dfin)


def test_finite_differences_packed_two_groups():
    d, dy, dfin = _inputs(1, 11, 4, 2, 3, 2, seed=1, nseq=3)
    _fd_check(d, dy, dfin, cu=np.array([0, 4, 5, 11]))


def test_finite_differences_active_clamp():
    d, dy, dfin = _inputs(1, 9, 2, 2, 2, 1, seed=2, dt_shift=0.0)
    sp = np.logaddexp(0.0, d["dt"] + d["dt_bias"])
    lo, hi = np.quantile(sp, 0.3), np.quantile(sp, 0.8)
    _fd_check(d, dy, dfin, dt_min=float(lo), dt_max=float(hi))


def test_finite_differences_no_init_no_skip():
    d, dy, dfin = _inputs(1, 8, 2, 3, 2, 1, seed=3, init=False)
    d["D"] = None
    d["dt_bias"] = None
    _fd_check(d, dy, dfin)


@pytest.mark.parametrize("cu", [None, np.array([0, 13, 14, 40])])
def test_dual_and_recurrence_forms_agree(cu):
    b = 1 if cu is not None else 2
    d, dy, dfin = _inputs(b, 40, 2, 4, 3, 1, seed=4, nseq=3 if cu is not None else 0)
    args = (d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"], dy, dfin)
    g1 = ssd_grads(*args, init=d["init"], cu_seqlens=cu, form="dual")
    g2 = ssd_grads(*args, init=d["init"], cu_seqlens=cu, form="recurrence")
    for name in NAMES:
        np.testing.assert_allclose(g1[name], g2[name], rtol=1e-10, atol=1e-10 * (np.abs(g2[name]).max() + 1))


def test_zero_steps_closed_form():
    d, dy, dfin = _inputs(1, 12, 2, 3, 4, 1, seed=5)
    d["dt"] = np.full_like(d["dt"], -1e4)      # softplus(-1e4 + bias) is exactly 0
    g = ssd_grads(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"], dy, dfin,
                  init=d["init"])
    C, h0 = d["C"][0, :, 0], d["init"][0]                       # (T, N), (H, P, N)
    dinit = np.einsum("thp,tn->hpn", dy[0], C) + dfin[0]
    np.testing.assert_allclose(g["init"][0], dinit, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["x"], d["D"][None, None, :, None] * dy, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["C"][0, :, 0], np.einsum("thp,hpn->tn", dy[0], h0),
                               rtol=1e-12, atol=1e-12)
    for name in ("B", "A", "dt", "dt_bias"):
        assert np.abs(g[name]).max() == 0.0, name


def test_skip_gradient_closed_form():
    d, dy, dfin = _inputs(2, 10, 3, 2, 2, 1, seed=6)
    g = ssd_grads(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"], dy, dfin,
                  init=d["init"])
    np.testing.assert_allclose(g["D"], (dy * d["x"]).sum(axis=(0, 1, 3)), rtol=1e-12)
