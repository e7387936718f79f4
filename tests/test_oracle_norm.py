"""Pins of the gated RMS norm oracle (CPU): a hand-derived fixture, torch's
rms_norm, scale invariance, closed forms of the weight gradient, an
orthogonality of the input gradient, and central finite differences of the
forward.  A mutation check plants plausible mistakes in a copy of the
oracle; each must fail at least one pin."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.gated_norm import gated_rmsnorm_bwd, gated_rmsnorm_fwd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "norm")


def _inputs(T=5, C=12, seed=0):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(T, C)), rng.normal(size=(T, C)) * 2, rng.normal(size=C)


def test_hand_derived_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "gated_norm_two_groups.json")))
    out, rstd = gated_rmsnorm_fwd(np.array(fx["y"]), np.array(fx["z"]), np.array(fx["w"]),
                                  fx["eps"], fx["group_size"])
    assert np.allclose(out, np.array(fx["out"]), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("gs", [1, 3, 4, 12])
def test_equals_torch_rms_norm_of_the_gated_input(gs):
    # a library routine: torch's rms_norm over each group of the gated input
    y, z, w = _inputs()
    eps = 1e-5
    out, _ = gated_rmsnorm_fwd(y, z, w, eps, gs)
    g = torch.from_numpy(y) * torch.nn.functional.silu(torch.from_numpy(z))
    ref = torch.nn.functional.rms_norm(g.view(5, 12 // gs, gs), (gs,), eps=eps).view(5, 12)
    ref = ref * torch.from_numpy(w)
    assert np.allclose(out, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_scale_invariance_and_unit_rms():
    y, z, w = _inputs()
    out, _ = gated_rmsnorm_fwd(y, z, w, 0.0, 4)
    out2, _ = gated_rmsnorm_fwd(3.5 * y, z, w, 0.0, 4)
    assert np.allclose(out, out2, rtol=1e-13)
    u = (out / w).reshape(5, 3, 4)
    assert np.allclose(np.sqrt(np.mean(u * u, axis=2)), 1.0, rtol=1e-13)


def test_groups_are_independent():
    y, z, w = _inputs()
    y2 = y.copy()
    y2[:, 4:8] *= -7.0
    a, _ = gated_rmsnorm_fwd(y, z, w, 1e-3, 4)
    b, _ = gated_rmsnorm_fwd(y2, z, w, 1e-3, 4)
    assert np.array_equal(a[:, :4], b[:, :4]) and np.array_equal(a[:, 8:], b[:, 8:])


def _fd(f, x, dout, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        g[i] = (np.sum(f(xp) * dout) - np.sum(f(xm) * dout)) / (2 * h)
    return g


@pytest.mark.parametrize("gs,eps", [(4, 1e-5), (12, 0.0), (3, 0.5)])
def test_backward_matches_finite_differences(gs, eps):
    y, z, w = _inputs(T=3, C=12, seed=gs)
    dout = np.random.default_rng(9).normal(size=y.shape)
    dy, dz, dw = gated_rmsnorm_bwd(y, z, w, eps, gs, dout)
    f = lambda **kw: gated_rmsnorm_fwd(kw.get("y", y), kw.get("z", z), kw.get("w", w), eps, gs)[0]
    assert np.allclose(dy, _fd(lambda v: f(y=v), y, dout), rtol=1e-6, atol=1e-7)
    assert np.allclose(dz, _fd(lambda v: f(z=v), z, dout), rtol=1e-6, atol=1e-7)
    assert np.allclose(dw, _fd(lambda v: f(w=v), w, dout), rtol=1e-6, atol=1e-7)


def test_backward_closed_forms():
    y, z, w = _inputs(T=7, C=12, seed=4)
    dout = np.random.default_rng(2).normal(size=y.shape)
    out, _ = gated_rmsnorm_fwd(y, z, w, 0.0, 6)
    dy, dz, dw = gated_rmsnorm_bwd(y, z, w, 0.0, 6, dout)
    # dw = sum over tokens of dout * (out / w)
    assert np.allclose(dw, np.sum(dout * out / w, axis=0), rtol=1e-13)
    # with eps = 0 the output does not change when y is scaled, so the
    # gradient is orthogonal to y within every (token, group)
    assert np.allclose(np.sum((dy * y).reshape(7, 2, 6), axis=2), 0.0, atol=1e-12)
    # a zero gate (z = 0) passes no gradient to y and the derivative
    # of silu at 0 is 1/2
    z0 = z.copy()
    z0[:, 0] = 0.0
    dy0, dz0, _ = gated_rmsnorm_bwd(y, z0, w, 1e-3, 6, dout)
    assert np.all(dy0[:, 0] == 0.0)


def _mutant(kind, y, z, w, eps, gs):
    sg = 1.0 / (1.0 + np.exp(-z))
    gate = {"no_gate": np.ones_like(z), "sigmoid_gate": sg}.get(kind, z * sg)
    g = y * gate
    T, Cn = y.shape
    gsz = Cn if kind == "one_group" else gs
    out = np.zeros_like(y)
    for k in range(Cn // gsz):
        sl = slice(k * gsz, (k + 1) * gsz)
        s2 = np.sum(g[:, sl] ** 2, axis=1)
        ms = s2 if kind == "sum_not_mean" else s2 / gsz
        r = 1 / (np.sqrt(ms) + eps) if kind == "eps_outside" else 1 / np.sqrt(ms + eps)
        out[:, sl] = g[:, sl] * r[:, None] * (1.0 if kind == "no_weight" else w[None, sl])
    return out


@pytest.mark.parametrize("kind", ["no_gate", "sigmoid_gate", "one_group", "sum_not_mean",
                                  "eps_outside", "no_weight"])
def test_pins_reject_planted_mistakes(kind):
    fx = json.load(open(os.path.join(GOLDEN, "gated_norm_two_groups.json")))
    y, z, w = _inputs()
    eps = 1e-2
    bad_fx = _mutant(kind, np.array(fx["y"]), np.array(fx["z"]), np.array(fx["w"]), fx["eps"],
                     fx["group_size"])
    fx_ok = np.allclose(bad_fx, np.array(fx["out"]), rtol=1e-12)
    g = torch.from_numpy(y) * torch.nn.functional.silu(torch.from_numpy(z))
    ref = (torch.nn.functional.rms_norm(g.view(5, 3, 4), (4,), eps=eps).view(5, 12)
           * torch.from_numpy(w)).numpy()
    lib_ok = np.allclose(_mutant(kind, y, z, w, eps, 4), ref, rtol=1e-12)
    assert not (fx_ok and lib_ok), kind


def test_backward_pins_reject_a_dropped_silu_derivative_term():
    y, z, w = _inputs(T=3, C=12, seed=3)
    dout = np.random.default_rng(5).normal(size=y.shape)
    _, dz, _ = gated_rmsnorm_bwd(y, z, w, 1e-5, 4, dout)
    # the mistake: d silu / dz taken as sigma(z) alone
    sg = 1.0 / (1.0 + np.exp(-z))
    wrong = dz / (1.0 + z * (1.0 - sg))
    fd = _fd(lambda v: gated_rmsnorm_fwd(y, v, w, 1e-5, 4)[0], z, dout)
    assert np.allclose(dz, fd, rtol=1e-6, atol=1e-7)
    assert not np.allclose(wrong, fd, rtol=1e-3, atol=1e-5)
