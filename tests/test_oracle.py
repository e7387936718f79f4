"""Pins of the fp64 oracle against things other than itself (CPU only).

The pages print no worked example and no formula, so each formulation of
the oracle is tied to: hand-derived fixtures (tests/golden), the
independently written quadratic dual form, closed forms (zero step, zero
decay, geometric series), a library IIR filter (scipy.signal.lfilter),
invariants (chunk-size independence, split-and-resume, packed = separate,
linearity) and a head-to-group reduction.  Chosen so that a dropped term, a
wrong sign, an off-by-one token, a transposed state or a wrong group map each
fails at least one of them.
"""
import glob
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import torch

from oracle.recurrence import ssd_recurrence
from oracle.dual import ssd_dual
from oracle.chunked import ssd_chunked
from state_space_model_ssd_amd.inputs import Problem, Recipe, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TIGHT = 1e-12


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def run_all(inp, **kw):
    return ssd_recurrence(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                          inp["D"], init=inp.get("init"), cu_seqlens=inp.get("cu_seqlens"), **kw)


def small(b=1, T=40, H=4, P=3, N=5, G=2, dtype="f32", init_std=None, seed=0, lens=None,
          recipe=None):
    if lens is not None:
        b, T = 1, sum(lens)
        lens = tuple(lens)
    prob = Problem(b, T, H, P, N, G, 16, dtype, seq_lens=lens)
    rec = recipe or Recipe(init_std=init_std)
    return make_inputs(prob, rec, seed=seed)


# ---------------------------------------------------------------- fixtures

def load_golden():
    out = []
    for f in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        d = json.load(open(f))
        arr = lambda k: None if d[k] is None else np.asarray(d[k], dtype=np.float64)
        inp = dict(x=arr("x"), dt=arr("dt"), dt_bias=arr("dt_bias"), A=arr("A"), B=arr("B"),
                   C=arr("C"), D=arr("D"), init=arr("init"),
                   cu_seqlens=None if d["cu_seqlens"] is None else np.asarray(d["cu_seqlens"]))
        out.append((d["name"], inp, arr("y"), arr("final")))
    return out


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c[0])
def test_golden_recurrence(case):
    name, inp, y_exp, f_exp = case
    y, f = run_all(inp)
    np.testing.assert_allclose(y, y_exp, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(f, f_exp, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c[0])
def test_golden_dual_and_chunked(case):
    name, inp, y_exp, f_exp = case
    kw = dict(init=inp["init"], cu_seqlens=inp["cu_seqlens"])
    y, f = ssd_dual(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"], **kw)
    np.testing.assert_allclose(y, y_exp, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(f, f_exp, rtol=1e-13, atol=1e-13)
    for L in (1, 2, 4):
        r = ssd_chunked(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                        inp["D"], L, **kw)
        np.testing.assert_allclose(r["y"], y_exp, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(r["final"], f_exp, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------- recurrence = dual

@pytest.mark.parametrize("shape", [
    dict(b=1, T=17, H=2, P=3, N=5, G=1),
    dict(b=2, T=33, H=4, P=4, N=2, G=2),
    dict(b=1, T=64, H=4, P=8, N=4, G=4),
    dict(b=3, T=9, H=6, P=2, N=7, G=3),
])
@pytest.mark.parametrize("init_std", [None, 0.3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recurrence_equals_dual(shape, init_std, dtype):
    inp = small(**shape, init_std=init_std, dtype=dtype, seed=7)
    y, f = run_all(inp)
    yd, fd = ssd_dual(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                      inp["D"], init=inp["init"])
    assert rel(y, yd) < TIGHT and rel(f, fd) < TIGHT


def test_recurrence_equals_dual_packed():
    inp = small(lens=[5, 1, 23, 16, 3], H=4, G=2, init_std=0.5, seed=3)
    y, f = run_all(inp)
    yd, fd = ssd_dual(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                      inp["D"], init=inp["init"], cu_seqlens=inp["cu_seqlens"])
    assert rel(y, yd) < TIGHT and rel(f, fd) < TIGHT


# -------------------------------------------------- chunk-size independence

@pytest.mark.parametrize("T", [64, 50])
def test_chunked_is_chunk_size_independent(T):
    inp = small(b=2, T=T, H=4, P=4, N=6, G=2, init_std=0.2, seed=11)
    y, f = run_all(inp)
    for L in (1, 3, 16, 64, T):
        r = ssd_chunked(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                        inp["D"], L, init=inp["init"])
        assert rel(r["y"], y) < TIGHT, L
        assert rel(r["final"], f) < TIGHT, L


def test_chunked_intermediates_match_recurrence_pieces():
    """S_c is the state a zero-started recurrence reaches over chunk c alone;
    Hin_c is the state the full recurrence holds before chunk c."""
    inp = small(lens=[37, 16, 5], H=2, P=3, N=4, G=1, init_std=0.4, seed=5)
    L = 16
    r = ssd_chunked(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                    inp["D"], L, init=inp["init"], cu_seqlens=inp["cu_seqlens"])
    x, dt, B, C = inp["x"], inp["dt"], inp["B"], inp["C"]
    for c, (s, t0, n, k) in enumerate(r["chunks"]):
        sl = slice(t0, t0 + n)
        _, fS = ssd_recurrence(x[:, sl], dt[:, sl], inp["dt_bias"], inp["A"], B[:, sl], C[:, sl],
                               inp["D"])
        assert rel(r["S"][c], fS[0]) < TIGHT
        seq_t0 = int(inp["cu_seqlens"][s])
        if t0 == seq_t0:
            assert np.array_equal(r["Hin"][c], inp["init"][s].double().numpy())
        else:
            pre = slice(seq_t0, t0)
            _, fH = ssd_recurrence(x[:, pre], dt[:, pre], inp["dt_bias"], inp["A"], B[:, pre],
                                   C[:, pre], inp["D"], init=inp["init"][s:s + 1])
            assert rel(r["Hin"][c], fH[0]) < TIGHT


def test_chunked_cumsum_stage():
    """delta is softplus(dt + bias) (checked against the library logaddexp),
    zero past a chunk's end; dAcs is its running sum times A, flat past the end."""
    inp = small(lens=[20, 7], H=3, P=2, N=2, G=1, seed=2)
    L = 8
    r = ssd_chunked(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                    inp["D"], L, cu_seqlens=inp["cu_seqlens"])
    dt = inp["dt"].double().numpy()[0]
    A = inp["A"].double().numpy()
    for c, (s, t0, n, k) in enumerate(r["chunks"]):
        d = np.logaddexp(0.0, dt[t0:t0 + n] + inp["dt_bias"].double().numpy()).T
        np.testing.assert_allclose(r["delta"][c, :, :n], d, rtol=1e-14)
        assert np.all(r["delta"][c, :, n:] == 0)
        run = np.zeros(3)
        for l in range(L):
            if l < n:
                run = run + d[:, l] * A
            np.testing.assert_allclose(r["dAcs"][c, :, l], run, rtol=1e-13)


# ------------------------------------------------------------ closed forms

def test_zero_step_gives_skip_only():
    inp = small(b=2, T=30, H=4, P=3, N=4, G=2, init_std=None, seed=4)
    inp["dt"] = torch.full_like(inp["dt"], -1e4)          # softplus -> exactly 0
    y, f = run_all(inp)
    xs = inp["x"].double().numpy()
    assert np.array_equal(y, inp["D"].double().numpy()[None, None, :, None] * xs)
    assert np.all(f == 0.0)


def test_zero_step_with_initial_state():
    inp = small(b=2, T=30, H=4, P=3, N=4, G=2, init_std=0.5, seed=4)
    inp["dt"] = torch.full_like(inp["dt"], -1e4)
    y, f = run_all(inp)
    xs = inp["x"].double().numpy()
    h0 = inp["init"].double().numpy()                      # (b, H, P, N)
    Cg = np.repeat(inp["C"].double().numpy(), 2, axis=2)   # (b, T, H, N)
    exp_y = np.einsum("bthn,bhpn->bthp", Cg, h0) + inp["D"].double().numpy()[None, None, :, None] * xs
    assert rel(y, exp_y) < 1e-14
    assert np.array_equal(f, h0)


def test_zero_decay_is_prefix_sum():
    inp = small(b=1, T=25, H=2, P=3, N=4, G=1, init_std=0.5, seed=9)
    inp["A"] = torch.zeros_like(inp["A"])
    y, f = run_all(inp)
    x = inp["x"].double().numpy()[0]                       # (T, H, P)
    Bv = inp["B"].double().numpy()[0, :, 0]                # (T, N)
    Cv = inp["C"].double().numpy()[0, :, 0]
    d = np.logaddexp(0.0, inp["dt"].double().numpy()[0])   # (T, H)
    upd = np.einsum("th,thp,tn->thpn", d, x, Bv)
    h = inp["init"].double().numpy()[0][None] + np.cumsum(upd, axis=0)
    exp_y = np.einsum("tn,thpn->thp", Cv, h) + inp["D"].double().numpy()[None, :, None] * x
    assert rel(y[0], exp_y) < 1e-13
    assert rel(f[0], h[-1]) < 1e-13


@pytest.mark.parametrize("A", [-0.3, -4.0])
def test_scalar_case_is_first_order_iir(A):
    T = 200
    g = np.random.default_rng(1)
    x = g.standard_normal((1, T, 1, 1))
    Bv = g.standard_normal((1, T, 1, 1))
    Cv = g.standard_normal((1, T, 1, 1))
    dt = np.full((1, T, 1), 0.25)
    D = np.array([0.7])
    y, f = ssd_recurrence(x, dt, None, np.array([A]), Bv, Cv, D)
    d = math.log1p(math.exp(0.25))
    a = math.exp(d * A)
    h = scipy.signal.lfilter([d], [1.0, -a], (x * Bv).ravel())
    exp_y = h * Cv.ravel() + D[0] * x.ravel()
    assert rel(y.ravel(), exp_y) < 1e-12
    assert abs(f.ravel()[0] - h[-1]) < 1e-12 * max(1.0, abs(h[-1]))


def test_constant_step_clamp():
    """dt_min = dt_max = c forces delta = c whatever dt is: the scalar case is
    then the IIR filter with gain c."""
    T, c, A = 64, 0.05, -2.0
    g = np.random.default_rng(2)
    x = g.standard_normal((1, T, 1, 1))
    Bv = g.standard_normal((1, T, 1, 1))
    Cv = np.ones((1, T, 1, 1))
    dt = g.standard_normal((1, T, 1)) * 5
    y, f = ssd_recurrence(x, dt, None, np.array([A]), Bv, Cv, np.array([0.0]), dt_min=c, dt_max=c)
    h = scipy.signal.lfilter([c], [1.0, -math.exp(c * A)], (x * Bv).ravel())
    assert rel(y.ravel(), h) < 1e-12


# --------------------------------------------------------------- invariants

@pytest.mark.parametrize("t_split", [1, 17, 39])
def test_split_and_resume(t_split):
    inp = small(b=2, T=40, H=4, P=3, N=5, G=2, init_std=0.3, seed=6)
    y, f = run_all(inp)
    sl1, sl2 = slice(0, t_split), slice(t_split, 40)
    cut = lambda k, s: inp[k][:, s]
    y1, f1 = ssd_recurrence(cut("x", sl1), cut("dt", sl1), inp["dt_bias"], inp["A"], cut("B", sl1),
                            cut("C", sl1), inp["D"], init=inp["init"])
    y2, f2 = ssd_recurrence(cut("x", sl2), cut("dt", sl2), inp["dt_bias"], inp["A"], cut("B", sl2),
                            cut("C", sl2), inp["D"], init=torch.from_numpy(f1))
    assert rel(np.concatenate([y1, y2], axis=1), y) < TIGHT
    assert rel(f2, f) < TIGHT


def test_packed_equals_separate_runs():
    lens = [7, 1, 30, 16]
    inp = small(lens=lens, H=4, P=3, N=4, G=2, init_std=0.3, seed=8)
    y, f = run_all(inp)
    cu = inp["cu_seqlens"].tolist()
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        ys, fs = ssd_recurrence(inp["x"][:, sl], inp["dt"][:, sl], inp["dt_bias"], inp["A"],
                                inp["B"][:, sl], inp["C"][:, sl], inp["D"],
                                init=inp["init"][s:s + 1])
        assert np.array_equal(ys[0], y[0, sl])             # same arithmetic order: bitwise
        assert np.array_equal(fs[0], f[s])


def test_linearity_in_input_and_state():
    a = small(b=1, T=33, H=2, P=3, N=4, G=1, init_std=0.5, seed=12)
    b2 = small(b=1, T=33, H=2, P=3, N=4, G=1, init_std=0.5, seed=13)
    for k in ("dt", "dt_bias", "A", "B", "C", "D"):
        b2[k] = a[k]
    al, be = 0.7, -1.9
    mix = dict(a)
    mix["x"] = al * a["x"].double() + be * b2["x"].double()
    mix["init"] = al * a["init"].double() + be * b2["init"].double()
    ya, fa = run_all(a)
    yb, fb = run_all(b2)
    ym, fm = run_all(mix)
    assert rel(ym, al * ya + be * yb) < 1e-12 and rel(fm, al * fa + be * fb) < 1e-12


def test_head_to_group_map_is_contiguous():
    """H=4, G=2 equals two G=1 problems: heads {0,1} on group 0, {2,3} on group 1."""
    inp = small(b=2, T=21, H=4, P=3, N=4, G=2, init_std=0.3, seed=14)
    y, f = run_all(inp)
    for g, hs in ((0, [0, 1]), (1, [2, 3])):
        idx = torch.tensor(hs)
        sub = dict(x=inp["x"][:, :, idx], dt=inp["dt"][:, :, idx], dt_bias=inp["dt_bias"][idx],
                   A=inp["A"][idx], B=inp["B"][:, :, g:g + 1], C=inp["C"][:, :, g:g + 1],
                   D=inp["D"][idx], init=inp["init"][:, idx])
        ys, fs = run_all(sub)
        assert np.array_equal(ys, y[:, :, hs]) and np.array_equal(fs, f[:, hs])


def test_head_subset_matches_full_run():
    inp = small(b=1, T=20, H=6, P=2, N=3, G=3, init_std=0.1, seed=15)
    y, f = run_all(inp)
    ys, fs = run_all(inp, heads=[5, 0, 3])
    assert np.array_equal(ys, y[:, :, [5, 0, 3]]) and np.array_equal(fs, f[:, [5, 0, 3]])


def test_long_run_is_finite_and_bounded():
    inp = small(b=1, T=4096, H=2, P=4, N=4, G=1, init_std=0.1, seed=16)
    y, f = run_all(inp)
    assert np.isfinite(y).all() and np.isfinite(f).all()
    assert np.abs(f).max() < 1e3


def test_empty_sequence_keeps_initial_state():
    inp = small(lens=[4, 3], H=2, P=2, N=2, G=1, init_std=1.0, seed=17)
    cu = np.array([0, 4, 4, 7])                            # middle sequence is empty
    init = torch.cat([inp["init"][:1], inp["init"][:1] * 3, inp["init"][1:]], 0)
    y, f = ssd_recurrence(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                          inp["D"], init=init, cu_seqlens=cu)
    assert np.array_equal(f[1], init[1].double().numpy())
    r = ssd_chunked(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                    inp["D"], 2, init=init, cu_seqlens=cu)
    assert rel(r["y"], y) < TIGHT and rel(r["final"], f) < TIGHT


# ------------------------------------------- the pins catch planted mistakes

def _mutant(inp, mutation):
    """A deliberately wrong per-token recurrence (tiny inputs, numpy loops);
    each mutation is a plausible slip that the pins above must reject."""
    x, dt = inp["x"], inp["dt"]
    b, T, H, P = x.shape
    G, N = inp["B"].shape[2], inp["B"].shape[3]
    cu = inp["cu_seqlens"]
    ranges = [(i * T, T) for i in range(b)] if cu is None else \
        [(int(cu[s]), int(cu[s + 1] - cu[s])) for s in range(len(cu) - 1)]
    X, Bm, Cm = x.reshape(b * T, H, P), inp["B"].reshape(b * T, G, N), inp["C"].reshape(b * T, G, N)
    DT = dt.reshape(b * T, H)
    y = np.zeros((b * T, H, P))
    fin = np.zeros((len(ranges), H, P, N))
    for s, (t0, n) in enumerate(ranges):
        for h in range(H):
            g = h % G if mutation == "group_mod" else h // (H // G)
            st = np.zeros((P, N)) if inp["init"] is None else inp["init"][s, h].copy()
            bias = 0.0 if mutation == "no_bias" else inp["dt_bias"][h]
            for t in range(t0, t0 + n):
                d = np.logaddexp(0.0, DT[t, h] + bias)
                a = math.exp(-d * inp["A"][h]) if mutation == "decay_sign" else math.exp(d * inp["A"][h])
                prev = st.copy()
                # "transpose": the state kept as (N, P), final returned that way
                upd = np.outer(Bm[t, g], X[t, h]) if mutation == "transpose" else np.outer(X[t, h], Bm[t, g])
                if mutation == "transpose" and t == t0:
                    st = st.T.copy()
                st = a * st + d * upd
                use = prev if mutation == "y_prev_state" else st
                skip = 0.0 if mutation == "no_skip" else inp["D"][h] * X[t, h]
                y[t, h] = (Cm[t, g] @ use if mutation == "transpose" else use @ Cm[t, g]) + skip
                if mutation == "init_undecayed" and t == t0 and inp["init"] is not None:
                    st = inp["init"][s, h] + d * upd
                    y[t, h] = st @ Cm[t, g] + skip
            fin[s, h] = st
    return y.reshape(b, T, H, P), fin


@pytest.mark.parametrize("mutation", ["none", "group_mod", "no_bias", "decay_sign", "transpose",
                                      "y_prev_state", "no_skip", "init_undecayed"])
def test_fixtures_reject_planted_mistakes(mutation):
    caught = []
    for name, inp, y_exp, f_exp in load_golden():
        y, f = _mutant(inp, mutation)
        ok = np.allclose(y, y_exp, rtol=1e-12, atol=1e-12) and np.allclose(f, f_exp, rtol=1e-12, atol=1e-12)
        if not ok:
            caught.append(name)
    if mutation == "none":
        assert caught == []          # the loop itself is right
    else:
        assert caught, f"no fixture catches {mutation}"
