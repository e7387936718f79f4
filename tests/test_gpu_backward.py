"""Parity of the HIP backward with the fp64 gradient oracle (GPU).

Both sides get the same seeded inputs (bf16 values upcast exactly for the
oracle) and the same output gradients dy (in x's dtype) and dfinal (fp32).
Every gradient is compared over the whole tensor by relative L2:
  - fp32 inputs: <= 1e-4.  The backward sums products over whole chunks in
    fp32 (token loops of up to 256 terms, P*N-term state contractions); the
    forward's 1e-5 bound covers one such sum, a gradient chains several.
  - bf16 inputs: <= 2e-2, the forward's bound.  CB and the entering states
    are stored in bf16 as in the forward, and dx, dB, dC are rounded once
    to bf16.
"""
import math

import numpy as np
import pytest
import torch

from oracle.backward import ssd_grads
from state_space_model_ssd_amd import binding
from state_space_model_ssd_amd.inputs import Problem, Recipe, make_inputs
from tests.helpers import f64, rel_l2, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _grads_case(prob, rec, seed, with_dfinal=True, dt_min=0.0, dt_max=math.inf):
    inp = make_inputs(prob, rec, seed=seed)
    gen = torch.Generator().manual_seed(1000 + seed)
    xdt = inp["x"].dtype
    dy = torch.randn(inp["x"].shape, generator=gen, dtype=torch.float32).to(xdt)
    nst = prob.nseq
    dfin = torch.randn((nst, prob.nheads, prob.headdim, prob.dstate), generator=gen,
                       dtype=torch.float32) if with_dfinal else None
    d = to_dev(inp)
    got = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size,
                          dy.cuda(), None if dfin is None else dfin.cuda(), D=d["D"],
                          dt_bias=d["dt_bias"], initial_states=d["init"],
                          cu_seqlens=d["cu_seqlens"], dt_min=dt_min, dt_max=dt_max)
    torch.cuda.synchronize()
    # with no initial state given, the gradient is the one at a zero state
    init = inp["init"] if inp["init"] is not None else \
        torch.zeros((nst, prob.nheads, prob.headdim, prob.dstate))
    ref = ssd_grads(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"],
                    dy, dfin, init=init, cu_seqlens=inp["cu_seqlens"], dt_min=dt_min,
                    dt_max=dt_max)
    tol = TOL[prob.dtype]
    report = {}
    for name, key in (("x", "x"), ("dt", "dt"), ("A", "A"), ("B", "B"), ("C", "C"), ("D", "D"),
                      ("dt_bias", "dt_bias"), ("init", "initial_states")):
        g = got[key].float().cpu()
        assert torch.isfinite(g).all(), name
        err = rel_l2(g, ref[name])
        report[name] = err
        assert err <= tol, (name, err, report)
    print("  rel_l2 " + " ".join(f"{k}={v:.2e}" for k, v in report.items()), flush=True)
    return got, ref


SHAPES = [
    # (b, T, H, P, N, G, L, dtype)
    (2, 150, 4, 32, 16, 2, 64, "f32"),
    (1, 200, 2, 64, 128, 1, 64, "f32"),
    (1, 300, 2, 64, 128, 1, 256, "f32"),
    (2, 130, 4, 32, 32, 2, 64, "bf16"),
    (1, 520, 4, 64, 128, 2, 256, "bf16"),
    (1, 300, 2, 64, 128, 1, 128, "bf16"),
    (2, 100, 2, 64, 128, 1, 64, "bf16"),
    # more heads per group than head blocks: blocks of one and two heads
    (1, 300, 12, 32, 32, 1, 64, "bf16"),
    (1, 200, 20, 32, 16, 2, 64, "f32"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_backward_shapes(shape):
    b, T, H, P, N, G, L, dt = shape
    prob = Problem(b, T, H, P, N, G, L, dt)
    _grads_case(prob, Recipe(init_std=0.3), seed=T + H)


def test_backward_long_memory_small_steps():
    prob = Problem(1, 600, 2, 64, 128, 1, 64, "f32")
    _grads_case(prob, Recipe(dt_bias="inv_softplus_uniform", init_std=0.5), seed=9)


@pytest.mark.parametrize("shape,lens", [((1, 520, 4, 64, 128, 2, 256, "bf16"), None),
                                        ((1, 300, 2, 64, 128, 1, 128, "bf16"), None),
                                        ((2, 100, 2, 64, 128, 1, 64, "bf16"), None),
                                        ((2, 130, 4, 32, 32, 2, 64, "bf16"), None),
                                        ((1, 230, 2, 32, 32, 1, 64, "bf16"), (100, 1, 64, 65))],
                         ids=["L256", "L128", "P64N128L64", "L64", "packed"])
def test_backward_small_steps_bf16(shape, lens):
    # small steps (dt near dt_bias in [1e-3, 1e-1]): every chunk's total
    # decay stays within 2^64, so dx takes its factored-decay path (CB^T
    # pieces scaled by exp(a_l), rows rescaled by delta_s exp(-a_s)); the
    # default recipe's larger steps exercise the masked path
    b, T, H, P, N, G, L, dt = shape
    prob = Problem(b, T, H, P, N, G, L, dt, seq_lens=lens)
    _grads_case(prob, Recipe(dt_bias="inv_softplus_uniform", dt_shift=-4.0, init_std=0.3), seed=T + L)


@pytest.mark.parametrize("lens,L,dt", [((100, 1, 64, 65), 64, "bf16"), ((70, 200, 3), 64, "f32")],
                         ids=lambda v: str(v))
def test_backward_packed(lens, L, dt):
    P, N = (32, 32) if dt == "bf16" else (64, 128)
    prob = Problem(1, sum(lens), 2, P, N, 1, L, dt, seq_lens=tuple(lens))
    _grads_case(prob, Recipe(init_std=0.4), seed=len(lens))


def test_backward_one_head_block_per_group():
    # 64 sequences of 256 tokens in 64-token chunks: 512 workgroups per head
    # block in the dCB launch, so on a GPU of up to 256 CUs each group's two
    # heads are walked by one workgroup and no partial dCB sums are added
    lens = (256,) * 64
    prob = Problem(1, sum(lens), 4, 32, 32, 2, 64, "bf16", seq_lens=lens)
    _grads_case(prob, Recipe(init_std=0.4), seed=11)


def test_backward_without_optional_inputs():
    prob = Problem(1, 140, 2, 32, 16, 1, 64, "f32")
    inp_rec = Recipe()                      # no initial state
    got, ref = _grads_case(prob, inp_rec, seed=3, with_dfinal=False)
    assert got["initial_states"].abs().max().item() > 0    # gradient at a zero initial state


def test_backward_active_clamp():
    prob = Problem(1, 130, 2, 32, 16, 1, 64, "f32")
    _grads_case(prob, Recipe(init_std=0.2), seed=4, dt_min=0.08, dt_max=0.3)


def test_backward_deterministic():
    prob = Problem(1, 300, 2, 64, 128, 1, 128, "bf16")
    a, _ = _grads_case(prob, Recipe(init_std=0.3), seed=5)
    b, _ = _grads_case(prob, Recipe(init_std=0.3), seed=5)
    for k in ("x", "dt", "A", "B", "C", "D", "dt_bias", "initial_states"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("packed", [False, True], ids=["batch", "packed"])
def test_backward_after_forward_reuses_its_intermediates(packed):
    # ssd_bwd_after_fwd on the workspace an ssd_fwd call (library's own kernel
    # choices) left: the same stages computed the same intermediates, so the
    # gradients equal ssd_bwd's bit for bit; stale bytes past the forward's
    # part of the workspace must not matter
    if packed:
        lens = (100, 300, 64, 200)
        prob = Problem(1, sum(lens), 4, 64, 128, 2, 64, "bf16", seq_lens=lens)
    else:
        prob = Problem(2, 520, 4, 64, 128, 2, 256, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.3), seed=21)
    gen = torch.Generator().manual_seed(1021)
    dy = torch.randn(inp["x"].shape, generator=gen, dtype=torch.float32).to(inp["x"].dtype).cuda()
    dfin = torch.randn((prob.nseq, prob.nheads, prob.headdim, prob.dstate), generator=gen).cuda()
    d = to_dev(inp)
    kw = dict(D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"], cu_seqlens=d["cu_seqlens"])
    ref = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, dy, dfin, **kw)
    ws = torch.full_like(ref["workspace"], 0x7f)           # stale bytes everywhere
    binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, workspace=ws,
                    tuning=None, **kw)
    got = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, dy, dfin,
                          workspace=ws, after_fwd=True, **kw)
    torch.cuda.synchronize()
    for k in ("x", "dt", "A", "B", "C", "D", "dt_bias", "initial_states"):
        assert torch.equal(got[k], ref[k]), k


def test_backward_repeated_calls_on_one_workspace():
    # every call on one workspace (first filled with stale bytes) gives the
    # fresh-workspace gradients bit for bit: nothing a call reads from the
    # workspace is left over from an earlier call
    prob = Problem(1, 700, 6, 64, 128, 2, 256, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.3), seed=31)
    gen = torch.Generator().manual_seed(1031)
    dy = torch.randn(inp["x"].shape, generator=gen, dtype=torch.float32).to(inp["x"].dtype).cuda()
    dfin = torch.randn((prob.nseq, prob.nheads, prob.headdim, prob.dstate), generator=gen).cuda()
    d = to_dev(inp)
    kw = dict(D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"], cu_seqlens=d["cu_seqlens"])
    ref = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, dy, dfin, **kw)
    ws = torch.full_like(ref["workspace"], 0x5a)
    for _ in range(3):
        got = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, dy, dfin,
                              workspace=ws, **kw)
        torch.cuda.synchronize()
        for k in ("A", "D", "dt_bias", "dt", "x"):
            assert torch.equal(got[k], ref[k]), k


def test_backward_after_forward_needs_a_workspace():
    prob = Problem(1, 100, 2, 32, 32, 1, 64, "bf16")
    d = to_dev(make_inputs(prob, Recipe(), seed=1))
    with pytest.raises(ValueError):
        binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size,
                        torch.zeros_like(d["x"]), after_fwd=True)


# ------------------------------------------------- full-size shapes, sampled
# Heads are independent for every gradient but dB and dC (sums over a
# group's heads), and batch rows for every gradient but dA, dD and ddt_bias
# (sums over rows), so the oracle runs on sub-problems of the full inputs.

def _sub_heads(inp, dy, dfin, rows, heads, groups):
    hs = torch.tensor(heads)
    gs = torch.tensor(groups)
    pick = lambda v, dim, idx: None if v is None else v.index_select(dim, idx)
    r = torch.tensor(rows)
    return dict(x=pick(inp["x"], 0, r)[:, :, hs], dt=pick(inp["dt"], 0, r)[:, :, hs],
                dt_bias=pick(inp["dt_bias"], 0, hs), A=inp["A"][hs],
                B=pick(inp["B"], 0, r)[:, :, gs], C=pick(inp["C"], 0, r)[:, :, gs],
                D=pick(inp["D"], 0, hs), dy=pick(dy, 0, r)[:, :, hs],
                dfin=None if dfin is None else pick(dfin, 0, r)[:, hs])


def test_backward_layer_shape_sampled_heads():
    # the layer shape in the launch configuration the bench times; heads 0
    # and 23 of both rows: every gradient but dB and dC
    from state_space_model_ssd_amd.inputs import workload_inputs
    prob, inp = workload_inputs(2)
    gen = torch.Generator().manual_seed(2024)
    dy = torch.randn(inp["x"].shape, generator=gen).to(inp["x"].dtype)
    dfin = torch.randn((prob.nseq, prob.nheads, prob.headdim, prob.dstate), generator=gen)
    d = to_dev(inp)
    got = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, dy.cuda(),
                          dfin.cuda(), D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"])
    torch.cuda.synchronize()
    heads = [0, prob.nheads - 1]
    s = _sub_heads(inp, dy, dfin, [0, 1], heads, [0])
    init = torch.zeros((prob.nseq, len(heads), prob.headdim, prob.dstate))
    ref = ssd_grads(s["x"], s["dt"], s["dt_bias"], s["A"], s["B"], s["C"], s["D"], s["dy"],
                    s["dfin"], init=init)
    hs = torch.tensor(heads)
    report = {}
    for name, key, dim in (("x", "x", 2), ("dt", "dt", 2), ("A", "A", 0), ("D", "D", 0),
                           ("dt_bias", "dt_bias", 0), ("init", "initial_states", 1)):
        g = got[key].float().cpu().index_select(dim, hs)
        assert torch.isfinite(g).all(), name
        report[name] = rel_l2(g, ref[name])
        assert report[name] <= TOL["bf16"], (name, report)
    print("  rel_l2 " + " ".join(f"{k}={v:.2e}" for k, v in report.items()), flush=True)


def test_backward_training_batch_one_group():
    # the training-batch shape: batch row 3 and group 7 (heads 56-63), so
    # that dB and dC of that group are complete; per-head sums over rows
    # (dA, dD, ddt_bias) are covered by the layer-shape case
    from state_space_model_ssd_amd.inputs import workload_inputs
    prob, inp = workload_inputs(3)
    gen = torch.Generator().manual_seed(2025)
    dy = torch.randn(inp["x"].shape, generator=gen).to(inp["x"].dtype)
    d = to_dev(inp)
    got = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, dy.cuda(),
                          None, D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"])
    torch.cuda.synchronize()
    row, g = 3, 7
    hpg = prob.nheads // prob.ngroups
    heads = list(range(g * hpg, (g + 1) * hpg))
    s = _sub_heads(inp, dy, None, [row], heads, [g])
    init = torch.zeros((1, hpg, prob.headdim, prob.dstate))
    ref = ssd_grads(s["x"], s["dt"], s["dt_bias"], s["A"], s["B"], s["C"], s["D"], s["dy"], None,
                    init=init)
    hs = torch.tensor(heads)
    cut = {"x": got["x"][row:row + 1][:, :, hs], "dt": got["dt"][row:row + 1][:, :, hs],
           "B": got["B"][row:row + 1][:, :, g:g + 1], "C": got["C"][row:row + 1][:, :, g:g + 1],
           "init": got["initial_states"][row:row + 1][:, hs]}
    report = {}
    for name, g_ in cut.items():
        g_ = g_.float().cpu()
        assert torch.isfinite(g_).all(), name
        report[name] = rel_l2(g_, ref[name])
        assert report[name] <= TOL["bf16"], (name, report)
    print("  rel_l2 " + " ".join(f"{k}={v:.2e}" for k, v in report.items()), flush=True)
