"""The forward with the gated RMS norm (ssd_fwd_gated) against ssd_fwd
followed by the standalone norm, bit for bit, and against the fp64 oracles
composed (GPU).

Norm groups inside a head run in chunk_scan's store (both scan paths, both
tile sizes); groups across heads run the norm as a launch of its own."""
import math

import numpy as np
import pytest
import torch

from oracle.gated_norm import gated_rmsnorm_fwd
from state_space_model_ssd_amd import binding
from state_space_model_ssd_amd.inputs import Problem, Recipe, make_inputs, workload_inputs
from tests.helpers import assert_close, oracle_forward, to_dev

pytestmark = pytest.mark.gpu


def run(prob, inp, gs, eps=1e-5, seed=0):
    d = to_dev(inp)
    g = torch.Generator().manual_seed(seed)
    z = (torch.randn(inp["x"].shape, generator=g) * 2).to(inp["x"].dtype)
    w = torch.randn(prob.nheads * prob.headdim, generator=g) * 0.5 + 1.0
    zc, wc = z.cuda(), w.cuda()
    out, fin, _ = binding.ssd_fwd_gated(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size,
                                        zc, wc, gs, eps, D=d["D"], dt_bias=d["dt_bias"],
                                        initial_states=d["init"], cu_seqlens=d["cu_seqlens"])
    y, fin2, _ = binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size,
                                 D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"],
                                 cu_seqlens=d["cu_seqlens"], tuning=None)
    C = prob.nheads * prob.headdim
    ref = binding.gated_norm_fwd(y.view(-1, C), zc.view(-1, C), wc, gs, eps).view(y.shape)
    torch.cuda.synchronize()
    return out, fin, ref, fin2, z, w


def check_oracle(prob, inp, out, z, w, gs, eps=1e-5):
    """y of the forward against the SSD oracle, and the gated output against
    the norm oracle applied to that y.  (The norm of a small group divides by
    that group's rms, so the SSD's own rounding of y, within its bound, can
    move the composed result by more than a bf16 bound: each stage is held
    to its own oracle.)"""
    d = to_dev(inp)
    y, _, _ = binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, D=d["D"],
                              dt_bias=d["dt_bias"], initial_states=d["init"],
                              cu_seqlens=d["cu_seqlens"], tuning=None)
    torch.cuda.synchronize()
    y_ref, _ = oracle_forward(inp)
    assert_close(y.float().cpu(), y_ref, prob.dtype, "y")
    C = prob.nheads * prob.headdim
    o_ref, _ = gated_rmsnorm_fwd(y.float().cpu().reshape(-1, C), z.reshape(-1, C), w, eps, gs)
    assert_close(out.float().cpu().reshape(-1, C), o_ref, prob.dtype, "gated out")


@pytest.mark.parametrize("gs", [64, 32, 16, 8, 128, 1536])
def test_gated_layer_shape(gs):
    prob, inp = workload_inputs(2)
    out, fin, ref, fin2, z, w = run(prob, inp, gs)
    assert torch.equal(out, ref) and torch.equal(fin, fin2)
    check_oracle(prob, inp, out, z, w, gs)


@pytest.mark.parametrize("L", [128, 256])
def test_gated_both_scan_paths(L):
    # heads whose whole-chunk decay takes the rescaled path and heads that
    # take the masked one, in one launch
    H = 6
    prob = Problem(2, 3 * L + 37, H, 64, 128, 2, L, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.3), seed=L)
    delta = torch.nn.functional.softplus(inp["dt"].double() + inp["dt_bias"].double())
    md = float(delta.mean())
    A = inp["A"].clone()
    for h in range(H):
        A[h] = (-1e-4, -60.0 / (L * md / math.log(2.0)), -16.0)[h % 3]
    inp["A"] = A
    for gs in (64, 16):
        out, fin, ref, fin2, z, w = run(prob, inp, gs, seed=gs)
        assert torch.equal(out, ref) and torch.equal(fin, fin2)
        check_oracle(prob, inp, out, z, w, gs)


def test_gated_many_tiles_and_packed():
    # a grid of many tiles per CU (8-wave tiles with the gate in their store)
    prob = Problem(1, 65536 + 77, 8, 64, 128, 1, 256, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.1), seed=2)
    cp = binding.make_problem(1, prob.seqlen, 8, 64, 128, 1, 256, binding.SSD_BF16)
    assert binding.fwd_choices(cp)["scan_kernel"] == 1
    out, fin, ref, fin2, z, w = run(prob, inp, 64)
    assert torch.equal(out, ref) and torch.equal(fin, fin2)
    check_oracle(prob, inp, out, z, w, 64)
    lens = (700, 0, 1025, 3)
    pp = Problem(1, sum(lens), 4, 64, 128, 2, 256, "bf16", seq_lens=lens)
    pin = make_inputs(pp, Recipe(init_std=0.3), seed=4)
    out, fin, ref, fin2, z, w = run(pp, pin, 32)
    assert torch.equal(out, ref) and torch.equal(fin, fin2)
    check_oracle(pp, pin, out, z, w, 32)


def test_gated_fp32_runs_the_norm_after():
    prob, inp = workload_inputs(1)
    out, fin, ref, fin2, z, w = run(prob, inp, 32)
    assert torch.equal(out, ref) and torch.equal(fin, fin2)
    check_oracle(prob, inp, out, z, w, 32)
