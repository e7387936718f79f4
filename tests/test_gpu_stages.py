"""Each HIP stage against the fp64 chunked oracle's intermediates (GPU).

The chunked oracle (oracle/chunked.py) splits the recurrence at the same
sequence-local chunk boundaries, so every intermediate has a counterpart:
delta and dA_cumsum (stage 1), CB (stage 2), chunk states (stage 3), states
entering each chunk (stage 4).  Stages can also be run one by one through
the stage mask, which must give the same result as the full call.
"""
import numpy as np
import pytest
import torch

from oracle.chunked import ssd_chunked
from state_space_model_ssd_amd import binding
from state_space_model_ssd_amd.inputs import Problem, Recipe, make_inputs
from tests.helpers import gpu_forward, rel_l2, f64

pytestmark = pytest.mark.gpu

CASES = [
    # (b, T, H, P, N, G, L, dtype, lens)
    (2, 300, 4, 64, 128, 2, 64, "f32", None),
    (1, 600, 4, 64, 128, 2, 256, "bf16", None),
    (1, 0, 4, 64, 128, 2, 64, "bf16", (100, 1, 64, 130)),
    (1, 0, 2, 32, 16, 1, 64, "f32", (65, 3, 128)),
]


def case_id(c):
    return "b{}T{}H{}P{}N{}G{}L{}{}{}".format(*c[:8], "" if c[8] is None else "-packed")


@pytest.fixture(params=CASES, ids=case_id, scope="module")
def run(request):
    b, T, H, P, N, G, L, dt, lens = request.param
    if lens is not None:
        T = sum(lens)
    prob = Problem(b, T, H, P, N, G, L, dt, seq_lens=lens)
    inp = make_inputs(prob, Recipe(init_std=0.3), seed=T)
    out, fin, ws = gpu_forward(prob, inp)
    torch.cuda.synchronize()
    cp = binding.make_problem(b, T, H, P, N, G, L, 0 if dt == "f32" else 1,
                              nseq=len(lens) if lens else 0)
    mid = binding.intermediates(ws, cp)
    ref = ssd_chunked(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                      inp["D"], L, init=inp["init"], cu_seqlens=inp["cu_seqlens"])
    return prob, inp, out, fin, ws, mid, ref


def test_chunk_table(run):
    prob, inp, out, fin, ws, mid, ref = run
    nc = len(ref["chunks"])
    if prob.seq_lens is None:
        return   # rows mode: the map is arithmetic, no table is written
    tab = mid["chunk_table"].cpu().numpy()
    want = np.array([(t0, n, s, k) for (s, t0, n, k) in ref["chunks"]], dtype=np.int64)
    assert np.array_equal(tab[:nc], want)
    assert np.all(tab[nc:, 1] == 0)
    sc = mid["seq_chunks"].cpu().numpy()
    firsts = [c for c, ch in enumerate(ref["chunks"]) if ch[3] == 0]
    assert list(sc[:-1]) == firsts and sc[-1] == nc


def test_cumsum_stage(run):
    prob, inp, out, fin, ws, mid, ref = run
    nc = len(ref["chunks"])
    d = f64(mid["delta"][:nc])
    a = f64(mid["dA_cumsum"][:nc])
    for c, (s, t0, n, k) in enumerate(ref["chunks"]):
        np.testing.assert_allclose(d[c, :, :n], ref["delta"][c, :, :n], rtol=2e-6, atol=1e-30)
        scale = np.abs(ref["dAcs"][c, :, :n]).max() + 1e-30
        assert np.abs(a[c, :, :n] - ref["dAcs"][c, :, :n]).max() <= 2e-6 * scale


def test_bmm_stage(run):
    prob, inp, out, fin, ws, mid, ref = run
    cb = f64(mid["cb"])
    Bf = np.abs(f64(inp["B"])).reshape(-1, prob.ngroups, prob.dstate)
    Cf = np.abs(f64(inp["C"])).reshape(-1, prob.ngroups, prob.dstate)
    for c, (s, t0, n, k) in enumerate(ref["chunks"]):
        tri = np.tril(np.ones((n, n), dtype=bool))
        for g in range(prob.ngroups):
            got = cb[c, g, :n, :n][tri]
            want = ref["CB"][c, g, :n, :n][tri]
            # fp32 accumulation of exact products: |err| <= ~N eps sum|c||b|,
            # plus one rounding to the stored dtype (bf16: 2^-8 relative)
            scale = (Cf[t0:t0 + n, g] @ Bf[t0:t0 + n, g].T)[tri]
            store = 0.0 if prob.dtype == "f32" else 2.0 ** -8
            assert np.max(np.abs(got - want) / (2e-6 * scale + store * np.abs(want) + 1e-30)) <= 1.0
            # the stored CB is causal: 0 above the diagonal of every diagonal
            # 64x64 block the chunk's rows reach (chunk_scan multiplies them
            # unmasked)
            for b0 in range(0, n, 64):
                blk = cb[c, g, b0:b0 + 64, b0:b0 + 64]
                assert not np.triu(blk, 1).any()


def test_chunk_state_stage(run):
    prob, inp, out, fin, ws, mid, ref = run
    nc = len(ref["chunks"])
    tol = 1e-5 if prob.dtype == "f32" else 5e-3      # bf16: one rounding of x * w
    assert rel_l2(mid["chunk_states"][:nc], ref["S"]) < tol


def test_state_passing_stage(run):
    prob, inp, out, fin, ws, mid, ref = run
    nc = len(ref["chunks"])
    tol = 1e-5 if prob.dtype == "f32" else 5e-3      # bf16 storage of entering states
    assert rel_l2(mid["states_in"][:nc].float(), ref["Hin"]) < tol
    assert rel_l2(fin, ref["final"]) < (1e-5 if prob.dtype == "f32" else 5e-3)


def test_stage_by_stage_equals_full_call(run):
    prob, inp, out, fin, ws, mid, ref = run
    ws2 = torch.zeros_like(ws)
    o2 = f2 = None
    for name in ("plan", "chunk_cumsum", "bmm_chunk", "chunk_state", "state_passing",
                 "chunk_scan"):
        o2, f2, ws2 = gpu_forward(prob, inp, workspace=ws2, out=o2, final_states=f2,
                                  stages=binding.STAGES[name])
    torch.cuda.synchronize()
    assert torch.equal(o2, out) and torch.equal(f2, fin)
