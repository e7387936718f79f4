"""The fused forward (ssd_tuning_t.fused = 2: stages 1-5 in one persistent
launch) against the fp64 oracle and against the separate launches (GPU).

The fused launch runs the same device functions in the same order as the
separate launches with the one-chain state passing and the 8-wave scan tile,
so the two must agree bit for bit; the oracle bounds both.  After every
fused call the error word of its counters must be 0 (no wait gave up).
"""
import math

import pytest
import torch

from state_space_model_ssd_amd import binding
from state_space_model_ssd_amd.inputs import Problem, Recipe, make_inputs, workload_inputs
from tests.helpers import assert_close, gpu_forward, oracle_forward, to_dev

pytestmark = pytest.mark.gpu

FUSED = {"fused": 2}
SEPARATE = {"fused": 1, "sp_blocks": 1}    # the same scan tile as the fused launch picks


def err_word(prob, ws):
    cp = binding.make_problem(prob.batch, prob.seqlen, prob.nheads, prob.headdim, prob.dstate,
                              prob.ngroups, prob.chunk_size, binding.SSD_BF16,
                              nseq=len(prob.seq_lens) if prob.seq_lens else 0)
    lay = binding.workspace_layout(cp)
    off = lay.sync + 4 * lay.max_chunks * prob.nheads
    return int(ws[off:off + 4].view(torch.int32).item())


def run_both(prob, inp, **kw):
    of, ff, ws = gpu_forward(prob, inp, tuning=FUSED, **kw)
    torch.cuda.synchronize()
    if prob.tokens > 0:                      # (no chunk: no counter is used or cleared)
        assert err_word(prob, ws) == 0
    os_, fs, _ = gpu_forward(prob, inp, tuning=SEPARATE, **kw)
    torch.cuda.synchronize()
    return of, ff, os_, fs


def check_oracle(prob, inp, y, f, head_batch=None):
    hs = list(range(prob.nheads))
    step = head_batch or len(hs)
    import numpy as np
    yr, fr = [], []
    for i in range(0, len(hs), step):
        a, b = oracle_forward(inp, heads=hs[i:i + step])
        yr.append(a)
        fr.append(b)
    assert_close(y.float().cpu(), np.concatenate(yr, 2), prob.dtype, "y")
    assert_close(f.cpu(), np.concatenate(fr, 1), prob.dtype, "final_states")


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_fused_workloads(k):
    prob, inp = workload_inputs(k)
    of, ff, os_, fs = run_both(prob, inp)
    assert torch.equal(of, os_) and torch.equal(ff, fs)
    check_oracle(prob, inp, of, ff, head_batch=None if k == 2 else 8)


SMALL = [
    # (b, T, H, P, N, G, L, init)
    (3, 520, 6, 64, 128, 3, 256, 0.5),
    (1, 777, 8, 64, 128, 4, 128, None),
    (2, 300, 4, 64, 128, 2, 128, 0.3),
    (1, 1, 4, 64, 128, 2, 256, 0.3),
    (1, 255, 4, 64, 128, 2, 256, None),
    (1, 257, 4, 64, 128, 1, 256, 0.3),
    (1, 65536, 2, 64, 128, 1, 256, 0.1),    # few heads, long chain (64 segments of the walk)
    (2, 0, 4, 64, 128, 2, 256, 1.0),        # no tokens: the initial state passes through
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "b{}T{}H{}P{}N{}G{}L{}init{}".format(*s))
def test_fused_shapes(shape):
    b, T, H, P, N, G, L, init = shape
    prob = Problem(b, T, H, P, N, G, L, "bf16")
    inp = make_inputs(prob, Recipe(init_std=init), seed=T + H + L)
    of, ff, os_, fs = run_both(prob, inp)
    assert torch.equal(of, os_) and torch.equal(ff, fs)
    if T == 0:
        assert torch.equal(ff.cpu(), inp["init"])
        return
    check_oracle(prob, inp, of, ff)


@pytest.mark.parametrize("lens,L", [((100, 0, 300, 0, 640, 1), 128),
                                    ((0, 257, 1024, 3, 511), 256)], ids=lambda v: str(v))
def test_fused_packed(lens, L):
    prob = Problem(1, sum(lens), 4, 64, 128, 2, L, "bf16", seq_lens=tuple(lens))
    inp = make_inputs(prob, Recipe(init_std=0.4), seed=len(lens) + L)
    of, ff, os_, fs = run_both(prob, inp)
    assert torch.equal(of, os_) and torch.equal(ff, fs)
    check_oracle(prob, inp, of, ff)
    o2, f2, ws = gpu_forward(prob, inp, use_seq_idx=True, tuning=FUSED)
    torch.cuda.synchronize()
    assert err_word(prob, ws) == 0
    assert torch.equal(o2, of) and torch.equal(f2, ff)


@pytest.mark.parametrize("L", [128, 256])
def test_fused_both_scan_paths(L):
    # heads with a negligible, a near-2^60 and a far larger whole-chunk decay:
    # one launch runs the rescaled and the masked scan tiles
    H = 6
    prob = Problem(2, 3 * L + 37, H, 64, 128, 2, L, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.3), seed=L)
    delta = torch.nn.functional.softplus(inp["dt"].double() + inp["dt_bias"].double())
    md = float(delta.mean())
    log2e = 1.0 / math.log(2.0)
    A = inp["A"].clone()
    for h in range(H):
        A[h] = (-1e-4, -60.0 / (log2e * L * md), -16.0)[h % 3]
    inp["A"] = A
    of, ff, os_, fs = run_both(prob, inp)
    assert torch.equal(of, os_) and torch.equal(ff, fs)
    check_oracle(prob, inp, of, ff)


def test_fused_graph_replays():
    """The fused forward captured in a HIP graph, replayed with new inputs and
    eager work in between: every replay equals an eager call."""
    prob, inp = workload_inputs(2)
    d = to_dev(inp)
    out = torch.empty_like(d["x"])
    fin = torch.empty((prob.nseq, prob.nheads, prob.headdim, prob.dstate), device="cuda")
    _, _, ws = binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size,
                               D=d["D"], dt_bias=d["dt_bias"], tuning=FUSED)

    def call():
        binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, D=d["D"],
                        dt_bias=d["dt_bias"], out=out, final_states=fin, workspace=ws,
                        tuning=FUSED)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(3)
    for rep in range(4):
        d["x"].copy_(torch.randn(d["x"].shape, generator=gen).to(torch.bfloat16))
        d["dt"].copy_(torch.randn(d["dt"].shape, generator=gen) - 2)
        g.replay()
        torch.cuda.synchronize()
        got_o, got_f = out.clone(), fin.clone()
        assert err_word(prob, ws) == 0
        eo, ef, _ = binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size,
                                    D=d["D"], dt_bias=d["dt_bias"], tuning=SEPARATE)
        torch.cuda.synchronize()
        assert torch.equal(got_o, eo) and torch.equal(got_f, ef), rep


def test_fused_then_backward_after_fwd():
    """The fused forward leaves the intermediates ssd_bwd_after_fwd reads,
    bit for bit those of the separate launches."""
    prob = Problem(1, 700, 4, 64, 128, 2, 256, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.2), seed=5)
    d = to_dev(inp)
    gen = torch.Generator().manual_seed(1)
    dy = torch.randn(d["x"].shape, generator=gen).to(torch.bfloat16).cuda()
    grads = []
    for tune in (FUSED, SEPARATE):
        cp = binding.make_problem(1, 700, 4, 64, 128, 2, 256, binding.SSD_BF16)
        ws = torch.empty(binding.bwd_workspace_size(cp), dtype=torch.uint8, device="cuda")
        binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], 256, D=d["D"],
                        dt_bias=d["dt_bias"], initial_states=d["init"], workspace=ws, tuning=tune)
        r = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], 256, dy, None, D=d["D"],
                            dt_bias=d["dt_bias"], initial_states=d["init"], workspace=ws,
                            after_fwd=True)
        torch.cuda.synchronize()
        grads.append({k: v.clone() for k, v in r.items() if k != "workspace" and v is not None})
    for k in grads[0]:
        assert torch.equal(grads[0][k], grads[1][k]), k
