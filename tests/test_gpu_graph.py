"""The forward captured in a HIP graph and replayed (the way bench.py times
it), against eager calls on the same inputs.  GPU only.

Each graph is replayed several times with eager work and synchronizations
in between; between replays the inputs are rewritten in place, so a replay
that read stale data or kept state from an earlier one would differ.  The
captured forward records no memset nodes: every buffer it reads is fully
written by an earlier kernel of the same forward.
"""
import pytest
import torch

from state_space_model_ssd_amd import binding
from state_space_model_ssd_amd.inputs import Problem, Recipe, make_inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "bf16-small-decay": (Problem(2, 1000, 6, 64, 128, 2, 256, "bf16"),
                         Recipe(dt_bias="inv_softplus_uniform", init_std=0.3)),
    "bf16-large-decay": (Problem(1, 777, 4, 64, 128, 1, 128, "bf16"), Recipe(init_std=0.3)),
    "bf16-packed": (Problem(1, 900, 4, 64, 128, 1, 64, "bf16", seq_lens=(300, 1, 599)),
                    Recipe(init_std=0.3)),
    "f32": (Problem(1, 333, 4, 32, 16, 1, 64, "f32"), Recipe(init_std=0.3)),
}


def _call(d, prob, out, fin, ws):
    binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, D=d["D"],
                    dt_bias=d["dt_bias"], initial_states=d["init"], cu_seqlens=d["cu_seqlens"],
                    out=out, final_states=fin, workspace=ws)


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_equal_eager_calls(name):
    prob, rec = CASES[name]
    d = to_dev(make_inputs(prob, rec, seed=7))
    g_out, g_fin, g_ws = binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size,
                                         D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"],
                                         cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        _call(d, prob, g_out, g_fin, g_ws)
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            _call(d, prob, g_out, g_fin, g_ws)
    torch.cuda.synchronize()
    e_out, e_fin = torch.empty_like(g_out), torch.empty_like(g_fin)
    e_ws = torch.empty_like(g_ws)
    for rep in range(4):
        if rep:
            # new inputs in the same buffers the graph reads
            fresh = to_dev(make_inputs(prob, rec, seed=100 + rep))
            for k in ("x", "dt", "B", "C", "init"):
                d[k].copy_(fresh[k])
        g_out.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _call(d, prob, e_out, e_fin, e_ws)
        torch.cuda.synchronize()
        assert torch.equal(g_out, e_out) and torch.equal(g_fin, e_fin), f"replay {rep}"
