"""The allocation-free forward (ssd_fwd_noalloc) against ssd_fwd (GPU).

Both run the same kernels on the same workspace layout, so their outputs
must be identical bit for bit.  Two calls in a row share the library's
static scratch array; the second has a smaller input.  Problems larger than
the array are refused before anything is enqueued.
"""
import pytest
import torch

from state_space_model_ssd_amd import binding
from state_space_model_ssd_amd.inputs import Problem, Recipe, make_inputs, workload_inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def _both(prob, inp, use_seq_idx=False):
    d = to_dev(inp)
    ref_out, ref_fin, _ = binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"],
                                          prob.chunk_size, D=d["D"], dt_bias=d["dt_bias"],
                                          initial_states=d["init"], cu_seqlens=d["cu_seqlens"],
                                          tuning=None)
    out = torch.full_like(d["x"], float("nan"))
    fin = torch.full((prob.nseq, prob.nheads, prob.headdim, prob.dstate), float("nan"),
                     device=d["x"].device)
    kw = dict(seq_idx=d["seq_idx"], nseq=prob.nseq) if use_seq_idx else \
        dict(cu_seqlens=d["cu_seqlens"])
    binding.ssd_fwd_noalloc(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, out, fin,
                            D=d["D"], dt_bias=d["dt_bias"], initial_states=d["init"], **kw)
    torch.cuda.synchronize()
    return ref_out, ref_fin, out, fin


@pytest.mark.parametrize("first,second", [
    # the layer shape (47.7 MB of workspace), then a smaller ragged one
    ((2, 4096, 24, 64, 128, 1, 256, "bf16", None), (1, 777, 8, 64, 128, 4, 128, "bf16", None)),
    # a packed batch, then a smaller fp32 problem
    ((1, 0, 8, 64, 128, 2, 64, "bf16", (300, 0, 1000, 65)), (1, 500, 4, 32, 16, 1, 64, "f32", None)),
])
def test_noalloc_equals_ssd_fwd_twice(first, second):
    for i, spec in enumerate((first, second)):
        b, T, H, P, N, G, L, dt, lens = spec
        if lens is not None:
            T = sum(lens)
        prob = Problem(b, T, H, P, N, G, L, dt, seq_lens=lens)
        inp = make_inputs(prob, Recipe(init_std=0.3), seed=7 + i)
        ro, rf, o, f = _both(prob, inp)
        print(f"  call {i}: {spec} equal={torch.equal(ro, o) and torch.equal(rf, f)}", flush=True)
        assert torch.equal(ro, o) and torch.equal(rf, f)
        if lens is not None:
            _, _, o2, f2 = _both(prob, inp, use_seq_idx=True)
            assert torch.equal(o2, o) and torch.equal(f2, f)


def test_noalloc_refuses_problems_beyond_the_scratch():
    prob = binding.make_problem(4, 8192, 64, 64, 128, 8, 256, binding.SSD_BF16)
    assert binding.workspace_size(prob) > binding.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((4, 8192, 64, 64), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((4, 8192, 64), device="cuda")
    A = torch.zeros(64, device="cuda")
    B = torch.zeros((4, 8192, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(binding.SsdError) as e:
        binding.ssd_fwd_noalloc(x, dt, A, B, B, 256, out)
    assert e.value.code == binding.SSD_ERR_TOO_LARGE
