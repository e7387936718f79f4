"""Every pinned kernel choice (ssd_tuning_t) against the fp64 oracle, and
the offline tuner end to end.  GPU only.

The choices move no arithmetic except chunk_scan's kernel: runs that differ
only in the state_passing vector width or in fusing the front are compared
bit for bit, and every run is compared with the oracle at the dtype's
tolerance.
"""
import itertools

import pytest
import torch

from state_space_model_ssd_amd import binding, tuning
from state_space_model_ssd_amd.inputs import Problem, Recipe, make_inputs
from tests.helpers import assert_close, gpu_forward, oracle_forward, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    # (problem, recipe, seed): a small decay (the per-tile kernel's rescaled
    # path) and a large one (its masked path), with initial states
    "bf16-L256-small-decay": (Problem(2, 700, 6, 64, 128, 2, 256, "bf16"),
                              Recipe(dt_bias="inv_softplus_uniform", init_std=0.3), 31),
    "bf16-L64-large-decay": (Problem(1, 333, 4, 64, 128, 1, 64, "bf16"), Recipe(init_std=0.3), 32),
    "bf16-L256-large-decay": (Problem(1, 600, 4, 64, 128, 1, 256, "bf16"), Recipe(init_std=0.3), 35),
    "f32-L64": (Problem(1, 300, 4, 32, 16, 1, 64, "f32"), Recipe(init_std=0.3), 33),
    "bf16-L128-packed": (Problem(1, 650, 4, 64, 128, 2, 128, "bf16", seq_lens=(200, 1, 449)),
                         Recipe(init_std=0.3), 34),
}


def _problem_c(prob):
    return binding.make_problem(prob.batch, prob.seqlen, prob.nheads, prob.headdim, prob.dstate,
                                prob.ngroups, prob.chunk_size,
                                torch.bfloat16 if prob.dtype == "bf16" else torch.float32,
                                prob.nseq if prob.seq_lens is not None else 0)


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    prob, rec, seed = CASES[request.param]
    inp = make_inputs(prob, rec, seed=seed)
    ref_y, ref_fin = oracle_forward(inp)
    return request.param, prob, inp, ref_y, ref_fin


def test_every_choice_matches_the_oracle(case):
    name, prob, inp, ref_y, ref_fin = case
    runs = {}
    for cand in tuning.candidates(_problem_c(prob)):
        print(f"  {name} {cand}", flush=True)
        out, fin, _ = gpu_forward(prob, inp, tuning=cand)
        assert_close(out, ref_y, prob.dtype, f"y {cand}")
        assert_close(fin, ref_fin, prob.dtype, f"final {cand}")
        runs[tuple(sorted(cand.items()))] = (out.cpu(), fin.cpu())
    # sp_vec and front change no rounding: equal bits within one scan kernel;
    # the four-wave tile kernel does each row group's arithmetic in the same
    # order as the eight-wave one
    by_scan = {}
    for key, (o, f) in runs.items():
        sk = dict(key).get("scan_kernel", 0)
        by_scan.setdefault(1 if sk == 3 else sk, []).append((key, o, f))
    for group in by_scan.values():
        _, o0, f0 = group[0]
        for key, o, f in group[1:]:
            assert torch.equal(o, o0) and torch.equal(f, f0), key
    # the final states never depend on the chunk_scan kernel
    fins = [f for _, f in runs.values()]
    assert all(torch.equal(f, fins[0]) for f in fins[1:])


def test_tuner_records_a_choice_the_binding_then_uses(tmp_path, monkeypatch):
    prob, rec, seed = CASES["bf16-L256-small-decay"]
    inp = make_inputs(prob, rec, seed=seed)
    pc = _problem_c(prob)
    d = to_dev(inp)
    entry = tuning.autotune(pc, d, reps=3, rounds=2)
    assert entry["choice"] == {} or entry["choice"] in tuning.candidates(pc)
    assert len(entry["candidates"]) == len(tuning.candidates(pc)) + 1   # and the library's own
    assert entry["us"] <= entry["default_us"]
    # a choice recorded as pinned, and one recorded as the library's own
    path = str(tmp_path / "cfg.json")
    pinned_choice = {"scan_kernel": 1, "sp_vec": 1, "front": 2}
    tuning.save_config({tuning.shape_key(pc): dict(entry, choice=pinned_choice)}, path)
    monkeypatch.setattr(tuning, "CONFIG_PATH", path)
    assert tuning.lookup(pc) == pinned_choice
    tuned, fin_t, _ = gpu_forward(prob, inp)                       # tuning="config"
    pinned, fin_p, _ = gpu_forward(prob, inp, tuning=pinned_choice)
    assert torch.equal(tuned, pinned) and torch.equal(fin_t, fin_p)
    tuning.save_config({tuning.shape_key(pc): dict(entry, choice={})}, path)
    assert tuning.lookup(pc) is None
