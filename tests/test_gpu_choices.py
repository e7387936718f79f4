"""The library's own kernel choices depend on the problem and the device,
never on earlier calls (GPU).

ssd_fwd_choices reports what the default path runs; a call sequence that
first runs other chunk sizes must report (and run) the same choices as a
fresh process, and the default output must equal ssd_fwd_tuned with those
choices pinned, bit for bit.
"""
import json
import os
import subprocess
import sys

import pytest
import torch

from state_space_model_ssd_amd import binding
from state_space_model_ssd_amd.inputs import Problem, Recipe, make_inputs, workload
from tests.helpers import gpu_forward

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (b, T, H, P, N, G, L, nseq): the layer shape, the training batch, the long
# context, and a 64-token-chunk shape whose tile count lies between the
# thresholds a persistent-grid size taken from 256-token chunks and its own
# would give
SHAPES = [
    (2, 4096, 24, 64, 128, 1, 256, 0),
    (4, 8192, 64, 64, 128, 8, 256, 0),
    (1, 131072, 32, 64, 128, 1, 256, 0),
    (1, 6400, 32, 64, 128, 2, 64, 0),
    (1, 65536, 2, 64, 128, 1, 256, 0),
]


def _cprob(s):
    b, T, H, P, N, G, L, nseq = s
    return binding.make_problem(b, T, H, P, N, G, L, binding.SSD_BF16, nseq=nseq)


def _fresh_process_choices():
    code = ("import json, sys; sys.path.insert(0, %r)\n"
            "from state_space_model_ssd_amd import binding\n"
            "from tests.test_gpu_choices import SHAPES, _cprob\n"
            "print(json.dumps([binding.fwd_choices(_cprob(s)) for s in SHAPES]))" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_choices_do_not_depend_on_earlier_calls():
    # run every chunk size first, the longest last
    for L in (64, 128, 256):
        prob = Problem(1, 3000, 8, 64, 128, 2, L, "bf16")
        gpu_forward(prob, make_inputs(prob, Recipe(), seed=L))
    torch.cuda.synchronize()
    here = [binding.fwd_choices(_cprob(s)) for s in SHAPES]
    fresh = _fresh_process_choices()
    print("choices:", here, flush=True)
    assert here == fresh
    for c in here:
        assert c["scan_kernel"] in (1, 2, 3) and c["sp_vec"] in (1, 2, 4) and c["front"] == 1
        assert c["sp_blocks"] in (1, 2, 4, 8, 16)
    # few state elements over a long chain: the blocked state passing
    assert here[-1]["sp_blocks"] > 1


@pytest.mark.parametrize("idx", [0, 3])
def test_default_equals_pinned_choices(idx):
    b, T, H, P, N, G, L, _ = SHAPES[idx]
    prob = Problem(b, T, H, P, N, G, L, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.1), seed=idx)
    # a forward at another chunk size first
    other = Problem(1, 2000, 4, 64, 128, 1, 256 if L != 256 else 64, "bf16")
    gpu_forward(other, make_inputs(other, Recipe(), seed=1))
    ch = binding.fwd_choices(_cprob(SHAPES[idx]))
    o1, f1, _ = gpu_forward(prob, inp, tuning=None)
    o2, f2, _ = gpu_forward(prob, inp, tuning=ch)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
