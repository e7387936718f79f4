"""Parity of the HIP forward with the fp64 oracle (GPU).

Every input is drawn on the CPU by the seeded generators; the oracle reads
the same values upcast exactly to fp64.  Tolerances: relative L2 <= 1e-5 for
fp32 x/B/C; relative L2 <= 2e-2 and max|err|/max|ref| <= 5e-2 for bf16 x/B/C
(tests/helpers.py gives the reason for normalising by max|ref|).  The five
workloads are compared in full (every token of every head, batch row or
sequence) in the launch configuration the bench times; the oracle runs over
groups of heads to bound its fp64 memory.
"""
import numpy as np
import math

import pytest
import torch

from state_space_model_ssd_amd.inputs import (Problem, Recipe, make_inputs, workload,
                                              workload_inputs, pick_heads)
from tests.helpers import assert_close, gpu_forward, oracle_forward, rel_l2, f64

pytestmark = pytest.mark.gpu


def check(prob, inp, heads=None, head_batch=None, **kw):
    """GPU forward against the oracle on `heads` (default: all).  With
    head_batch, the oracle runs that many heads at a time and the metrics are
    taken over the concatenation of all of them, as over one tensor."""
    out, fin, _ = gpu_forward(prob, inp, **kw)
    torch.cuda.synchronize()
    hs = list(range(prob.nheads)) if heads is None else list(heads)
    step = head_batch or len(hs)
    y_parts, f_parts = [], []
    for i in range(0, len(hs), step):
        y_r, f_r = oracle_forward(inp, heads=hs[i:i + step])
        y_parts.append(y_r)
        f_parts.append(f_r)
    y_ref = np.concatenate(y_parts, axis=2)
    f_ref = np.concatenate(f_parts, axis=1)
    y = out[:, :, hs].float().cpu()
    f = fin[:, hs].cpu()
    assert torch.isfinite(y).all() and torch.isfinite(f).all()
    ey = assert_close(y, y_ref, prob.dtype, "y")
    ef = assert_close(f, f_ref, prob.dtype, "final_states")
    print(f"  rel_l2 y={ey:.3e} final={ef:.3e} over {len(hs)} heads", flush=True)
    return out, fin


# ------------------------------------------------------------ the workloads

def test_workload1_tiny_f32():
    prob, inp = workload_inputs(1)
    check(prob, inp)


def test_workload2_layer_shape():
    prob, inp = workload_inputs(2)
    check(prob, inp)


def test_workload3_training_batch():
    prob, inp = workload_inputs(3)
    check(prob, inp, head_batch=16)


def test_workload4_long_context():
    prob, inp = workload_inputs(4)
    check(prob, inp, head_batch=8)


def test_workload5_packed():
    prob, inp = workload_inputs(5)
    out_cu, fin_cu = check(prob, inp, head_batch=8)
    out_si, fin_si, _ = gpu_forward(prob, inp, use_seq_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(out_cu, out_si) and torch.equal(fin_cu, fin_si)


# ----------------------------------------------------- shapes and ragged tails

SMALL = [
    # (b, T, H, P, N, G, L, dtype)
    (2, 300, 4, 64, 128, 2, 64, "bf16"),
    (1, 777, 8, 64, 128, 4, 128, "bf16"),
    (3, 520, 6, 64, 128, 3, 256, "bf16"),
    (2, 200, 4, 32, 32, 1, 64, "bf16"),
    (2, 333, 4, 64, 128, 2, 64, "f32"),
    (1, 600, 2, 64, 128, 1, 256, "f32"),
    (2, 130, 4, 32, 16, 4, 64, "f32"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "b{}T{}H{}P{}N{}G{}L{}{}".format(*s))
@pytest.mark.parametrize("init_std", [None, 0.5])
def test_ragged_shapes(shape, init_std):
    b, T, H, P, N, G, L, dt = shape
    prob = Problem(b, T, H, P, N, G, L, dt)
    inp = make_inputs(prob, Recipe(init_std=init_std), seed=T + H)
    check(prob, inp)


# Shapes with enough (chunk, head) tiles that the bf16 chunk_scan runs its
# persistent kernel (at least 6 tiles per resident workgroup; the sizes below
# leave a margin of 2-5x for every supported chunk size and tile shape), with
# ragged tails and initial states; the small shapes above run the one
# workgroup per tile kernel.
PERSISTENT = [
    # (b, T, H, P, N, G, L)
    (1, 16384 + 40, 128, 64, 128, 4, 64),
    (1, 16384 + 100, 96, 64, 128, 8, 128),
    (3, 5000, 64, 64, 128, 4, 256),
    (2, 20000, 32, 32, 32, 2, 64),
]


@pytest.mark.parametrize("shape", PERSISTENT, ids=lambda s: "b{}T{}H{}P{}N{}G{}L{}".format(*s))
def test_persistent_path_configs(shape):
    b, T, H, P, N, G, L = shape
    prob = Problem(b, T, H, P, N, G, L, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.2), seed=L + H)
    check(prob, inp, heads=[0, H // 2 + 1, H - 1])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_chain_longer_than_one_decay_batch(dt):
    # 1094 chunks in one sequence: the state chain crosses the 1024-chunk
    # batches in which state_passing stages the chunk decays
    prob = Problem(1, 70000, 4, 64, 128, 1, 64, dt)
    inp = make_inputs(prob, Recipe(init_std=0.2), seed=11)
    check(prob, inp)


@pytest.mark.parametrize("P,N,L", [(32, 32, 64), (64, 128, 64), (64, 128, 128), (64, 128, 256)])
def test_decay_regimes_per_head(P, N, L):
    # Heads cycle through a negligible decay, a whole-chunk decay near 2^-60
    # and one far below 2^-64, so one launch runs both chunk_scan paths (the
    # rescaled one for a chunk decay within 2^64, the masked one beyond).
    H = 6
    prob = Problem(2, 3 * L + 37, H, P, N, 2, L, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.3), seed=P + L)
    delta = torch.nn.functional.softplus(inp["dt"].double() + inp["dt_bias"].double())
    mean_delta = float(delta.mean())
    log2e = 1.0 / math.log(2.0)
    A = inp["A"].clone()
    for h in range(H):
        if h % 3 == 0:
            A[h] = -1e-4
        elif h % 3 == 1:
            A[h] = -60.0 / (log2e * L * mean_delta)
        else:
            A[h] = -16.0
    assert 16.0 * L * mean_delta * log2e > 4 * 64    # the third kind is far past the switch
    inp["A"] = A
    check(prob, inp)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 255, 256, 257])
def test_edge_lengths(T):
    prob = Problem(1, T, 4, 64, 128, 2, 64 if T < 200 else 256, "bf16")
    inp = make_inputs(prob, Recipe(init_std=0.3), seed=T)
    check(prob, inp)


def test_long_memory_small_steps():
    """Small steps (the layer-shape workload's dt_bias) keep the state alive
    across many chunks: the chain's accuracy is what is tested."""
    prob = Problem(1, 4096, 4, 64, 128, 1, 256, "f32")
    inp = make_inputs(prob, Recipe(dt_bias="inv_softplus_uniform", init_std=0.5), seed=3)
    check(prob, inp)


# ---------------------------------------------------------------- packed

PACKED = [
    ((1, 63, 64, 65, 200), 64, "bf16"),
    ((500, 1, 1, 300, 257), 256, "bf16"),
    ((130, 7, 64), 64, "f32"),
    ((1,), 64, "f32"),
]


@pytest.mark.parametrize("lens,L,dt", PACKED, ids=lambda v: str(v))
def test_packed_batches(lens, L, dt):
    P, N = (64, 128)
    prob = Problem(1, sum(lens), 4, P, N, 2, L, dt, seq_lens=tuple(lens))
    inp = make_inputs(prob, Recipe(init_std=0.4), seed=len(lens))
    out, fin = check(prob, inp)
    out2, fin2, _ = gpu_forward(prob, inp, use_seq_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(fin, fin2)


@pytest.mark.parametrize("lens,L", [((100, 0, 300, 0, 64, 0), 64),
                                    ((0, 257, 0, 0, 511, 3), 256),
                                    ((0,), 64)], ids=lambda v: str(v))
def test_packed_zero_length_sequences(lens, L):
    """A zero-length sequence inside a packed batch passes its initial state
    through as its final state, and the other sequences get exactly what
    the same batch without it gives."""
    H, P, N, G = 4, 64, 128, 2
    prob = Problem(1, sum(lens), H, P, N, G, L, "bf16", seq_lens=tuple(lens))
    inp = make_inputs(prob, Recipe(init_std=0.4), seed=sum(lens) + len(lens))
    out, fin = check(prob, inp)
    out2, fin2, _ = gpu_forward(prob, inp, use_seq_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(fin, fin2)
    for s, n in enumerate(lens):
        if n == 0:
            assert torch.equal(fin[s].cpu(), inp["init"][s]), s
    keep = [s for s, n in enumerate(lens) if n > 0]
    if not keep:
        assert out.numel() == 0
        return
    kl = tuple(lens[s] for s in keep)
    kprob = Problem(1, sum(kl), H, P, N, G, L, "bf16", seq_lens=kl)
    kinp = dict(inp)
    kinp["init"] = inp["init"][keep].contiguous()
    cu = [0]
    for n in kl:
        cu.append(cu[-1] + n)
    kinp["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32)
    kout, kfin, _ = gpu_forward(kprob, kinp)
    torch.cuda.synchronize()
    assert torch.equal(kout, out)
    assert torch.equal(kfin, fin[keep])


def test_packed_equals_isolated_runs():
    lens = (70, 300, 1, 129)
    prob = Problem(1, sum(lens), 4, 64, 128, 2, 64, "bf16", seq_lens=lens)
    inp = make_inputs(prob, Recipe(init_std=0.4), seed=21)
    out, fin, _ = gpu_forward(prob, inp)
    cu = inp["cu_seqlens"].tolist()
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        sub = dict(inp)
        for k in ("x", "dt", "B", "C"):
            sub[k] = inp[k][:, sl].contiguous()
        sub["init"] = inp["init"][s:s + 1].contiguous()
        sub["cu_seqlens"] = None
        sprob = Problem(1, lens[s], 4, 64, 128, 2, 64, "bf16")
        o, f, _ = gpu_forward(sprob, sub)
        torch.cuda.synchronize()
        # chunks start at each sequence's first token in both runs: same
        # arithmetic, so the results are identical
        assert torch.equal(o[0], out[0, sl]) and torch.equal(f[0], fin[s])


def test_packed_boundaries_leak_nothing():
    """Perturbing one sequence's inputs leaves every other sequence's outputs
    bitwise unchanged."""
    lens = (100, 37, 300, 64, 200)
    prob = Problem(1, sum(lens), 4, 64, 128, 2, 64, "bf16", seq_lens=lens)
    inp = make_inputs(prob, Recipe(init_std=0.4), seed=5)
    out, fin, _ = gpu_forward(prob, inp)
    cu = inp["cu_seqlens"].tolist()
    for victim in range(len(lens)):
        pert = dict(inp)
        sl = slice(cu[victim], cu[victim + 1])
        for k, scale in (("x", 3.0), ("dt", 1.5), ("B", -2.0), ("C", 0.5)):
            t = inp[k].clone()
            t[:, sl] = (t[:, sl].float() * scale + 0.25).to(t.dtype)
            pert[k] = t
        ini = inp["init"].clone()
        ini[victim] = ini[victim] * -3 + 1
        pert["init"] = ini
        o2, f2, _ = gpu_forward(prob, pert)
        torch.cuda.synchronize()
        for s in range(len(lens)):
            if s == victim:
                continue
            ss = slice(cu[s], cu[s + 1])
            assert torch.equal(o2[0, ss], out[0, ss]), (victim, s)
            assert torch.equal(f2[s], fin[s]), (victim, s)


# ----------------------------------------------------------- invariants

def test_deterministic():
    prob, inp = workload_inputs(2)
    a, fa, _ = gpu_forward(prob, inp)
    b, fb, _ = gpu_forward(prob, inp)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(fa, fb)


def test_split_and_resume():
    prob = Problem(2, 1024, 4, 64, 128, 2, 256, "f32")
    inp = make_inputs(prob, Recipe(init_std=0.2), seed=9)
    out, fin, _ = gpu_forward(prob, inp)
    cut = 512   # a chunk boundary: identical chunking on both sides
    p1 = Problem(2, cut, 4, 64, 128, 2, 256, "f32")
    p2 = Problem(2, 1024 - cut, 4, 64, 128, 2, 256, "f32")
    i1, i2 = dict(inp), dict(inp)
    for k in ("x", "dt", "B", "C"):
        i1[k] = inp[k][:, :cut].contiguous()
        i2[k] = inp[k][:, cut:].contiguous()
    o1, f1, _ = gpu_forward(p1, i1)
    i2["init"] = f1.cpu()
    o2, f2, _ = gpu_forward(p2, i2)
    torch.cuda.synchronize()
    assert rel_l2(torch.cat([o1, o2], 1), out) < 1e-6
    assert rel_l2(f2, fin) < 1e-6


def test_zero_step_gives_skip_only():
    prob = Problem(1, 300, 4, 64, 128, 2, 64, "f32")
    inp = make_inputs(prob, Recipe(), seed=2)
    inp["dt"] = torch.full_like(inp["dt"], -1e4)
    out, fin, _ = gpu_forward(prob, inp)
    torch.cuda.synchronize()
    exp = inp["D"][None, None, :, None] * inp["x"]
    assert torch.equal(out.cpu(), exp)
    assert torch.count_nonzero(fin) == 0


def test_empty_input_passes_initial_state_through():
    prob = Problem(2, 0, 4, 64, 128, 2, 64, "bf16")
    inp = make_inputs(prob, Recipe(init_std=1.0), seed=1)
    out, fin, _ = gpu_forward(prob, inp)
    torch.cuda.synchronize()
    assert out.numel() == 0
    assert torch.equal(fin.cpu(), inp["init"])


def test_no_skip_no_bias_no_final():
    prob = Problem(1, 500, 4, 64, 128, 1, 256, "bf16")
    inp = make_inputs(prob, Recipe(), seed=4)
    d = dict(inp)
    d["D"] = None
    d["dt_bias"] = None
    out, fin, _ = gpu_forward(prob, d, return_final_states=False)
    torch.cuda.synchronize()
    assert fin is None
    ref = dict(inp)
    ref["D"] = torch.zeros_like(inp["D"])
    ref["dt_bias"] = torch.zeros_like(inp["dt_bias"])
    y_ref, _ = oracle_forward(ref)
    assert_close(out.float().cpu(), y_ref, "bf16", "y")


def test_clamped_step():
    prob = Problem(1, 400, 4, 64, 128, 1, 64, "f32")
    inp = make_inputs(prob, Recipe(), seed=8)
    out, fin, _ = gpu_forward(prob, inp, dt_min=0.05, dt_max=0.2)
    torch.cuda.synchronize()
    from oracle.recurrence import ssd_recurrence
    y_ref, f_ref = ssd_recurrence(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"],
                                  inp["C"], inp["D"], dt_min=0.05, dt_max=0.2)
    assert_close(out.cpu(), y_ref, "f32", "y")
    assert_close(fin.cpu(), f_ref, "f32", "final")
