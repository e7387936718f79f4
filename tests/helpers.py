"""Shared helpers of the tests: metrics, device transfer, GPU and oracle runs."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances of the forward against the fp64 oracle:
#   fp32 x/B/C: relative L2 <= 1e-5
#   bf16 x/B/C (fp32 accumulation): relative L2 <= 2e-2 and
#   max|err| / max|ref| <= 5e-2.
# The max-abs bound is normalised by max|ref|: normalised by rms(ref) it
# would fail for any bf16 output, because rounding the exact result to bf16
# alone gives max|err|/rms of 0.052 (layer-shape workload) and 0.176
# (training-batch workload), whose outputs reach 23x and 61x their rms.
TOL_F32_REL_L2 = 1e-5
TOL_BF16_REL_L2 = 2e-2
TOL_BF16_MAX_NORM = 5e-2


def f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().cpu().to(torch.float64).numpy()


def rel_l2(got, ref) -> float:
    g, r = f64(got), f64(ref)
    return float(np.linalg.norm((g - r).ravel()) / max(np.linalg.norm(r.ravel()), 1e-300))


def max_norm(got, ref) -> float:
    """max |got - ref| / max |ref|."""
    g, r = f64(got), f64(ref)
    if not r.size:
        return 0.0
    return float(np.max(np.abs(g - r))) / max(float(np.max(np.abs(r))), 1e-300)


def max_rms(got, ref) -> float:
    """max |got - ref| / rms(ref) (reported, not a bound: see above)."""
    g, r = f64(got), f64(ref)
    if not r.size:
        return 0.0
    return float(np.max(np.abs(g - r))) / max(float(np.sqrt(np.mean(r * r))), 1e-300)


def pages_criterion_fraction(got, ref, atol=1e-2, rtol=1e-2) -> float:
    """Fraction of elements outside |got - ref| <= atol + rtol |ref|, the
    elementwise criterion of the clova.ai precision table (section "Faster
    kernels: Does the math still hold?")."""
    g, r = f64(got), f64(ref)
    if not r.size:
        return 0.0
    return float(np.mean(np.abs(g - r) > atol + rtol * np.abs(r)))


def assert_close(got, ref, dtype: str, what: str = ""):
    e = rel_l2(got, ref)
    print(f"  {what}: rel_l2={e:.3e} max/max={max_norm(got, ref):.3e} "
          f"max/rms={max_rms(got, ref):.3e} "
          f"outside(1e-2+1e-2|ref|)={pages_criterion_fraction(got, ref):.2e}", flush=True)
    if dtype == "f32":
        assert e <= TOL_F32_REL_L2, f"{what}: rel L2 {e:.3e} > {TOL_F32_REL_L2}"
    else:
        m = max_norm(got, ref)
        assert e <= TOL_BF16_REL_L2, f"{what}: rel L2 {e:.3e} > {TOL_BF16_REL_L2}"
        assert m <= TOL_BF16_MAX_NORM, f"{what}: max/max {m:.3e} > {TOL_BF16_MAX_NORM}"
    return e


def to_dev(inp: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_forward(prob, inp: dict, use_seq_idx: bool = False, **kw):
    """Run the HIP forward on inputs drawn on the CPU.  Returns device tensors
    (out, final_states, workspace)."""
    from state_space_model_ssd_amd import binding
    d = to_dev(inp)
    if use_seq_idx:
        return binding.ssd_fwd_seq_idx(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size,
                                       d["seq_idx"], prob.nseq, D=d["D"], dt_bias=d["dt_bias"],
                                       initial_states=d["init"], **kw)
    return binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], prob.chunk_size, D=d["D"],
                           dt_bias=d["dt_bias"], initial_states=d["init"],
                           cu_seqlens=d["cu_seqlens"], **kw)


def oracle_forward(inp: dict, heads=None):
    from oracle.recurrence import ssd_recurrence
    return ssd_recurrence(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"],
                          inp["D"], init=inp["init"], cu_seqlens=inp["cu_seqlens"], heads=heads)
