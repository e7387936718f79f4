"""The gated RMS norm kernels against the fp64 oracle (GPU).

Inputs are drawn on the CPU and rounded to the dtype; the oracle reads the
same values upcast exactly.  Tolerances: relative L2 <= 1e-5 for fp32 and
<= 2e-2 with max|err|/max|ref| <= 5e-2 for bf16 outputs (one rounding of
each output to bf16 is about 2^-9 relative); dw accumulates in fp32 in
either case and must be within 1e-5 relative L2 for fp32 inputs and 1e-4
for bf16 inputs (the bf16 dy/dz/out roundings do not enter it, but its sum
of 8192 fp32 products does).
"""
import numpy as np
import pytest
import torch

from oracle.gated_norm import gated_rmsnorm_bwd, gated_rmsnorm_fwd
from state_space_model_ssd_amd import binding
from tests.helpers import assert_close, rel_l2

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def draw(T, C, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    y = torch.randn((T, C), generator=g).to(DT[dtype])
    z = (torch.randn((T, C), generator=g) * 2).to(DT[dtype])
    w = torch.randn(C, generator=g) * 0.5 + 1.0
    dout = torch.randn((T, C), generator=g).to(DT[dtype])
    return y, z, w, dout


CASES = [
    # (tokens, channels, group_size, dtype)
    (8192, 1536, 1536, "bf16"),     # the layer shape: 24 heads x 64, one group per token
    (777, 4096, 512, "bf16"),       # 64 heads x 64 in 8 groups of 8 heads
    (300, 1536, 64, "bf16"),        # one group per head
    (129, 8192, 8192, "bf16"),      # the widest row
    (65, 256, 8, "bf16"),           # groups of one vector
    (500, 1024, 256, "f32"),
    (33, 4096, 4096, "f32"),
    (17, 96, 32, "f32"),            # a row of 24 vectors: most threads idle
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}C{}G{}{}".format(*c))
def test_gated_norm_forward(case):
    T, C, gs, dtype = case
    y, z, w, _ = draw(T, C, dtype, T + C)
    eps = 1e-5
    out, rstd = binding.gated_norm_fwd(y.cuda(), z.cuda(), w.cuda(), gs, eps, return_rstd=True)
    torch.cuda.synchronize()
    ref, rref = gated_rmsnorm_fwd(y, z, w, eps, gs)
    assert torch.isfinite(out.float()).all()
    assert_close(out.float().cpu(), ref, dtype, "out")
    assert rel_l2(rstd.cpu(), rref) < 1e-5


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}C{}G{}{}".format(*c))
def test_gated_norm_backward(case):
    T, C, gs, dtype = case
    y, z, w, dout = draw(T, C, dtype, 7 * T + C)
    eps = 1e-5
    dy, dz, dw = binding.gated_norm_bwd(y.cuda(), z.cuda(), w.cuda(), dout.cuda(), gs, eps)
    torch.cuda.synchronize()
    rdy, rdz, rdw = gated_rmsnorm_bwd(y, z, w, eps, gs, dout)
    assert_close(dy.float().cpu(), rdy, dtype, "dy")
    assert_close(dz.float().cpu(), rdz, dtype, "dz")
    e = rel_l2(dw.cpu(), rdw)
    print(f"  dw: rel_l2={e:.3e}", flush=True)
    assert e <= (1e-5 if dtype == "f32" else 1e-4)


def test_gated_norm_in_place_and_deterministic():
    y, z, w, dout = draw(2048, 1536, "bf16", 3)
    yc, zc, wc, dc = y.cuda(), z.cuda(), w.cuda(), dout.cuda()
    out = binding.gated_norm_fwd(yc, zc, wc, 1536)
    buf = yc.clone()
    binding.gated_norm_fwd(buf, zc, wc, 1536, out=buf)          # out is y itself
    a = binding.gated_norm_bwd(yc, zc, wc, dc, 1536)
    b = binding.gated_norm_bwd(yc, zc, wc, dc, 1536)
    torch.cuda.synchronize()
    assert torch.equal(buf, out)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_gated_norm_no_rows():
    y = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(512, device="cuda")
    out = binding.gated_norm_fwd(y, y, w, 64)
    dy, dz, dw = binding.gated_norm_bwd(y, y, w, y, 64)
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.count_nonzero(dw) == 0
