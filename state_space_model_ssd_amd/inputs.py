"""Seeded synthetic inputs for the Mamba-2 SSD chunked-scan forward.

This module only draws random tensors with the shapes and value
distributions of the workloads; it holds none of the method's arithmetic.
Both the HIP path (through the binding) and the fp64 oracle consume the
exact same CPU tensors made here, so the two sides can never disagree about
their inputs.

Layouts (row-major, contiguous):
  x      (batch, seqlen, nheads, headdim)        fp32 or bf16
  dt     (batch, seqlen, nheads)                 fp32, raw (before softplus)
  dt_bias(nheads)                                fp32
  A      (nheads)                                fp32, negative
  B, C   (batch, seqlen, ngroups, dstate)        same dtype as x
  D      (nheads)                                fp32
  init   (batch or nseq, nheads, headdim, dstate) fp32, or None
  cu_seqlens (nseq + 1) int32, seq_idx (seqlen) int32 for a packed batch

The generation order inside one generator is fixed: sequence lengths (packed
batches only), x, dt_raw, dt_bias, A, B, C, D, initial states.  bf16 tensors
are drawn in fp32 and rounded to nearest-even by the cast.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch


@dataclasses.dataclass(frozen=True)
class Problem:
    batch: int
    seqlen: int            # per row; for a packed batch: total tokens
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int
    dtype: str = "bf16"    # "f32" or "bf16" for x, B, C and the output
    seq_lens: Optional[tuple] = None   # packed batch: lengths of the sequences

    @property
    def nseq(self) -> int:
        return len(self.seq_lens) if self.seq_lens is not None else self.batch

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


@dataclasses.dataclass(frozen=True)
class Recipe:
    """Value distributions of one workload."""
    dt_shift: float = -2.0                 # dt_raw ~ N(0, 1) + dt_shift
    dt_bias: str = "zero"                  # "zero" | "inv_softplus_uniform"
    dt_bias_range: tuple = (1e-3, 1e-1)    # for inv_softplus_uniform
    log_neg_a_range: tuple = (0.0, math.log(16.0))  # A = -exp(U(lo, hi))
    init_std: Optional[float] = None       # None: no initial state given


def _torch_dtype(name: str) -> torch.dtype:
    if name == "f32":
        return torch.float32
    if name == "bf16":
        return torch.bfloat16
    raise ValueError(f"unsupported dtype {name!r}")


def draw_seq_lens(gen: torch.Generator, nseq: int, lo: int, hi: int) -> tuple:
    """Integer lengths uniform on [lo, hi] inclusive."""
    return tuple(int(v) for v in torch.randint(lo, hi + 1, (nseq,), generator=gen))


def make_inputs(prob: Problem, recipe: Recipe = Recipe(), seed: int = 0,
                gen: Optional[torch.Generator] = None) -> dict:
    """Draw one problem's inputs on the CPU.  Returns a dict of tensors."""
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    b, T, H, P, N, G = prob.batch, prob.seqlen, prob.nheads, prob.headdim, prob.dstate, prob.ngroups
    dt_ = _torch_dtype(prob.dtype)
    if prob.seq_lens is not None:
        assert b == 1 and sum(prob.seq_lens) == T, "packed batch: batch == 1, seqlen == sum(lens)"

    x = torch.randn((b, T, H, P), generator=gen, dtype=torch.float32).to(dt_)
    dt = torch.randn((b, T, H), generator=gen, dtype=torch.float32) + recipe.dt_shift
    if recipe.dt_bias == "zero":
        dt_bias = torch.zeros(H, dtype=torch.float32)
    elif recipe.dt_bias == "inv_softplus_uniform":
        lo, hi = recipe.dt_bias_range
        u = torch.rand(H, generator=gen, dtype=torch.float64) * (hi - lo) + lo
        dt_bias = torch.log(torch.expm1(u)).to(torch.float32)
    else:
        raise ValueError(recipe.dt_bias)
    lo, hi = recipe.log_neg_a_range
    A = -torch.exp(torch.rand(H, generator=gen, dtype=torch.float32) * (hi - lo) + lo)
    B = torch.randn((b, T, G, N), generator=gen, dtype=torch.float32).to(dt_)
    C = torch.randn((b, T, G, N), generator=gen, dtype=torch.float32).to(dt_)
    D = torch.randn(H, generator=gen, dtype=torch.float32)
    init = None
    if recipe.init_std is not None:
        init = torch.randn((prob.nseq, H, P, N), generator=gen, dtype=torch.float32) * recipe.init_std

    out = dict(x=x, dt=dt, dt_bias=dt_bias, A=A, B=B, C=C, D=D, init=init,
               cu_seqlens=None, seq_idx=None)
    if prob.seq_lens is not None:
        cu = [0]
        for n in prob.seq_lens:
            cu.append(cu[-1] + int(n))
        out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32)
        out["seq_idx"] = torch.repeat_interleave(
            torch.arange(len(prob.seq_lens), dtype=torch.int32),
            torch.tensor(prob.seq_lens, dtype=torch.int64))
    return out


# --------------------------------------------------------------------------
# The named workloads.  Workload k is drawn from seed k - 1.  Workloads 1-5
# are the five configurations of the forward; workload 6 is a shape where one
# state chain per element leaves the HBM idle (two heads at long context),
# for the blocked state_passing.
# --------------------------------------------------------------------------

def _cfg5_lens(seed: int) -> tuple:
    return draw_seq_lens(torch.Generator().manual_seed(seed), 16, 256, 16384)


def workload(k: int):
    """Return (Problem, Recipe, seed) of workload k in 1..6."""
    if k == 1:   # tiny, fp32 everywhere
        return (Problem(1, 512, 4, 32, 16, 1, 64, "f32"), Recipe(), 0)
    if k == 2:   # Mamba-2 layer shape, short context
        return (Problem(2, 4096, 24, 64, 128, 1, 256, "bf16"),
                Recipe(dt_bias="inv_softplus_uniform"), 1)
    if k == 3:   # training batch, 8 heads per B/C group
        return (Problem(4, 8192, 64, 64, 128, 8, 256, "bf16"), Recipe(), 2)
    if k == 4:   # long context, 512-chunk state chain, nonzero initial state
        return (Problem(1, 131072, 32, 64, 128, 1, 256, "bf16"), Recipe(init_std=0.1), 3)
    if k == 5:   # 16 packed sequences, boundaries mid-chunk
        lens = _cfg5_lens(4)
        return (Problem(1, sum(lens), 32, 64, 128, 4, 256, "bf16", seq_lens=lens),
                Recipe(init_std=0.1), 4)
    if k == 6:   # two heads, 256-chunk chain: 16384 state elements
        return (Problem(1, 65536, 2, 64, 128, 1, 256, "bf16"), Recipe(init_std=0.1), 5)
    raise ValueError(f"workload {k} does not exist (1..6)")


def workload_inputs(k: int) -> tuple:
    """(Problem, inputs dict) of workload k.  For the packed workload the
    sequence lengths are the first draw of the seeded generator and the
    tensors follow from the same generator."""
    prob, rec, seed = workload(k)
    gen = torch.Generator().manual_seed(seed)
    if prob.seq_lens is not None:
        lens = draw_seq_lens(gen, len(prob.seq_lens), 256, 16384)
        assert lens == prob.seq_lens
    return prob, make_inputs(prob, rec, gen=gen)


WORKLOAD_NAMES = {
    1: "tiny-f32 b1 T512 H4 P32 N16 G1 L64",
    2: "mamba2-layer b2 T4096 H24 P64 N128 G1 L256 bf16",
    3: "train-batch b4 T8192 H64 P64 N128 G8 L256 bf16",
    4: "long-context b1 T131072 H32 P64 N128 G1 L256 bf16 init",
    5: "packed-16seq H32 P64 N128 G4 L256 bf16 init",
    6: "few-heads-long b1 T65536 H2 P64 N128 G1 L256 bf16 init",
}


def pick_heads(H: int, G: int, count: int) -> list:
    """A deterministic head sample that touches the first and last group."""
    if count >= H:
        return list(range(H))
    hs = sorted({0, H - 1} | {int(round(i * (H - 1) / max(count - 1, 1))) for i in range(count)})
    return hs[:max(count, 2)]
