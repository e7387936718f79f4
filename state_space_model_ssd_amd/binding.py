"""Thin Python binding of the C ABI in include/ssd.h (argument marshalling only).

Every stage of the SSD forward runs in the HIP kernels of libssd_hip.so;
this module only checks tensor metadata, allocates outputs and the workspace
with torch (device memory) and passes raw pointers plus the current HIP
stream.  If the library is not built, every call raises: there is no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd_hip.so")

SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP, \
    SSD_ERR_TOO_LARGE = range(6)
NOALLOC_SCRATCH_BYTES = 64 << 20     # SSD_NOALLOC_SCRATCH_BYTES of include/ssd.h
SSD_F32, SSD_BF16 = 0, 1
STAGE_PLAN, STAGE_CUMSUM, STAGE_BMM, STAGE_CHUNK_STATE, STAGE_STATE_PASSING, STAGE_CHUNK_SCAN = \
    (1 << i for i in range(6))
STAGE_ALL = 0x3F
STAGES = {"plan": STAGE_PLAN, "chunk_cumsum": STAGE_CUMSUM, "bmm_chunk": STAGE_BMM,
          "chunk_state": STAGE_CHUNK_STATE, "state_passing": STAGE_STATE_PASSING,
          "chunk_scan": STAGE_CHUNK_SCAN}

EXPORTED = ("ssd_fwd_workspace_size", "ssd_workspace_layout", "ssd_config_supported",
            "ssd_fwd", "ssd_fwd_stages", "ssd_fwd_tuned", "ssd_bwd_workspace_size", "ssd_bwd",
            "ssd_bwd_after_fwd", "ssd_fwd_choices", "ssd_fwd_noalloc", "ssd_gated_norm_fwd",
            "ssd_gated_norm_bwd_workspace_size", "ssd_gated_norm_bwd", "ssd_fwd_gated",
            "ssd_status_string")


class SsdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"ssd: {msg} (status {code})")
        self.code = code


class ProblemC(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk_size", ctypes.c_int64), ("nseq", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float)]


class LayoutC(ctypes.Structure):
    _fields_ = [("max_chunks", ctypes.c_int64), ("chunk_table", ctypes.c_size_t),
                ("seq_chunks", ctypes.c_size_t), ("delta", ctypes.c_size_t),
                ("dA_cumsum", ctypes.c_size_t), ("cb", ctypes.c_size_t),
                ("chunk_states", ctypes.c_size_t), ("states_in", ctypes.c_size_t),
                ("block_states", ctypes.c_size_t), ("block_logdecay", ctypes.c_size_t),
                ("sync", ctypes.c_size_t),
                ("sp_blocks", ctypes.c_int64), ("total_bytes", ctypes.c_size_t)]


class NormProblemC(ctypes.Structure):
    """ssd_norm_problem_t: the gated RMS norm after the SSD."""
    _fields_ = [("tokens", ctypes.c_int64), ("channels", ctypes.c_int64),
                ("group_size", ctypes.c_int64), ("dtype", ctypes.c_int32), ("eps", ctypes.c_float)]


class GateC(ctypes.Structure):
    """ssd_gate_t: the gated RMS norm ssd_fwd_gated applies to its output."""
    _fields_ = [("z", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("group_size", ctypes.c_int64)]


class TuningC(ctypes.Structure):
    """ssd_tuning_t: pinned kernel choices, 0 = the library's own."""
    _fields_ = [("scan_kernel", ctypes.c_int32), ("sp_vec", ctypes.c_int32),
                ("front", ctypes.c_int32), ("sp_blocks", ctypes.c_int32),
                ("fused", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libssd_hip.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing; build it with "
            "`python -m state_space_model_ssd_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    PP = ctypes.POINTER(ProblemC)
    lib.ssd_fwd_workspace_size.argtypes = [PP]
    lib.ssd_fwd_workspace_size.restype = sz
    lib.ssd_workspace_layout.argtypes = [PP, ctypes.POINTER(LayoutC)]
    lib.ssd_workspace_layout.restype = ctypes.c_int
    lib.ssd_config_supported.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64]
    lib.ssd_config_supported.restype = ctypes.c_int
    lib.ssd_fwd.argtypes = [PP] + [vp] * 12 + [vp, sz, vp]
    lib.ssd_fwd.restype = ctypes.c_int
    lib.ssd_fwd_stages.argtypes = [PP] + [vp] * 12 + [vp, sz, ctypes.c_uint32, vp]
    lib.ssd_fwd_stages.restype = ctypes.c_int
    lib.ssd_fwd_tuned.argtypes = [PP] + [vp] * 12 + [vp, sz, ctypes.c_uint32,
                                                     ctypes.POINTER(TuningC), vp]
    lib.ssd_fwd_tuned.restype = ctypes.c_int
    lib.ssd_bwd_workspace_size.argtypes = [PP]
    lib.ssd_bwd_workspace_size.restype = sz
    lib.ssd_bwd.argtypes = [PP] + [vp] * 20 + [vp, sz, vp]
    lib.ssd_bwd.restype = ctypes.c_int
    lib.ssd_bwd_after_fwd.argtypes = [PP] + [vp] * 20 + [vp, sz, vp]
    lib.ssd_bwd_after_fwd.restype = ctypes.c_int
    NP = ctypes.POINTER(NormProblemC)
    lib.ssd_gated_norm_fwd.argtypes = [NP] + [vp] * 5 + [vp]
    lib.ssd_gated_norm_fwd.restype = ctypes.c_int
    lib.ssd_gated_norm_bwd_workspace_size.argtypes = [NP]
    lib.ssd_gated_norm_bwd_workspace_size.restype = sz
    lib.ssd_gated_norm_bwd.argtypes = [NP] + [vp] * 8 + [sz, vp]
    lib.ssd_gated_norm_bwd.restype = ctypes.c_int
    lib.ssd_fwd_gated.argtypes = [PP] + [vp] * 10 + [ctypes.POINTER(GateC), vp, vp, vp, sz, vp]
    lib.ssd_fwd_gated.restype = ctypes.c_int
    lib.ssd_fwd_noalloc.argtypes = [PP] + [vp] * 12 + [vp]
    lib.ssd_fwd_noalloc.restype = ctypes.c_int
    lib.ssd_fwd_choices.argtypes = [PP, ctypes.POINTER(TuningC)]
    lib.ssd_fwd_choices.restype = ctypes.c_int
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().ssd_status_string(code).decode()


def _check(code: int):
    if code != SSD_OK:
        raise SsdError(code, status_string(code))


def make_problem(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype,
                 nseq=0, dt_min=0.0, dt_max=math.inf) -> ProblemC:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}.get(dtype, -1)
    return ProblemC(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate),
                    int(ngroups), int(chunk_size), int(nseq), int(dtype), float(dt_min),
                    float(dt_max))


def workspace_size(prob: ProblemC) -> int:
    return int(load_library().ssd_fwd_workspace_size(ctypes.byref(prob)))


def workspace_layout(prob: ProblemC) -> LayoutC:
    lay = LayoutC()
    _check(load_library().ssd_workspace_layout(ctypes.byref(prob), ctypes.byref(lay)))
    return lay


def config_supported(dtype, headdim, dstate, chunk_size) -> bool:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}.get(dtype, -1)
    return bool(load_library().ssd_config_supported(int(dtype), int(headdim), int(dstate),
                                                    int(chunk_size)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape, device):
    if t is None:
        return
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def ssd_fwd(x, dt, A, B, C, chunk_size, D=None, dt_bias=None, initial_states=None,
            cu_seqlens=None, seq_idx=None, dt_min=0.0, dt_max=math.inf, out=None,
            final_states=None, return_final_states=True, workspace=None,
            stages: int = STAGE_ALL, tuning="config"):
    """SSD forward on the GPU through the C ABI.

    x (b, T, H, P) fp32|bf16; dt (b, T, H) fp32; A (H) fp32; B, C (b, T, G, N)
    in x's dtype; D, dt_bias (H) fp32 or None; initial_states (nstates, H, P, N)
    fp32 or None; cu_seqlens (nseq + 1) / seq_idx (T) int32 for a packed batch
    (b == 1).  Returns (out, final_states, workspace).

    tuning: "config" looks the shape up in the tuned config file (see
    tuning.py) and keeps the library's own choices for shapes it does not
    list; None keeps the library's choices; a dict with any of scan_kernel,
    sp_vec, front pins them (ssd_tuning_t in include/ssd.h).
    """
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_fwd runs on the GPU only; x is on " + str(dev))
    nseq = 0
    if cu_seqlens is not None:
        nseq = cu_seqlens.numel() - 1
    elif seq_idx is not None:
        raise ValueError("pass nseq through cu_seqlens, or use ssd_fwd_seq_idx")
    return _run(x, dt, A, B, C, chunk_size, D, dt_bias, initial_states, cu_seqlens, None, nseq,
                dt_min, dt_max, out, final_states, return_final_states, workspace, stages,
                tuning)


def bwd_workspace_size(prob: ProblemC) -> int:
    return int(load_library().ssd_bwd_workspace_size(ctypes.byref(prob)))


def ssd_bwd(x, dt, A, B, C, chunk_size, dout, dfinal_states=None, D=None, dt_bias=None,
            initial_states=None, cu_seqlens=None, dt_min=0.0, dt_max=math.inf, workspace=None,
            after_fwd=False):
    """SSD backward on the GPU through the C ABI: gradients of
    sum(out * dout) + sum(final_states * dfinal_states) for the inputs of
    ssd_fwd (same arguments).  Returns a dict with x, dt, A, B, C, D,
    dt_bias, initial_states (gradients; D, dt_bias and initial_states always
    computed) and the workspace.

    after_fwd: call ssd_bwd_after_fwd, which reuses the forward's
    intermediates left in `workspace` (required, ssd_bwd_workspace_size
    bytes) by an ssd_fwd call on the same inputs."""
    lib = load_library()
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_bwd runs on the GPU only; x is on " + str(dev))
    f32 = torch.float32
    nseq = cu_seqlens.numel() - 1 if cu_seqlens is not None else 0
    nstates = nseq if nseq > 0 else b
    _need(x, "x", x.dtype, (b, T, H, P), dev)
    _need(dt, "dt", f32, (b, T, H), dev)
    _need(A, "A", f32, (H,), dev)
    _need(B, "B", x.dtype, (b, T, G, N), dev)
    _need(C, "C", x.dtype, (b, T, G, N), dev)
    _need(D, "D", f32, (H,), dev)
    _need(dt_bias, "dt_bias", f32, (H,), dev)
    _need(initial_states, "initial_states", f32, (nstates, H, P, N), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,), dev)
    _need(dout, "dout", x.dtype, (b, T, H, P), dev)
    _need(dfinal_states, "dfinal_states", f32, (nstates, H, P, N), dev)
    prob = make_problem(b, T, H, P, N, G, chunk_size, x.dtype, nseq, dt_min, dt_max)
    # every token lies in a sequence (cu_seqlens runs from 0 to T), so the
    # library writes every entry of these
    g = {"x": torch.empty_like(x), "dt": torch.empty_like(dt), "A": torch.empty(H, dtype=f32, device=dev),
         "B": torch.empty_like(B), "C": torch.empty_like(C), "D": torch.empty(H, dtype=f32, device=dev),
         "dt_bias": torch.empty(H, dtype=f32, device=dev),
         "initial_states": torch.empty((nstates, H, P, N), dtype=f32, device=dev)}
    need = lib.ssd_bwd_workspace_size(ctypes.byref(prob))
    if workspace is None:
        if after_fwd:
            raise ValueError("after_fwd needs the workspace the forward ran with")
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        fn = lib.ssd_bwd_after_fwd if after_fwd else lib.ssd_bwd
        code = fn(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B),
                           _ptr(C), _ptr(D), _ptr(initial_states), _ptr(cu_seqlens), None,
                           _ptr(dout), _ptr(dfinal_states), _ptr(g["x"]), _ptr(g["dt"]),
                           _ptr(g["A"]), _ptr(g["B"]), _ptr(g["C"]), _ptr(g["D"]),
                           _ptr(g["dt_bias"]), _ptr(g["initial_states"]), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), stream)
    _check(code)
    g["workspace"] = workspace
    return g


def ssd_fwd_seq_idx(x, dt, A, B, C, chunk_size, seq_idx, nseq, **kw):
    """As ssd_fwd for a packed batch described by per-token sequence ids."""
    return _run(x, dt, A, B, C, chunk_size, kw.get("D"), kw.get("dt_bias"),
                kw.get("initial_states"), None, seq_idx, int(nseq), kw.get("dt_min", 0.0),
                kw.get("dt_max", math.inf), kw.get("out"), kw.get("final_states"),
                kw.get("return_final_states", True), kw.get("workspace"),
                kw.get("stages", STAGE_ALL), kw.get("tuning", "config"))


def ssd_fwd_noalloc(x, dt, A, B, C, chunk_size, out, final_states=None, D=None, dt_bias=None,
                    initial_states=None, cu_seqlens=None, seq_idx=None, nseq=0, dt_min=0.0,
                    dt_max=math.inf):
    """The forward through ssd_fwd_noalloc: the library's static scratch array
    is the workspace, and the caller passes the outputs (`out`, and
    `final_states` or None), so nothing is allocated here either.  For a
    packed batch pass cu_seqlens, or seq_idx with nseq."""
    lib = load_library()
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    f32 = torch.float32
    if dev.type != "cuda":
        raise ValueError("ssd_fwd_noalloc runs on the GPU only; x is on " + str(dev))
    if cu_seqlens is not None:
        nseq = cu_seqlens.numel() - 1
    nstates = nseq if nseq > 0 else b
    for t, name, dtp, shape in ((x, "x", x.dtype, (b, T, H, P)), (dt, "dt", f32, (b, T, H)),
                                (A, "A", f32, (H,)), (B, "B", x.dtype, (b, T, G, N)),
                                (C, "C", x.dtype, (b, T, G, N)), (D, "D", f32, (H,)),
                                (dt_bias, "dt_bias", f32, (H,)),
                                (initial_states, "initial_states", f32, (nstates, H, P, N)),
                                (cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,)),
                                (seq_idx, "seq_idx", torch.int32, (T,)),
                                (out, "out", x.dtype, (b, T, H, P)),
                                (final_states, "final_states", f32, (nstates, H, P, N))):
        _need(t, name, dtp, shape, dev)
    prob = make_problem(b, T, H, P, N, G, chunk_size, x.dtype, nseq, dt_min, dt_max)
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        code = lib.ssd_fwd_noalloc(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A),
                                   _ptr(B), _ptr(C), _ptr(D), _ptr(initial_states),
                                   _ptr(cu_seqlens), _ptr(seq_idx), _ptr(out),
                                   _ptr(final_states), stream)
    _check(code)
    return out, final_states


def _norm_problem(y, group_size, eps):
    dtype = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}.get(y.dtype, -1)
    C = y.shape[-1]
    return NormProblemC(int(y.numel() // max(C, 1)), int(C), int(group_size), int(dtype),
                        float(eps))


def gated_norm_fwd(y, z, w, group_size, eps=1e-5, out=None, return_rstd=False):
    """ssd_gated_norm_fwd: rmsnorm(y * silu(z)) * w over groups of group_size
    consecutive channels of the last axis.  y, z: (..., channels) in fp32 or
    bf16 on the GPU, w: (channels,) fp32.  out may be y (in place).  Returns
    out, or (out, rstd) with rstd (rows, channels // group_size) fp32."""
    lib = load_library()
    dev = y.device
    if dev.type != "cuda":
        raise ValueError("gated_norm_fwd runs on the GPU only; y is on " + str(dev))
    C = y.shape[-1]
    _need(y, "y", y.dtype, tuple(y.shape), dev)
    _need(z, "z", y.dtype, tuple(y.shape), dev)
    _need(w, "w", torch.float32, (C,), dev)
    if out is None:
        out = torch.empty_like(y)
    _need(out, "out", y.dtype, tuple(y.shape), dev)
    p = _norm_problem(y, group_size, eps)
    rstd = None
    if return_rstd:
        rstd = torch.empty((p.tokens, C // max(int(group_size), 1)), dtype=torch.float32,
                           device=dev)
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        code = lib.ssd_gated_norm_fwd(ctypes.byref(p), _ptr(y), _ptr(z), _ptr(w), _ptr(out),
                                      _ptr(rstd), stream)
    _check(code)
    return (out, rstd) if return_rstd else out


def gated_norm_bwd(y, z, w, dout, group_size, eps=1e-5, workspace=None):
    """ssd_gated_norm_bwd: (dy, dz, dw) of sum(gated_norm_fwd(y, z, w) * dout)."""
    lib = load_library()
    dev = y.device
    if dev.type != "cuda":
        raise ValueError("gated_norm_bwd runs on the GPU only; y is on " + str(dev))
    C = y.shape[-1]
    for t, name in ((y, "y"), (z, "z"), (dout, "dout")):
        _need(t, name, y.dtype, tuple(y.shape), dev)
    _need(w, "w", torch.float32, (C,), dev)
    p = _norm_problem(y, group_size, eps)
    dy, dz = torch.empty_like(y), torch.empty_like(y)
    dw = torch.empty(C, dtype=torch.float32, device=dev)
    need = int(lib.ssd_gated_norm_bwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        code = lib.ssd_gated_norm_bwd(ctypes.byref(p), _ptr(y), _ptr(z), _ptr(w), _ptr(dout),
                                      _ptr(dy), _ptr(dz), _ptr(dw), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), stream)
    _check(code)
    return dy, dz, dw


def ssd_fwd_gated(x, dt, A, B, C, chunk_size, z, norm_weight, group_size, eps=1e-5, D=None,
                  dt_bias=None, initial_states=None, cu_seqlens=None, out=None,
                  final_states=None, workspace=None):
    """ssd_fwd_gated: the forward, then rmsnorm(y * silu(z)) * norm_weight over
    groups of group_size channels of each token's nheads * headdim channels.
    Returns (out, final_states, workspace) like ssd_fwd, out being the
    normalised output."""
    lib = load_library()
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_fwd_gated runs on the GPU only; x is on " + str(dev))
    f32 = torch.float32
    nseq = cu_seqlens.numel() - 1 if cu_seqlens is not None else 0
    nstates = nseq if nseq > 0 else b
    for t, name, dtp, shape in ((x, "x", x.dtype, (b, T, H, P)), (dt, "dt", f32, (b, T, H)),
                                (A, "A", f32, (H,)), (B, "B", x.dtype, (b, T, G, N)),
                                (C, "C", x.dtype, (b, T, G, N)), (D, "D", f32, (H,)),
                                (dt_bias, "dt_bias", f32, (H,)),
                                (initial_states, "initial_states", f32, (nstates, H, P, N)),
                                (cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,)),
                                (z, "z", x.dtype, (b, T, H, P)),
                                (norm_weight, "norm_weight", f32, (H * P,))):
        _need(t, name, dtp, shape, dev)
    prob = make_problem(b, T, H, P, N, G, chunk_size, x.dtype, nseq)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.dtype, (b, T, H, P), dev)
    if final_states is None:
        final_states = torch.empty((nstates, H, P, N), dtype=f32, device=dev)
    _need(final_states, "final_states", f32, (nstates, H, P, N), dev)
    need = lib.ssd_fwd_workspace_size(ctypes.byref(prob))
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=dev)
    gate = GateC(_ptr(z), _ptr(norm_weight), float(eps), int(group_size))
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        code = lib.ssd_fwd_gated(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A),
                                 _ptr(B), _ptr(C), _ptr(D), _ptr(initial_states), _ptr(cu_seqlens),
                                 None, ctypes.byref(gate), _ptr(out), _ptr(final_states),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 stream)
    _check(code)
    return out, final_states, workspace


def fwd_choices(prob: ProblemC) -> dict:
    """The library's own kernel choices for this problem on the current
    device (ssd_fwd_choices), as a dict of the ssd_tuning_t fields."""
    t = TuningC(0, 0, 0, 0, 0)
    _check(load_library().ssd_fwd_choices(ctypes.byref(prob), ctypes.byref(t)))
    return {k: int(getattr(t, k)) for k, _ in TuningC._fields_}


def make_tuning(choice) -> TuningC:
    """TuningC from None or a dict of scan_kernel / sp_vec / front / sp_blocks /
    fused."""
    t = TuningC(0, 0, 0, 0, 0)
    if choice:
        unknown = set(choice) - {"scan_kernel", "sp_vec", "front", "sp_blocks", "fused"}
        if unknown:
            raise ValueError(f"unknown tuning fields {sorted(unknown)}")
        for k, v in choice.items():
            setattr(t, k, int(v))
    return t


def _run(x, dt, A, B, C, chunk_size, D, dt_bias, init, cu, sidx, nseq, dt_min, dt_max, out,
         final_states, return_final, workspace, stages, tuning="config"):
    lib = load_library()
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    f32 = torch.float32
    _need(x, "x", x.dtype, (b, T, H, P), dev)
    _need(dt, "dt", f32, (b, T, H), dev)
    _need(A, "A", f32, (H,), dev)
    _need(B, "B", x.dtype, (b, T, G, N), dev)
    _need(C, "C", x.dtype, (b, T, G, N), dev)
    _need(D, "D", f32, (H,), dev)
    _need(dt_bias, "dt_bias", f32, (H,), dev)
    nstates = nseq if nseq > 0 else b
    _need(init, "initial_states", f32, (nstates, H, P, N), dev)
    _need(cu, "cu_seqlens", torch.int32, (nseq + 1,), dev)
    _need(sidx, "seq_idx", torch.int32, (T,), dev)
    prob = make_problem(b, T, H, P, N, G, chunk_size, x.dtype, nseq, dt_min, dt_max)
    if isinstance(tuning, str):
        if tuning != "config":
            raise ValueError("tuning is 'config', None or a dict")
        from state_space_model_ssd_amd import tuning as _tuning
        tuning = _tuning.lookup(prob)
    tune = make_tuning(tuning)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.dtype, (b, T, H, P), dev)
    if final_states is None and return_final:
        final_states = torch.empty((nstates, H, P, N), dtype=f32, device=dev)
    _need(final_states, "final_states", f32, (nstates, H, P, N), dev)
    need = lib.ssd_fwd_workspace_size(ctypes.byref(prob))
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        code = lib.ssd_fwd_tuned(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A),
                                 _ptr(B), _ptr(C), _ptr(D), _ptr(init), _ptr(cu), _ptr(sidx),
                                 _ptr(out), _ptr(final_states), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), int(stages),
                                 ctypes.byref(tune), stream)
    _check(code)
    return out, final_states, workspace


def intermediates(workspace: torch.Tensor, prob: ProblemC) -> dict:
    """Views of the stage intermediates inside a workspace (layout of
    ssd_workspace_layout): chunk_table (mc,4), seq_chunks (nstates+1),
    delta/dA_cumsum (mc,H,L), chunk_states (mc,H,P,N) fp32, cb (mc,G,L,L)
    and states_in (mc,H,P,N) in the problem dtype."""
    lay = workspace_layout(prob)
    mc, H, L, G = lay.max_chunks, prob.nheads, prob.chunk_size, prob.ngroups
    P, N = prob.headdim, prob.dstate
    nstates = prob.nseq if prob.nseq > 0 else prob.batch

    def view(off, dtype, shape):
        n = 1
        for s in shape:
            n *= s
        es = torch.tensor([], dtype=dtype).element_size()
        return workspace[off:off + n * es].view(dtype).view(*shape)

    sdt = torch.bfloat16 if prob.dtype == SSD_BF16 else torch.float32
    return dict(
        max_chunks=mc,
        chunk_table=view(lay.chunk_table, torch.int32, (mc, 4)),
        seq_chunks=view(lay.seq_chunks, torch.int32, (nstates + 1,)),
        delta=view(lay.delta, torch.float32, (mc, H, L)),
        dA_cumsum=view(lay.dA_cumsum, torch.float32, (mc, H, L)),
        cb=view(lay.cb, sdt, (mc, G, L, L)),
        chunk_states=view(lay.chunk_states, torch.float32, (mc, H, P, N)),
        states_in=view(lay.states_in, sdt, (mc, H, P, N)),
    )
