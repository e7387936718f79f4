"""Host-side checks of the C ABI (CPU only: no kernel is ever launched).

The library must load without a GPU, export every function include/ssd.h
declares, size its workspace as documented, and reject bad arguments on the
host before anything reaches a device.
"""
import ctypes
import math
import os
import re

import pytest

from state_space_model_ssd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(6):
        assert binding.status_string(code)
    assert binding.status_string(99) == "unknown status"


def _prob(**kw):
    base = dict(batch=2, seqlen=1000, nheads=8, headdim=64, dstate=128, ngroups=2,
                chunk_size=256, dtype=binding.SSD_BF16, nseq=0)
    base.update(kw)
    return binding.make_problem(**base)


def _expected_layout(b, T, H, P, N, G, L, nseq, esize):
    al = lambda v: (v + 255) // 256 * 256
    mc = (min((T + nseq * (L - 1)) // L, T) if nseq else b * ((T + L - 1) // L))
    nst = nseq if nseq else b
    kb = 16 if nst * H * P * N < 2 ** 18 else 0      # blocked state_passing reserve
    sync = 4 * (mc * H + 1)                          # counters of the fused forward
    sizes = [16 * mc, 4 * (nst + 1), 4 * mc * H * L, 4 * mc * H * L, esize * mc * G * L * L,
             4 * mc * H * P * N, esize * mc * H * P * N, 4 * nst * kb * H * P * N, 4 * nst * kb * H,
             sync]
    offs, off = [], 0
    for s in sizes:
        offs.append(off)
        off = al(off + s)
    return mc, offs, off, max(kb, 1)


@pytest.mark.parametrize("shape", [
    dict(batch=2, seqlen=1000, nheads=8, headdim=64, dstate=128, ngroups=2, chunk_size=256),
    dict(batch=1, seqlen=99932, nheads=32, headdim=64, dstate=128, ngroups=4, chunk_size=256, nseq=16),
    dict(batch=3, seqlen=64, nheads=4, headdim=32, dstate=16, ngroups=1, chunk_size=64,
         dtype=binding.SSD_F32),
    dict(batch=1, seqlen=0, nheads=4, headdim=64, dstate=128, ngroups=1, chunk_size=64),
])
def test_workspace_layout_matches_documentation(shape):
    p = _prob(**shape)
    lay = binding.workspace_layout(p)
    es = 2 if p.dtype == binding.SSD_BF16 else 4
    mc, offs, total, kb = _expected_layout(p.batch, p.seqlen, p.nheads, p.headdim, p.dstate,
                                           p.ngroups, p.chunk_size, p.nseq, es)
    assert lay.max_chunks == mc and lay.sp_blocks == kb
    got = [lay.chunk_table, lay.seq_chunks, lay.delta, lay.dA_cumsum, lay.cb, lay.chunk_states,
           lay.states_in, lay.block_states, lay.block_logdecay, lay.sync]
    assert got == offs and lay.total_bytes == total == binding.workspace_size(p)


def test_packed_chunk_bound_covers_every_length_mix():
    # sum ceil(len/L) never exceeds the bound the workspace is sized for
    import random
    rnd = random.Random(0)
    L = 256
    for _ in range(200):
        nseq = rnd.randint(1, 40)
        lens = [rnd.randint(0, 3 * L) for _ in range(nseq)]
        T = sum(lens)
        if T == 0:
            continue
        lay = binding.workspace_layout(_prob(batch=1, seqlen=T, nseq=nseq))
        assert sum((n + L - 1) // L for n in lens) <= lay.max_chunks


def test_supported_configs():
    assert binding.config_supported(binding.SSD_BF16, 64, 128, 256)
    assert binding.config_supported(binding.SSD_F32, 32, 16, 64)
    assert not binding.config_supported(binding.SSD_BF16, 64, 128, 512)
    assert not binding.config_supported(binding.SSD_BF16, 48, 128, 256)
    assert not binding.config_supported(7, 64, 128, 256)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails on the host


def _call(lib, p, ws=FAKE, ws_bytes=1 << 40, cu=None, sidx=None, x=FAKE, stages=binding.STAGE_ALL,
          nulls=()):
    ptr = {k: FAKE for k in ("x", "dt", "dtb", "A", "B", "C", "D", "init", "out", "fin")}
    ptr["x"] = x
    for k in nulls:
        ptr[k] = None
    return lib.ssd_fwd_stages(ctypes.byref(p), ptr["x"], ptr["dt"], ptr["dtb"], ptr["A"], ptr["B"],
                              ptr["C"], ptr["D"], ptr["init"], cu, sidx, ptr["out"], ptr["fin"],
                              ws, ws_bytes, stages, None)


@pytest.mark.parametrize("kw,code", [
    (dict(nheads=6, ngroups=4), binding.SSD_ERR_INVALID_ARG),        # H % G
    (dict(dtype=3), binding.SSD_ERR_INVALID_ARG),
    (dict(batch=0), binding.SSD_ERR_INVALID_ARG),
    (dict(seqlen=-1), binding.SSD_ERR_INVALID_ARG),
    (dict(headdim=0), binding.SSD_ERR_INVALID_ARG),
    (dict(nseq=4), binding.SSD_ERR_INVALID_ARG),                      # packed needs batch 1
    (dict(chunk_size=512), binding.SSD_ERR_UNSUPPORTED),
    (dict(headdim=48), binding.SSD_ERR_UNSUPPORTED),
    (dict(nheads=70000, ngroups=1), binding.SSD_ERR_UNSUPPORTED),
    (dict(batch=1 << 20, seqlen=1 << 20), binding.SSD_ERR_UNSUPPORTED),
])
def test_invalid_problems_rejected(lib, kw, code):
    p = _prob(**kw)
    assert _call(lib, p) == code
    assert lib.ssd_fwd_workspace_size(ctypes.byref(p)) == 0


def test_clamp_range_checked(lib):
    p = _prob()
    p.dt_min, p.dt_max = 1.0, 0.5
    assert _call(lib, p) == binding.SSD_ERR_INVALID_ARG
    p.dt_min, p.dt_max = float("nan"), 1.0
    assert _call(lib, p) == binding.SSD_ERR_INVALID_ARG


def test_packing_arguments_checked(lib):
    packed = _prob(batch=1, nseq=3)
    assert _call(lib, packed) == binding.SSD_ERR_INVALID_ARG                   # neither
    assert _call(lib, packed, cu=FAKE, sidx=FAKE) == binding.SSD_ERR_INVALID_ARG   # both
    assert _call(lib, _prob(), cu=FAKE) == binding.SSD_ERR_INVALID_ARG          # unpacked + cu
    # no tokens: a packed batch of empty sequences may name neither (checked
    # up to the workspace, the first check that needs no device)
    empty = _prob(batch=1, seqlen=0, nseq=3)
    assert _call(lib, empty, ws=None) == binding.SSD_ERR_WORKSPACE


@pytest.mark.parametrize("null", ["x", "dt", "A", "B", "C", "out"])
def test_required_pointers_checked(lib, null):
    assert _call(lib, _prob(), nulls=(null,)) == binding.SSD_ERR_INVALID_ARG


def test_workspace_checked(lib):
    p = _prob()
    need = lib.ssd_fwd_workspace_size(ctypes.byref(p))
    assert _call(lib, p, ws=None) == binding.SSD_ERR_WORKSPACE
    assert _call(lib, p, ws_bytes=need - 1) == binding.SSD_ERR_WORKSPACE
    assert _call(lib, p, ws=ctypes.c_void_p(0x1008)) == binding.SSD_ERR_WORKSPACE   # misaligned


def test_stage_mask_checked(lib):
    assert _call(lib, _prob(), stages=1 << 7) == binding.SSD_ERR_INVALID_ARG


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError):
        binding.ssd_fwd(x, torch.zeros(1, 4, 2), torch.zeros(2), torch.zeros(1, 4, 1, 128),
                        torch.zeros(1, 4, 1, 128), 64)


def test_missing_library_fails_loudly(tmp_path):
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="no fallback"):
            binding.load_library(str(tmp_path / "absent.so"))
    finally:
        binding._lib = saved


def test_choices_query_checked_on_host(lib):
    t = binding.TuningC(0, 0, 0, 0)
    assert lib.ssd_fwd_choices(ctypes.byref(_prob(nheads=7, ngroups=2)), ctypes.byref(t)) == \
        binding.SSD_ERR_INVALID_ARG
    assert lib.ssd_fwd_choices(ctypes.byref(_prob(headdim=48)), ctypes.byref(t)) == \
        binding.SSD_ERR_UNSUPPORTED
    assert lib.ssd_fwd_choices(ctypes.byref(_prob()), None) == binding.SSD_ERR_INVALID_ARG
    import torch
    if not torch.cuda.is_available():
        # the choices depend on the device, so without one the query fails
        assert lib.ssd_fwd_choices(ctypes.byref(_prob()), ctypes.byref(t)) == binding.SSD_ERR_HIP


@pytest.mark.parametrize("kw,code", [
    (dict(channels=96, group_size=32), binding.SSD_OK),                 # 4 vectors per group
    (dict(channels=1536, group_size=1536), binding.SSD_OK),             # 3 chunks of 64 vectors
    (dict(channels=100, group_size=30), binding.SSD_ERR_INVALID_ARG),   # does not divide
    (dict(channels=96, group_size=12), binding.SSD_ERR_UNSUPPORTED),    # not whole vectors
    (dict(channels=96, group_size=48), binding.SSD_ERR_UNSUPPORTED),    # 6 vectors: not 2^k
    (dict(channels=16384, group_size=64), binding.SSD_ERR_UNSUPPORTED), # too wide a row
    (dict(eps=-1.0), binding.SSD_ERR_INVALID_ARG),
    (dict(tokens=-1), binding.SSD_ERR_INVALID_ARG),
    (dict(dtype=5), binding.SSD_ERR_INVALID_ARG),
])
def test_norm_problems_checked_on_host(lib, kw, code):
    base = dict(tokens=10, channels=128, group_size=64, dtype=binding.SSD_BF16, eps=1e-5)
    base.update(kw)
    p = binding.NormProblemC(base["tokens"], base["channels"], base["group_size"], base["dtype"],
                             base["eps"])
    size = lib.ssd_gated_norm_bwd_workspace_size(ctypes.byref(p))
    assert (size > 0) == (code == binding.SSD_OK)
    if code != binding.SSD_OK:
        assert lib.ssd_gated_norm_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None) == code
    else:
        # required pointers, then the workspace, are checked before any launch
        assert lib.ssd_gated_norm_fwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, None, None) == \
            binding.SSD_ERR_INVALID_ARG
        assert lib.ssd_gated_norm_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, size - 1, None) == binding.SSD_ERR_WORKSPACE
