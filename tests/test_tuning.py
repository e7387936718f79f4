"""Host-side checks of the tuning config (CPU only: no kernel is launched).

The shape key, the config file's round trip and its fallback, the candidate
list, and the C ABI's rejection of out-of-range choices before anything is
enqueued.
"""
import ctypes
import json

import pytest

from state_space_model_ssd_amd import binding, tuning


def _prob(**kw):
    base = dict(batch=2, seqlen=4096, nheads=24, headdim=64, dstate=128, ngroups=1,
                chunk_size=256, dtype=binding.SSD_BF16, nseq=0)
    base.update(kw)
    return binding.make_problem(**base)


def test_shape_key_names_what_the_choices_depend_on():
    k = tuning.shape_key(_prob())
    assert k == "bf16/P64/N128/L256/G1/H24/chunks32/seqs2"
    others = [_prob(nheads=32), _prob(seqlen=8192), _prob(batch=1, seqlen=8192, nseq=3),
              _prob(dtype=binding.SSD_F32, headdim=32, dstate=16, chunk_size=64), _prob(ngroups=8)]
    keys = {tuning.shape_key(p) for p in others}
    assert k not in keys and len(keys) == len(others)


def test_candidates_cover_every_choice():
    bf = tuning.candidates(_prob())
    assert len(bf) == 19 and len({json.dumps(c, sort_keys=True) for c in bf}) == 19
    assert {c["scan_kernel"] for c in bf[:18]} == {1, 2, 3}
    assert {c["sp_vec"] for c in bf[:18]} == {1, 2, 4}
    assert {c["front"] for c in bf[:18]} == {1, 2}
    assert {c["fused"] for c in bf} == {1, 2} and bf[18] == {"fused": 2}
    assert all("fused" not in c for c in tuning.candidates(_prob(chunk_size=64)))
    f32 = tuning.candidates(_prob(dtype=binding.SSD_F32, headdim=32, dstate=16, chunk_size=64))
    assert f32[:3] == [{"sp_vec": 1}, {"sp_vec": 2}, {"sp_vec": 4}]
    # few state elements: the workspace reserves 16 blocks, so every block
    # count is a candidate, with every vector width
    assert len(f32) == 3 + 15
    assert {c["sp_blocks"] for c in f32[3:]} == {1, 2, 4, 8, 16}


def test_workspace_reserves_blocks_only_for_few_state_elements():
    small = binding.workspace_layout(_prob(dtype=binding.SSD_F32, headdim=32, dstate=16,
                                           chunk_size=64))
    assert small.sp_blocks == 16
    nst, H, PN = 2, 24, 32 * 16
    assert small.block_logdecay - small.block_states >= 4 * nst * 16 * H * PN
    assert small.total_bytes - small.block_logdecay >= 4 * nst * 16 * H
    big = binding.workspace_layout(_prob())          # 2 * 24 * 64 * 128 >= 2^18 elements
    assert big.sp_blocks == 1
    assert big.block_logdecay == big.block_states == big.sync


def test_config_round_trip_and_fallback(tmp_path, monkeypatch):
    path = str(tmp_path / "cfg.json")
    p = _prob()
    assert tuning.load_config(path) == {}
    tuning.save_config({tuning.shape_key(p): {"choice": {"scan_kernel": 1, "sp_vec": 4, "front": 1},
                                              "us": 50.0}}, path)
    assert tuning.lookup(p, path) == {"scan_kernel": 1, "sp_vec": 4, "front": 1}
    assert tuning.lookup(_prob(nheads=32), path) is None          # not tuned: library's choice
    monkeypatch.setattr(tuning, "CONFIG_PATH", path)
    assert tuning.lookup(p) == {"scan_kernel": 1, "sp_vec": 4, "front": 1}


def test_malformed_config_rejected(tmp_path):
    path = tmp_path / "bad.json"
    path.write_text(json.dumps({"k": {"choice": {"tile": 3}}}))
    with pytest.raises(ValueError):
        tuning.load_config(str(path))


def test_committed_config_is_well_formed():
    table = tuning.load_config()
    for key, entry in table.items():
        assert key.count("/") == 7
        assert entry["us"] <= entry["default_us"] * 1.05
        assert entry["choice"] in [c["choice"] for c in entry["candidates"]]
        assert entry["choice"] == {} or entry["us"] < entry["default_us"] * (1 - tuning.MARGIN)


def test_make_tuning_rejects_unknown_fields():
    t = binding.make_tuning({"sp_vec": 2})
    assert (t.scan_kernel, t.sp_vec, t.front, t.sp_blocks) == (0, 2, 0, 0)
    with pytest.raises(ValueError):
        binding.make_tuning({"tile": 1})


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails on the host


@pytest.mark.parametrize("dtype,fields", [
    (binding.SSD_BF16, dict(scan_kernel=4)),
    (binding.SSD_BF16, dict(scan_kernel=-1)),
    (binding.SSD_BF16, dict(sp_vec=3)),
    (binding.SSD_BF16, dict(sp_vec=8)),
    (binding.SSD_BF16, dict(front=3)),
    (binding.SSD_BF16, dict(sp_blocks=3)),
    (binding.SSD_BF16, dict(sp_blocks=32)),
    (binding.SSD_BF16, dict(sp_blocks=2)),      # a layer-size problem reserves no blocks
    (binding.SSD_F32, dict(scan_kernel=1)),     # fp32 has one chunk_scan kernel
    (binding.SSD_F32, dict(front=1)),           # and no fused front
    (binding.SSD_BF16, dict(fused=3)),
    (binding.SSD_F32, dict(fused=2)),           # the fused forward is bf16 only
    (binding.SSD_BF16, dict(fused=2, front=2)),
    (binding.SSD_BF16, dict(fused=2, scan_kernel=2)),
    (binding.SSD_BF16, dict(fused=2, sp_vec=2)),
])
def test_out_of_range_tuning_rejected_on_host(dtype, fields):
    lib = binding.load_library()
    p = _prob(dtype=dtype) if dtype == binding.SSD_BF16 else \
        _prob(dtype=dtype, headdim=32, dstate=16, chunk_size=64)
    t = binding.TuningC(0, 0, 0, 0)
    for k, v in fields.items():
        setattr(t, k, v)
    code = lib.ssd_fwd_tuned(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                             None, FAKE, FAKE, FAKE, 1 << 40, binding.STAGE_ALL, ctypes.byref(t),
                             None)
    assert code == binding.SSD_ERR_INVALID_ARG
