"""Host-side checks of bench.py's bookkeeping (no GPU): the per-launch
algorithmic bytes, the source hash that ties a committed counter summary to
the kernel it measured, the readers of those summaries, and the one-GPU
contract of the command line."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    """A copy of the kernel sources and an empty profiles/ under a temp root."""
    src = os.path.join(ROOT, "state_space_model_ssd_amd", "csrc")
    dst = tmp_path / "state_space_model_ssd_amd" / "csrc"
    shutil.copytree(src, dst)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _write_traffic(root, kernel, tag, nbytes, digest):
    (root / "profiles" / f"{kernel}_{tag}_traffic.md").write_text(
        f"# HBM traffic of {kernel}\n\n| counter | x |\n|---|---|\n\n"
        f"traffic_bytes_per_launch: {nbytes}\nkernel_source_sha256_16: {digest}\n")


def test_hash_ignores_comments_and_blank_space(fake_root):
    h0 = bench.kernel_source_hash("chunk_scan")
    f = fake_root / "state_space_model_ssd_amd" / "csrc" / "ssd_scan_tile.h"
    f.write_text("// a new comment\n" + f.read_text().replace(";\n", ";\n\n", 3) + "\n/* more */\n")
    assert bench.kernel_source_hash("chunk_scan") == h0
    f.write_text(f.read_text() + "\nstatic int extra_code_line;\n")
    assert bench.kernel_source_hash("chunk_scan") != h0


def test_hash_covers_the_kernels_own_headers(fake_root):
    h_scan, h_front = bench.kernel_source_hash("chunk_scan"), bench.kernel_source_hash("front")
    f = fake_root / "state_space_model_ssd_amd" / "csrc" / "ssd_state_tile.h"
    f.write_text(f.read_text() + "\nstatic int extra_code_line;\n")
    assert bench.kernel_source_hash("front") != h_front       # the front includes it
    assert bench.kernel_source_hash("chunk_scan") == h_scan   # chunk_scan does not


def test_traffic_only_while_the_source_matches(fake_root):
    assert bench.measured_traffic("chunk_scan", "w") is None            # no summary
    _write_traffic(fake_root, "chunk_scan", "w", 12345, bench.kernel_source_hash("chunk_scan"))
    assert bench.measured_traffic("chunk_scan", "w") == 12345
    _write_traffic(fake_root, "chunk_scan", "w", 12345, "0000000000000000")
    assert bench.measured_traffic("chunk_scan", "w") is None            # stale summary


def test_counters_only_while_the_source_matches(fake_root):
    h = bench.kernel_source_hash("front")
    (fake_root / "profiles" / "counters_w.md").write_text(
        "# counters\n\n| launch | waves |\n|---|---|\n| front | 1 |\n\n"
        f"mfma_busy front: 0.0890\nlds_conflict_ratio front: 0.119\nl2_hit front: 0.650\n"
        f"kernel_source_sha256_16 front: {h}\n"
        f"mfma_busy chunk_scan: 0.5\nkernel_source_sha256_16 chunk_scan: 0000000000000000\n")
    c = bench.measured_counters("front", "w")
    assert c["mfma_busy"] == pytest.approx(0.089) and c["l2_hit"] == pytest.approx(0.65)
    assert c["lds_conflict_ratio"] == pytest.approx(0.119)
    assert bench.measured_counters("chunk_scan", "w") is None          # stale hash
    assert bench.measured_counters("state_passing", "w") is None       # not listed


def test_committed_summaries_parse():
    # every committed traffic summary carries a byte count and a source hash
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.endswith("_traffic.md")]
    assert names
    for n in names:
        text = open(os.path.join(prof, n)).read()
        assert "traffic_bytes_per_launch:" in text and "kernel_source_sha256_16:" in text, n
        assert "Command" in text or "rocprofv3" in text, n


def test_chunk_scan_bytes_match_the_formula():
    # chunk_scan per (chunk, head): x in and y out, C and CB shared by the
    # group's heads (CB on and below the diagonal), the running sums and
    # steps, the entering state -- for the layer workload, 768 units
    from state_space_model_ssd_amd.inputs import workload_inputs
    prob, _ = workload_inputs(2)
    work = bench.algorithmic_work(prob, 32)
    L, P, N, H, G, e = 256, 64, 128, 24, 1, 2
    tri = L * (L + 1) // 2
    per_tile = 2 * e * L * P + e * L * N * G / H + e * tri * G / H + 8 * L + e * P * N
    assert work["chunk_scan"][0] == pytest.approx(768 * per_tile, rel=1e-9)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
