"""Host-side checks of bench.py: the one-GPU contract, the algorithmic byte counts it
reports, and how it picks up the recorded HBM traffic of a counter summary."""
import os
import subprocess
import sys

import pytest

import bench
import datagen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_benchmarked_forward():
    # 4 x 8192 x 4096 bf16: x, delta in and y out (6 B per element), B and C per token,
    # A and Dskip, and the final state when it is written
    wl = datagen.workload("mamba1p4b_bf16")
    elems = 4 * 8192 * 4096
    plain = elems * 6 + 2 * 4 * 8192 * 16 * 2 + 4096 * 16 * 4 + 4096 * 4
    assert bench.algorithmic_bytes(wl, False) == plain == 807_682_048
    assert bench.algorithmic_bytes(wl, True) == plain + 4 * 4096 * 16 * 4 == 808_730_624


def test_algorithmic_bytes_of_an_fp32_workload():
    wl = datagen.workload("mamba130m_f32")
    elems = wl.batch * wl.seqlen * wl.dim
    want = elems * 12 + 2 * wl.batch * wl.seqlen * wl.dstate * 4 + wl.dim * wl.dstate * 4 + wl.dim * 4
    assert bench.algorithmic_bytes(wl, False) == want == 304_191_488


def _summary(tmp_path, name, body):
    d = tmp_path / "profiles"
    d.mkdir(exist_ok=True)
    (d / name).write_text(body)
    return str(tmp_path)


def test_recorded_traffic_needs_a_matching_fingerprint(tmp_path, monkeypatch):
    root = _summary(tmp_path, "k.md", "# x\n\ntraffic_bytes: 12345\nkernel_src_sha256_16: 00112233aabbccdd\n")
    monkeypatch.setattr(bench, "ROOT", root)
    monkeypatch.setattr(bench, "source_fingerprint", lambda files: "00112233aabbccdd")
    assert bench.recorded_traffic("k.md", bench.FWD_SOURCES) == 12345
    monkeypatch.setattr(bench, "source_fingerprint", lambda files: "ffffffffffffffff")
    assert bench.recorded_traffic("k.md", bench.FWD_SOURCES) is None
    assert bench.recorded_traffic("missing.md", bench.FWD_SOURCES) is None


def test_recorded_traffic_ignores_a_summary_without_the_fields(tmp_path, monkeypatch):
    root = _summary(tmp_path, "k.md", "# x\n\nno figures here\n")
    monkeypatch.setattr(bench, "ROOT", root)
    monkeypatch.setattr(bench, "source_fingerprint", lambda files: "00112233aabbccdd")
    assert bench.recorded_traffic("k.md", bench.FWD_SOURCES) is None


@pytest.mark.parametrize("name,sources", [
    ("k_lockstep_mamba1p4b_bf16_hbm_counters.md", bench.FWD_SOURCES),
    ("k_lockstep_fused_mamba1p4b_bf16_hbm_counters.md", bench.FWD_SOURCES),
    ("k_step_decode_bf16_hbm_counters.md", bench.FWD_SOURCES),
    ("k_bwd_mamba1p4b_bf16_hbm_counters.md", bench.BWD_SOURCES),
    ("k_ssd_mamba2_bf16_hbm_counters.md", bench.SSD_SOURCES),
    ("k_ssd_step_mamba2_decode_bf16_hbm_counters.md", bench.SSD_SOURCES),
])
def test_every_counter_summary_records_traffic_and_sources(name, sources):
    """Each committed counter summary carries the two lines bench.py reads (whether the
    fingerprint still matches depends on later source edits, so it is not asserted)."""
    import re
    text = open(os.path.join(ROOT, "profiles", name)).read()
    assert re.search(r"^traffic_bytes: \d+$", text, re.M)
    assert re.search(r"^kernel_src_sha256_16: [0-9a-f]{16}$", text, re.M)
