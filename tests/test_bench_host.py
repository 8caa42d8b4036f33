"""Host-side pieces of bench.py: the one-GPU guard, launch statistics, the
gate that keeps a stale traffic profile out of the JSON line, the coded-size
accounting of both coders, and the CPU-baseline record (no GPU needed)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_launch_percentiles():
    pct = bench.launch_pct([1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0, 9.0, 10.0, 11.0])
    assert pct == {"launch_ms_p10": 2.0, "launch_ms_p50": 6.0, "launch_ms_p90": 10.0}


def test_traffic_profile_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_src_sha", lambda: "abc123")
    (prof / "traffic_w_m.txt").write_text("# header: with a colon\nconfig: C=1 W=2\nkernel_src_sha: abc123\n"
                                          "hbm_bytes_per_launch: 1234567\n")
    assert bench.read_traffic("w_m", "C=1 W=2") == 1234567.0
    assert bench.read_traffic("w_m", "C=1 W=4") is None          # taken on another configuration
    (prof / "traffic_w_m.txt").write_text("config: C=1 W=2\nkernel_src_sha: other\nhbm_bytes_per_launch: 1234567\n")
    assert bench.read_traffic("w_m", "C=1 W=2") is None          # taken on other kernel sources
    assert bench.read_traffic("missing", "C=1 W=2") is None


def test_committed_traffic_summary_matches_the_default_command():
    """The committed summary applies to the configuration bench.py runs by
    default (it is null in the JSON line otherwise)."""
    import argparse

    a = argparse.Namespace(refill_steps=2, refill_ahead=1)
    text = open(os.path.join(ROOT, "profiles", "traffic_tensor_4096_bf16.txt")).read()
    assert f"config: {bench.traffic_config(8192, 32, a, 16)}" in text


def test_kernel_source_hash_covers_every_kernel_source():
    for p in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, p)), p
    assert len(bench.kernel_src_sha()) == 16


@pytest.fixture(scope="module")
def lib():
    import entropy_coded_weight_canonical_amd as ent

    try:
        ent.load()
    except ent.LibraryNotBuilt:
        pytest.skip("library not built")
    return ent


def test_coded_size_accounting(lib):
    """in_bytes counts the stream and the chunk offsets, as the roofline's
    algorithmic bytes do; bits per weight follow from it."""
    rng = np.random.default_rng(5)
    q = np.clip(np.rint(rng.laplace(8, 1.2, size=(64, 512))), 0, 15).astype(np.uint8)
    c = bench.Coded(q, np.float32(0.01), 8, "unsigned", 4, 12, 4096, 32, 64, 512, 2, ahead=True)
    assert c.n_chunks == 8
    assert c.in_bytes == 4 * c.words.size + 8 * 9
    assert c.coded_bits_per_weight == pytest.approx(8.0 * c.in_bytes / q.size)
    r = bench.RansCoded(q, np.float32(0.01), 8, 4, 4096, 32, 64, 512)
    assert r.n_chunks == 8
    assert r.in_bytes == 2 * r.units.size + 8 * 9
    # each chunk carries at least its 32 lane states (two units each)
    assert r.units.size >= 8 * 64


def test_cpu_baseline_record(lib):
    rng = np.random.default_rng(6)
    q = np.clip(np.rint(rng.laplace(8, 1.0, size=(32, 256))), 0, 15).astype(np.uint8)
    c = bench.Coded(q, np.float32(0.02), 8, "unsigned", 4, 12, 1024, 32, 32, 256, 2, ahead=True)
    rec = bench.cpu_baseline(c, budget_s=0.2, single_budget_s=0.1)
    assert rec["kind"] == "oracle" and rec["unit"] == "Gsym/s"
    assert rec["value"] > 0 and rec["single_thread_value"] > 0 and rec["decode_only_value"] > 0
    assert rec["cores"] >= 1 and rec["nproc"] >= 1 and isinstance(rec["cpu_model"], str)


def test_profiles_apply_only_to_their_sources_and_configuration(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_src_sha", lambda: "abc123")
    (prof / "counters_k.txt").write_text("config: cfg A\nkernel_src_sha: abc123\n"
                                         "valu_lane_ops_per_symbol: 8.0   # a comment\n")
    r = bench.gemv_roofline("k", "cfg A", 2e12, 1e9, 1.0)
    assert r["bound"] == "alu" and r["valu_lane_ops_per_symbol"] == 8.0
    assert r["achieved"] == pytest.approx(16000.0) and r["frac"] == pytest.approx(16000.0 / r["peak"], rel=1e-3)
    assert r["peak"] == pytest.approx(256 * 4 * 16 * 2.4)
    assert r["hbm"]["achieved"] == pytest.approx(1000.0) and r["hbm"]["frac"] == pytest.approx(0.125)
    r = bench.gemv_roofline("k", "cfg B", 2e12, 1e9, 1.0)       # taken on another configuration
    assert r["achieved"] is None and r["frac"] is None and r["hbm"]["frac"] == pytest.approx(0.125)


def test_workload_table_matches_the_stated_configurations():
    """configs[0..4] in order: sizes and code widths as stated; GEMV chunks
    hold whole rows."""
    w = bench.WORKLOADS
    assert [w[k]["config"] for k in ("tensor_2048", "tensor_4096", "smollm_stack", "phi3_stack", "mistral_stack")] \
        == [1, 2, 3, 4, 5]
    assert (w["tensor_2048"]["bits"], w["tensor_2048"]["scheme"], w["tensor_2048"]["chunk"]) == (8, "asymmetric", 4096)
    assert (w["tensor_4096"]["bits"], w["tensor_4096"]["scheme"], w["tensor_4096"]["chunk"],
            w["tensor_4096"]["lanes"]) == (4, "unsigned", 8192, 32)
    assert w["smollm_stack"]["bits"] == 8 and w["phi3_stack"]["bits"] == 4 and w["mistral_stack"]["bits"] == 4
    # no lane count is stated for configs[0] and [2]: 64, the faster layout
    assert w["tensor_2048"]["lanes"] == 64 and w["smollm_stack"]["lanes"] == 64
    for cols in (1024, 3072, 4096, 8192, 14336):
        c = bench.gemv_chunk(cols, 4096)
        assert c % cols == 0 and c >= cols
