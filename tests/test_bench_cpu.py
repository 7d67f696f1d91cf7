"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the byte
accounting its roofline figures rest on, and the counter-table lookup."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)


def test_algorithmic_bytes_per_expert():
    b = _bench()
    # bf16: w13 [1024][2048] and w2 [2048][512], two bytes each.
    assert b.EXPERT_BYTES["bf16"] == (4_194_304, 2_097_152)
    # NVFP4: half a byte per code, one E4M3 byte per 16 codes, one fp32 tensor scale.
    assert b.EXPERT_BYTES["nvfp4"] == (1_048_576 + 131_072 + 4, 524_288 + 65_536 + 4)
    assert b.ROUTER_BYTES == 1_048_576


def test_kernel_names_follow_the_launch_counts():
    b = _bench()
    assert b.kernel_names(3, False) == ["route", "gateup", "down"]
    assert b.kernel_names(5, False)[2] == "gateup"
    assert b.kernel_names(6, False)[0] == "norm"
    assert b.kernel_names(2, True) == ["gateup", "down"]


def test_counter_rows_are_used_only_for_matching_sources(tmp_path, monkeypatch):
    b = _bench()
    table = tmp_path / "t.md"
    table.write_text("| workload | kernel | sources sha | FETCH KiB | WRITE KiB | bytes |\n"
                     "|---|---|---|---|---|---|\n"
                     "| decode_t8 | gateup | abcdef0123456789 | 1.0 | 2.0 | 12345 |\n")
    monkeypatch.setattr(b, "TRAFFIC_TABLE", str(table))
    assert b.measured_traffic("decode_t8", "gateup", "abcdef0123456789") == 12345
    assert b.measured_traffic("decode_t8", "gateup", "0000000000000000") is None
    assert b.measured_traffic("decode_t8", "down", "abcdef0123456789") is None
    sha = b.kernel_sources_sha("decode.hip")
    assert len(sha) == 16 and int(sha, 16) >= 0
