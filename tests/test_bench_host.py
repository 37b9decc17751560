"""Host logic of bench.py (no GPU): the compulsory byte counts behind the roofline,
the counter-summary reader and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def desc(name):
    s = workloads.spec(name)
    return {k: s[k] for k in workloads.DESC_KEYS}


def test_forward_bytes_ssd_siso():
    # per (token, head): x and y rows of 64 bf16, one fp32 step; per (token, group)
    # with one group per head: B and C rows of 128 bf16
    per_token_head = 64 * 2 + 64 * 2 + 4 + 128 * 2 + 128 * 2
    assert per_token_head == 772
    assert bench.algorithmic_bytes(desc("ssd_siso"), 2, "fwd") == 8 * 2048 * 24 * 772


def test_reverse_bytes_ssd_siso():
    # reads x, dy, B, C and dt, writes dx, dB, dC and ddt
    per_token_head = 3 * 64 * 2 + 2 * 4 + 2 * (2 * 128 * 2)
    assert per_token_head == 1416
    assert bench.algorithmic_bytes(desc("ssd_siso"), 2, "bwd") == 8 * 2048 * 24 * 1416


def test_forward_bytes_hybrid_two_endpoint():
    # rank 2: x and y rows 2 x 64 bf16; dt, beta, gamma fp32; B and C rows 2 x 64 bf16
    per_token_head = 2 * 64 * 2 * 2 + 3 * 4 + 2 * (2 * 64 * 2)
    assert bench.algorithmic_bytes(desc("hybrid"), 2, "fwd") == 4 * 8192 * 32 * per_token_head


def test_decode_bytes_ssd_siso():
    # per slice: the fp32 state read and written, x and y rows, B and C rows, dt
    per_slice = 2 * 128 * 64 * 4 + 2 * 64 * 2 + 2 * 128 * 2 + 4
    assert per_slice == 66308
    d = desc("ssd_siso")
    d["batch"] = 256
    assert bench.decode_bytes(d, 2) == 256 * 24 * per_slice


def test_traffic_needs_matching_kernel_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    f = prof / "hbm_counters_w_m.md"
    f.write_text("kernel_hash: 0000000000000000\n"
                 "traffic_bytes_per_launch ssm_bwd_chunk: 1234\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0000000000000000")
    assert bench.measured_traffic("ssm_bwd_chunk", "w", "m") == 1234
    assert bench.measured_traffic("ssm_fwd_kernel", "w", "m") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "ffffffffffffffff")
    assert bench.measured_traffic("ssm_bwd_chunk", "w", "m") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
