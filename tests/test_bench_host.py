"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic work
formulas the rooflines divide by, and the traffic lookup's source check."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_bytes_by_hand():
    # two sequences of 1 and 17 tokens, 8 KV heads of 64: every context
    # token's K and V rows (8 * 64 * 2 B each), q and bf16 out rows of
    # 32 heads, one block id for the first sequence and two for the second,
    # and the two lengths
    kv = (1 + 17) * 2 * 8 * 64 * 2
    q_out = 2 * 32 * 64 * 2 * 2
    ids = (1 + 2) * 4
    assert bench.decode_bytes([1, 17], 2, 32, 8, 64, 2) == kv + q_out + ids + 8
    assert bench.decode_bytes([], 0, 32, 8, 64, 2) == 0


def test_append_and_rope_bytes():
    # one token: K and V rows of 8 heads, read once and stored once
    assert bench.append_bytes(1, 8, 64) == 8 * 64 * 2 * 2 * 2
    # with q (32 heads) read and written, and one cos and one sin row
    assert bench.rope_append_bytes(1, 32, 8, 64) == (32 + 16) * 64 * 2 * 2 + 2 * 32 * 4


def test_prefill_flops_of_the_workload():
    """Q.K^T and P.V over the visible (causal) keys only: the figure the
    prefill roofline divides by for prompts 4 x 512 + 2 x 2048."""
    Hq, D = 32, 64
    flops = sum(Hq * 2 * 2 * D * L * (L + 1) // 2 for L in [512] * 4 + [2048] * 2)
    assert flops == 38679871488
    # brute force on a small prompt: count the visible pairs one by one
    L = 37
    pairs = sum(1 for t in range(L) for j in range(L) if j <= t)
    assert Hq * 2 * 2 * D * pairs == Hq * 2 * 2 * D * L * (L + 1) // 2


def test_traffic_lookup_needs_the_same_kernel_source(tmp_path, monkeypatch):
    rec = {"kernel_source_hash": "abc", "bytes_per_planned_append_decode_call": 123,
           "bytes_per_append_decode_call": 456, "bytes_per_decode_call": 789}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "decode_ragged_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles("abc", "planned") == 123
    assert bench.traffic_from_profiles("abc", "two-calls") == 789
    assert bench.traffic_from_profiles("other", "planned") is None


def test_committed_traffic_matches_the_committed_decode_source():
    """The counter summary under profiles/ was taken on this decode.hip, so
    the benchmark reports it (a stale file would make traffic null)."""
    h = bench.source_hash("decode.hip")
    assert bench.traffic_from_profiles(h, "planned") is not None


def test_dpm_clock_tables_parse():
    """The driver's DPM tables as printed on the GPU host: levels in MHz and
    the one marked current ('S' is the sleep level)."""
    assert bench.parse_dpm("S: 125Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == ([125, 500, 2400], 125)
    assert bench.parse_dpm("0: 500Mhz\n1: 2400Mhz *\n") == ([500, 2400], 2400)
    assert bench.parse_dpm("0: 2000Mhz *\n") == ([2000], 2000)
    assert bench.parse_dpm("") == ([], None)
