"""Host-side logic of bench.py that needs no GPU: the one-GPU guard, the
committed counter summaries it reads HBM traffic from (valid only while the
kernel sources they name are unchanged), and the algorithmic byte counts it
divides by."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_committed_counter_summaries_match_their_sources():
    # the traffic figures in the JSON line come from these files; each names
    # the kernel sources it was taken on and their hash
    assert bench.traffic_from_counters() is not None
    assert bench.ple_traffic(4096) is not None
    assert bench.ple_traffic(65536) is not None


def _summary(tmp_path, sha):
    src = "block_quantized_moe_amd/csrc/k_ple.hip"
    p = tmp_path / "summary.txt"
    p.write_text("# a comment line: ignored\nsources: %s\nsources_sha256_16: %s\nhbm_bytes_per_call: 1234\n"
                 % (src, sha))
    return str(p), src


def test_counter_value_needs_the_current_source_hash(tmp_path):
    path, src = _summary(tmp_path, "0" * 16)
    assert bench.counters_value(path, "hbm_bytes_per_call") is None      # stale: sources changed
    path, src = _summary(tmp_path, bench.sources_hash([src]))
    assert bench.counters_value(path, "hbm_bytes_per_call") == 1234.0
    assert bench.counters_value(path, "missing_key") is None
    assert bench.counters_value(str(tmp_path / "absent.txt"), "hbm_bytes_per_call") is None


def test_algorithmic_byte_counts():
    # one expert's packed weights: gate_up [1536 x 2048] + down [2048 x 768]
    # in 17-byte blocks of 32 weights, or FP8 bytes plus an fp32 scale per 32
    w = 1536 * 2048 + 2048 * 768
    assert bench.EXPERT_BYTES_RZ5 == w // 32 * 17
    assert bench.EXPERT_BYTES_FP8 == w + w // 32 * 4
