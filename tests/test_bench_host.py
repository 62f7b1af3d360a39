"""Host-side arithmetic of bench.py (no GPU): the algorithmic work its
throughput figures divide by, the one-GPU guard, and the gate that keeps a
stale HBM-traffic profile out of the bench line.

The flop counts are pinned to closed forms of the six workload shapes (4·D
flop per visible (query, key) pair per query head; a causal square block
of n rows sees n(n+1)/2 pairs, a 1024-key window clips each row at 1024),
and the visible-pair count to brute force over the mask definition."""

import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _pairs_brute(Sq, Skv, causal, window):
    n = 0
    for i in range(Sq):
        p = i + Skv - Sq                      # bottom-right aligned position of row i
        for k in range(Skv):
            if causal and k > p:
                continue
            if causal and window > 0 and k <= p - window:
                continue
            n += 1
    return n


@pytest.mark.parametrize("Sq,Skv,causal,window", [
    (1, 1, True, 0), (7, 7, True, 0), (5, 19, True, 0), (19, 5, True, 0), (33, 33, True, 4),
    (17, 40, True, 1), (40, 17, False, 0), (64, 64, True, 64), (64, 64, True, 65), (8, 300, True, 50),
])
def test_visible_pairs_match_brute_force(Sq, Skv, causal, window):
    assert bench.visible_pairs(Sq, Skv, causal, window) == _pairs_brute(Sq, Skv, causal, window)


def test_visible_pairs_of_sampled_rows():
    Sq, Skv, w = 11, 14, 3
    per_row = [sum(1 for k in range(Skv) if r + Skv - Sq - w < k <= r + Skv - Sq) for r in range(Sq)]
    rows = [0, 3, 9, 10]
    assert bench.visible_pairs(Sq, Skv, True, w, rows=rows) == sum(per_row[r] for r in rows)


def test_workload_flops_match_closed_forms():
    tri = lambda n: n * (n + 1) // 2
    assert bench.prefill_flops(workloads.C1) == 4 * 64 * 2 * 1 * tri(128) == 4_227_072
    assert bench.prefill_flops(workloads.C2) == 4 * 128 * 32 * 2 * tri(4096) == 274_945_015_808
    win = tri(1024) + (8192 - 1024) * 1024               # rows past the first 1024 see 1024 keys
    assert win == 7_864_832
    assert bench.prefill_flops(workloads.C4A) == 4 * 256 * 16 * win == 128_857_407_488
    assert bench.prefill_flops(workloads.C4B) == 4 * 512 * 16 * tri(8192) == 1_099_645_845_504


def test_decode_bytes_count_kv_once_per_kv_head():
    s = workloads.C5
    kv = 4 * 32768 * 8 * 128 * 2 * 2                        # K and V, bf16, every token of 4 sequences
    q_o = 2 * 4 * 8 * 64 * 128 * 2                          # Q read and O written, bf16
    lse = 4 * 64 * 8 * 4
    meta = 4 * 4 + 4 * (32768 // 16) * 4                   # lengths and the block table
    assert bench.decode_bytes(s, [32768] * 4) == kv + q_o + lse + meta == 537_960_464
    c = workloads.C3                                        # contiguous: no block table
    assert bench.decode_bytes(c, [1024] * 16) == 16 * 1024 * 8 * 128 * 4 + 2 * 16 * 32 * 128 * 2 + 16 * 32 * 4 + 16 * 4


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_traffic_is_read_only_for_the_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("# header\nhbm_bytes_per_launch = 123456\nsource_hash = abc\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic("abc") == 123456
    assert bench.read_traffic("def") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.read_traffic("abc") is None


def test_committed_profiles_name_their_kernel_sources():
    """The traffic and counter summaries under profiles/ each name the hash
    of the kernel sources they were taken on (one line, 16 hex digits); the
    bench line uses a traffic figure only when that hash is the current one
    (test_traffic_is_read_only_for_the_current_sources)."""
    import re

    for name in ("traffic_prefill_c2.txt", "traffic_decode_c3_verify_c5.txt",
                 "mfma_lds_counters_six_workloads.txt"):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        hashes = [l.split("=", 1)[1].strip() for l in text.splitlines() if l.startswith("source_hash")]
        assert len(hashes) == 1 and re.fullmatch(r"[0-9a-f]{16}", hashes[0]), name
