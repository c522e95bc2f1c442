"""Host-side checks of bench.py's contract: the one-GPU refusal, the
algorithmic byte count behind its roofline, and the counter figure that is
reported only for the scan sources it was measured on."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _headline_shape():
    # 8 sequences x 262,144 tokens, 4 groups, 64 heads, top-16, FP8, bf16 queries
    table = np.random.default_rng(0).permutation(8 * 2048).reshape(8, 2048).astype(np.int32)
    return SimpleNamespace(index_k_dtype=2, kv_dtype=2, q_dtype=1, seq_lens=np.full(8, 262144),
                           rows=8, num_seqs=8, num_groups=4, max_blocks=2048, top_k=16,
                           num_q_heads=64, block_table=table, num_phys_blocks=8 * 2048)


def test_shared_blocks_count_once_in_the_scan_bytes():
    # requests 0 and 1 share physical blocks 0..2 and have private tails of
    # 10 and 5 tokens (blocks 3, 4); request 2 sees 100 tokens of block 2
    shape = SimpleNamespace(index_k_dtype=2, kv_dtype=2, q_dtype=1,
                            seq_lens=np.array([3 * 128 + 10, 3 * 128 + 5, 2 * 128 + 100]),
                            rows=3, num_seqs=3, num_groups=1, max_blocks=4, top_k=16,
                            num_q_heads=16,
                            block_table=np.array([[0, 1, 2, 3], [0, 1, 2, 4], [0, 1, 2, 0]],
                                                 np.int32),
                            num_phys_blocks=5)
    idx, _, _ = bench.algorithmic_bytes(shape, topk_counts=0)
    small = 3 * 1 * 128 * 2 + (4 + 4 + 3) * 4 + 3 * 1 * 4 * 4
    assert idx == (3 * 128 + 10 + 5) * 128 + small


def test_scan_bytes_of_the_headline_are_the_keys_plus_small_arrays():
    idx, topk, att = bench.algorithmic_bytes(_headline_shape(), topk_counts=8 * 4 * 16 * 128)
    keys = 8 * 262144 * 128              # one FP8 index key of 128 B per token
    queries = 8 * 4 * 128 * 2            # bf16 index query per (row, group)
    table = 8 * 2048 * 4                 # one int32 table entry per block
    scores = 8 * 4 * 2048 * 4            # one fp32 pooled score per (row, group, block)
    assert idx == keys + queries + table + scores == 268771328
    assert topk == scores + 8 * 4 * 16 * 4
    # selected K and V: 256 B per token per group; q in and out; ids and table entries
    assert att == 8 * 4 * 16 * 128 * 256 + 8 * 64 * 128 * 2 * 2 + 8 * 4 * 16 * 8


def test_counter_traffic_is_reported_only_for_its_workload_and_sources(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "index_scan_traffic.json")) as fh:
        t = json.load(fh)
    if t["scan_sources_sha256"] == bench.scan_fingerprint():
        assert bench.measured_traffic(t["workload"]) == t["traffic_bytes_per_launch"]
    assert bench.measured_traffic("nvfp4_512k") is None
    monkeypatch.setattr(bench, "scan_fingerprint", lambda: "0" * 16)
    assert bench.measured_traffic(t["workload"]) is None


def test_share_correlation_applies_to_the_share_workload_only():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "fp8_256k",
                        "--share-corr", "0.9"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "fp8_share64" in r.stderr and r.stdout == ""
