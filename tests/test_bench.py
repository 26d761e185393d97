"""CPU tests of the benchmark's accounting: the FLOP and byte counts it reports
and its refusal of multi-GPU runs."""

import os
import subprocess
import sys

import numpy as np

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _visible_pairs(lengths, causal, window):
    """Visible (query, key) pairs counted from the oracle's mask."""
    return sum(int(oracle.allowed_mask(L, L, causal, window).sum()) for L in lengths)


def test_flops_of_packed_windowed_batches_count_visible_pairs():
    for causal, window in [(True, 0), (True, 7), (False, 5), (False, 0)]:
        lengths = [1, 5, 16, 33]
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        inp = dict(d=64, Hq=3, B=len(lengths), cu_seqlens=cu, causal=causal, window=window,
                   Nq=33, Nk=33)
        assert bench.attention_flops(inp) == 4.0 * 3 * 64 * _visible_pairs(lengths, causal,
                                                                           window)


def test_flops_of_dense_workloads():
    # 4 B Hq Nq Nk d, halved for causal
    gqa = workloads.WORKLOADS["gqa_causal_prefill"]
    inp = dict(gqa, Nq=8192, Nk=8192, cu_seqlens=None)
    assert bench.attention_flops(inp) == 4.0 * 32 * 8192 * 8192 * 128 / 2
    mha = dict(workloads.WORKLOADS["mha_d64"], Nq=2048, Nk=2048, cu_seqlens=None)
    assert bench.attention_flops(mha) == 4.0 * 4 * 16 * 2048 * 2048 * 64


def test_algorithmic_bytes_of_the_gqa_prefill():
    # Q, K, V read once, O and LSE written once (bf16 tensors, fp32 LSE)
    q = np.empty((1, 8192, 32, 128), np.uint16)
    k = np.empty((1, 8192, 8, 128), np.uint16)
    inp = dict(q=q, k=k, dtype="bf16", Hq=32)
    expect = 2 * (2 * q.size + 2 * k.size) + 4 * 8192 * 32
    assert bench.algorithmic_bytes(inp) == expect == 168820736


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
