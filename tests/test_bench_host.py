"""Host-side arithmetic of bench.py (CPU only): the algorithmic byte and flop
counts that the reported roofline figures divide by, checked against closed
forms written from the definitions (each latent row read once per request; 2
flop per multiply-add, 576 for the scores and 512 for the output, per visible
(row, key) pair), and the multi-GPU refusal."""

import subprocess
import sys

import numpy as np

import bench
from workloads import make_custom, make_workload


def test_bytes_tiny_closed_form():
    w = make_workload("tiny")            # lengths 37 and 130, 16 heads, q_len 1, bf16
    b = bench._algorithmic_bytes(w)
    assert b["kv"] == (37 + 130) * 576 * 2
    assert b["q"] == 2 * 16 * 576 * 2 and b["o"] == 2 * 16 * 512 * 2 and b["lse"] == 2 * 16 * 4
    assert b["bt"] == (1 + 3) * 4
    assert b["total"] == b["kv"] + b["q"] + b["o"] + b["lse"] + b["bt"]


def test_flops_decode_and_causal_verify():
    w = make_workload("tiny")
    assert bench._algorithmic_flops(w) == 2 * 1088 * 16 * (37 + 130)
    # q_len 4, causal: row i of a request of length L sees L - 4 + i + 1 keys
    v = make_custom("v", bs=2, heads=16, q_len=4, seq_lens=[10, 3], seed=1, with_values=False)
    vis = sum(max(0, L - 4 + i + 1) for L in (10, 3) for i in range(4))
    assert bench._algorithmic_flops(v) == 2 * 1088 * 16 * vis
    nc = make_custom("nc", bs=1, heads=8, q_len=3, seq_lens=[20], seed=1, causal=False,
                     with_values=False)
    assert bench._algorithmic_flops(nc) == 2 * 1088 * 8 * 3 * 20


def test_fp8_bytes_are_one_per_element():
    w = make_custom("f", bs=1, heads=16, q_len=1, seq_lens=[100], seed=1, kv_dtype="fp8_e4m3",
                    with_values=False)
    assert bench._algorithmic_bytes(w)["kv"] == 100 * 576


def test_q8_query_bytes_and_mfma_floor():
    """An e4m3 query is one byte per value; its matrix floor prices the
    algorithmic flops (1088 per pair: scores and output, both on e4m3
    operands) at the 5 PFLOP/s e4m3 peak."""
    w = make_custom("f", bs=2, heads=16, q_len=1, seq_lens=[100, 64], seed=1,
                    kv_dtype="fp8_e4m3", with_values=False)
    assert bench._algorithmic_bytes(w, q8=True)["q"] == 2 * 16 * 576
    assert bench._algorithmic_bytes(w)["q"] == 2 * 16 * 576 * 2
    pairs = 16 * (100 + 64)
    want = 2 * 1088 * pairs / 5000e12 * 1e3
    assert abs(bench.mfma_floor_ms(w, True) - want) <= 1e-12 * want
    assert abs(bench.mfma_floor_ms(w, False) - 2 * 1088 * pairs / 2500e12 * 1e3) <= 1e-18


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                       text=True, cwd=bench.__file__.rsplit("/", 1)[0])
    assert r.returncode == 2 and "one GPU" in r.stderr
