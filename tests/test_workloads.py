"""Seeded generator: reproducible, page-aligned, oversized pools (CPU only)."""

import numpy as np
import torch

import oracle
from workloads import make_custom, make_workload, poison_unused, PAGE_SIZE


def test_tiny_is_reproducible_and_shaped():
    a, b = make_workload("tiny"), make_workload("tiny")
    assert np.array_equal(a.q_bits, b.q_bits) and np.array_equal(a.kv, b.kv)
    assert np.array_equal(a.req_to_token, b.req_to_token)
    assert a.q_bits.shape == (2, 1, 16, 576) and a.kv.shape == (8, 64, 576)
    assert list(a.seq_lens) == [37, 130]


def test_slots_are_page_aligned_and_pages_disjoint():
    w = make_custom("x", bs=5, heads=1, q_len=1, seq_lens=[1, 63, 64, 65, 300], seed=1)
    owned = []
    for b in range(w.bs):
        row = w.req_to_token[w.req_pool_indices[b]]
        L = int(w.seq_lens[b])
        for j in range(L):
            assert row[j] % PAGE_SIZE == j % PAGE_SIZE
            assert row[j] // PAGE_SIZE == row[(j // PAGE_SIZE) * PAGE_SIZE] // PAGE_SIZE
        owned.extend(w.pages[b].tolist())
    assert len(owned) == len(set(owned))
    assert w.pool_pages == 2 * len(owned)
    assert len(set(w.req_pool_indices.tolist())) == w.bs


def test_fp8_pool_round_trips_within_e4m3_precision():
    w = make_custom("f", bs=1, heads=1, q_len=1, seq_lens=[64], kv_dtype="fp8_e4m3", seed=3)
    assert w.kv.dtype == np.uint8
    vals = torch.from_numpy(w.kv).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.isfinite(vals).all() and np.abs(vals).max() <= 448
    assert np.abs(vals).max() >= 400          # the scale maps max|x| near 448
    assert 0 < w.kv_descale < 1


def test_poison_hits_only_unreachable_slots():
    w = make_custom("p", bs=2, heads=2, q_len=1, seq_lens=[37, 130], seed=4)
    kv = poison_unused(w, "nan")
    o1, l1 = oracle.paged_decode(w.q_bits, w.kv, "bf16", 1.0, w.req_to_token, w.req_pool_indices,
                                 w.seq_lens, w.softmax_scale)
    o2, l2 = oracle.paged_decode(w.q_bits, kv, "bf16", 1.0, w.req_to_token, w.req_pool_indices,
                                 w.seq_lens, w.softmax_scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert (kv == 0x7FC0).sum() == (w.pool_pages * 64 - 37 - 130) * 576
