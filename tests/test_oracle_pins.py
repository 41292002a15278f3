"""Pins of the fp64 oracle against things other than itself (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle
from tests import brute_force
from workloads import make_custom, make_workload, SOFTMAX_SCALE


def _oracle(w, **kw):
    return oracle.paged_decode(w.q_bits, w.kv, w.kv_dtype, w.kv_descale, w.req_to_token,
                               w.req_pool_indices, w.seq_lens, w.softmax_scale, w.causal, **kw)


# ---------------------------------------------------------------- dtype decoders

def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.int64).astype(np.uint16)
    bits[:4] = [0x0000, 0x8000, 0x7F80, 0xFF80]  # +-0, +-inf
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3fn_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7F and 0xFF only
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


# ---------------------------------------------------------------- block table

@pytest.mark.parametrize("lens", [[37, 130], [1, 64, 65, 128, 129], [640]])
def test_block_table_maps_every_token_to_its_slot(lens):
    w = make_custom("bt", bs=len(lens), heads=1, q_len=1, seq_lens=lens, seed=len(lens))
    width = w.bt_width + 3
    bt = oracle.block_table(w.req_to_token, w.req_pool_indices, w.seq_lens, width)
    assert bt.dtype == np.int32 and bt.shape == (w.bs, width)
    for b, L in enumerate(lens):
        row = w.req_to_token[w.req_pool_indices[b]]
        npg = -(-L // 64)
        for j in range(L):
            assert bt[b, j // 64] * 64 + j % 64 == row[j]
        assert np.all(bt[b, npg:] == -1)
        assert np.all(bt[b, :npg] >= 0)


def test_block_table_custom_pad_and_narrow_width():
    w = make_custom("bt", bs=2, heads=1, q_len=1, seq_lens=[10, 200], seed=3)
    bt = oracle.block_table(w.req_to_token, w.req_pool_indices, w.seq_lens, 6, pad=7)
    assert np.all(bt[0, 1:] == 7) and np.all(bt[1, 4:] == 7)
    with pytest.raises(ValueError):
        oracle.block_table(w.req_to_token, w.req_pool_indices, w.seq_lens, 3)


# ---------------------------------------------------------------- brute force

def _compare_brute(w, tol=1e-12, requests=None, rows=None):
    o, lse = _oracle(w)
    ref = brute_force.decode(w, requests=requests, rows=rows)
    H = w.heads
    for (b, r), (ob, lb) in ref.items():
        i, h = divmod(r, H)
        np.testing.assert_allclose(o[b, i, h], ob, rtol=0, atol=tol)
        if math.isinf(lb):
            assert lse[b, i, h] == lb
        else:
            assert abs(lse[b, i, h] - lb) <= tol * max(1.0, abs(lb))


def test_oracle_matches_brute_force_tiny():
    w = make_workload("tiny")
    _compare_brute(w)


@pytest.mark.parametrize("case", [
    dict(bs=3, heads=2, q_len=3, seq_lens=[3, 5, 70]),          # causal verify rows
    dict(bs=2, heads=3, q_len=1, seq_lens=[65, 1]),              # page-boundary tail, single token
    dict(bs=1, heads=2, q_len=2, seq_lens=[129]),
    dict(bs=2, heads=2, q_len=1, seq_lens=[64, 100], kv_dtype="fp8_e4m3"),
    dict(bs=1, heads=2, q_len=2, seq_lens=[66], kv_dtype="fp8_e4m3"),
])
def test_oracle_matches_brute_force_micro(case):
    w = make_custom("micro", seed=17, **case)
    _compare_brute(w)


def test_oracle_matches_brute_force_non_causal():
    w = make_custom("nc", bs=1, heads=2, q_len=3, seq_lens=[40], seed=5, causal=False)
    _compare_brute(w)


# ---------------------------------------------------------------- closed forms

def test_single_token_output_is_v0_exactly():
    w = make_custom("one", bs=3, heads=4, q_len=1, seq_lens=[1, 1, 1], seed=9)
    o, lse = _oracle(w)
    for b in range(3):
        slot = int(w.req_to_token[w.req_pool_indices[b], 0])
        k0 = w.kv[slot // 64, slot % 64]
        v0 = (k0[:512].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        kf = (k0.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        for h in range(4):
            assert np.array_equal(o[b, 0, h], v0)
            qf = (w.q_bits[b, 0, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            s = w.softmax_scale * math.fsum(qf * kf)
            assert abs(lse[b, 0, h] - s) <= 1e-12 * max(1, abs(s))


@pytest.mark.parametrize("L", [5, 64, 200])
def test_identical_keys_give_that_row(L):
    w = make_custom("same", bs=1, heads=3, q_len=1, seq_lens=[L], seed=L)
    row = w.req_to_token[w.req_pool_indices[0]]
    first = w.kv[row[0] // 64, row[0] % 64].copy()
    for j in range(L):
        w.kv[row[j] // 64, row[j] % 64] = first
    o, lse = _oracle(w)
    v = (first[:512].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kf = (first.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for h in range(3):
        assert np.array_equal(o[0, 0, h], v)
        qf = (w.q_bits[0, 0, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        s = w.softmax_scale * math.fsum(qf * kf)
        assert abs(lse[0, 0, h] - (s + math.log(L))) <= 1e-11 * max(1, abs(s))


def test_zero_scale_gives_mean_of_visible_values():
    w = make_custom("zero", bs=2, heads=2, q_len=3, seq_lens=[7, 150], seed=4, softmax_scale=0.0)
    o, lse = _oracle(w)
    for b in range(2):
        L = int(w.seq_lens[b])
        row = w.req_to_token[w.req_pool_indices[b]]
        vals = np.stack([(w.kv[row[j] // 64, row[j] % 64, :512].astype(np.uint32) << 16)
                         .view(np.float32).astype(np.float64) for j in range(L)])
        for i in range(3):
            nv = L - 3 + i + 1
            for h in range(2):
                np.testing.assert_allclose(o[b, i, h], vals[:nv].mean(axis=0), rtol=0, atol=1e-14)
                assert abs(lse[b, i, h] - math.log(nv)) <= 1e-14


def test_empty_request_gives_zero_and_neg_inf():
    w = make_custom("empty", bs=2, heads=2, q_len=1, seq_lens=[0, 9], seed=2)
    o, lse = _oracle(w)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------------- invariants

def test_split_then_merge_equals_unsplit():
    w = make_custom("split", bs=1, heads=4, q_len=1, seq_lens=[777], seed=11)
    bt = oracle.block_table(w.req_to_token, w.req_pool_indices, w.seq_lens, w.bt_width)
    K = oracle.request_keys(w.kv, "bf16", 1.0, bt[0], 777)
    Q = oracle.bf16_to_f64(w.q_bits[0].reshape(4, 576))
    full_o, full_l = oracle.attend(Q, K, w.softmax_scale, np.full(4, 776))
    rng = np.random.default_rng(1)
    for k in (1, 2, 5, 13):
        cuts = np.sort(rng.choice(np.arange(1, 777), size=k - 1, replace=False)) if k > 1 else []
        bounds = [0, *cuts, 777]
        po, pl = [], []
        for a, c in zip(bounds[:-1], bounds[1:]):
            oo, ll = oracle.attend(Q, K[a:c], w.softmax_scale, np.full(4, c - a - 1))
            po.append(oo)
            pl.append(ll)
        mo, ml = oracle.merge_states(np.stack(po), np.stack(pl), np.array([0, k]))
        np.testing.assert_allclose(mo[0], full_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml[0], full_l, rtol=1e-13, atol=0)


def test_merge_with_itself_adds_ln2_and_with_empty_is_identity():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((1, 5, 512))
    l = rng.standard_normal((1, 5)) * 3
    mo, ml = oracle.merge_states(np.concatenate([o, o]), np.concatenate([l, l]), np.array([0, 2]))
    np.testing.assert_allclose(mo[0], o[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ml[0], l[0] + math.log(2), rtol=0, atol=1e-14)
    empty_o = rng.standard_normal((1, 5, 512))
    empty_l = np.full((1, 5), -np.inf)
    mo, ml = oracle.merge_states(np.concatenate([empty_o, o]), np.concatenate([empty_l, l]), np.array([0, 2]))
    np.testing.assert_allclose(mo[0], o[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(ml[0], l[0], rtol=0, atol=1e-15)
    mo, ml = oracle.merge_states(np.concatenate([empty_o, empty_o]),
                                 np.concatenate([empty_l, empty_l]), np.array([0, 2]))
    assert np.all(mo == 0) and np.all(ml == -np.inf)


def test_page_permutation_invariance():
    w = make_custom("perm", bs=3, heads=2, q_len=2, seq_lens=[70, 3, 200], seed=21)
    o1, l1 = _oracle(w)
    rng = np.random.default_rng(3)
    perm = rng.permutation(w.pool_pages)          # new page index of old page i
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    r2t = w.req_to_token.astype(np.int64)
    r2t2 = (perm[r2t // 64] * 64 + r2t % 64).astype(np.int32)
    o2, l2 = oracle.paged_decode(w.q_bits, kv2, "bf16", 1.0, r2t2, w.req_pool_indices,
                                 w.seq_lens, w.softmax_scale, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_verify_rows_equal_shorter_decodes():
    n, H = 4, 3
    w = make_custom("ver", bs=2, heads=H, q_len=n, seq_lens=[9, 131], seed=8)
    o, lse = _oracle(w)
    for i in range(n):
        o1, l1 = oracle.paged_decode(w.q_bits[:, i:i + 1].copy(), w.kv, "bf16", 1.0, w.req_to_token,
                                     w.req_pool_indices, w.seq_lens - n + i + 1, w.softmax_scale, True)
        np.testing.assert_allclose(o[:, i], o1[:, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, i], l1[:, 0], rtol=0, atol=1e-13)


def test_sampled_rows_match_full_result():
    w = make_custom("rows", bs=2, heads=4, q_len=2, seq_lens=[50, 90], seed=6)
    o, l = _oracle(w)
    os_, ls_ = _oracle(w, rows={1: np.array([0, 5, 7])})
    for r in (0, 5, 7):
        i, h = divmod(r, 4)
        np.testing.assert_allclose(os_[1, i, h], o[1, i, h], rtol=0, atol=1e-14)
    assert np.isnan(os_[0]).all()
