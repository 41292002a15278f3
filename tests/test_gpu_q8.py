"""GPU parity of the fp8-query decode (mla_decode_q8) against the fp64 oracle,
and of every decode kernel on block tables with bad entries.

The fp8 branch of the FlashMLA page's forward_decode quantises q with the
cache scale (scaled_fp8_quant) and hands descale_q, descale_k to the kernel.
The oracle (``oracle.paged_decode_q8``) is attention with the query row
e4m3fn(code) * q_descale over the dequantised cache, in fp64; the codes come
from the oracle's own quantiser, so the decode is checked on its own.
Tolerances as for the other decode tests: max |o - o_ref| <= 1e-2, mean
<= 1e-3, |lse - lse_ref| <= 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_custom, make_workload, poison_unused
from workloads.device import to_device
from tests.test_gpu_parity import SMALL, _np, assert_close, run, ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_mla_req_amd as m
    return m


def _q_scale(w):
    """The page's choice: q_scale = descale_q = the cache's k_scale."""
    return float(np.float32(w.kv_descale))


def run_q8(mla, w, q_scale, num_parts=None, kv=None, table=None):
    """Decode the oracle's codes of w's query on the GPU; returns (o, lse, codes)."""
    d = to_device(w, kv=kv)
    codes = oracle.quantize_q(w.q_bits, q_scale)
    qd = torch.tensor([q_scale], dtype=torch.float32, device="cuda")
    if table is None:
        table = mla.build_block_table(d.req_to_token, d.req_pool_indices, d.seq_lens, w.bt_width,
                                      max_seq_len_hint=int(w.seq_lens.max()))
    plan = mla.plan_splits(d.seq_lens, w.rows_per_req, num_parts, "fp8_e4m3")
    out, lse = mla.decode(torch.from_numpy(codes).cuda(), d.kv, table, d.seq_lens,
                          w.softmax_scale, kv_dtype="fp8_e4m3", kv_descale=d.kv_descale,
                          q_descale=qd, causal=w.causal, plan=plan)
    torch.cuda.synchronize()
    return _np(out), _np(lse), codes


def ref_q8(w, codes, q_scale, rows=None):
    return oracle.paged_decode_q8(codes, q_scale, w.kv, w.kv_dtype, w.kv_descale,
                                  w.req_to_token, w.req_pool_indices, w.seq_lens,
                                  w.softmax_scale, w.causal, rows=rows)


Q8_CASES = [
    dict(bs=3, heads=16, q_len=1, seq_lens=[1, 63, 64]),
    dict(bs=4, heads=16, q_len=1, seq_lens=[65, 127, 128, 129]),
    dict(bs=2, heads=128, q_len=1, seq_lens=[700, 1500]),
    dict(bs=2, heads=16, q_len=4, seq_lens=[4, 300]),        # verify rows (R = 64), causal
    dict(bs=2, heads=32, q_len=4, seq_lens=[5, 267]),        # R = 128, causal tail
    dict(bs=2, heads=128, q_len=2, seq_lens=[90, 600]),      # R = 256: two row blocks
    dict(bs=1, heads=128, q_len=4, seq_lens=[260]),          # R = 512: four row blocks
    dict(bs=5, heads=20, q_len=1, seq_lens=[64, 1, 200, 3, 129]),  # R not a multiple of 32
]


@pytest.mark.parametrize("case", Q8_CASES, ids=lambda c: f"b{c['bs']}h{c['heads']}n{c['q_len']}")
@pytest.mark.parametrize("parts", [1, 5, 64])
def test_q8_small_shapes(mla, case, parts):
    w = make_custom("q8", seed=51, kv_dtype="fp8_e4m3", **SMALL, **case)
    qs = _q_scale(w)
    o, lse, codes = run_q8(mla, w, qs, num_parts=parts)
    assert_close(o, lse, *ref_q8(w, codes, qs))


def test_q8_non_causal_multi_token(mla):
    w = make_custom("q8nc", bs=2, heads=16, q_len=3, seq_lens=[50, 200], seed=52, causal=False,
                    kv_dtype="fp8_e4m3", **SMALL)
    qs = _q_scale(w)
    o, lse, codes = run_q8(mla, w, qs, num_parts=9)
    assert_close(o, lse, *ref_q8(w, codes, qs))


@pytest.mark.parametrize("q_factor", [-1.0, 0.0, 0.25, 3.0, 12.0, 40.0])
def test_q8_query_descale_sign_zero_and_size(mla, q_factor):
    """descale_q enters the scores only: a negative one flips their sign, zero
    weighs every visible key the same.  The codes stay those of the cache
    scale; only the descale handed to the kernel changes.  Large factors
    spread the scores over tens to hundreds of log2 units, so later pages'
    maxima exceed a row's first one by more than the weights' range: those
    pages take an output scale exponent, and jumps past its limit move the
    reference max (and rescale the output)."""
    w = make_custom("q8d", bs=2, heads=64, q_len=2, seq_lens=[100, 333], seed=53,
                    kv_dtype="fp8_e4m3", **SMALL)
    qs = _q_scale(w)
    codes = oracle.quantize_q(w.q_bits, qs)
    qd = float(np.float32(qs * q_factor))
    d = to_device(w)
    bt = mla.build_block_table(d.req_to_token, d.req_pool_indices, d.seq_lens, w.bt_width)
    plan = mla.plan_splits(d.seq_lens, w.rows_per_req, 7, "fp8_e4m3")
    out, lse = mla.decode(torch.from_numpy(codes).cuda(), d.kv, bt, d.seq_lens, w.softmax_scale,
                          kv_dtype="fp8_e4m3", kv_descale=d.kv_descale,
                          q_descale=torch.tensor([qd], dtype=torch.float32, device="cuda"),
                          plan=plan)
    torch.cuda.synchronize()
    assert_close(_np(out), _np(lse), *ref_q8(w, codes, qd))


@pytest.mark.parametrize("kind", ["nan", "big"])
def test_q8_poisoned_unused_slots_are_never_read(mla, kind):
    w = make_custom("q8p", bs=4, heads=32, q_len=2, seq_lens=[1, 70, 129, 250], seed=54,
                    kv_dtype="fp8_e4m3", **SMALL)
    qs = _q_scale(w)
    o1, l1, codes = run_q8(mla, w, qs, num_parts=6)
    o2, l2, _ = run_q8(mla, w, qs, num_parts=6, kv=poison_unused(w, kind))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert_close(o2, l2, *ref_q8(w, codes, qs))


def test_q8_page_permutation_is_bit_exact(mla):
    w = make_custom("q8perm", bs=3, heads=64, q_len=1, seq_lens=[300, 64, 1000], seed=55,
                    kv_dtype="fp8_e4m3", **SMALL)
    qs = _q_scale(w)
    o1, l1, _ = run_q8(mla, w, qs, num_parts=16)
    perm = np.random.default_rng(4).permutation(w.pool_pages)
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    r2t = w.req_to_token.astype(np.int64)
    w.req_to_token = (perm[r2t // 64] * 64 + r2t % 64).astype(np.int32)
    o2, l2, _ = run_q8(mla, w, qs, num_parts=16, kv=kv2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_q8_split_counts_all_match_oracle(mla):
    w = make_custom("q8s", bs=2, heads=128, q_len=1, seq_lens=[3000, 5000], seed=56,
                    kv_dtype="fp8_e4m3")
    qs = _q_scale(w)
    codes = oracle.quantize_q(w.q_bits, qs)
    o_ref, lse_ref = ref_q8(w, codes, qs)
    for parts in (1, 2, 17, 256):
        o, lse, _ = run_q8(mla, w, qs, num_parts=parts)
        assert_close(o, lse, o_ref, lse_ref)


def test_q8_identical_keys_return_that_value_row(mla):
    """Every key the same latent row: all weights are equal whatever the
    scores, so the output is that row's V (times the cache scale) exactly."""
    w = make_custom("q8same", bs=2, heads=16, q_len=1, seq_lens=[200, 77], seed=57,
                    kv_dtype="fp8_e4m3", **SMALL)
    w.kv_descale = 0.125
    for b in range(2):
        row = w.req_to_token[w.req_pool_indices[b]]
        first = w.kv[row[0] // 64, row[0] % 64].copy()
        for j in range(int(w.seq_lens[b])):
            w.kv[row[j] // 64, row[j] % 64] = first
    qs = 0.0625
    o, lse, codes = run_q8(mla, w, qs, num_parts=4)
    assert_close(o, lse, *ref_q8(w, codes, qs))
    for b in range(2):
        slot = int(w.req_to_token[w.req_pool_indices[b], 0])
        v = oracle.e4m3fn_to_f64(w.kv[slot // 64, slot % 64, :512]) * 0.125
        assert np.array_equal(o[b, 0], np.broadcast_to(v, o[b, 0].shape))


def test_q8_matches_the_bf16_query_path_within_the_bar(mla):
    """With a power-of-two scale the dequantised query is exact in bf16, so the
    fp8-query kernel and the bf16-query kernel compute the same attention
    (different accumulation orders only)."""
    w = make_custom("q8vs", bs=2, heads=128, q_len=1, seq_lens=[300, 1000], seed=58,
                    kv_dtype="fp8_e4m3", **SMALL)
    qs = 2.0 ** -6
    o8, l8, codes = run_q8(mla, w, qs, num_parts=9)
    vals = oracle.e4m3fn_to_f64(codes) * qs
    w.q_bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f64(w.q_bits), vals)  # exact
    ob, lb = run(mla, w, num_parts=9)
    assert np.abs(o8 - ob).max() <= 1e-2 and np.abs(l8 - lb).max() <= 1e-3


def test_q8_full_size_all_rows(mla):
    """The fp8 configuration (batch 128, 128 heads, 4096 tokens each) with its
    query quantised, one part per CU, every row."""
    w = make_workload("fp8")
    qs = _q_scale(w)
    o, lse, codes = run_q8(mla, w, qs)
    assert_close(o, lse, *ref_q8(w, codes, qs))


def test_q8_rejects_a_bf16_cache_and_missing_descale(mla):
    w = make_custom("q8x", bs=1, heads=16, q_len=1, seq_lens=[10], seed=59, **SMALL)
    d = to_device(w)
    codes = torch.zeros((1, 1, 16, 576), dtype=torch.uint8, device="cuda")
    bt = mla.build_block_table(d.req_to_token, d.req_pool_indices, d.seq_lens, w.bt_width)
    with pytest.raises(ValueError):
        mla.decode(codes, d.kv, bt, d.seq_lens, w.softmax_scale, kv_dtype="bf16",
                   q_descale=torch.ones(1, device="cuda"))
    w8 = make_custom("q8x", bs=1, heads=16, q_len=1, seq_lens=[10], seed=59,
                     kv_dtype="fp8_e4m3", **SMALL)
    d8 = to_device(w8)
    with pytest.raises(ValueError):
        mla.decode(codes, d8.kv, bt, d8.seq_lens, w.softmax_scale, kv_dtype="fp8_e4m3",
                   kv_descale=d8.kv_descale)


# ------------------------------------------------------------------ bad block-table entries

def _bad_table_case(mla, kv_dtype, q8):
    """Block-table entries that name no page of the pool (-1, -7, past the
    pool) and a table narrower than a request's page count: those pages are
    never read and contribute nothing, so each row is attention over the keys
    of its request's remaining pages (all of a request's pages bad: o = 0,
    lse = -inf)."""
    w = make_custom("bad", bs=4, heads=32, q_len=1, seq_lens=[300, 130, 64, 200], seed=60,
                    kv_dtype=kv_dtype, **SMALL)
    d = to_device(w)
    width = 4  # request 0 needs 5 pages: its page 4 lies past the table
    good = oracle.block_table(w.req_to_token, w.req_pool_indices, w.seq_lens, 5)
    bad = {(0, 1): -1, (1, 2): w.pool_pages + 3, (2, 0): -1, (3, 0): -7}
    table = good[:, :width].copy()
    for (b, p), v in bad.items():
        table[b, p] = v
    tdev = torch.from_numpy(np.ascontiguousarray(table)).cuda()
    qs = _q_scale(w) if q8 else None
    codes = oracle.quantize_q(w.q_bits, qs) if q8 else None
    o_ref = np.zeros((w.bs, 1, 32, 512))
    lse_ref = np.full((w.bs, 1, 32), -np.inf)
    for b in range(w.bs):
        L = int(w.seq_lens[b])
        K = oracle.request_keys(w.kv, w.kv_dtype, w.kv_descale, good[b], L)
        keep = np.array([(j // 64) < width and (b, j // 64) not in bad for j in range(L)])
        Q = (oracle.e4m3fn_to_f64(codes[b, 0]) * qs if q8 else oracle.bf16_to_f64(w.q_bits[b, 0]))
        Kv = K[keep]
        o_ref[b, 0], lse_ref[b, 0] = oracle.attend(Q, Kv, w.softmax_scale,
                                                   np.full(32, Kv.shape[0] - 1))
    for parts in (1, 5, 64):
        if q8:
            o, lse, _ = run_q8(mla, w, qs, num_parts=parts, table=tdev)
        else:
            plan = mla.plan_splits(d.seq_lens, w.rows_per_req, parts, kv_dtype)
            out, l = mla.decode(d.q, d.kv, tdev, d.seq_lens, w.softmax_scale, kv_dtype=kv_dtype,
                                kv_descale=d.kv_descale, plan=plan)
            torch.cuda.synchronize()
            o, lse = _np(out), _np(l)
        assert_close(o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("kv_dtype,q8", [("bf16", False), ("fp8_e4m3", False),
                                         ("fp8_e4m3", True)])
def test_bad_table_entries_contribute_nothing(mla, kv_dtype, q8):
    _bad_table_case(mla, kv_dtype, q8)
