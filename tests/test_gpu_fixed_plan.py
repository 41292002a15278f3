"""GPU: the deterministic fixed-tile plan (mla_plan_fixed_splits).

The plan is integer work and must equal the oracle's rule bit for bit; a
decode over it must match the fp64 oracle within the parity tolerances; and a
request must decode bit for bit the same alone, in another batch, or with
another max_parts (the point of fixed tiles).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_gpu_parity import _np, assert_close, ref
from workloads import make_custom, make_workload, workload_seq_lens, CONFIGS
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_mla_req_amd as m
    return m


def _need(lens, T):
    return int(sum(-(-(-(-int(L) // 64)) // T) for L in lens))


@pytest.mark.parametrize("lens,T,extra", [
    ([37, 130], 1, 0), ([37, 130], 1, 5), ([0], 32, 1), ([1], 32, 0), ([2048, 2049, 4096], 32, 2),
    ([0, 5, 0, 700], 4, 0), ("dsv3", 32, 0), ("long", 32, 0), ("verify", 32, 0),
    ("fp8", 32, 7), ("dsv3", 8, 0), ("rand1000", 16, 3), ("many16384", 32, 0),
])
def test_fixed_plan_bit_exact(mla, lens, T, extra):
    if lens == "rand1000":
        lens = np.random.default_rng(3).integers(0, 20000, size=1000)
    elif lens == "many16384":
        lens = np.random.default_rng(4).integers(1, 200, size=16384)
    elif isinstance(lens, str):
        lens = workload_seq_lens(lens)
    lens = np.asarray(lens, dtype=np.int32)
    max_parts = max(1, _need(lens, T) + extra)
    sl = torch.from_numpy(lens).cuda()
    t, ip = mla.plan_fixed_splits(sl, T, max_parts)
    t_ref, ip_ref = oracle.plan_fixed(lens, T, max_parts)
    assert np.array_equal(_np(t), t_ref)
    assert np.array_equal(_np(ip), ip_ref)
    oracle.check_fixed_plan(_np(t), _np(ip), lens, T)


def test_fixed_plan_overflow_plans_nothing(mla):
    lens = np.array([4096, 100, 70000], dtype=np.int32)
    sl = torch.from_numpy(lens).cuda()
    t, ip = mla.plan_fixed_splits(sl, 4, 5)            # no hint: the device finds 291 > 5
    assert not _np(t).any() and not _np(ip).any()


def _fixed_decode(mla, d, w, bt_width, T, max_parts, idx=None):
    """Block table, fixed plan, decode and merge for the requests `idx` of w
    (all by default), sharing w's pool and req_to_token."""
    q, sl, rpi = d.q, d.seq_lens, d.req_pool_indices
    if idx is not None:
        ii = torch.as_tensor(idx, dtype=torch.long, device="cuda")
        q, sl, rpi = q[ii].contiguous(), sl[ii].contiguous(), rpi[ii].contiguous()
    bt = mla.build_block_table(d.req_to_token, rpi, sl, bt_width)
    plan = mla.plan_fixed_splits(sl, T, max_parts)
    out, lse = mla.decode(q, d.kv, bt, sl, w.softmax_scale, kv_dtype=w.kv_dtype,
                          kv_descale=d.kv_descale, causal=w.causal, plan=plan)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    dict(bs=2, heads=16, q_len=1, lens=[37, 130], T=1, kv="bf16"),
    dict(bs=6, heads=128, q_len=1, lens=[100, 3000, 5000, 64, 2049, 777], T=4, kv="bf16"),
    dict(bs=4, heads=16, q_len=4, lens=[5, 300, 1500, 4100], T=2, kv="bf16"),
    dict(bs=3, heads=128, q_len=1, lens=[129, 2500, 4096], T=8, kv="fp8_e4m3"),
]


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"b{c['bs']}h{c['heads']}n{c['q_len']}T{c['T']}{c['kv']}")
def test_fixed_plan_decode_matches_oracle(mla, c):
    w = make_custom("fixed", bs=c["bs"], heads=c["heads"], q_len=c["q_len"], seq_lens=c["lens"],
                    seed=41, kv_dtype=c["kv"], value_scale=0.5)
    d = to_device(w)
    out, lse = _fixed_decode(mla, d, w, w.bt_width, c["T"], _need(c["lens"], c["T"]) + 2)
    o_ref, lse_ref = ref(w)
    assert_close(_np(out), _np(lse), o_ref, lse_ref)


def test_fixed_plan_batch_invariance_bit_exact(mla):
    """The same requests decoded in the whole batch, in a reordered sub-batch
    and with more plan rows give bit-identical bf16 outputs and fp32 LSEs."""
    lens = [100, 3000, 5000, 64, 2049, 777, 4097, 1]
    w = make_custom("inv", bs=len(lens), heads=128, q_len=1, seq_lens=lens, seed=43,
                    value_scale=0.5)   # short contexts: |o| < 4, so one bf16 rounding stays < 1e-2
    d = to_device(w)
    T = 4
    out_a, lse_a = _fixed_decode(mla, d, w, w.bt_width, T, _need(lens, T))
    idx = [6, 1, 2, 4]
    sub = [lens[i] for i in idx]
    out_b, lse_b = _fixed_decode(mla, d, w, w.bt_width + 3, T, _need(sub, T) + 9, idx=idx)
    ii = torch.as_tensor(idx, device="cuda")
    assert torch.equal(out_b.view(torch.int16), out_a[ii].view(torch.int16))
    assert torch.equal(lse_b, lse_a[ii])
    # and each request alone
    for j, i in enumerate(idx):
        out_c, lse_c = _fixed_decode(mla, d, w, w.bt_width, T, _need([lens[i]], T), idx=[i])
        assert torch.equal(out_c.view(torch.int16), out_a[i:i + 1].view(torch.int16))
        assert torch.equal(lse_c, lse_a[i:i + 1])
    o_ref, lse_ref = ref(w)
    assert_close(_np(out_a), _np(lse_a), o_ref, lse_ref)


@pytest.mark.parametrize("name", ["dsv3", "verify", "fp8"])
def test_fixed_plan_full_size_all_rows(mla, name):
    """Full-size workloads with the page's 2048-token tiles (32 pages), every
    row against the oracle."""
    w = make_workload(name)
    d = to_device(w)
    T = 32
    out, lse = _fixed_decode(mla, d, w, w.bt_width, T, _need(w.seq_lens, T))
    assert_close(_np(out), _np(lse), *ref(w))


def test_captured_append_and_fixed_plan_step_replays(mla):
    """KV append, block table, fixed plan, decode and merge captured in one HIP
    graph (the fixed plan's part count is fixed by the capacity, so the launch
    shapes do not change between replays): every replay, with eager work and
    synchronisation in between, equals the eager step bit for bit, and the
    result matches the oracle's append + decode."""
    from tests.test_gpu_append import _bf16_rows, _dev_u16

    lens = [900, 130, 2000]
    w = make_custom("graph_fixed", bs=3, heads=128, q_len=1, seq_lens=lens, seed=52,
                    value_scale=0.5)
    d = to_device(w)
    rows, T = w.rows_per_req, 4
    max_parts = _need(lens, T) + 3
    slots = np.array([int(w.req_to_token[int(w.req_pool_indices[b]), lens[b] - 1])
                      for b in range(w.bs)], dtype=np.int64)
    k = _bf16_rows(np.random.default_rng(8), w.bs, 0.5)
    loc, kd = torch.from_numpy(slots).cuda(), _dev_u16(k)
    bt = torch.empty((w.bs, w.bt_width), dtype=torch.int32, device="cuda")
    tp = torch.empty((max_parts, 8), dtype=torch.int32, device="cuda")
    ip = torch.empty((w.bs + 1,), dtype=torch.int32, device="cuda")
    po, pl = mla.partial_buffers(w.bs, rows, max_parts)
    out = torch.empty((w.bs, 1, w.heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.bs, 1, w.heads), dtype=torch.float32, device="cuda")

    def step():
        mla.set_kv_buffer(d.kv, loc, kd)
        mla.build_block_table(d.req_to_token, d.req_pool_indices, d.seq_lens, w.bt_width, out=bt)
        mla.plan_fixed_splits(d.seq_lens, T, max_parts, tile_plan=tp, split_indptr=ip)
        mla.mla_decode(d.q, d.kv, bt, d.seq_lens, tp, ip, w.softmax_scale, partial_o=po,
                       partial_lse=pl, out=out, lse=lse)
        mla.merge_states(po, pl, ip, out, lse)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.zero_()
        lse.zero_()
        po.zero_()
        tp.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    kv_ref = oracle.set_kv_buffer(w.kv, slots, k, "bf16")
    o_ref, lse_ref = oracle.paged_decode(w.q_bits, kv_ref, "bf16", 1.0, w.req_to_token,
                                         w.req_pool_indices, w.seq_lens, w.softmax_scale, w.causal)
    assert_close(_np(out), _np(lse), o_ref, lse_ref)


def test_fixed_plan_decode_with_empty_and_one_token_requests(mla):
    """Empty requests (no piece: the merge writes o = 0, lse = -inf), a
    one-token request, and requests ending exactly on a tile boundary."""
    lens = [0, 1, 256, 0, 257, 64]
    w = make_custom("fixed_edge", bs=len(lens), heads=16, q_len=1, seq_lens=lens, seed=44,
                    value_scale=0.5)
    d = to_device(w)
    T = 4                                      # 256 tokens = exactly one tile
    out, lse = _fixed_decode(mla, d, w, w.bt_width, T, _need(lens, T) + 1)
    o, l = _np(out), _np(lse)
    o_ref, lse_ref = ref(w)
    assert_close(o, l, o_ref, lse_ref)
    for b in (0, 3):
        assert np.all(o[b] == 0) and np.all(l[b] == -np.inf)


# ------------------------------------------------------------ packed fixed tiles

@pytest.mark.parametrize("lens,T,parts,rows", [
    ([37, 130], 1, 4, 16), ([0], 32, 3, 128), ([1], 32, 256, 128), ([0, 5, 0, 700], 4, 7, 64),
    ([130, 64, 300, 4000], 8, 5, 128), ("dsv3", 32, 256, 128), ("dsv3", 16, 256, 128),
    ("long", 32, 256, 128), ("verify", 16, 256, 64), ("fp8", 32, 256, 128),
    ("rand1000", 16, 200, 128), ("many16384", 32, 256, 16),
])
def test_fixed_packed_plan_bit_exact(mla, lens, T, parts, rows):
    if lens == "rand1000":
        lens = np.random.default_rng(3).integers(0, 20000, size=1000)
    elif lens == "many16384":
        lens = np.random.default_rng(4).integers(1, 200, size=16384)
    elif isinstance(lens, str):
        lens = workload_seq_lens(lens)
    lens = np.asarray(lens, dtype=np.int32)
    parts = min(parts, mla.device_num_cus())
    sl = torch.from_numpy(lens).cuda()
    t, ip = mla.plan_fixed_packed(sl, rows, T, parts)
    t_ref, ip_ref = oracle.plan_fixed_packed(lens, T, parts, rows)
    assert np.array_equal(_np(ip), ip_ref)
    assert np.array_equal(_np(t), t_ref)
    oracle.check_fixed_packed_plan(_np(t), _np(ip), lens, T, parts, rows)


def _packed_decode(mla, d, w, bt_width, T, parts, idx=None, q8=False):
    q, sl, rpi = d.q, d.seq_lens, d.req_pool_indices
    if idx is not None:
        ii = torch.as_tensor(idx, dtype=torch.long, device="cuda")
        q, sl, rpi = q[ii].contiguous(), sl[ii].contiguous(), rpi[ii].contiguous()
    bt = mla.build_block_table(d.req_to_token, rpi, sl, bt_width)
    plan = mla.plan_fixed_packed(sl, w.rows_per_req, T, parts)
    tiles = int(_np(plan[1])[-1])
    ws = mla.partial_buffers(sl.shape[0], w.rows_per_req, parts, num_slots=tiles)
    kw = {}
    if q8:
        qs = float(np.float32(w.kv_descale))
        kw["q_descale"] = torch.tensor([qs], dtype=torch.float32, device="cuda")
        q = torch.from_numpy(oracle.quantize_q(w.q_bits, qs)).cuda()
        if idx is not None:
            q = q[ii].contiguous()
    out, lse = mla.decode(q, d.kv, bt, sl, w.softmax_scale, kv_dtype=w.kv_dtype,
                          kv_descale=d.kv_descale, causal=w.causal, plan=plan, workspace=ws,
                          **kw)
    torch.cuda.synchronize()
    return out, lse


PACKED_CASES = [
    dict(bs=2, heads=16, q_len=1, lens=[37, 130], T=1, parts=2, kv="bf16"),
    dict(bs=6, heads=128, q_len=1, lens=[100, 3000, 5000, 64, 2049, 777], T=4, parts=7, kv="bf16"),
    dict(bs=4, heads=16, q_len=4, lens=[5, 300, 1500, 4100], T=2, parts=9, kv="bf16"),
    dict(bs=3, heads=128, q_len=1, lens=[129, 2500, 4096], T=8, parts=3, kv="fp8_e4m3"),
    dict(bs=5, heads=20, q_len=1, lens=[64, 1, 900, 3, 2000], T=3, parts=4, kv="bf16"),
]


@pytest.mark.parametrize("c", PACKED_CASES,
                         ids=lambda c: f"b{c['bs']}h{c['heads']}n{c['q_len']}T{c['T']}P{c['parts']}{c['kv']}")
def test_fixed_packed_decode_matches_oracle(mla, c):
    """Parts holding several tiles, of one request or of several: each tile
    a piece of its own, every row at the bar."""
    w = make_custom("packed", bs=c["bs"], heads=c["heads"], q_len=c["q_len"], seq_lens=c["lens"],
                    seed=44, kv_dtype=c["kv"], value_scale=0.5)
    d = to_device(w)
    out, lse = _packed_decode(mla, d, w, w.bt_width, c["T"], c["parts"])
    assert_close(_np(out), _np(lse), *ref(w))


def test_fixed_packed_q8_decode_matches_oracle(mla):
    from tests.test_gpu_q8 import ref_q8
    w = make_custom("packed8", bs=4, heads=128, q_len=1, seq_lens=[700, 64, 3000, 1290], seed=45,
                    kv_dtype="fp8_e4m3")
    d = to_device(w)
    qs = float(np.float32(w.kv_descale))
    out, lse = _packed_decode(mla, d, w, w.bt_width, 5, 6, q8=True)
    assert_close(_np(out), _np(lse), *ref_q8(w, oracle.quantize_q(w.q_bits, qs), qs))


@pytest.mark.parametrize("q8", [False, True])
def test_fixed_packed_batch_invariance_bit_exact(mla, q8):
    """A request gives the same bits packed with others (whatever part its
    tiles land in), in a reordered sub-batch with another part count, and
    alone -- and the same bits as the one-tile-per-part fixed plan."""
    lens = [100, 3000, 5000, 64, 2049, 777, 4097, 1]
    kv = "fp8_e4m3" if q8 else "bf16"
    w = make_custom("pinv", bs=len(lens), heads=128, q_len=1, seq_lens=lens, seed=46,
                    value_scale=0.5, kv_dtype=kv)
    d = to_device(w)
    T = 4
    out_a, lse_a = _packed_decode(mla, d, w, w.bt_width, T, 13, q8=q8)
    idx = [6, 1, 2, 4]
    out_b, lse_b = _packed_decode(mla, d, w, w.bt_width + 3, T, 5, idx=idx, q8=q8)
    ii = torch.as_tensor(idx, device="cuda")
    assert torch.equal(out_b.view(torch.int16), out_a[ii].view(torch.int16))
    assert torch.equal(lse_b, lse_a[ii])
    for i in idx:
        out_c, lse_c = _packed_decode(mla, d, w, w.bt_width, T, 3, idx=[i], q8=q8)
        assert torch.equal(out_c.view(torch.int16), out_a[i:i + 1].view(torch.int16))
        assert torch.equal(lse_c, lse_a[i:i + 1])
    if not q8:
        out_f, lse_f = _fixed_decode(mla, d, w, w.bt_width, T, _need(lens, T))
        assert torch.equal(out_f.view(torch.int16), out_a.view(torch.int16))
        assert torch.equal(lse_f, lse_a)


@pytest.mark.parametrize("name,T", [("dsv3", 16), ("dsv3", 32), ("verify", 16), ("fp8", 32)])
def test_fixed_packed_full_size_all_rows(mla, name, T):
    w = make_workload(name)
    d = to_device(w)
    out, lse = _packed_decode(mla, d, w, w.bt_width, T, mla.device_num_cus())
    assert_close(_np(out), _np(lse), *ref(w))
