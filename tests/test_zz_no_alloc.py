"""mla_decode_static (the allocation-free decode + merge) against mla_decode
followed by mla_merge_states on the same inputs and plan: identical outputs,
bit for bit, on two calls in a row (the second smaller), and the workspace
limit."""

import numpy as np
import pytest
import torch

from workloads import make_custom, make_workload
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_mla_req_amd as m
    return m


def _both(mla, w, num_parts=None):
    d = to_device(w)
    rows = w.rows_per_req
    parts = num_parts or mla.device_num_cus()
    bt, tp, ip = mla.build_table_and_plan(d.req_to_token, d.req_pool_indices, d.seq_lens,
                                          w.bt_width, rows, parts)
    shape = (w.bs, w.q_len, w.heads, 512)
    kw = dict(kv_dtype=w.kv_dtype, kv_descale=d.kv_descale, causal=w.causal)
    # the existing path: caller workspace, decode, then merge
    po, pl = mla.partial_buffers(w.bs, rows, tp.shape[0])
    out_ref = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse_ref = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    mla.mla_decode(d.q, d.kv, bt, d.seq_lens, tp, ip, w.softmax_scale, partial_o=po,
                   partial_lse=pl, out=out_ref, lse=lse_ref, **kw)
    mla.merge_states(po, pl, ip, out_ref, lse_ref)
    # the static-workspace path, into poisoned outputs
    out = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode_static(d.q, d.kv, bt, d.seq_lens, tp, ip, w.softmax_scale, out=out, lse=lse,
                          **kw)
    torch.cuda.synchronize()
    return out_ref, lse_ref, out, lse


def _assert_same(out_ref, lse_ref, out, lse):
    assert torch.isfinite(out.float()).all()
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
    a, b = lse.cpu().numpy(), lse_ref.cpu().numpy()
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    assert np.array_equal(a.view(np.int32), b.view(np.int32))


def test_static_workspace_matches_the_workspace_path_twice(mla):
    """A full-size headline batch, then a smaller one (fewer requests, fewer
    parts) on the same array: both bit-identical to decode + merge."""
    print("[static] dsv3 full size", flush=True)
    _assert_same(*_both(mla, make_workload("dsv3")))
    print("[static] small ragged batch, 7 parts", flush=True)
    w = make_custom("st", bs=5, heads=16, q_len=2, seq_lens=[1, 70, 300, 0, 129], seed=71)
    _assert_same(*_both(mla, w, num_parts=7))


def test_static_workspace_fp8_cache(mla):
    print("[static] fp8 cache small", flush=True)
    w = make_custom("st8", bs=3, heads=128, q_len=1, seq_lens=[500, 64, 1000], seed=72,
                    kv_dtype="fp8_e4m3")
    _assert_same(*_both(mla, w, num_parts=11))


def test_static_workspace_limit(mla):
    """Partial states past the array's 64 MiB are refused, nothing launched."""
    w = make_custom("stbig", bs=520, heads=128, q_len=1, seq_lens=[64] * 520, seed=73,
                    with_values=False)
    d = to_device(w)
    out = torch.empty((520, 1, 128, 512), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((520, 1, 128, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((4, 64, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((520, 1), dtype=torch.int32, device="cuda")
    tp = torch.zeros((256, 8), dtype=torch.int32, device="cuda")
    ip = torch.zeros((521,), dtype=torch.int32, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_static(q, kv, bt, d.seq_lens, tp, ip, 0.1, out=out)
    assert e.value.status == mla._lib.MLA_ERR_CAPACITY
