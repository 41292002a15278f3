"""The debug build's precondition checks (libmla_decode_debug.so, -DMLA_DEBUG)
and the launch log (MLA_TRACE), on the GPU.

The release build trusts two preconditions: a request's tokens sit
page-aligned in the pool (the block table keeps only the page of token 64p),
and the block-table entries a decode reads name pages of the pool.  The debug
build checks both on the device and returns MLA_ERR_PRECONDITION naming the
first violation; where they hold it returns what the release build returns.
"""

import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from workloads import make_custom
from workloads.device import to_device

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_mla_req_amd import _lib
    return _lib, _lib.lib(), _lib.debug_lib()


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _table(lib, d, width):
    bt = torch.full((d.seq_lens.shape[0], width), -1, dtype=torch.int32, device="cuda")
    st = lib.mla_build_block_table(_p(d.req_to_token), d.req_to_token.shape[0],
                                   d.req_to_token.stride(0), _p(d.req_pool_indices),
                                   _p(d.seq_lens), d.seq_lens.shape[0], 64, _p(bt), width, -1, -1,
                                   None)
    torch.cuda.synchronize()
    return st, bt


def _decode(lib, w, d, bt, parts=5):
    import paged_kv_mla_req_amd as mla
    tp, ip = mla.plan_splits(d.seq_lens, w.rows_per_req, parts)
    po, pl = mla.partial_buffers(w.bs, w.rows_per_req, parts)
    out = torch.empty((w.bs, w.q_len, w.heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.bs, w.q_len, w.heads), dtype=torch.float32, device="cuda")
    st = lib.mla_decode(_p(d.q), w.bs, w.q_len, w.heads, _p(d.kv), 0, d.kv.shape[0], _p(bt),
                        bt.shape[1], _p(d.seq_lens), _p(tp), tp.shape[0], _p(ip),
                        w.softmax_scale, 1, None, _p(po), _p(pl), po.shape[0], _p(out), _p(lse),
                        None)
    if st == 0:
        st = lib.mla_merge_states(_p(po), _p(pl), po.shape[0], _p(ip), w.bs, w.rows_per_req, 512,
                                  _p(out), _p(lse), None)
    torch.cuda.synchronize()
    return st, out, lse


def _work():
    w = make_custom("dbg", bs=3, heads=16, q_len=1, seq_lens=[130, 64, 300], seed=70,
                    value_scale=0.5)
    return w, to_device(w)


def test_debug_build_accepts_what_holds_and_matches_release(libs):
    _lib, rel, dbg = libs
    w, d = _work()
    st_r, bt_r = _table(rel, d, w.bt_width)
    st_d, bt_d = _table(dbg, d, w.bt_width)
    assert st_r == 0 and st_d == 0, dbg.mla_last_error_message()
    assert torch.equal(bt_r, bt_d)
    s1, o1, l1 = _decode(rel, w, d, bt_r)
    s2, o2, l2 = _decode(dbg, w, d, bt_d)
    assert s1 == 0 and s2 == 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_debug_build_reports_slots_that_are_not_page_aligned(libs):
    _lib, rel, dbg = libs
    w, _ = _work()
    # move token 5 of request 2 to a slot of another page
    row = int(w.req_pool_indices[2])
    w.req_to_token[row, 5] = (w.req_to_token[row, 5] + 64 * 3) % (w.pool_pages * 64)
    d = to_device(w)
    st_r, _ = _table(rel, d, w.bt_width)
    assert st_r == 0  # the release build trusts the layout
    st_d, _ = _table(dbg, d, w.bt_width)
    assert st_d == _lib.MLA_ERR_PRECONDITION
    msg = dbg.mla_last_error_message().decode()
    assert "request 2, token 5" in msg, msg


def test_debug_build_reports_table_entries_outside_the_pool(libs):
    _lib, rel, dbg = libs
    w, d = _work()
    _, bt = _table(rel, d, w.bt_width)
    good = bt.clone()
    bt[2, 3] = w.pool_pages + 5
    st_r, _, _ = _decode(rel, w, d, bt)
    assert st_r == 0  # the release build masks the page
    st_d, _, _ = _decode(dbg, w, d, bt)
    assert st_d == _lib.MLA_ERR_PRECONDITION
    msg = dbg.mla_last_error_message().decode()
    assert "request 2, page 3" in msg, msg
    # a table narrower than request 2's five pages
    st_n, _, _ = _decode(dbg, w, d, good[:, :4].contiguous())
    assert st_n == _lib.MLA_ERR_PRECONDITION
    assert "request 2, page 4" in dbg.mla_last_error_message().decode()


def test_trace_logs_each_launch(libs):
    """MLA_TRACE=1: one stderr line per launch, naming the entry point and its
    sizes; without it, nothing."""
    code = (
        "import torch, paged_kv_mla_req_amd as mla\n"
        "from workloads import make_custom\n"
        "from workloads.device import to_device\n"
        "w = make_custom('tr', bs=2, heads=16, q_len=1, seq_lens=[37, 130], seed=1)\n"
        "d = to_device(w)\n"
        "bt = mla.build_block_table(d.req_to_token, d.req_pool_indices, d.seq_lens, w.bt_width)\n"
        "mla.decode(d.q, d.kv, bt, d.seq_lens, w.softmax_scale, num_parts=3)\n"
        "torch.cuda.synchronize()\n")
    for on in (True, False):
        env = dict(os.environ, PYTHONPATH=ROOT)
        env.pop("MLA_TRACE", None)
        if on:
            env["MLA_TRACE"] = "1"
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                           cwd=ROOT, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        lines = [l for l in r.stderr.splitlines() if l.startswith("[mla] ")]
        if on:
            names = [l.split()[1] for l in lines]
            assert names == ["mla_build_block_table:", "mla_plan_splits:", "mla_decode:",
                             "mla_merge_states:"], lines
            assert "bs 2 q_len 1 heads 16" in lines[2]
        else:
            assert lines == []
