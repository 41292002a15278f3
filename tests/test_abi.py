"""The C ABI library loads and exports every declared symbol; argument errors
come back as status codes before any launch (CPU only, no GPU calls)."""

import ctypes
import os
import re

import pytest

from paged_kv_mla_req_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    names = _declared()
    assert "mla_decode" in names and "mla_merge_states" in names
    assert "mla_build_block_table" in names and "mla_plan_splits" in names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"
    assert set(_lib.SIGNATURES) == set(names)


def test_version_and_status_strings():
    lib = _lib.lib()
    assert lib.mla_abi_version() == 2
    assert lib.mla_status_string(0) == b"ok"
    assert lib.mla_status_string(2) == b"unsupported"
    assert lib.mla_max_total_splits(64, 256) == 320
    # bf16 partial o (1024 bytes a row) and fp32 lse (4 bytes a row) per slot
    assert lib.mla_workspace_bytes(64, 128, 256) == 320 * 128 * (512 * 2 + 4)
    assert lib.mla_partial_bytes(64, 128, 256) == lib.mla_workspace_bytes(64, 128, 256)
    assert lib.mla_workspace_bytes(-1, 128, 256) == 0


P = ctypes.c_void_p
FAKE = P(0x1000)  # never dereferenced: every case below fails argument checks first


def _decode(**kw):
    a = dict(q=FAKE, bs=2, q_len=1, heads=16, kv=FAKE, dtype=0, pages=8, bt=FAKE, bts=3,
             sl=FAKE, tp=FAKE, parts=4, ip=FAKE, scale=0.07, causal=1, desc=None, po=FAKE,
             pl=FAKE, slots=6, out=FAKE, lse=None)
    a.update(kw)
    return _lib.lib().mla_decode(a["q"], a["bs"], a["q_len"], a["heads"], a["kv"], a["dtype"],
                                 a["pages"], a["bt"], a["bts"], a["sl"], a["tp"], a["parts"],
                                 a["ip"], a["scale"], a["causal"], a["desc"], a["po"], a["pl"],
                                 a["slots"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(out=None), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(bs=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(heads=-1), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=-0.5), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), _lib.MLA_ERR_UNSUPPORTED),
    (dict(dtype=1), _lib.MLA_ERR_INVALID_ARGUMENT),          # fp8 without descale
    (dict(heads=513), _lib.MLA_ERR_UNSUPPORTED),              # rows > 512
    (dict(q_len=5, heads=128), _lib.MLA_ERR_UNSUPPORTED),     # 640 rows
    (dict(slots=5), _lib.MLA_ERR_CAPACITY),                   # < bs + parts
    (dict(parts=65537, slots=70000), _lib.MLA_ERR_CAPACITY),
])
def test_decode_argument_errors(kw, status):
    assert _decode(**kw) == status
    assert _lib.lib().mla_last_error_message().startswith(b"mla_decode")


def _decode_q8(**kw):
    a = dict(q=FAKE, qd=FAKE, bs=2, q_len=1, heads=16, kv=FAKE, pages=8, bt=FAKE, bts=3,
             sl=FAKE, tp=FAKE, parts=4, ip=FAKE, scale=0.07, causal=1, desc=FAKE, po=FAKE,
             pl=FAKE, slots=6, out=FAKE, lse=None)
    a.update(kw)
    return _lib.lib().mla_decode_q8(a["q"], a["qd"], a["bs"], a["q_len"], a["heads"], a["kv"],
                                    a["pages"], a["bt"], a["bts"], a["sl"], a["tp"], a["parts"],
                                    a["ip"], a["scale"], a["causal"], a["desc"], a["po"],
                                    a["pl"], a["slots"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(qd=None), _lib.MLA_ERR_INVALID_ARGUMENT),           # no query descale
    (dict(desc=None), _lib.MLA_ERR_INVALID_ARGUMENT),         # no cache descale
    (dict(bs=0), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), _lib.MLA_ERR_INVALID_ARGUMENT),
    (dict(heads=513), _lib.MLA_ERR_UNSUPPORTED),
    (dict(slots=5), _lib.MLA_ERR_CAPACITY),
])
def test_decode_q8_argument_errors(kw, status):
    assert _decode_q8(**kw) == status
    assert _lib.lib().mla_last_error_message().startswith(b"mla_decode_q8")


def test_block_table_argument_errors():
    lib = _lib.lib()
    f = lib.mla_build_block_table
    assert f(None, 4, 256, FAKE, FAKE, 2, 64, FAKE, 3, -1, -1, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 4, 256, FAKE, FAKE, 0, 64, FAKE, 3, -1, -1, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 4, 256, FAKE, FAKE, 2, 32, FAKE, 3, -1, -1, None) == _lib.MLA_ERR_UNSUPPORTED
    # hint needs 4 pages, table has 3
    assert f(FAKE, 4, 256, FAKE, FAKE, 2, 64, FAKE, 3, -1, 200, None) == _lib.MLA_ERR_CAPACITY
    # hint needs a slot past the end of req_to_token rows
    assert f(FAKE, 4, 128, FAKE, FAKE, 2, 64, FAKE, 8, -1, 200, None) == _lib.MLA_ERR_CAPACITY


def test_plan_and_merge_argument_errors():
    lib = _lib.lib()
    g = lib.mla_plan_splits
    assert g(None, 2, 16, 4, 0, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert g(FAKE, 2, 16, 0, 0, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert g(FAKE, 2, 16, 4, 3, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert g(FAKE, 2, 0, 4, 0, FAKE, FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    assert g(FAKE, 2, 600, 4, 0, FAKE, FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    assert g(FAKE, 20000, 16, 4, 0, FAKE, FAKE, None) == _lib.MLA_ERR_CAPACITY
    assert g(FAKE, 2, 16, 600, 0, FAKE, FAKE, None) == _lib.MLA_ERR_CAPACITY
    assert g(FAKE, 2, 16, 4, 0, P(0x1004), FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    m = lib.mla_merge_states
    # (partial_o, partial_lse, partial_slots, split_indptr, bs, rows, dv, out, lse, stream)
    assert m(None, FAKE, 4, FAKE, 2, 16, 512, FAKE, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert m(FAKE, FAKE, 4, FAKE, 0, 16, 512, FAKE, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert m(FAKE, FAKE, -1, FAKE, 2, 16, 512, FAKE, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert m(FAKE, FAKE, 4, FAKE, 2, 513, 512, FAKE, None, None) == _lib.MLA_ERR_UNSUPPORTED
    assert m(FAKE, FAKE, 4, FAKE, 2, 16, 256, FAKE, None, None) == _lib.MLA_ERR_UNSUPPORTED
    assert m(P(0x1008), FAKE, 4, FAKE, 2, 16, 512, FAKE, None, None) == _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_last_error_message().startswith(b"mla_merge_states")


def test_table_and_plan_argument_errors():
    """The fused call checks both calls' arguments before any launch."""
    f = _lib.lib().mla_build_table_and_plan
    ok = dict(r2t=FAKE, rows=4, stride=256, rpi=FAKE, sl=FAKE, bs=2, page=64, bt=FAKE, bts=3,
              pad=-1, hint=-1, rpr=16, parts=4, dtype=0, tp=FAKE, ip=FAKE)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["r2t"], a["rows"], a["stride"], a["rpi"], a["sl"], a["bs"], a["page"], a["bt"],
                 a["bts"], a["pad"], a["hint"], a["rpr"], a["parts"], a["dtype"], a["tp"],
                 a["ip"], None)

    assert call(r2t=None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(bt=None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(tp=None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(bs=0) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(page=32) == _lib.MLA_ERR_UNSUPPORTED
    assert call(hint=200) == _lib.MLA_ERR_CAPACITY          # needs 4 pages, table has 3
    assert call(rpr=0) == _lib.MLA_ERR_UNSUPPORTED
    assert call(parts=600) == _lib.MLA_ERR_CAPACITY
    assert call(dtype=5) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert _lib.lib().mla_last_error_message().startswith(b"mla_build_table_and_plan")


def test_set_kv_buffer_argument_errors():
    f = _lib.lib().mla_set_kv_buffer
    ok = dict(k=FAKE, stride=576, loc=FAKE, n=4, kv=FAKE, dtype=0, pages=8, scale=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["k"], a["stride"], a["loc"], a["n"], a["kv"], a["dtype"], a["pages"],
                 a["scale"], None)

    assert call(k=None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(loc=None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(kv=None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(n=-1) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(pages=0) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(stride=575) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert call(dtype=1) == _lib.MLA_ERR_INVALID_ARGUMENT     # fp8 without a scale
    assert call(dtype=9) == _lib.MLA_ERR_UNSUPPORTED
    assert call(stride=580) == _lib.MLA_ERR_UNSUPPORTED       # not a multiple of 8
    assert call(k=P(0x1008)) == _lib.MLA_ERR_UNSUPPORTED      # k not 16-byte aligned
    assert _lib.lib().mla_last_error_message().startswith(b"mla_set_kv_buffer")
    assert call(n=0) == _lib.MLA_OK                           # nothing to store: no launch
    assert call(n=0, k=None, loc=None) == _lib.MLA_OK         # nothing is read then
    assert call(n=0, kv=None) == _lib.MLA_ERR_INVALID_ARGUMENT


def test_fixed_plan_argument_errors_and_bound():
    lib = _lib.lib()
    f = lib.mla_plan_fixed_splits
    assert f(None, 2, 32, 8, -1, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 0, 32, 8, -1, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 2, 0, 8, -1, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 2, 32, 0, -1, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 20000, 32, 8, -1, FAKE, FAKE, None) == _lib.MLA_ERR_CAPACITY
    assert f(FAKE, 2, 32, 65537, -1, FAKE, FAKE, None) == _lib.MLA_ERR_CAPACITY
    assert f(FAKE, 2, 32, 8, -1, P(0x1004), FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    # 2 requests of up to 4097 tokens = 65 pages = 3 tiles of 32 pages each: 6 > 5
    assert f(FAKE, 2, 32, 5, 4097, FAKE, FAKE, None) == _lib.MLA_ERR_CAPACITY
    assert lib.mla_last_error_message().startswith(b"mla_plan_fixed_splits")
    b = lib.mla_fixed_split_parts_bound
    assert b(2, 4097, 32) == 6 and b(64, 8192, 32) == 256 and b(3, 0, 32) == 0
    assert b(1, 1, 1) == 1 and b(-1, 5, 32) == -1 and b(2, 5, 0) == -1
    assert b(16384, 2**31 - 1, 1) == 2**31 - 1


def test_fixed_packed_plan_argument_errors():
    lib = _lib.lib()
    f = lib.mla_plan_fixed_packed  # (seq_lens, bs, tile_pages, rows, parts, tile_plan, indptr, stream)
    assert f(None, 2, 32, 128, 8, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 2, 32, 128, 8, None, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 0, 32, 128, 8, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 2, 0, 128, 8, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 2, -3, 128, 8, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 2, 32, 128, 0, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 2, 32, 0, 8, FAKE, FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    assert f(FAKE, 2, 32, 513, 8, FAKE, FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    assert f(FAKE, 2, 32, 128, 8, P(0x1004), FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    assert f(FAKE, 20000, 32, 128, 8, FAKE, FAKE, None) == _lib.MLA_ERR_CAPACITY
    assert f(FAKE, 2, 32, 128, 65537, FAKE, FAKE, None) == _lib.MLA_ERR_CAPACITY
    assert lib.mla_last_error_message().startswith(b"mla_plan_fixed_packed")


def test_quantize_q_argument_errors():
    f = _lib.lib().mla_quantize_q_fp8
    assert f(None, 576, 4, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 576, 4, None, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 576, 4, FAKE, None, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 576, -1, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 500, 4, FAKE, FAKE, None) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 580, 4, FAKE, FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    assert f(P(0x1008), 576, 4, FAKE, FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    assert f(FAKE, 576, 2**31, FAKE, FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    assert _lib.lib().mla_last_error_message().startswith(b"mla_quantize_q_fp8")
    assert f(None, 576, 0, FAKE, FAKE, None) == _lib.MLA_OK


def test_decode_static_rejects_before_any_launch():
    """mla_decode_static checks its sizes and its workspace limit on the host:
    a call whose partial states exceed MLA_STATIC_WORKSPACE_BYTES comes back
    CAPACITY without touching the device."""
    f = _lib.lib().mla_decode_static
    FAKE = ctypes.c_void_p(16)
    args = lambda bs, q_len, heads, parts: (FAKE, bs, q_len, heads, FAKE, 0, 100, FAKE, 8, FAKE,
                                           FAKE, parts, FAKE, 0.1, 1, None, FAKE, None, None)
    assert f(*args(0, 1, 16, 1)) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(*args(2, 1, 16, 0)) == _lib.MLA_ERR_INVALID_ARGUMENT
    assert f(*args(2, 1, 600, 1)) == _lib.MLA_ERR_UNSUPPORTED
    # (512 + 256) slots * 128 rows * 1028 bytes = 101 MB > 64 MiB
    assert f(*args(512, 1, 128, 256)) == _lib.MLA_ERR_CAPACITY
    assert b"static workspace" in _lib.lib().mla_last_error_message()
