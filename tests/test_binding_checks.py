"""The Python binding's argument checks, on the CPU: every shape, size or
dtype mismatch raises before the library is reached (the C ABI is handed only
pointers and the sizes the binding derives, so a mismatched buffer would
otherwise be written past its end on the device).

The tests stand CPU tensors in for device tensors (the binding's device test
is patched to accept them) and replace the library with a stub that raises
``Reached``: a correct call ends in ``Reached``, a mismatched one in
ValueError/TypeError without reaching it."""

import pytest
import torch

import paged_kv_mla_req_amd as mla
from paged_kv_mla_req_amd import _lib


class Reached(Exception):
    pass


@pytest.fixture
def m(monkeypatch):
    monkeypatch.setattr(mla, "_on_gpu", lambda t: True)

    def stub():
        raise Reached()

    monkeypatch.setattr(_lib, "lib", stub)
    return mla


BS, QL, H, PAGES, W, PARTS = 3, 2, 16, 10, 4, 5
R = QL * H


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def decode_args(**over):
    a = dict(q=bf16(BS, QL, H, 576), kv_cache=bf16(PAGES, 64, 576), block_table=i32(BS, W),
             seq_lens=i32(BS), tile_plan=i32(PARTS, 8), split_indptr=i32(BS + 1),
             partial_o=bf16(BS + PARTS, R, 512), partial_lse=f32(BS + PARTS, R),
             out=bf16(BS, QL, H, 512), lse=f32(BS, QL, H))
    a.update(over)
    return a


def call_decode(m, a):
    m.mla_decode(a["q"], a["kv_cache"], a["block_table"], a["seq_lens"], a["tile_plan"],
                 a["split_indptr"], 0.1, partial_o=a["partial_o"], partial_lse=a["partial_lse"],
                 out=a["out"], lse=a["lse"])


def test_decode_correct_shapes_reach_the_library(m):
    with pytest.raises(Reached):
        call_decode(m, decode_args())


@pytest.mark.parametrize("over", [
    dict(out=bf16(BS, 1, H, 512)),                  # q_len 2 into a q_len-1 output
    dict(out=bf16(BS, QL, H, 256)),
    dict(lse=f32(BS, QL, H + 1)),
    dict(partial_o=bf16(BS + PARTS, R - 1, 512)),
    dict(partial_lse=f32(BS + PARTS + 1, R)),
    dict(block_table=i32(BS - 1, W)),
    dict(seq_lens=i32(BS + 1)),
    dict(split_indptr=i32(BS)),
    dict(tile_plan=i32(PARTS, 7)),
    dict(kv_cache=bf16(PAGES, 32, 576)),
    dict(q=bf16(BS, QL, H, 512)),
    dict(q=torch.zeros((BS, QL, H, 576), dtype=torch.float16)),
    dict(block_table=torch.zeros((BS, W), dtype=torch.int64)),
])
def test_decode_mismatches_raise_before_the_library(m, over):
    with pytest.raises((ValueError, TypeError)):
        call_decode(m, decode_args(**over))


def test_decode_q8_checks(m):
    a = decode_args(q=torch.zeros((BS, QL, H, 576), dtype=torch.uint8),
                    kv_cache=torch.zeros((PAGES, 64, 576), dtype=torch.uint8))
    kw = dict(partial_o=a["partial_o"], partial_lse=a["partial_lse"], out=a["out"], lse=a["lse"])
    args = (a["kv_cache"], a["block_table"], a["seq_lens"], a["tile_plan"], a["split_indptr"], 0.1)
    with pytest.raises(Reached):
        m.mla_decode_q8(a["q"], f32(1), *args, kv_descale=f32(1), **kw)
    with pytest.raises(ValueError):                      # no query descale
        m.mla_decode_q8(a["q"], None, *args, kv_descale=f32(1), **kw)
    with pytest.raises(ValueError):                      # an empty one
        m.mla_decode_q8(a["q"], f32(0), *args, kv_descale=f32(1), **kw)
    with pytest.raises(TypeError):                       # bf16 query
        m.mla_decode_q8(bf16(BS, QL, H, 576), f32(1), *args, kv_descale=f32(1), **kw)
    with pytest.raises(TypeError):                       # bf16 cache
        m.mla_decode_q8(a["q"], f32(1), bf16(PAGES, 64, 576), *args[1:], kv_descale=f32(1), **kw)


def test_decode_static_checks(m):
    a = decode_args()
    args = (a["q"], a["kv_cache"], a["block_table"], a["seq_lens"], a["tile_plan"],
            a["split_indptr"], 0.1)
    with pytest.raises(Reached):
        m.mla_decode_static(*args, out=a["out"], lse=a["lse"])
    with pytest.raises(ValueError):
        m.mla_decode_static(*args, out=bf16(BS, QL, H + 1, 512), lse=a["lse"])


def test_merge_checks(m):
    po, pl, ip = bf16(BS + PARTS, R, 512), f32(BS + PARTS, R), i32(BS + 1)
    with pytest.raises(Reached):
        m.merge_states(po, pl, ip, bf16(BS, QL, H, 512), f32(BS, QL, H))
    for bad in (dict(po=bf16(BS + PARTS, R, 256)), dict(pl=f32(BS + PARTS, R + 1)),
                dict(out=bf16(BS, QL, H, 511)), dict(lse=f32(BS, QL)), dict(ip=i32(1))):
        a = dict(po=po, pl=pl, ip=ip, out=bf16(BS, QL, H, 512), lse=f32(BS, QL, H))
        a.update(bad)
        with pytest.raises(ValueError):
            m.merge_states(a["po"], a["pl"], a["ip"], a["out"], a["lse"])


def test_table_and_plan_checks(m):
    r2t, rpi, sl = i32(2 * BS, 256), i32(BS), i32(BS)
    with pytest.raises(Reached):
        m.build_block_table(r2t, rpi, sl, W, out=i32(BS, W))
    with pytest.raises(ValueError):
        m.build_block_table(r2t, rpi, sl, W, out=i32(BS - 1, W))
    with pytest.raises(ValueError):
        m.build_block_table(r2t, i32(BS + 1), sl, W, out=i32(BS, W))
    with pytest.raises(ValueError):
        m.plan_splits(sl, R, PARTS, tile_plan=i32(PARTS - 1, 8))
    with pytest.raises(ValueError):
        m.plan_splits(sl, R, PARTS, split_indptr=i32(BS))
    with pytest.raises(ValueError):
        m.build_table_and_plan(r2t, rpi, sl, W, R, PARTS, out=i32(BS, W),
                               tile_plan=i32(PARTS, 7))


def test_append_and_quantize_checks(m):
    kv = bf16(PAGES, 64, 576)
    with pytest.raises(Reached):
        m.set_kv_buffer(kv, torch.zeros(4, dtype=torch.int64), bf16(4, 576))
    with pytest.raises(ValueError):        # 4 rows, 3 slots
        m.set_kv_buffer(kv, torch.zeros(3, dtype=torch.int64), bf16(4, 576))
    with pytest.raises(ValueError):        # rows not 576 wide
        m.set_kv_buffer(kv, torch.zeros(4, dtype=torch.int64), bf16(4, 512))
    q = bf16(BS, QL, H, 576)
    with pytest.raises(Reached):
        m.quantize_q_fp8(q, f32(1), out=torch.zeros((BS, QL, H, 576), dtype=torch.uint8))
    with pytest.raises(ValueError):
        m.quantize_q_fp8(q, f32(1), out=torch.zeros((BS, QL, H, 575), dtype=torch.uint8))
