"""GPU parity of the KV append (mla_set_kv_buffer) against the oracle.

Byte work: the pool after the append must equal the oracle's pool bit for bit
(bf16 rows copied, fp8 rows quantised to e4m3fn of the fp32 quotient).
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload, CONFIGS
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_mla_req_amd as m
    return m


def _bf16_rows(rng, n, scale=1.0):
    x = (rng.standard_normal((n, 576)) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _pool_np(kv, dtype):
    t = kv.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else t.numpy()


def _slots(rng, n, pages, extra_invalid=True):
    s = rng.permutation(pages * 64)[:n].astype(np.int64)
    if extra_invalid and n >= 4:
        s[1], s[2] = -5, pages * 64          # outside the pool: skipped
        s[3] = 1 << 40
    return s


@pytest.mark.parametrize("n", [1, 3, 64, 257, 4099])
def test_append_bf16_bit_exact(mla, n):
    rng = np.random.default_rng(100 + n)
    pages = max(8, -(-2 * n // 64))
    kv = rng.integers(0, 1 << 16, size=(pages, 64, 576), dtype=np.int64).astype(np.uint16)
    slots = _slots(rng, n, pages)
    k = _bf16_rows(rng, n)
    kv_d = _dev_u16(kv)
    mla.set_kv_buffer(kv_d, torch.from_numpy(slots).cuda(), _dev_u16(k), kv_dtype="bf16")
    torch.cuda.synchronize()
    assert np.array_equal(_pool_np(kv_d, "bf16"), oracle.set_kv_buffer(kv, slots, k, "bf16"))


@pytest.mark.parametrize("scale", [1.0, 0.0125, 3.0, 2.0 ** -7])
def test_append_fp8_bit_exact(mla, scale):
    rng = np.random.default_rng(7)
    # Values that hit every e4m3 rounding case for scale 1: the midpoints between
    # neighbouring codes (exact in bf16), both signs, saturating and subnormal ones.
    v = oracle.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = np.concatenate([(v[:-1] + v[1:]) / 2, -(v[:-1] + v[1:]) / 2, v, -v,
                           [500.0, -1e4, 2.0 ** -12, -(2.0 ** -11), 0.0, -0.0]])
    mid_bits = (mids.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    n_mid_rows = -(-mid_bits.size // 576)
    special = np.resize(mid_bits, (n_mid_rows, 576))
    k = np.concatenate([special, _bf16_rows(rng, 300, 2.0), _bf16_rows(rng, 40, 1e-3)])
    n = k.shape[0]
    pages = 16
    kv = rng.integers(0, 256, size=(pages, 64, 576), dtype=np.int64).astype(np.uint8)
    slots = _slots(rng, n, pages)
    kv_d = torch.from_numpy(kv.copy()).cuda()
    sc = torch.tensor([scale], dtype=torch.float32, device="cuda")
    mla.set_kv_buffer(kv_d, torch.from_numpy(slots).cuda(), _dev_u16(k), kv_dtype="fp8_e4m3",
                      kv_scale=sc)
    torch.cuda.synchronize()
    want = oracle.set_kv_buffer(kv, slots, k, "fp8_e4m3", scale)
    assert np.array_equal(_pool_np(kv_d, "fp8_e4m3"), want)


def test_append_strided_rows_and_empty(mla):
    rng = np.random.default_rng(5)
    n, pages = 50, 4
    kv = rng.integers(0, 1 << 16, size=(pages, 64, 576), dtype=np.int64).astype(np.uint16)
    wide = _bf16_rows(rng, n * 2)[:, :]                     # [2n, 576]
    big = np.zeros((n, 640), dtype=np.uint16)
    big[:, :576] = wide[:n]
    big[:, 576:] = 0x7FC0                                   # NaN padding, never stored
    k_view = _dev_u16(big)[:, :576]                         # row stride 640
    slots = _slots(rng, n, pages, extra_invalid=False)
    kv_d = _dev_u16(kv)
    mla.set_kv_buffer(kv_d, torch.from_numpy(slots).cuda(), k_view, kv_dtype="bf16")
    empty = torch.empty((0, 576), dtype=torch.bfloat16, device="cuda")
    mla.set_kv_buffer(kv_d, torch.empty(0, dtype=torch.int64, device="cuda"), empty)
    torch.cuda.synchronize()
    assert np.array_equal(_pool_np(kv_d, "bf16"), oracle.set_kv_buffer(kv, slots, wide[:n], "bf16"))


@pytest.mark.parametrize("name", ["tiny", "verify_small"])
def test_append_then_decode_matches_oracle(mla, name):
    """The step the pages run: store the new tokens' rows at their slots, then
    decode over the updated pool; compared with the oracle's append + decode."""
    from tests.test_gpu_parity import assert_close, run
    from workloads import make_custom

    if name == "tiny":
        w = make_workload("tiny")
    else:
        w = make_custom("verify_small", bs=3, heads=16, q_len=4, seq_lens=np.array([5, 70, 300]), seed=31,
                        kv_dtype="bf16", value_scale=0.5)
    rng = np.random.default_rng(9)
    slots = []
    for b in range(w.bs):
        L = int(w.seq_lens[b])
        row = w.req_to_token[int(w.req_pool_indices[b])]
        slots.extend(int(row[L - w.q_len + i]) for i in range(w.q_len))
    slots = np.array(slots, dtype=np.int64)
    k = _bf16_rows(rng, slots.size, 0.5)
    kv_ref = oracle.set_kv_buffer(w.kv, slots, k, w.kv_dtype)
    d = to_device(w)
    mla.set_kv_buffer(d.kv, torch.from_numpy(slots).cuda(), _dev_u16(k), kv_dtype=w.kv_dtype)
    torch.cuda.synchronize()
    assert np.array_equal(_pool_np(d.kv, w.kv_dtype), kv_ref)
    o, lse = run(mla, w, num_parts=3, kv=_pool_np(d.kv, w.kv_dtype))
    o_ref, lse_ref = oracle.paged_decode(w.q_bits, kv_ref, w.kv_dtype, w.kv_descale,
                                         w.req_to_token, w.req_pool_indices, w.seq_lens,
                                         w.softmax_scale, w.causal)
    assert_close(o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("name", ["dsv3", "fp8", "verify"])
def test_append_full_size_step(mla, name):
    """The append at a full workload's step size (one row per new token: 64, 128
    and 256 tokens) into its full-size pool: the written rows bit-exact, every
    other byte of the pool unchanged."""
    cfg = CONFIGS[name]
    bs, q_len = cfg["bs"], cfg.get("q_len", 1)
    fp8 = cfg["kv_dtype"] == "fp8_e4m3"
    rng = np.random.default_rng(77)
    pages = bs * 2 * 128 if name != "verify" else bs * 2 * 257
    n = bs * q_len
    slots = rng.permutation(pages * 64)[:n].astype(np.int64)
    k = _bf16_rows(rng, n)
    if fp8:
        kv_d = torch.randint(0, 256, (pages, 64, 576), dtype=torch.uint8, device="cuda")
        scale = 4.5 / 448
        sc = torch.tensor([scale], dtype=torch.float32, device="cuda")
    else:
        kv_d = torch.randint(-32768, 32767, (pages, 64, 576), dtype=torch.int16,
                             device="cuda").view(torch.bfloat16)
        sc = None
    before = kv_d.clone()
    mla.set_kv_buffer(kv_d, torch.from_numpy(slots).cuda(), _dev_u16(k), kv_dtype=cfg["kv_dtype"],
                      kv_scale=sc)
    torch.cuda.synchronize()
    flat = kv_d.view(pages * 64, 576)
    got = flat[torch.from_numpy(slots).cuda()].cpu()
    if fp8:
        assert np.array_equal(got.numpy(), oracle.quantize_rows(k, scale))
    else:
        assert np.array_equal(got.view(torch.int16).numpy().view(np.uint16), k)
    mask = torch.ones(pages * 64, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(slots).cuda()] = False
    assert torch.equal(flat[mask].view(torch.uint8) if fp8 else flat[mask].view(torch.int16),
                       before.view(pages * 64, 576)[mask].view(torch.uint8) if fp8
                       else before.view(pages * 64, 576)[mask].view(torch.int16))


# ------------------------------------------------------------ query quantisation

@pytest.mark.parametrize("name,scale", [("tiny", 1.0), ("fp8", 4.5 / 448), ("verify", 0.0125),
                                        ("dsv3", 2.0 ** -6)])
def test_quantize_q_fp8_bit_exact(mla, name, scale):
    """The fp8 branch's query quantisation at the workloads' query shapes."""
    w = make_workload(name)
    d = to_device(w)
    sc = torch.tensor([scale], dtype=torch.float32, device="cuda")
    codes = mla.quantize_q_fp8(d.q, sc)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oracle.quantize_q(w.q_bits, scale))


def test_quantize_q_fp8_rounding_cases(mla):
    v = oracle.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    vals = np.concatenate([(v[:-1] + v[1:]) / 2, -(v[:-1] + v[1:]) / 2, v, -v,
                           [500.0, -1e4, 2.0 ** -12, 0.0, -0.0]])
    bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q = np.resize(bits, (3, 576))
    for scale in (1.0, 3.0):
        sc = torch.tensor([scale], dtype=torch.float32, device="cuda")
        codes = mla.quantize_q_fp8(_dev_u16(q), sc)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), oracle.quantize_q(q, scale))


def test_quantized_query_decodes_as_the_fp8_query_oracle(mla):
    """The fp8 branch end to end on small shapes: the query quantised on the GPU
    (mla_quantize_q_fp8) and, with a power-of-two scale, taken back to bf16
    exactly (code value * scale, a test-side step), then decoded on the GPU over
    an fp8 cache, matches the oracle's fp8-query decode of the GPU's codes."""
    from tests.test_gpu_parity import _np, assert_close, run
    from workloads import make_custom

    w = make_custom("q8dec", bs=3, heads=16, q_len=1, seq_lens=[37, 300, 1100], seed=61,
                    kv_dtype="fp8_e4m3", value_scale=0.5)
    d = to_device(w)
    dq = 2.0 ** -4
    sc = torch.tensor([dq], dtype=torch.float32, device="cuda")
    codes = mla.quantize_q_fp8(d.q, sc)
    torch.cuda.synchronize()
    c_np = codes.cpu().numpy()
    assert np.array_equal(c_np, oracle.quantize_q(w.q_bits, dq))
    q_deq = (codes.view(torch.float8_e4m3fn).to(torch.float32) * dq).to(torch.bfloat16)
    vals = oracle.e4m3fn_to_f64(c_np) * dq
    assert np.array_equal(q_deq.float().cpu().numpy().astype(np.float64), vals)   # exact
    bt = mla.build_block_table(d.req_to_token, d.req_pool_indices, d.seq_lens, w.bt_width)
    plan = mla.plan_splits(d.seq_lens, w.rows_per_req, 5, w.kv_dtype)
    out, lse = mla.decode(q_deq.contiguous(), d.kv, bt, d.seq_lens, w.softmax_scale,
                          kv_dtype=w.kv_dtype, kv_descale=d.kv_descale, causal=w.causal,
                          plan=plan)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.paged_decode_q8(c_np, dq, w.kv, w.kv_dtype, w.kv_descale,
                                            w.req_to_token, w.req_pool_indices, w.seq_lens,
                                            w.softmax_scale, w.causal)
    assert_close(_np(out), _np(lse), o_ref, lse_ref)
