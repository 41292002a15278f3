"""Pins of the KV-append oracle (e4m3fn encoder and slot scatter), CPU only.

The encoder is checked against closed-form codes written from the format
(1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormal step 2^-9,
largest finite 448, NaN S.1111.111), against torch's float8_e4m3fn cast
(a library routine; torch does not saturate, so inputs are clipped to +-448
for that comparison), and against the decoder (every finite code round-trips).
"""

import numpy as np
import torch

import oracle
from oracle.kv_append import E4M3_MAX


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    y = torch.from_numpy(np.clip(x, -E4M3_MAX, E4M3_MAX).astype(np.float32))
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_closed_forms():
    cases = [(0.0, 0x00), (-0.0, 0x80)]   # a dict would merge +0 and -0
    cases += list({
        1.0: 0x38, -2.0: 0xC0, 1.125: 0x39, 0.5: 0x30,
        448.0: 0x7E, -448.0: 0xFE, 449.0: 0x7E, 1e6: 0x7E, np.inf: 0x7E, -np.inf: 0xFE,
        2.0 ** -6: 0x08,            # smallest normal
        2.0 ** -9: 0x01,            # smallest subnormal
        7 * 2.0 ** -9: 0x07,        # largest subnormal
        2.0 ** -10: 0x00,           # tie between 0 and 2^-9: even code 0
        3 * 2.0 ** -10: 0x02,       # tie between codes 1 and 2: even code 2
        1.0625: 0x38,               # tie between 1.0 (0x38) and 1.125 (0x39): even 0x38
        1.1875: 0x3A,               # tie between 0x39 and 0x3A: even 0x3A
        432.0: 0x7E,                # tie between 416 (0x7D) and 448 (0x7E): even 0x7E
        240.0: 0x77, 256.0: 0x78,
    }.items())
    xs = np.array([c[0] for c in cases], dtype=np.float64)
    want = np.array([c[1] for c in cases], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3fn_encode(xs), want)
    nan = oracle.e4m3fn_encode(np.array([np.nan, -np.nan]))
    assert nan[0] & 0x7F == 0x7F and nan[1] & 0x7F == 0x7F


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3fn_to_f64(codes)
    assert np.array_equal(oracle.e4m3fn_encode(vals), codes)


def test_e4m3_encode_midpoints_go_to_even_code():
    codes = np.arange(0x7F, dtype=np.uint8)
    v = oracle.e4m3fn_to_f64(codes)
    mid = (v[:-1] + v[1:]) / 2
    even = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(oracle.e4m3fn_encode(mid), even)
    eps = np.spacing(mid) * 4
    assert np.array_equal(oracle.e4m3fn_encode(mid - eps), codes[:-1])
    assert np.array_equal(oracle.e4m3fn_encode(mid + eps), codes[1:])
    assert np.array_equal(oracle.e4m3fn_encode(-mid), even | 0x80)


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000) * np.exp2(rng.uniform(-14, 10, 200000))
    x = x.astype(np.float32).astype(np.float64)
    codes = np.arange(0x7F, dtype=np.uint8)
    v = oracle.e4m3fn_to_f64(codes)
    mids = np.concatenate([(v[:-1] + v[1:]) / 2, -(v[:-1] + v[1:]) / 2])
    x = np.concatenate([x, mids, [500.0, -500.0, 448.0, 460.0, 470.0]])
    assert np.array_equal(oracle.e4m3fn_encode(x), _torch_e4m3(x))


def test_quantize_rows_uses_fp32_quotient():
    # k = 1.0 and scale = 3: the fp32 quotient 0.33333334 is encoded (code 0x2B = 0.34375
    # is nearer than 0x2A = 0.3125); the closed form is the same in any precision here.
    k = np.full(oracle.paged_mla.LATENT_DIM, 0x3F80, dtype=np.uint16)   # bf16 1.0
    codes = oracle.quantize_rows(k, 3.0)
    assert np.all(codes == 0x2B)
    # The quotient is rounded once, to fp32, then to e4m3: scale 1 gives the plain encode.
    rng = np.random.default_rng(3)
    bits = (rng.standard_normal(576).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vals = oracle.bf16_to_f64(bits)
    assert np.array_equal(oracle.quantize_rows(bits, 1.0), oracle.e4m3fn_encode(vals))


def test_set_kv_buffer_bf16_scatter():
    rng = np.random.default_rng(11)
    pages = 6
    kv = rng.integers(0, 1 << 16, size=(pages, 64, 576), dtype=np.int64).astype(np.uint16)
    slots = np.array([0, 63, 64, 200, 383, -1, 384, 1000], dtype=np.int64)
    k = rng.integers(0, 1 << 16, size=(len(slots), 576), dtype=np.int64).astype(np.uint16)
    out = oracle.set_kv_buffer(kv, slots, k, "bf16")
    touched = np.zeros((pages, 64), dtype=bool)
    for i, s in enumerate(slots):
        if 0 <= s < pages * 64:
            assert np.array_equal(out[s // 64, s % 64], k[i])
            touched[s // 64, s % 64] = True
    assert np.array_equal(out[~touched], kv[~touched])      # everything else as it was
    assert np.array_equal(kv, kv.copy())                    # input not modified


def test_set_kv_buffer_fp8_error_bound_and_decode_sees_new_rows():
    rng = np.random.default_rng(12)
    pages, scale = 4, 0.0125
    kv = rng.integers(0, 256, size=(pages, 64, 576), dtype=np.int64).astype(np.uint8)
    slots = rng.permutation(pages * 64)[:40]
    x = rng.standard_normal((40, 576)).astype(np.float32)
    k = (x.view(np.uint32) >> 16).astype(np.uint16)          # truncated to bf16 bits
    out = oracle.set_kv_buffer(kv, slots, k, "fp8_e4m3", scale)
    kval = oracle.bf16_to_f64(k)
    got = oracle.e4m3fn_to_f64(out.reshape(-1, 576)[slots]) * scale
    # Relative error of a normal e4m3 value is at most 2^-4; subnormals err by at
    # most half the step 2^-9 (times the scale).
    bound = np.maximum(np.abs(kval) * 2.0 ** -4, 2.0 ** -10 * scale) * (1 + 1e-9)
    assert np.all(np.abs(got - kval) <= bound)
    # The decode oracle reads an appended token back as that latent row.
    L = 130
    seq_pages = rng.permutation(pages)[:3]
    r2t = np.zeros((1, 192), dtype=np.int32)
    r2t[0] = (seq_pages[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
    new_slot = int(r2t[0, L - 1])
    row = rng.standard_normal(576).astype(np.float32)
    row_bits = (row.view(np.uint32) >> 16).astype(np.uint16)[None, :]
    out2 = oracle.set_kv_buffer(kv, [new_slot], row_bits, "fp8_e4m3", scale)
    bt = oracle.block_table(r2t, np.array([0]), np.array([L]), 3)
    K = oracle.request_keys(out2, "fp8_e4m3", scale, bt[0], L)
    assert np.array_equal(K[L - 1], oracle.e4m3fn_to_f64(oracle.quantize_rows(row_bits[0], scale)) * scale)


# ------------------------------------------------------------ fp8 query

def test_quantize_q_shape_and_codes():
    rng = np.random.default_rng(21)
    q = (rng.standard_normal((2, 1, 4, 576)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    c = oracle.quantize_q(q, 0.02)
    assert c.shape == q.shape and c.dtype == np.uint8
    assert np.array_equal(c.reshape(-1), oracle.quantize_rows(q.reshape(-1), 0.02))


def _tiny_q8_case():
    from workloads import make_custom
    w = make_custom("q8", bs=2, heads=4, q_len=2, seq_lens=[70, 5], seed=23, value_scale=0.5)
    rng = np.random.default_rng(24)
    codes = rng.integers(0, 0x7E, size=w.q_bits.shape).astype(np.uint8)
    codes |= (rng.random(w.q_bits.shape) < 0.5).astype(np.uint8) << 7     # random signs
    return w, codes


def test_decode_q8_equals_decode_of_the_dequantised_query():
    """With a power-of-two q scale, code * scale is exact in bf16: the fp8-query
    decode must equal the bf16 decode of those values."""
    w, codes = _tiny_q8_case()
    dq = 2.0 ** -5
    vals = oracle.e4m3fn_to_f64(codes) * dq
    q_bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f64(q_bits), vals)             # exact in bf16
    args = (w.kv, w.kv_dtype, w.kv_descale, w.req_to_token, w.req_pool_indices, w.seq_lens,
            w.softmax_scale, w.causal)
    o8, l8 = oracle.paged_decode_q8(codes, dq, *args)
    o, l = oracle.paged_decode(q_bits, *args)
    assert np.allclose(o8, o, rtol=0, atol=1e-12) and np.allclose(l8, l, rtol=0, atol=1e-12)
    # and quantising those values gives the codes back
    assert np.array_equal(oracle.quantize_q(q_bits, dq), codes)


def test_decode_q8_descale_scales_the_scores_only():
    """q_descale multiplies every score: it is the same as folding it into the
    softmax scale, and the output stays a weighted mean of the value rows."""
    w, codes = _tiny_q8_case()
    base = (w.kv, w.kv_dtype, w.kv_descale, w.req_to_token, w.req_pool_indices, w.seq_lens)
    o_a, l_a = oracle.paged_decode_q8(codes, 0.37, *base, w.softmax_scale, w.causal)
    o_b, l_b = oracle.paged_decode_q8(codes, 1.0, *base, w.softmax_scale * 0.37, w.causal)
    assert np.allclose(o_a, o_b, rtol=0, atol=1e-12) and np.allclose(l_a, l_b, rtol=0, atol=1e-12)
    # a zero scale leaves the plain mean of the visible value rows (lse = ln count)
    o_0, l_0 = oracle.paged_decode_q8(codes, 0.0, *base, w.softmax_scale, w.causal)
    L0 = int(w.seq_lens[1])
    K = oracle.request_keys(w.kv, w.kv_dtype, w.kv_descale,
                            oracle.block_table(w.req_to_token, w.req_pool_indices, w.seq_lens,
                                               w.bt_width)[1], L0)
    # request 1, token 0 of q_len 2 (causal) sees keys 0 .. L - 2
    assert np.allclose(o_0[1, 0], K[:L0 - 1, :512].mean(axis=0), atol=1e-12)
    assert np.allclose(l_0[1, 0], np.log(L0 - 1), atol=1e-12)
