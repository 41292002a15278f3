"""Pure-Python brute force for MLA decode, independent of ``oracle/``.

Contiguous keys are copied out token by token through ``req_to_token``
(no block table), values are decoded with ``struct`` (bf16) or torch's
float8_e4m3fn cast (fp8), and softmax attention is evaluated with scalar
loops in Python floats.  Small inputs only.
"""

import math
import struct


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _fp8_table():
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return [float(v) for v in codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()]


def contiguous_keys(w, b):
    """Request b's latent rows 0..L-1 as lists of floats."""
    L = int(w.seq_lens[b])
    row = w.req_to_token[int(w.req_pool_indices[b])]
    tab = _fp8_table() if w.kv_dtype == "fp8_e4m3" else None
    keys = []
    for j in range(L):
        slot = int(row[j])
        page, off = slot // 64, slot % 64
        raw = w.kv[page, off]
        if tab is None:
            keys.append([_bf16(x) for x in raw])
        else:
            keys.append([tab[int(x)] * w.kv_descale for x in raw])
    return keys


def decode_row(qrow, keys, scale, n_visible):
    """(o, lse) for one query row over the first n_visible keys."""
    if n_visible <= 0:
        return [0.0] * 512, -math.inf
    s = []
    for j in range(n_visible):
        k = keys[j]
        acc = 0.0
        for d in range(576):
            acc += qrow[d] * k[d]
        s.append(scale * acc)
    m = max(s)
    p = [math.exp(x - m) for x in s]
    l = sum(p)
    o = [0.0] * 512
    for j in range(n_visible):
        pj = p[j] / l
        k = keys[j]
        for d in range(512):
            o[d] += pj * k[d]
    return o, m + math.log(l)


def decode(w, requests=None, rows=None):
    """{(b, r): (o, lse)} for the chosen requests/rows; r = i*H + h."""
    out = {}
    H, n = w.heads, w.q_len
    for b in (range(w.bs) if requests is None else requests):
        keys = contiguous_keys(w, b)
        L = int(w.seq_lens[b])
        for r in (range(n * H) if rows is None else rows):
            i, h = divmod(r, H)
            qrow = [_bf16(x) for x in w.q_bits[b, i, h]]
            nv = (L - n + i + 1) if w.causal else L
            out[(b, r)] = decode_row(qrow, keys, w.softmax_scale, nv)
    return out
