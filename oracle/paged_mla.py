"""Plain fp64 MLA paged-KV decode: the definition, written out.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages fix it:

* Block table (FlashMLA backend page, ``init_forward_metadata``, decode and
  target-verify branches): a ``[bs, width]`` int32 table, pre-filled with -1,
  whose first ceil(seq_len/64) entries of row b name request b's pages.  The
  page body of the index kernel is not on the pages; the plainest reading,
  consistent with the cache being viewed as ``[-1, 64, 1, 576]`` in
  ``forward_decode``, is entry p = (slot of token 64p) // 64.
* Latent cache and V (``forward_decode``): q is ``[bs, q_len, H, 576]``; K is
  the 576-wide latent row; V is its first ``kv_lora_rank`` = 512 columns
  (``head_dim_v=self.kv_lora_rank``); scores use ``softmax_scale=layer.scaling``
  and ``causal=True``.
* Verify lengths (``forward_extend``, non-EXTEND branch): the cache length
  passed is prefix + draft tokens; with causal masking aligned bottom-right,
  draft token i of n sees keys 0 .. L-n+i.
* fp8 cache (``forward_decode`` fp8 branch; AITER helper page,
  ``forward_decode_vectorized_5d``): the stored byte is an fp8 value that must
  be multiplied by the per-tensor scale to recover the latent value.
* LSE and merge (FlashInfer backend page, ``forward_extend``: two partial
  attentions over disjoint key sets each return (o, lse) and ``merge_state``
  combines them; FlashMLA page, ``forward_decode``: lse is returned so that
  decode-context-parallel ranks can correct the output by online softmax).
  lse is the natural log of the sum of exp(scaled score) over visible keys.
"""

from __future__ import annotations

import numpy as np

PAGE_SIZE = 64
LATENT_DIM = 576
V_DIM = 512


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64.  A bf16 value is the upper half of the
    fp32 with the same bits, so the conversion is exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP float8 e4m3fn bytes -> float64, from the format's definition:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.ldexp(1.0, (exp - 7).astype(np.int64))
    sub = (man / 8.0) * np.ldexp(1.0, -6)
    val = sign * np.where(exp == 0, sub, normal)
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return val


def block_table(req_to_token: np.ndarray, req_pool_indices: np.ndarray,
                seq_lens: np.ndarray, width: int, pad: int = -1,
                page_size: int = PAGE_SIZE) -> np.ndarray:
    """bt[b, p] = req_to_token[rpi[b], page_size*p] // page_size for
    p < ceil(seq_lens[b] / page_size), and ``pad`` elsewhere."""
    bs = len(seq_lens)
    bt = np.full((bs, width), pad, dtype=np.int32)
    for b in range(bs):
        n = -(-int(seq_lens[b]) // page_size)
        if n > width:
            raise ValueError("block table too narrow")
        row = req_to_token[int(req_pool_indices[b])]
        for p in range(n):
            bt[b, p] = int(row[p * page_size]) // page_size
    return bt


def request_keys(kv: np.ndarray, kv_dtype: str, kv_descale: float,
                 bt_row: np.ndarray, seq_len: int) -> np.ndarray:
    """The request's latent rows 0..seq_len-1 in logical order, as float64
    ``[seq_len, 576]``: page bt_row[j // 64], row j % 64, times the
    per-tensor descale (1 for bf16)."""
    n = -(-seq_len // PAGE_SIZE)
    raw = kv[np.asarray(bt_row[:n], dtype=np.int64)].reshape(n * PAGE_SIZE, LATENT_DIM)[:seq_len]
    if kv_dtype == "bf16":
        return bf16_to_f64(raw)
    if kv_dtype == "fp8_e4m3":
        return e4m3fn_to_f64(raw) * float(kv_descale)
    raise ValueError(kv_dtype)


def attend(Q: np.ndarray, K: np.ndarray, scale: float, last_visible: np.ndarray):
    """Softmax attention of rows Q ``[R, 576]`` over keys K ``[L, 576]`` with
    V = K[:, :512].  Row r sees keys 0..last_visible[r] (inclusive).

    Returns (o ``[R, 512]``, lse ``[R]``): o = sum_j p_j V_j / sum_j p_j with
    p_j = exp(s_j - m), s_j = scale * <q, k_j>, m = max visible s_j, and
    lse = m + ln(sum_j p_j).  A row with no visible key gets o = 0, lse = -inf.
    """
    R = Q.shape[0]
    L = K.shape[0]
    o = np.zeros((R, V_DIM), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if L == 0 or R == 0:
        return o, lse
    S = float(scale) * (Q @ K.T)
    vis = np.arange(L)[None, :] <= np.asarray(last_visible)[:, None]
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1)
    has = np.isfinite(m)
    P = np.where(vis, np.exp(Sm - np.where(has, m, 0.0)[:, None]), 0.0)
    l = P.sum(axis=1)
    V = K[:, :V_DIM]
    o[has] = (P[has] @ V) / l[has, None]
    lse[has] = m[has] + np.log(l[has])
    return o, lse


def paged_decode(q_bits, kv, kv_dtype, kv_descale, req_to_token, req_pool_indices,
                 seq_lens, softmax_scale, causal=True, rows=None):
    """Batched MLA decode over the paged latent cache, in fp64.

    q_bits: uint16 ``[bs, q_len, H, 576]`` bf16 bits.  Row order inside a
    request is r = i*H + h.  Returns o ``[bs, q_len, H, 512]`` and lse
    ``[bs, q_len, H]``.  ``rows`` optionally restricts the work to a dict
    {b: array of row indices r}; other rows are left NaN.
    """
    bs, n, H, D = q_bits.shape
    assert D == LATENT_DIM
    width = max(1, -(-int(np.max(seq_lens)) // PAGE_SIZE)) if bs else 1
    bt = block_table(req_to_token, req_pool_indices, seq_lens, width)
    o = np.full((bs, n * H, V_DIM), np.nan)
    lse = np.full((bs, n * H), np.nan)
    for b in range(bs):
        sel = np.arange(n * H) if rows is None else np.asarray(rows.get(b, []), dtype=np.int64)
        if sel.size == 0:
            continue
        L = int(seq_lens[b])
        K = request_keys(kv, kv_dtype, kv_descale, bt[b], L)
        Q = bf16_to_f64(q_bits[b].reshape(n * H, D)[sel])
        i = sel // H
        last = (L - n + i) if causal else np.full(sel.size, L - 1)
        o[b, sel], lse[b, sel] = attend(Q, K, softmax_scale, last)
    return o.reshape(bs, n, H, V_DIM), lse.reshape(bs, n, H)


def paged_decode_q8(q_codes, q_descale, kv, kv_dtype, kv_descale, req_to_token,
                    req_pool_indices, seq_lens, softmax_scale, causal=True, rows=None):
    """paged_decode with an fp8 query (the fp8 branch of the FlashMLA page's
    forward_decode: q quantised to e4m3fn with the cache scale, then
    descale_q applied to the scores): the query row's value is
    e4m3fn(code) * q_descale.  q_codes: uint8 [bs, q_len, H, 576]."""
    bs, n, H, D = q_codes.shape
    assert D == LATENT_DIM
    width = max(1, -(-int(np.max(seq_lens)) // PAGE_SIZE)) if bs else 1
    bt = block_table(req_to_token, req_pool_indices, seq_lens, width)
    o = np.full((bs, n * H, V_DIM), np.nan)
    lse = np.full((bs, n * H), np.nan)
    for b in range(bs):
        sel = np.arange(n * H) if rows is None else np.asarray(rows.get(b, []), dtype=np.int64)
        if sel.size == 0:
            continue
        L = int(seq_lens[b])
        K = request_keys(kv, kv_dtype, kv_descale, bt[b], L)
        Q = e4m3fn_to_f64(q_codes[b].reshape(n * H, D)[sel]) * float(q_descale)
        i = sel // H
        last = (L - n + i) if causal else np.full(sel.size, L - 1)
        o[b, sel], lse[b, sel] = attend(Q, K, softmax_scale, last)
    return o.reshape(bs, n, H, V_DIM), lse.reshape(bs, n, H)


def merge_states(o_parts: np.ndarray, lse_parts: np.ndarray, indptr: np.ndarray):
    """Exact merge of partial attention states over disjoint key sets.

    Pieces indptr[b] .. indptr[b+1]-1 belong to request b.  For each row:
    LSE = M + ln(sum_k exp(lse_k - M)) with M = max_k lse_k, and
    o = sum_k exp(lse_k - LSE) * o_k.  Pieces with lse = -inf weigh 0; a row
    whose pieces are all empty gets o = 0, lse = -inf.
    """
    bs = len(indptr) - 1
    R, Dv = o_parts.shape[1], o_parts.shape[2]
    o = np.zeros((bs, R, Dv))
    lse = np.full((bs, R), -np.inf)
    for b in range(bs):
        k0, k1 = int(indptr[b]), int(indptr[b + 1])
        if k1 == k0:
            continue
        ls = lse_parts[k0:k1].astype(np.float64)        # [k, R]
        M = ls.max(axis=0)                               # [R]
        ok = np.isfinite(M)
        Msafe = np.where(ok, M, 0.0)
        w = np.where(np.isfinite(ls), np.exp(ls - Msafe[None, :]), 0.0)
        tot = w.sum(axis=0)
        LSE = np.where(ok, Msafe + np.log(np.where(ok, tot, 1.0)), -np.inf)
        wn = np.where(ok[None, :] & np.isfinite(ls), np.exp(ls - np.where(ok, LSE, 0.0)[None, :]), 0.0)
        o[b] = np.einsum("kr,krd->rd", wn, o_parts[k0:k1].astype(np.float64))
        lse[b] = LSE
    return o, lse
