"""Plain KV append into the paged latent cache: the definition, written out.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages fix it:

* The FlashMLA backend page's ``forward_decode`` (and the target-verify branch
  of ``forward_extend``) first stores the new tokens' latent rows:
  ``token_to_kv_pool.set_kv_buffer(layer, cache_loc, k, v)`` with
  ``cache_loc = forward_batch.out_cache_loc``, one pool slot per new token.
  In MLA the value is the first 512 columns of the same latent row, so only
  the 576-wide row k is stored.
* The pool is the one ``forward_decode`` reads, viewed as ``[-1, 64, 1, 576]``:
  slot s is row s % 64 of page s // 64.
* fp8 cache (``forward_decode`` fp8 branch): a stored byte times the
  per-tensor scale ``k_scale`` is the latent value.  The body of
  ``set_kv_buffer`` is not on the pages; the plainest reading consistent with
  that is byte = e4m3fn(k / k_scale), rounded to nearest (ties to even),
  saturating at the largest finite value 448 (e4m3fn has no infinity).  The
  quotient is taken in fp32 (the precision the quantised code is decided in),
  so both sides decide every byte from the same fp32 value.
"""

from __future__ import annotations

import numpy as np

from .paged_mla import LATENT_DIM, PAGE_SIZE, e4m3fn_to_f64

E4M3_MAX = 448.0

# Every non-negative finite e4m3fn value, indexed by its code 0x00..0x7E
# (0x7F is NaN), from the format's own definition in e4m3fn_to_f64.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3fn_to_f64(_POS_CODES)


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> OCP float8 e4m3fn codes: the nearest finite value, ties to
    the even code (mantissa LSB 0), |x| > 448 saturating to 448, NaN to
    0x7F with the sign bit of x.  The search is over the table of all 127
    non-negative values, so no bit trick of an encoder is assumed."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    sign = np.signbit(x)
    return np.where(sign, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows(k_bits: np.ndarray, kv_scale: float) -> np.ndarray:
    """bf16 latent rows -> e4m3fn bytes of k / kv_scale, the quotient rounded
    to fp32 first (IEEE division in fp32, which numpy performs)."""
    kf = (np.asarray(k_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        qf = kf / np.float32(kv_scale)
    return e4m3fn_encode(qf.astype(np.float64))


def set_kv_buffer(kv: np.ndarray, slots: np.ndarray, k_bits: np.ndarray, kv_dtype: str,
                  kv_scale: float = 1.0) -> np.ndarray:
    """A copy of the pool ``kv`` ``[num_pages, 64, 576]`` (uint16 bf16 bits,
    or uint8 e4m3fn bytes) with latent row i of ``k_bits`` ``[n, 576]``
    stored at slot ``slots[i]``: page slots[i] // 64, row slots[i] % 64.
    Slots outside the pool are skipped; slots are expected to be distinct."""
    out = np.array(kv, copy=True)
    n_slots = out.shape[0] * PAGE_SIZE
    flat = out.reshape(n_slots, LATENT_DIM)
    k_bits = np.asarray(k_bits, dtype=np.uint16).reshape(-1, LATENT_DIM)
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0 or s >= n_slots:
            continue
        if kv_dtype == "bf16":
            flat[s] = k_bits[i]
        elif kv_dtype == "fp8_e4m3":
            flat[s] = quantize_rows(k_bits[i], kv_scale)
        else:
            raise ValueError(kv_dtype)
    return out


def quantize_q(q_bits: np.ndarray, q_scale: float) -> np.ndarray:
    """The fp8 branch of the FlashMLA page's forward_decode quantises the
    query with the cache's scale before attention (scaled_fp8_quant with
    q_scale = k_scale): code = e4m3fn(q / q_scale), the same rounding and
    saturation as the cache bytes.  Returns uint8 codes of q's shape."""
    return quantize_rows(q_bits, q_scale)
