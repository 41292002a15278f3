"""Seeded synthetic workloads for MLA paged-KV decode.

Shapes follow the FlashMLA backend page:
  * ``PAGE_SIZE`` is 64 tokens (module constant at the top of the page).
  * q is viewed as ``[bs, q_len, heads, head_dim]`` with head_dim =
    kv_lora_rank + qk_rope_head_dim = 512 + 64 = 576
    (``FlashMLABackend.__init__`` and ``forward_decode``).
  * the latent cache is viewed as ``[pages, 64, 1, 576]``; V is its first
    kv_lora_rank = 512 columns (``head_dim_v`` in the ``forward_decode`` call).
  * ``req_to_token[req_pool_indices[b], j]`` is the pool slot of token j of
    request b (``init_forward_metadata``; the AITER helper page calls these
    "one slot id per logical token").
  * ``seq_lens`` are KV lengths including the q_len new tokens; in target-verify
    mode they are prefix + draft tokens (``forward_extend``, verify branch).

Nothing here computes attention.  The only numeric transformations are the
ones that produce stored input bits: fp32 -> bf16 round-to-nearest-even, and
fp32 -> float8_e4m3fn encoding (done by torch's cast) after dividing by a
per-tensor scale.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

PAGE_SIZE = 64
LATENT_DIM = 576  # kv_lora_rank 512 + rope 64
V_DIM = 512       # kv_lora_rank
E4M3_MAX = 448.0
# 1/sqrt(192): 192 = qk_nope_head_dim 128 + qk_rope_head_dim 64 (DeepSeek-V3
# shape).  Stored as the fp32 value every consumer uses.
SOFTMAX_SCALE = float(np.float32(1.0 / np.sqrt(192.0)))


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Workload:
    name: str
    bs: int
    heads: int
    q_len: int
    kv_dtype: str                 # "bf16" or "fp8_e4m3"
    q_bits: np.ndarray            # uint16 [bs, q_len, heads, 576] (bf16 bits)
    kv: np.ndarray                # uint16 (bf16 bits) or uint8 (e4m3 bytes) [pool_pages, 64, 576]
    kv_descale: float             # per-tensor dequant scale (fp32 value; 1.0 for bf16)
    req_to_token: np.ndarray      # int32 [rows, ctx_cap]
    req_pool_indices: np.ndarray  # int32 [bs]
    seq_lens: np.ndarray          # int32 [bs], KV length incl. the q_len new tokens
    softmax_scale: float          # fp32 value
    causal: bool
    pages: List[np.ndarray] = field(repr=False, default_factory=list)  # physical pages per request

    @property
    def rows_per_req(self) -> int:
        return self.heads * self.q_len

    @property
    def pool_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def bt_width(self) -> int:
        return _cdiv(int(self.seq_lens.max()), PAGE_SIZE) if self.bs else 0

    @property
    def kv_bytes_read(self) -> int:
        """Bytes of latent KV that one pass must read: each visible token once."""
        elem = 2 if self.kv_dtype == "bf16" else 1
        return int(self.seq_lens.astype(np.int64).sum()) * LATENT_DIM * elem


# name -> parameters.  Seeds are fixed per workload.
CONFIGS: Dict[str, dict] = {
    # batch 2, 16 heads, q_len 1, lengths {37, 130}, pool of 8 pages, N(0,1)*0.5
    "tiny": dict(bs=2, heads=16, q_len=1, seq_lens=[37, 130], pool_pages=8,
                 value_scale=0.5, kv_dtype="bf16", seed=1001),
    # DeepSeek-V3-shaped decode: batch 64, 128 heads, lengths U[1024, 8192]
    "dsv3": dict(bs=64, heads=128, q_len=1, len_range=(1024, 8192),
                 kv_dtype="bf16", seed=1002),
    # the same shape with every length at exactly 4096 ("4k context")
    "dsv3_4k": dict(bs=64, heads=128, q_len=1, seq_lens=[4096] * 64,
                    kv_dtype="bf16", seed=1006),
    # long-context split stress: batch 8, 128 heads, lengths U[32768, 65536]
    "long": dict(bs=8, heads=128, q_len=1, len_range=(32768, 65536),
                 kv_dtype="bf16", seed=1003),
    # fp8 e4m3 latent cache with a per-tensor scale, bf16 q
    "fp8": dict(bs=128, heads=128, q_len=1, seq_lens=[4096] * 128,
                kv_dtype="fp8_e4m3", seed=1004),
    # speculative target-verify: 4 draft tokens, prefix U[256, 16384], causal
    "verify": dict(bs=64, heads=16, q_len=4, prefix_range=(256, 16384),
                   kv_dtype="bf16", seed=1005),
}


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (finite inputs only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def _e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """fp32 -> float8_e4m3fn bytes via torch's cast (round to nearest even);
    the input is clipped to the finite range first."""
    import torch

    y = np.clip(x, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    t = torch.from_numpy(y).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _normal_pool(rng: np.random.Generator, pages: int, scale: float) -> np.ndarray:
    x = rng.standard_normal((pages, PAGE_SIZE, LATENT_DIM), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def make_custom(
    name: str,
    bs: int,
    heads: int,
    q_len: int,
    seq_lens,
    kv_dtype: str = "bf16",
    seed: int = 0,
    pool_pages: Optional[int] = None,
    value_scale: float = 1.0,
    softmax_scale: float = SOFTMAX_SCALE,
    causal: bool = True,
    ctx_slack: int = 64,
    with_values: bool = True,
) -> Workload:
    """Build a workload with explicit lengths.

    The pool holds ``pool_pages`` pages (default: twice the pages the batch
    uses), in a seeded random permutation.  ``req_to_token`` has 2*bs rows;
    the batch uses a seeded choice of bs distinct rows.  Slots are
    page-aligned: token j of request b lives at slot 64*page_b[j // 64] + j % 64.
    Cells that the batch does not use hold random valid slots, so a reader
    that strays gets wrong values rather than a bad address.  With
    ``with_values=False`` only the index data is made (the pool is a single
    zero page), for tests that never read latent values.
    """
    if kv_dtype not in ("bf16", "fp8_e4m3"):
        raise ValueError(kv_dtype)
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(bs)
    if bs and seq_lens.min() < 0:
        raise ValueError("negative length")
    n_pages = [_cdiv(int(L), PAGE_SIZE) for L in seq_lens]
    used = int(sum(n_pages))
    if pool_pages is None:
        pool_pages = max(2 * used, 1)
    if pool_pages < used:
        raise ValueError("pool too small")

    rows = max(2 * bs, 1)
    rpi = rng.choice(rows, size=bs, replace=False).astype(np.int32)
    perm = rng.permutation(pool_pages).astype(np.int64)
    pages: List[np.ndarray] = []
    off = 0
    for npg in n_pages:
        pages.append(perm[off:off + npg].copy())
        off += npg

    max_len = int(seq_lens.max()) if bs else 0
    ctx_cap = _cdiv(max_len, PAGE_SIZE) * PAGE_SIZE + ctx_slack
    r2t = rng.integers(0, pool_pages * PAGE_SIZE, size=(rows, ctx_cap), dtype=np.int64).astype(np.int32)
    for b in range(bs):
        npg = n_pages[b]
        if npg == 0:
            continue
        slots = (pages[b][:, None] * PAGE_SIZE + np.arange(PAGE_SIZE)[None, :]).reshape(-1)
        r2t[rpi[b], :npg * PAGE_SIZE] = slots.astype(np.int32)

    q = rng.standard_normal((bs, q_len, heads, LATENT_DIM), dtype=np.float32)
    if value_scale != 1.0:
        q *= np.float32(value_scale)
    q_bits = _bf16_bits(q)

    if not with_values:
        kv = np.zeros((1, PAGE_SIZE, LATENT_DIM), dtype=np.uint16 if kv_dtype == "bf16" else np.uint8)
        return Workload(
            name=name, bs=bs, heads=heads, q_len=q_len, kv_dtype=kv_dtype, q_bits=q_bits, kv=kv,
            kv_descale=1.0, req_to_token=r2t, req_pool_indices=rpi, seq_lens=seq_lens,
            softmax_scale=float(np.float32(softmax_scale)), causal=causal, pages=pages)
    x = _normal_pool(rng, pool_pages, value_scale)
    if kv_dtype == "bf16":
        kv = _bf16_bits(x)
        descale = 1.0
    else:
        amax = float(np.abs(x).max()) if x.size else 1.0
        descale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
        kv = np.empty(x.shape, dtype=np.uint8)
        step = 256
        for p0 in range(0, pool_pages, step):
            kv[p0:p0 + step] = _e4m3_bytes(x[p0:p0 + step] / np.float32(descale))
    del x

    return Workload(
        name=name, bs=bs, heads=heads, q_len=q_len, kv_dtype=kv_dtype,
        q_bits=q_bits, kv=kv, kv_descale=descale, req_to_token=r2t,
        req_pool_indices=rpi, seq_lens=seq_lens, softmax_scale=float(np.float32(softmax_scale)),
        causal=causal, pages=pages,
    )


def workload_seq_lens(name: str) -> np.ndarray:
    """The KV lengths (incl. the q_len new tokens) of a named workload,
    without generating its data."""
    c = CONFIGS[name]
    rng = np.random.Generator(np.random.PCG64(c["seed"]))
    bs, q_len = c["bs"], c["q_len"]
    if "seq_lens" in c:
        return np.asarray(c["seq_lens"], dtype=np.int32)
    if "len_range" in c:
        lo, hi = c["len_range"]
        return rng.integers(lo, hi + 1, size=bs).astype(np.int32)
    lo, hi = c["prefix_range"]
    return (rng.integers(lo, hi + 1, size=bs) + q_len).astype(np.int32)


def make_workload(name: str) -> Workload:
    """One of the named workloads in ``CONFIGS``."""
    c = dict(CONFIGS[name])
    seed = c.pop("seed")
    bs = c["bs"]
    q_len = c["q_len"]
    lens = workload_seq_lens(name)
    return make_custom(
        name, bs=bs, heads=c["heads"], q_len=q_len, seq_lens=lens,
        kv_dtype=c["kv_dtype"], seed=seed + 7919, pool_pages=c.get("pool_pages"),
        value_scale=c.get("value_scale", 1.0),
    )


def poison_unused(w: Workload, kind: str = "nan") -> np.ndarray:
    """Copy of the pool where every slot no request may read is poisoned:
    the tail of each request's last page and every page no request owns.
    ``kind``: "nan" or "big" (bf16 1e4 / e4m3 448)."""
    kv = w.kv.copy()
    if w.kv_dtype == "bf16":
        val = np.uint16(0x7FC0) if kind == "nan" else _bf16_bits(np.array([1e4], np.float32))[0]
    else:
        val = np.uint8(0x7F) if kind == "nan" else np.uint8(0x7E)
    owned = np.zeros(w.pool_pages, dtype=bool)
    for b in range(w.bs):
        pg = w.pages[b]
        owned[pg] = True
        L = int(w.seq_lens[b])
        if len(pg) and L % PAGE_SIZE:
            kv[pg[-1], L % PAGE_SIZE:, :] = val
    kv[~owned] = val
    return kv
