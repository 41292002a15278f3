"""MI355X (gfx950) MLA paged-KV decode: thin Python binding of the C ABI.

Every function here only checks tensor shapes/dtypes/devices, takes raw
device pointers and the current HIP stream, and calls the same-named entry
point of ``libmla_decode.so`` (declared in ``include/mla_decode.h``).  All
arithmetic runs in the library's HIP kernels; nothing falls back to torch or
to the CPU.  PyTorch is used for device memory and streams only.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import MLAError, MLA_KV_BF16, MLA_KV_FP8_E4M3  # noqa: F401

PAGE_SIZE = 64
LATENT_DIM = 576
V_DIM = 512

_KV_DTYPES = {"bf16": MLA_KV_BF16, "fp8_e4m3": MLA_KV_FP8_E4M3}


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_gpu(t: torch.Tensor) -> bool:
    return t.is_cuda


def _need(t: torch.Tensor, name: str, dtypes, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not _on_gpu(t):
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _same_device(*named):
    """All given tensors (None skipped) on one device."""
    devs = {(n, t.device) for n, t in named if t is not None}
    if len({d for _, d in devs}) > 1:
        raise ValueError("tensors on different devices: " +
                         ", ".join(f"{n}={d}" for n, d in sorted(devs, key=str)))


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")


def _kv_code(kv_dtype) -> int:
    if isinstance(kv_dtype, int):
        return kv_dtype
    try:
        return _KV_DTYPES[kv_dtype]
    except KeyError:
        raise ValueError(f"unknown kv_dtype {kv_dtype!r}") from None


def abi_version() -> int:
    return int(_lib.lib().mla_abi_version())


def device_num_cus() -> int:
    return int(_lib.lib().mla_device_num_cus())


def max_total_splits(bs: int, num_parts: int) -> int:
    return int(_lib.lib().mla_max_total_splits(bs, num_parts))


def workspace_bytes(bs: int, rows_per_req: int, num_parts: int) -> int:
    """Bytes of partial_o (bf16) + partial_lse (fp32) for bs + num_parts slots
    (mla_workspace_bytes)."""
    return int(_lib.lib().mla_workspace_bytes(bs, rows_per_req, num_parts))


def build_block_table(req_to_token: torch.Tensor, req_pool_indices: torch.Tensor,
                      seq_lens: torch.Tensor, width: int, pad_value: int = -1,
                      max_seq_len_hint: int = -1, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """int32 [bs, width] block table (mla_build_block_table)."""
    _need(req_to_token, "req_to_token", (torch.int32,), 2)
    _need(req_pool_indices, "req_pool_indices", (torch.int32,), 1)
    _need(seq_lens, "seq_lens", (torch.int32,), 1)
    bs = seq_lens.shape[0]
    if out is None:
        out = torch.empty((bs, width), dtype=torch.int32, device=seq_lens.device)
    _need(out, "out", (torch.int32,), 2)
    _shape(req_pool_indices, "req_pool_indices", (bs,))
    if out.shape[0] < bs:
        raise ValueError(f"out has {out.shape[0]} rows, needs {bs}")
    _same_device(("req_to_token", req_to_token), ("req_pool_indices", req_pool_indices),
                 ("seq_lens", seq_lens), ("out", out))
    _lib.check(_lib.lib().mla_build_block_table(
        _p(req_to_token), req_to_token.shape[0], req_to_token.stride(0), _p(req_pool_indices),
        _p(seq_lens), bs, PAGE_SIZE, _p(out), out.shape[1], pad_value, max_seq_len_hint,
        _stream(stream)))
    return out


def plan_splits(seq_lens: torch.Tensor, rows_per_req: int, num_parts: Optional[int] = None,
                kv_dtype="bf16", tile_plan: Optional[torch.Tensor] = None,
                split_indptr: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(tile_plan int32 [num_parts, 8], split_indptr int32 [bs+1]) (mla_plan_splits).
    ``num_parts`` defaults to the device's CU count."""
    _need(seq_lens, "seq_lens", (torch.int32,), 1)
    bs = seq_lens.shape[0]
    if num_parts is None:
        num_parts = device_num_cus()
    if tile_plan is None:
        tile_plan = torch.empty((num_parts, 8), dtype=torch.int32, device=seq_lens.device)
    if split_indptr is None:
        split_indptr = torch.empty((bs + 1,), dtype=torch.int32, device=seq_lens.device)
    _need(tile_plan, "tile_plan", (torch.int32,), 2)
    _need(split_indptr, "split_indptr", (torch.int32,), 1)
    if tile_plan.shape[0] < num_parts or tile_plan.shape[1] != 8 or \
            split_indptr.shape[0] < bs + 1:
        raise ValueError("plan buffers too small")
    _same_device(("seq_lens", seq_lens), ("tile_plan", tile_plan),
                 ("split_indptr", split_indptr))
    _lib.check(_lib.lib().mla_plan_splits(_p(seq_lens), bs, rows_per_req, num_parts,
                                          _kv_code(kv_dtype), _p(tile_plan), _p(split_indptr),
                                          _stream(stream)))
    return tile_plan[:num_parts], split_indptr[:bs + 1]


def plan_fixed_splits(seq_lens: torch.Tensor, tile_pages: int = 32,
                      max_parts: Optional[int] = None, max_seq_len_hint: int = -1,
                      tile_plan: Optional[torch.Tensor] = None,
                      split_indptr: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Deterministic fixed-tile plan (mla_plan_fixed_splits): every request cut at
    multiples of ``tile_pages`` pages (default 32 = 2048 tokens).  ``max_parts``
    defaults to the bound for ``max_seq_len_hint``, which is then required.
    Returns (tile_plan int32 [max_parts, 8], split_indptr int32 [bs + 1])."""
    _need(seq_lens, "seq_lens", (torch.int32,), 1)
    bs = seq_lens.shape[0]
    if max_parts is None:
        if max_seq_len_hint < 0:
            raise ValueError("plan_fixed_splits needs max_parts or max_seq_len_hint")
        max_parts = max(1, int(_lib.lib().mla_fixed_split_parts_bound(bs, max_seq_len_hint,
                                                                       tile_pages)))
    if tile_plan is None:
        tile_plan = torch.empty((max_parts, 8), dtype=torch.int32, device=seq_lens.device)
    if split_indptr is None:
        split_indptr = torch.empty((bs + 1,), dtype=torch.int32, device=seq_lens.device)
    _need(tile_plan, "tile_plan", (torch.int32,), 2)
    _need(split_indptr, "split_indptr", (torch.int32,), 1)
    if tile_plan.shape != (max_parts, 8) or split_indptr.shape != (bs + 1,):
        raise ValueError("tile_plan must be [max_parts, 8] and split_indptr [bs + 1]")
    _same_device(("seq_lens", seq_lens), ("tile_plan", tile_plan),
                 ("split_indptr", split_indptr))
    _lib.check(_lib.lib().mla_plan_fixed_splits(_p(seq_lens), bs, tile_pages, max_parts,
                                                max_seq_len_hint, _p(tile_plan),
                                                _p(split_indptr), _stream(stream)))
    return tile_plan, split_indptr


def plan_fixed_packed(seq_lens: torch.Tensor, rows_per_req: int, tile_pages: int = 32,
                      num_parts: Optional[int] = None,
                      tile_plan: Optional[torch.Tensor] = None,
                      split_indptr: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The fixed tiles of plan_fixed_splits packed into ``num_parts`` parts of
    about equal cost (mla_plan_fixed_packed; default: one per CU).  The decode
    needs partial slots for every tile: size its workspace with
    partial_buffers(..., num_slots=split_indptr[bs]) or an upper bound
    (fixed_split_parts_bound).  Returns (tile_plan int32 [num_parts, 8],
    split_indptr int32 [bs + 1])."""
    _need(seq_lens, "seq_lens", (torch.int32,), 1)
    bs = seq_lens.shape[0]
    if num_parts is None:
        num_parts = device_num_cus()
    if tile_plan is None:
        tile_plan = torch.empty((num_parts, 8), dtype=torch.int32, device=seq_lens.device)
    if split_indptr is None:
        split_indptr = torch.empty((bs + 1,), dtype=torch.int32, device=seq_lens.device)
    _need(tile_plan, "tile_plan", (torch.int32,), 2)
    _need(split_indptr, "split_indptr", (torch.int32,), 1)
    if tile_plan.shape != (num_parts, 8) or split_indptr.shape != (bs + 1,):
        raise ValueError("tile_plan must be [num_parts, 8] and split_indptr [bs + 1]")
    _same_device(("seq_lens", seq_lens), ("tile_plan", tile_plan),
                 ("split_indptr", split_indptr))
    _lib.check(_lib.lib().mla_plan_fixed_packed(_p(seq_lens), bs, tile_pages, rows_per_req,
                                                num_parts, _p(tile_plan), _p(split_indptr),
                                                _stream(stream)))
    return tile_plan, split_indptr


def fixed_split_parts_bound(bs: int, max_seq_len: int, tile_pages: int = 32) -> int:
    """Most tiles (pieces) a fixed-tile plan of bs requests of up to
    max_seq_len tokens can have (mla_fixed_split_parts_bound)."""
    return int(_lib.lib().mla_fixed_split_parts_bound(bs, max_seq_len, tile_pages))


def build_table_and_plan(req_to_token: torch.Tensor, req_pool_indices: torch.Tensor,
                         seq_lens: torch.Tensor, width: int, rows_per_req: int,
                         num_parts: Optional[int] = None, kv_dtype="bf16", pad_value: int = -1,
                         max_seq_len_hint: int = -1, out: Optional[torch.Tensor] = None,
                         tile_plan: Optional[torch.Tensor] = None,
                         split_indptr: Optional[torch.Tensor] = None, stream=None):
    """(block_table, tile_plan, split_indptr) from one launch
    (mla_build_table_and_plan): the results of build_block_table and
    plan_splits."""
    _need(req_to_token, "req_to_token", (torch.int32,), 2)
    _need(req_pool_indices, "req_pool_indices", (torch.int32,), 1)
    _need(seq_lens, "seq_lens", (torch.int32,), 1)
    bs = seq_lens.shape[0]
    dev = seq_lens.device
    if num_parts is None:
        num_parts = device_num_cus()
    if out is None:
        out = torch.empty((bs, width), dtype=torch.int32, device=dev)
    if tile_plan is None:
        tile_plan = torch.empty((num_parts, 8), dtype=torch.int32, device=dev)
    if split_indptr is None:
        split_indptr = torch.empty((bs + 1,), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.int32,), 2)
    _need(tile_plan, "tile_plan", (torch.int32,), 2)
    _need(split_indptr, "split_indptr", (torch.int32,), 1)
    if tile_plan.shape[0] < num_parts or tile_plan.shape[1] != 8 or \
            split_indptr.shape[0] < bs + 1:
        raise ValueError("plan buffers too small")
    _shape(req_pool_indices, "req_pool_indices", (bs,))
    if out.shape[0] < bs:
        raise ValueError(f"out has {out.shape[0]} rows, needs {bs}")
    _same_device(("req_to_token", req_to_token), ("req_pool_indices", req_pool_indices),
                 ("seq_lens", seq_lens), ("out", out), ("tile_plan", tile_plan),
                 ("split_indptr", split_indptr))
    _lib.check(_lib.lib().mla_build_table_and_plan(
        _p(req_to_token), req_to_token.shape[0], req_to_token.stride(0), _p(req_pool_indices),
        _p(seq_lens), bs, PAGE_SIZE, _p(out), out.shape[1], pad_value, max_seq_len_hint,
        rows_per_req, num_parts, _kv_code(kv_dtype), _p(tile_plan), _p(split_indptr),
        _stream(stream)))
    return out, tile_plan[:num_parts], split_indptr[:bs + 1]


def partial_buffers(bs: int, rows_per_req: int, num_parts: int, device="cuda",
                    num_slots: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Workspace for split pieces: partial o bf16 [S, R, 512] and partial lse
    fp32 [S, R], S = bs + num_parts (the most pieces of a balanced plan), or
    at least ``num_slots`` (a fixed-tile plan: its number of tiles)."""
    slots = max_total_splits(bs, num_parts)
    if num_slots is not None:
        slots = max(slots, int(num_slots))
    return (torch.empty((slots, rows_per_req, V_DIM), dtype=torch.bfloat16, device=device),
            torch.empty((slots, rows_per_req), dtype=torch.float32, device=device))


def _check_decode(q, q_dtypes, kv_cache, code, block_table, seq_lens, tile_plan, split_indptr,
                  out, lse, kv_descale, partial_o=None, partial_lse=None, q_descale=None):
    """Shape, dtype and device checks shared by the decode entry points;
    returns (bs, q_len, heads)."""
    _need(q, "q", q_dtypes, 4)
    kv_ok = (torch.bfloat16, torch.int16, torch.uint16) if code == MLA_KV_BF16 else (
        torch.uint8, torch.float8_e4m3fn)
    _need(kv_cache, "kv_cache", kv_ok, 3)
    if kv_cache.shape[1:] != (PAGE_SIZE, LATENT_DIM):
        raise ValueError(f"kv_cache must be [pages, 64, 576], got {tuple(kv_cache.shape)}")
    bs, q_len, heads, d = q.shape
    if d != LATENT_DIM:
        raise ValueError("q must be [bs, q_len, heads, 576]")
    _need(block_table, "block_table", (torch.int32,), 2)
    _need(seq_lens, "seq_lens", (torch.int32,), 1)
    _need(tile_plan, "tile_plan", (torch.int32,), 2)
    _need(split_indptr, "split_indptr", (torch.int32,), 1)
    _need(out, "out", (torch.bfloat16,), 4)
    _shape(out, "out", (bs, q_len, heads, V_DIM))
    if lse is not None:
        _need(lse, "lse", (torch.float32,), 3)
        _shape(lse, "lse", (bs, q_len, heads))
    for name, t in (("kv_descale", kv_descale), ("q_descale", q_descale)):
        if t is not None:
            _need(t, name, (torch.float32,))
            if t.numel() < 1:
                raise ValueError(f"{name} must hold one value")
    rows = q_len * heads
    if partial_o is not None or partial_lse is not None:
        _need(partial_o, "partial_o", (torch.bfloat16,), 3)
        _need(partial_lse, "partial_lse", (torch.float32,), 2)
        if partial_o.shape[1:] != (rows, V_DIM) or partial_lse.shape != (partial_o.shape[0], rows):
            raise ValueError("partial buffers do not match q")
    if block_table.shape[0] < bs:
        raise ValueError(f"block_table has {block_table.shape[0]} rows, needs {bs}")
    _shape(seq_lens, "seq_lens", (bs,))
    if split_indptr.shape[0] < bs + 1:
        raise ValueError(f"split_indptr needs bs + 1 = {bs + 1} entries")
    if tile_plan.shape[1] != 8:
        raise ValueError("tile_plan must be [num_parts, 8]")
    _same_device(("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                 ("seq_lens", seq_lens), ("tile_plan", tile_plan), ("split_indptr", split_indptr),
                 ("partial_o", partial_o), ("partial_lse", partial_lse), ("out", out),
                 ("lse", lse), ("kv_descale", kv_descale), ("q_descale", q_descale))
    return bs, q_len, heads


def mla_decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
               seq_lens: torch.Tensor, tile_plan: torch.Tensor, split_indptr: torch.Tensor,
               softmax_scale: float, *, partial_o: torch.Tensor, partial_lse: torch.Tensor,
               out: torch.Tensor, lse: Optional[torch.Tensor] = None, kv_dtype="bf16",
               kv_descale: Optional[torch.Tensor] = None, causal: bool = True,
               stream=None) -> None:
    """Split attention over the plan's pieces (mla_decode)."""
    code = _kv_code(kv_dtype)
    bs, q_len, heads = _check_decode(q, (torch.bfloat16,), kv_cache, code, block_table, seq_lens,
                                     tile_plan, split_indptr, out, lse, kv_descale, partial_o,
                                     partial_lse)
    _lib.check(_lib.lib().mla_decode(
        _p(q), bs, q_len, heads, _p(kv_cache), code, kv_cache.shape[0], _p(block_table),
        block_table.shape[1], _p(seq_lens), _p(tile_plan), tile_plan.shape[0], _p(split_indptr),
        float(softmax_scale), 1 if causal else 0, _p(kv_descale), _p(partial_o), _p(partial_lse),
        partial_o.shape[0], _p(out), _p(lse), _stream(stream)))


def mla_decode_q8(q_fp8: torch.Tensor, q_descale: torch.Tensor, kv_cache: torch.Tensor,
                  block_table: torch.Tensor, seq_lens: torch.Tensor, tile_plan: torch.Tensor,
                  split_indptr: torch.Tensor, softmax_scale: float, *, kv_descale: torch.Tensor,
                  partial_o: torch.Tensor, partial_lse: torch.Tensor, out: torch.Tensor,
                  lse: Optional[torch.Tensor] = None, causal: bool = True,
                  stream=None) -> None:
    """mla_decode with an e4m3 query (codes from quantize_q_fp8, value
    code * q_descale) over an e4m3 cache (mla_decode_q8)."""
    if q_descale is None or kv_descale is None:
        raise ValueError("q_descale and kv_descale are required")
    bs, q_len, heads = _check_decode(q_fp8, (torch.uint8, torch.float8_e4m3fn), kv_cache,
                                     MLA_KV_FP8_E4M3, block_table, seq_lens, tile_plan,
                                     split_indptr, out, lse, kv_descale, partial_o, partial_lse,
                                     q_descale)
    _lib.check(_lib.lib().mla_decode_q8(
        _p(q_fp8), _p(q_descale), bs, q_len, heads, _p(kv_cache), kv_cache.shape[0],
        _p(block_table), block_table.shape[1], _p(seq_lens), _p(tile_plan), tile_plan.shape[0],
        _p(split_indptr), float(softmax_scale), 1 if causal else 0, _p(kv_descale),
        _p(partial_o), _p(partial_lse), partial_o.shape[0], _p(out), _p(lse), _stream(stream)))


def mla_decode_static(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                      seq_lens: torch.Tensor, tile_plan: torch.Tensor, split_indptr: torch.Tensor,
                      softmax_scale: float, *, out: torch.Tensor,
                      lse: Optional[torch.Tensor] = None, kv_dtype="bf16",
                      kv_descale: Optional[torch.Tensor] = None, causal: bool = True,
                      stream=None) -> None:
    """Decode and merge with the library's own partial-state workspace
    (mla_decode_static): allocates nothing, takes no workspace."""
    code = _kv_code(kv_dtype)
    bs, q_len, heads = _check_decode(q, (torch.bfloat16,), kv_cache, code, block_table, seq_lens,
                                     tile_plan, split_indptr, out, lse, kv_descale)
    _lib.check(_lib.lib().mla_decode_static(
        _p(q), bs, q_len, heads, _p(kv_cache), code, kv_cache.shape[0], _p(block_table),
        block_table.shape[1], _p(seq_lens), _p(tile_plan), tile_plan.shape[0], _p(split_indptr),
        float(softmax_scale), 1 if causal else 0, _p(kv_descale), _p(out), _p(lse),
        _stream(stream)))


def time_next_decode(start: torch.cuda.Event, stop: torch.cuda.Event) -> None:
    """The next mla_decode on this thread records ``start``/``stop`` at its
    kernel's own begin and end (mla_decode_time_next_launch).  The events
    must have been recorded once before, so that they exist."""
    _lib.check(_lib.lib().mla_decode_time_next_launch(ctypes.c_void_p(start.cuda_event),
                                                      ctypes.c_void_p(stop.cuda_event)))


def merge_states(partial_o: torch.Tensor, partial_lse: torch.Tensor, split_indptr: torch.Tensor,
                 out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """Exact LSE merge of split pieces into out (bf16) and lse (mla_merge_states).
    partial_o: bf16 [slots, R, 512]; partial_lse: fp32 [slots, R]."""
    _need(partial_o, "partial_o", (torch.bfloat16,), 3)
    _need(partial_lse, "partial_lse", (torch.float32,), 2)
    _need(split_indptr, "split_indptr", (torch.int32,), 1)
    _need(out, "out", (torch.bfloat16,))
    bs = split_indptr.shape[0] - 1
    if bs < 1:
        raise ValueError("split_indptr must have at least 2 entries")
    slots, rows, dv = partial_o.shape
    if dv != V_DIM:
        raise ValueError("partial_o rows must be 512 wide")
    _shape(partial_lse, "partial_lse", (slots, rows))
    if out.numel() != bs * rows * V_DIM:
        raise ValueError("out does not match split_indptr and partial_o")
    if lse is not None:
        _need(lse, "lse", (torch.float32,))
        if lse.numel() != bs * rows:
            raise ValueError("lse does not match")
    _same_device(("partial_o", partial_o), ("partial_lse", partial_lse),
                 ("split_indptr", split_indptr), ("out", out), ("lse", lse))
    _lib.check(_lib.lib().mla_merge_states(_p(partial_o), _p(partial_lse), slots,
                                           _p(split_indptr), bs, rows, V_DIM, _p(out), _p(lse),
                                           _stream(stream)))


def decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, softmax_scale: float, *, kv_dtype="bf16",
           kv_descale: Optional[torch.Tensor] = None, causal: bool = True,
           num_parts: Optional[int] = None, plan=None, workspace=None,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           q_descale: Optional[torch.Tensor] = None,
           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode (mla_decode_q8 for a uint8 / e4m3 query, which needs
    ``q_descale`` and an fp8 cache) followed by mla_merge_states; returns
    (out bf16 [bs, q_len, H, 512], lse fp32 [bs, q_len, H]).  ``plan`` =
    (tile_plan, split_indptr) from plan_splits, ``workspace`` = (partial_o,
    partial_lse) from partial_buffers."""
    bs, q_len, heads, _ = q.shape
    rows = q_len * heads
    if plan is None:
        plan = plan_splits(seq_lens, rows, num_parts, kv_dtype, stream=stream)
    tile_plan, split_indptr = plan
    if workspace is None:
        workspace = partial_buffers(bs, rows, tile_plan.shape[0], q.device)
    if out is None:
        out = torch.empty((bs, q_len, heads, V_DIM), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((bs, q_len, heads), dtype=torch.float32, device=q.device)
    if q.dtype in (torch.uint8, torch.float8_e4m3fn):
        if _kv_code(kv_dtype) != MLA_KV_FP8_E4M3:
            raise ValueError("an e4m3 query needs kv_dtype='fp8_e4m3'")
        mla_decode_q8(q, q_descale, kv_cache, block_table, seq_lens, tile_plan, split_indptr,
                      softmax_scale, kv_descale=kv_descale, partial_o=workspace[0],
                      partial_lse=workspace[1], out=out, lse=lse, causal=causal, stream=stream)
    else:
        mla_decode(q, kv_cache, block_table, seq_lens, tile_plan, split_indptr, softmax_scale,
                   partial_o=workspace[0], partial_lse=workspace[1], out=out, lse=lse,
                   kv_dtype=kv_dtype, kv_descale=kv_descale, causal=causal, stream=stream)
    merge_states(workspace[0], workspace[1], split_indptr, out, lse, stream=stream)
    return out, lse


def set_kv_buffer(kv_cache: torch.Tensor, out_cache_loc: torch.Tensor, k: torch.Tensor, *,
                  kv_dtype="bf16", kv_scale: Optional[torch.Tensor] = None,
                  stream=None) -> None:
    """Store latent rows ``k`` (bf16 [n, 576], or a row-strided view whose rows
    start 16-byte aligned) at pool slots ``out_cache_loc`` (int64 [n]) of
    ``kv_cache`` [pages, 64, 576], in place (mla_set_kv_buffer).  For an fp8
    cache ``kv_scale`` is the device fp32 per-tensor scale."""
    code = _kv_code(kv_dtype)
    kv_ok = (torch.bfloat16, torch.int16, torch.uint16) if code == MLA_KV_BF16 else (
        torch.uint8, torch.float8_e4m3fn)
    _need(kv_cache, "kv_cache", kv_ok, 3)
    if kv_cache.shape[1:] != (PAGE_SIZE, LATENT_DIM):
        raise ValueError(f"kv_cache must be [pages, 64, 576], got {tuple(kv_cache.shape)}")
    _need(out_cache_loc, "out_cache_loc", (torch.int64,), 1)
    if not isinstance(k, torch.Tensor) or not _on_gpu(k) or k.dtype != torch.bfloat16:
        raise TypeError("k must be a bf16 GPU tensor")
    if k.dim() != 2 or k.shape[1] != LATENT_DIM or k.stride(1) != 1:
        raise ValueError("k must be [n, 576] with unit column stride")
    if k.shape[0] != out_cache_loc.shape[0]:
        raise ValueError("k and out_cache_loc disagree on the token count")
    if kv_scale is not None:
        _need(kv_scale, "kv_scale", (torch.float32,))
    _lib.check(_lib.lib().mla_set_kv_buffer(
        _p(k), k.stride(0) if k.shape[0] > 1 else LATENT_DIM, _p(out_cache_loc), k.shape[0],
        _p(kv_cache), code, kv_cache.shape[0], _p(kv_scale), _stream(stream)))


def quantize_q_fp8(q: torch.Tensor, q_scale: torch.Tensor, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """e4m3fn codes (uint8, q's shape) of q / q_scale (mla_quantize_q_fp8): the
    query quantisation of the fp8 branch.  q: bf16 [..., 576], contiguous;
    q_scale: device fp32 scalar."""
    _need(q, "q", (torch.bfloat16,))
    if q.shape[-1] != LATENT_DIM:
        raise ValueError("q rows must be 576 wide")
    _need(q_scale, "q_scale", (torch.float32,))
    if out is None:
        out = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    _need(out, "out", (torch.uint8, torch.float8_e4m3fn))
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    rows = q.numel() // LATENT_DIM
    _lib.check(_lib.lib().mla_quantize_q_fp8(_p(q), LATENT_DIM, rows, _p(q_scale), _p(out),
                                             _stream(stream)))
    return out
