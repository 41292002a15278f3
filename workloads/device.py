"""Copy a seeded workload to GPU tensors (bits unchanged, no arithmetic)."""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .synth import Workload


@dataclass
class DeviceWorkload:
    q: torch.Tensor                 # bf16 [bs, q_len, H, 576]
    kv: torch.Tensor                # bf16 or uint8 [pages, 64, 576]
    req_to_token: torch.Tensor      # int32
    req_pool_indices: torch.Tensor  # int32 [bs]
    seq_lens: torch.Tensor          # int32 [bs]
    kv_descale: Optional[torch.Tensor]  # fp32 [1] for fp8, else None
    kv_dtype: str


def to_device(w: Workload, device="cuda", kv: Optional[np.ndarray] = None) -> DeviceWorkload:
    kv = w.kv if kv is None else kv
    q = torch.from_numpy(np.ascontiguousarray(w.q_bits).view(np.int16)).to(device).view(torch.bfloat16)
    if w.kv_dtype == "bf16":
        kvt = torch.from_numpy(np.ascontiguousarray(kv).view(np.int16)).to(device).view(torch.bfloat16)
        descale = None
    else:
        kvt = torch.from_numpy(np.ascontiguousarray(kv)).to(device)
        descale = torch.tensor([w.kv_descale], dtype=torch.float32, device=device)
    return DeviceWorkload(
        q=q, kv=kvt,
        req_to_token=torch.from_numpy(np.ascontiguousarray(w.req_to_token)).to(device),
        req_pool_indices=torch.from_numpy(np.ascontiguousarray(w.req_pool_indices)).to(device),
        seq_lens=torch.from_numpy(np.ascontiguousarray(w.seq_lens)).to(device),
        kv_descale=descale, kv_dtype=w.kv_dtype)
