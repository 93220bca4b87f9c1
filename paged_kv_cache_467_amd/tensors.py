"""Move a workloads.DecodeBatch to device tensors and bring results back.

Plumbing only: element bits are reinterpreted (int16 -> float16/bfloat16),
never converted.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def to_device(bits: np.ndarray, dtype: str, device) -> torch.Tensor:
    a = np.ascontiguousarray(bits)
    if dtype == "f32":
        return torch.from_numpy(a.view(np.float32)).to(device)
    return torch.from_numpy(a.view(np.int16)).to(device).view(TORCH_DTYPE[dtype])


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy array of stored bits (float32 or uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def int32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


@dataclass
class DeviceBatch:
    query: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    new_key: torch.Tensor
    new_value: torch.Tensor
    slot_mapping: torch.Tensor
    out: torch.Tensor


def device_batch(batch, device="cuda") -> DeviceBatch:
    dt = batch.dtype
    q = to_device(batch.query, dt, device)
    return DeviceBatch(
        query=q,
        key_cache=to_device(batch.key_cache, dt, device),
        value_cache=to_device(batch.value_cache, dt, device),
        block_tables=int32(batch.block_tables, device),
        context_lens=int32(batch.context_lens, device),
        new_key=to_device(batch.new_key, dt, device),
        new_value=to_device(batch.new_value, dt, device),
        slot_mapping=int32(batch.slot_mapping, device),
        out=torch.empty_like(q),
    )


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Stored bits -> float64 values (exact)."""
    a = np.ascontiguousarray(bits)
    if dtype == "f32":
        return a.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
