"""Helpers shared by the GPU tests: uploads of seeded inputs and error metrics."""
from __future__ import annotations

import numpy as np
import torch


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a cuda bfloat16 tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return dev_bf16(x)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 cuda tensor -> uint16 bit patterns on the host."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return host_bits(t)
    return t.cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def rowwise_rel(o: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||o - ref||_inf / ||ref||_inf (last axis is the row)."""
    num = np.max(np.abs(o - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.max(num / den))


def say(*a) -> None:
    print(*a, flush=True)
