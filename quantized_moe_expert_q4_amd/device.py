"""Device-memory plumbing with PyTorch: aligned buffers and uploads.

PyTorch only provides memory and streams here; no part of the computation.
"""
from __future__ import annotations

import numpy as np
import torch

SLOT_ALIGN = 4096


def aligned_empty(nbytes: int, align: int = SLOT_ALIGN, device: str = "cuda") -> torch.Tensor:
    """uint8 device tensor of ``nbytes`` whose data pointer is ``align``-aligned.

    Over-allocates by ``align`` bytes and returns a view at the first aligned
    offset; the view keeps the allocation alive.
    """
    raw = torch.empty(nbytes + align, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % align
    view = raw[off:off + nbytes]
    assert view.data_ptr() % align == 0
    return view


def upload_slots(slots: np.ndarray, device: str = "cuda") -> torch.Tensor:
    """Copy a ``uint8 [num_slots, slot_stride]`` host array into aligned device memory."""
    flat = np.ascontiguousarray(slots, dtype=np.uint8).reshape(-1)
    dev = aligned_empty(flat.size, SLOT_ALIGN, device)
    dev.copy_(torch.from_numpy(flat))
    return dev


def upload_bf16_bits(bits: np.ndarray, device: str = "cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bf16 device tensor of the same shape."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)
