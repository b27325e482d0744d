"""Seeded generators for expert slots, activations and routing ids.

Every generator takes a ``numpy.random.Generator`` and draws in a fixed,
documented order, so a seed fixes every byte.  Workload shapes follow the
five benchmark configurations of the Q4 expert gate/up path:

1. one expert, H=256, I=128, M=1, scales U[0.005, 0.02];
2. one expert, H=4096, I=1536, M=1, one 4 KiB-aligned contiguous slot;
3. as 2 with M=8;
4. 64 expert slots (H=6144, I=2048) in one buffer, M=32 tokens, top-8 ids
   drawn without replacement per token;
5. one expert, H=7168, I=4096, M in {1, 4, 16, 32}; 1% of gate rows and 1% of
   up rows forced to the all-8 nibble pattern (zero weights), 1% of x entries
   set to +-9984 (the bf16 value nearest 1e4), scales U[0.001, 0.05].

Slot byte layout (an expert slot as described on diff page 52/51 of
@mlx-bun/inference 1.0.0, kernels/glm52/layout.ts: byte offsets of each field
from the slot base): ``[gate words | up words | gate scales | up scales]``
back to back, padded to a multiple of 4096 bytes.  Gate and up words are
little-endian uint32 ``[I][H/8]``; scales are little-endian float32 ``[I]``.

x values are standard normal float32 samples rounded to nearest-even bf16 by
torch's CPU conversion (a library routine, so the generator holds none of the
arithmetic under test).
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

OFFSET_ABSENT = (1 << 64) - 1

# bf16 bit patterns of +9984 and -9984 (9984 = 156 * 64 is the bf16 value
# nearest to 1e4).
BF16_POS_9984 = 0x461C
BF16_NEG_9984 = 0xC61C
ALL_EIGHT_WORD = 0x88888888


@dataclass(frozen=True)
class SlotLayout:
    """Byte offsets of each field from the slot base (down fields optional)."""

    slot_bytes: int
    gate_weight_offset: int
    up_weight_offset: int
    gate_scale_offset: int
    up_scale_offset: int
    down_weight_offset: int = OFFSET_ABSENT
    down_scale_offset: int = OFFSET_ABSENT


def _wbytes(rows: int, K: int, fmt: str) -> int:
    """Bytes of a ``[rows, K]`` weight matrix: packed nibbles (q4) or int8 (q8)."""
    return rows * K // 2 if fmt == "q4" else rows * K


def contiguous_layout(H: int, I: int, align: int = 4096, fmt: str = "q4") -> SlotLayout:
    """Gate words, up words, gate scales, up scales back to back.

    Each field starts on a 16-byte boundary (a no-op for the five workloads,
    whose fields are all multiples of 16 bytes long).  ``fmt="q8"`` sizes
    the weight fields for one int8 weight per byte.
    """
    def up16(n):
        return (n + 15) // 16 * 16

    wbytes = _wbytes(I, H, fmt)
    gate_w = 0
    up_w = up16(wbytes)
    gate_s = up16(up_w + wbytes)
    up_s = up16(gate_s + 4 * I)
    end = up_s + 4 * I
    slot = (end + align - 1) // align * align
    return SlotLayout(slot, gate_w, up_w, gate_s, up_s)


def expert_layout(H: int, I: int, align: int = 4096, fmt: str = "q4") -> SlotLayout:
    """A whole-expert slot: gate words, up words, down words, gate scales, up
    scales, down scales back to back (16-byte aligned fields), padded to
    ``align``.  Down words are ``[H][I/8]`` (int8 ``[H][I]`` for q8), down
    scales ``[H]``."""
    def up16(n):
        return (n + 15) // 16 * 16

    wbytes = _wbytes(I, H, fmt)
    gate_w = 0
    up_w = up16(wbytes)
    down_w = up16(up_w + wbytes)
    gate_s = up16(down_w + wbytes)
    up_s = up16(gate_s + 4 * I)
    down_s = up16(up_s + 4 * I)
    end = down_s + 4 * H
    slot = (end + align - 1) // align * align
    return SlotLayout(slot, gate_w, up_w, gate_s, up_s, down_w, down_s)


def pack_nibbles(nibbles: np.ndarray) -> np.ndarray:
    """Pack a ``[R, H]`` array of values 0..15 into ``[R, H/8]`` uint32 words.

    Nibble ``k`` of a row sits in word ``k // 8`` at bits ``4*(k % 8)``.
    Used by tests that want to choose weights nibble by nibble.
    """
    nib = np.asarray(nibbles, dtype=np.uint32)
    R, H = nib.shape
    assert H % 8 == 0
    words = np.zeros((R, H // 8), dtype=np.uint32)
    for p in range(8):
        words |= (nib[:, p::8] & 0xF) << np.uint32(4 * p)
    return words


def write_slot(layout: SlotLayout, H: int, I: int, gate_words, up_words, gate_scales, up_scales,
               out: Optional[np.ndarray] = None) -> np.ndarray:
    """Lay given gate/up words ``[I, H/8]`` and scales ``[I]`` into a slot."""
    if out is None:
        out = np.zeros(layout.slot_bytes, dtype=np.uint8)
    wb = I * H // 2
    gw = np.asarray(gate_words, dtype="<u4").reshape(I, H // 8)
    uw = np.asarray(up_words, dtype="<u4").reshape(I, H // 8)
    out[layout.gate_weight_offset:layout.gate_weight_offset + wb] = gw.view(np.uint8).ravel()
    out[layout.up_weight_offset:layout.up_weight_offset + wb] = uw.view(np.uint8).ravel()
    out[layout.gate_scale_offset:layout.gate_scale_offset + 4 * I] = \
        np.asarray(gate_scales, dtype="<f4").view(np.uint8)
    out[layout.up_scale_offset:layout.up_scale_offset + 4 * I] = \
        np.asarray(up_scales, dtype="<f4").view(np.uint8)
    return out


def _uniform_words(rng: np.random.Generator, I: int, H: int) -> np.ndarray:
    return rng.integers(0, 1 << 32, size=(I, H // 8), dtype=np.uint64).astype(np.uint32)


def _uniform_weights(rng: np.random.Generator, rows: int, K: int, fmt: str) -> np.ndarray:
    """A weight matrix as raw little-endian bytes: uniform nibbles packed in
    words (q4), or uniform int8 in [-128, 127] (q8, drawn as 32-bit words
    whose bytes are the weights, row-major)."""
    if fmt == "q4":
        return _uniform_words(rng, rows, K).astype("<u4").view(np.uint8).reshape(rows, K // 2)
    w = rng.integers(0, 1 << 32, size=(rows, (K + 3) // 4), dtype=np.uint64).astype("<u4")
    return w.view(np.uint8).reshape(rows, -1)[:, :K]


def _zero_weight_row(fmt: str, K: int) -> np.ndarray:
    """Bytes of a row of zero weights: all-8 nibbles (q4) or zero bytes (q8)."""
    return np.full(K // 2, 0x88, np.uint8) if fmt == "q4" else np.zeros(K, np.uint8)


def fill_slot(
    rng: np.random.Generator,
    H: int,
    I: int,
    layout: SlotLayout,
    scale_range=(0.005, 0.02),
    zero_row_fraction: float = 0.0,
    out: Optional[np.ndarray] = None,
    fmt: str = "q4",
) -> np.ndarray:
    """Draw one expert slot into a uint8 array of ``layout.slot_bytes``.

    Draw order: gate words, up words, gate scales, up scales, then (if
    ``zero_row_fraction``) the gate rows and the up rows forced to all-8.
    When the layout has down fields, then down words ``[H, I/8]``, down
    scales ``[H]`` and (if ``zero_row_fraction``) the down rows forced to
    all-8.  Padding bytes are zero.
    """
    if out is None:
        out = np.zeros(layout.slot_bytes, dtype=np.uint8)
    else:
        out[:] = 0
    gw = _uniform_weights(rng, I, H, fmt)
    uw = _uniform_weights(rng, I, H, fmt)
    lo, hi = scale_range
    gs = rng.uniform(lo, hi, size=I).astype(np.float32)
    us = rng.uniform(lo, hi, size=I).astype(np.float32)
    if zero_row_fraction:
        n = int(round(zero_row_fraction * I))
        gw[rng.choice(I, n, replace=False)] = _zero_weight_row(fmt, H)
        uw[rng.choice(I, n, replace=False)] = _zero_weight_row(fmt, H)
    wb = _wbytes(I, H, fmt)
    out[layout.gate_weight_offset:layout.gate_weight_offset + wb] = gw.ravel()
    out[layout.up_weight_offset:layout.up_weight_offset + wb] = uw.ravel()
    out[layout.gate_scale_offset:layout.gate_scale_offset + 4 * I] = gs.astype("<f4").view(np.uint8)
    out[layout.up_scale_offset:layout.up_scale_offset + 4 * I] = us.astype("<f4").view(np.uint8)
    if layout.down_weight_offset != OFFSET_ABSENT:
        dw = _uniform_weights(rng, H, I, fmt)
        ds = rng.uniform(lo, hi, size=H).astype(np.float32)
        if zero_row_fraction:
            dw[rng.choice(H, int(round(zero_row_fraction * H)), replace=False)] = _zero_weight_row(fmt, I)
        out[layout.down_weight_offset:layout.down_weight_offset + wb] = dw.ravel()
        out[layout.down_scale_offset:layout.down_scale_offset + 4 * H] = ds.astype("<f4").view(np.uint8)
    return out


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 samples rounded to nearest-even bf16 (torch's CPU
    conversion); returns uint16 bit patterns."""
    import torch
    f = rng.standard_normal(size=shape, dtype=np.float32)
    b = torch.from_numpy(np.ascontiguousarray(f)).to(torch.bfloat16)
    return b.view(torch.int16).numpy().view(np.uint16).copy()


def f32_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 samples (f32 activations)."""
    return rng.standard_normal(size=shape, dtype=np.float32)


def add_outliers_f32(rng: np.random.Generator, x: np.ndarray, fraction: float) -> np.ndarray:
    """Set ``round(fraction * x.size)`` distinct entries to +-1e4 (equal odds), f32."""
    x = x.copy()
    flat = x.reshape(-1)
    n = int(round(fraction * flat.size))
    pos = rng.choice(flat.size, n, replace=False)
    signs = rng.integers(0, 2, size=n)
    flat[pos] = np.where(signs == 1, -1e4, 1e4).astype(np.float32)
    return x


def add_outliers(rng: np.random.Generator, xbits: np.ndarray, fraction: float) -> np.ndarray:
    """Set ``round(fraction * x.size)`` distinct entries to +-9984 (equal odds)."""
    x = xbits.copy()
    flat = x.reshape(-1)
    n = int(round(fraction * flat.size))
    pos = rng.choice(flat.size, n, replace=False)
    signs = rng.integers(0, 2, size=n)
    flat[pos] = np.where(signs == 1, BF16_NEG_9984, BF16_POS_9984).astype(np.uint16)
    return x


def top_k_routing(rng: np.random.Generator, M: int, K: int, num_slots: int) -> np.ndarray:
    """Per token, K distinct slot ids drawn uniformly without replacement."""
    ids = np.empty((M, K), dtype=np.int32)
    for t in range(M):
        ids[t] = rng.choice(num_slots, K, replace=False)
    return ids


def sha256_hex(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


@dataclass
class Config:
    """One workload: slots (uint8 [num_slots, slot_stride]), x bits, ids."""

    name: str
    seed: int
    H: int
    I: int
    M: int
    layout: SlotLayout
    slots: np.ndarray            # uint8 [num_slots, slot_stride]
    x: np.ndarray                # uint16 [M, H] bf16 bits
    ids: Optional[np.ndarray] = None   # int32 [M, K] for the grouped call
    K: int = 0
    notes: Dict[str, str] = field(default_factory=dict)

    @property
    def num_slots(self) -> int:
        return self.slots.shape[0]

    @property
    def slot_stride(self) -> int:
        return self.slots.shape[1]


CONFIGS: Dict[str, dict] = {
    "cfg1": dict(seed=101, H=256, I=128, M=1, scale=(0.005, 0.02)),
    "cfg2": dict(seed=102, H=4096, I=1536, M=1, scale=(0.005, 0.02)),
    "cfg3": dict(seed=103, H=4096, I=1536, M=8, scale=(0.005, 0.02)),
    "cfg4": dict(seed=104, H=6144, I=2048, M=32, K=8, num_slots=64, scale=(0.005, 0.02)),
    "cfg5": dict(seed=105, H=7168, I=4096, M=None, scale=(0.001, 0.05), zero_rows=0.01, outliers=0.01),
}


def make_config(name: str, M: Optional[int] = None, num_slots: Optional[int] = None,
                H: Optional[int] = None, I: Optional[int] = None, seed: Optional[int] = None,
                with_down: bool = False, fmt: str = "q4") -> Config:
    """Build one of the five workloads (or a resized variant of it).

    ``cfg5`` needs ``M`` in {1, 4, 16, 32}; its x is drawn from seed 105+M.
    ``num_slots``/``H``/``I``/``seed`` override the defaults for scaled-down
    or scaled-up variants with the same distributions.  ``with_down`` lays
    the slots out as whole experts (``expert_layout``) and draws down weights
    and scales of the same distributions after each slot's gate/up fields.
    ``fmt="q8"`` draws int8 weights uniform on [-128, 127] (one byte each)
    in place of the packed nibbles; all-8 rows become zero rows.
    """
    spec = dict(CONFIGS[name])
    H = H or spec["H"]
    I = I or spec["I"]
    seed = spec["seed"] if seed is None else seed
    layout = expert_layout(H, I, fmt=fmt) if with_down else contiguous_layout(H, I, fmt=fmt)
    rng = np.random.default_rng(seed)
    if name == "cfg4":
        E = num_slots or spec["num_slots"]
        M = M or spec["M"]
        K = spec["K"] if E >= spec["K"] else E
        slots = np.zeros((E, layout.slot_bytes), dtype=np.uint8)
        for e in range(E):
            fill_slot(rng, H, I, layout, spec["scale"], out=slots[e], fmt=fmt)
        x = bf16_normal(rng, (M, H))
        ids = top_k_routing(rng, M, K, E)
        return Config(name, seed, H, I, M, layout, slots, x, ids, K)
    if name == "cfg5":
        if M is None:
            raise ValueError("cfg5 needs M")
        slots = fill_slot(rng, H, I, layout, spec["scale"], spec["zero_rows"], fmt=fmt)[None, :]
        xrng = np.random.default_rng(seed + M)
        x = bf16_normal(xrng, (M, H))
        x = add_outliers(xrng, x, spec["outliers"])
        return Config(name, seed, H, I, M, layout, slots, x)
    M = M or spec["M"]
    E = num_slots or 1
    slots = np.zeros((E, layout.slot_bytes), dtype=np.uint8)
    for e in range(E):
        fill_slot(rng, H, I, layout, spec["scale"], out=slots[e], fmt=fmt)
    x = bf16_normal(rng, (M, H))
    return Config(name, seed, H, I, M, layout, slots, x)
