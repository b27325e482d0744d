"""CPU oracle for the Q4 expert gate/up + SwiGLU path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, loads or calls
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP kernels.

What it computes, and where the pages define it (pages of the diff of
@mlx-bun/inference 1.0.0 on my.diffend.io; "page 52" is
.../0.0.0-stage/1.0.0/page/52):

* Slot layout and validation -- page 51, kernels/glm52/layout.ts
  (``Glm52CanonicalMetalLayout``, ``validateRange``) and page 52,
  kernels/glm52/streamed-experts.ts (``validateCall``): byte offsets from the
  slot base, each field must lie inside the slot.
* Weight decode -- page 52, streamed-experts.ts, ``GATE_UP_SOURCE``: row ``i``
  of a projection is ``H/8`` uint32 words; nibble ``p`` of word ``w`` (bits
  ``4p..4p+3``) is input position ``k = 8w + p``; its weight is ``q - 8``
  (zero point 8, the "affine zero-point 8" Q4 family of the same file).
* Gate/up -- same kernel: ``gate = (sum_k (q_k - 8) x_k) * scale_row`` in F32.
  The kernel's F32 FMA order is one of many valid orders; the oracle takes the
  plain definition: the exact sum, times the F32 scale, rounded once to F32
  (round to nearest, ties to even).
* SwiGLU tail -- same kernel, lane-0 tail: gate and up rounded to bf16, then
  ``s = bf16(1 / (1 + exp(-g)))`` evaluated in F32, ``silu = bf16(g * s)``,
  ``out = bf16(silu * u)``.  F32 -> bf16 rounding is round to nearest even,
  the rule of the ``trellis_bf16`` helper on page 54, kernels/trellis/codebook.ts.
* Down projection and the whole expert -- page 52, streamed-experts.ts,
  ``DOWN_SOURCE`` and ``Glm52CanonicalMetalExecutor.execute``: the gate/up
  kernel's bf16 output ``mid[M, I]`` is the input of the down kernel, whose row
  ``h`` (of ``H``) holds ``I/8`` words in the same nibble order;
  ``out[m, h] = bf16((sum_i (q_hi - 8) mid[m, i]) * down_scale[h])``, the sum
  again taken exactly and the F32 product rounded once.  ``validateCall``
  requires both dimensions divisible by 8 and every field inside the slot.
* Q8 family -- same page, ``Q8_GATE_UP_SOURCE``, ``Q8_DOWN_SOURCE`` and
  ``Glm52CanonicalQ8MetalExecutor``: the same computation with signed int8
  weights, one byte per weight, row-major (``[I][H]`` for gate/up,
  ``[H][I]`` for down), no zero point.  Every call below takes
  ``fmt="q4"`` or ``fmt="q8"``.
* f32 activations -- same page: ``validateCall`` accepts bfloat16 or float32
  input and ``execute`` gives every output the input's dtype ``T``.  With
  ``T = float`` the tail's conversions are identities: ``s = 1 / (1 +
  exp(-gate))``, ``silu = gate * s``, ``out = silu * up``, each an F32
  operation; the down output is the F32 value itself.  Calls take
  ``xdtype="bf16"`` (bit patterns, uint16) or ``xdtype="f32"`` (float32).
* Grouped call -- row independence stated on page 52 (one launch geometry for
  every batch width; each sample and row is computed on its own): output
  ``[t, j, :]`` is the single-expert result for token ``t`` on slot
  ``ids[t, j]``.  Ids outside ``[0, num_slots)`` give zero outputs and are
  counted (a reading: the pages have no grouped Q4 call).

Readings where the pages are silent (listed with reasons in the design notes):
``exp`` is evaluated in double and rounded once to F32 (the pages ask for a
precise F32 exp); non-finite activations are outside the contract.

Every function here is a plain, slow transcription of those definitions.
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

OFFSET_ABSENT = (1 << 64) - 1


# ---------------------------------------------------------------------------
# bf16 / f32 helpers
# ---------------------------------------------------------------------------

def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact: bf16 is the top half of f32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16(v) -> np.ndarray:
    """Round float32 values to bf16, nearest, ties to even; returns bit patterns.

    Definition-level implementation: for each finite value take the two bf16
    neighbours that bracket it (truncation toward zero and the next bf16 away
    from zero), compare the exact distances in float64, and on a tie keep the
    one with an even last significand bit.  Values beyond the largest bf16 by
    half an ulp or more round to infinity (IEEE).  NaN maps to the quiet NaN
    0x7FC0 with the input's sign.
    """
    u = np.ascontiguousarray(np.asarray(v, dtype=np.float32)).view(np.uint32).reshape(-1)
    sign = (u >> np.uint32(16)) & np.uint32(0x8000)
    mag = u & np.uint32(0x7FFFFFFF)
    is_nan = mag > np.uint32(0x7F800000)
    is_inf = mag == np.uint32(0x7F800000)
    lo_bits = (mag >> np.uint32(16)).astype(np.uint32)          # toward zero
    hi_bits = lo_bits + np.uint32(1)                             # away from zero
    a = mag.view(np.float32).astype(np.float64)
    lo_val = (lo_bits << np.uint32(16)).view(np.float32).astype(np.float64)
    # one bf16 ulp at lo, in an unbounded exponent range (so the neighbour
    # above the largest finite bf16 is 2**128, whose pattern is infinity)
    efield = ((lo_bits >> np.uint32(7)) & np.uint32(0xFF)).astype(np.int64)
    ulp = np.exp2(np.maximum(efield, 1) - 127 - 7).astype(np.float64)
    hi_val = lo_val + ulp
    d_lo = a - lo_val
    d_hi = hi_val - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo_bits & np.uint32(1)) == np.uint32(1)))
    take_hi &= d_lo != 0.0
    res = np.where(take_hi, hi_bits, lo_bits)
    res = np.where(is_inf, np.uint32(0x7F80), res)
    res = np.where(is_nan, np.uint32(0x7FC0), res)
    res = (res | sign).astype(np.uint16)
    return res.reshape(np.shape(v))


def f32_round_dyadic(n: int, e: int, zero_sign: float = 1.0) -> float:
    """Round the exact value ``n * 2**e`` (integers) to float32, ties to even.

    Returns a Python float holding the float32 value.  Handles subnormals and
    overflow to infinity.  ``zero_sign`` gives the sign of an exact zero.
    """
    if n == 0:
        return math.copysign(0.0, zero_sign)
    neg = n < 0
    a = -n if neg else n
    top = a.bit_length() - 1 + e                # floor(log2 |value|)
    q_exp = max(top - 23, -149)                 # exponent of one f32 ulp here
    shift = q_exp - e
    if shift <= 0:
        m = a << (-shift)
    else:
        m = a >> shift
        r = a - (m << shift)
        half = 1 << (shift - 1)
        if r > half or (r == half and (m & 1)):
            m += 1
    if m.bit_length() + q_exp > 128:
        val = math.inf
    else:
        val = math.ldexp(m, q_exp)
    return -val if neg else val


def f32_parts(v: float) -> Tuple[int, int]:
    """Exact integer decomposition of a finite float: ``v == n * 2**e``."""
    if v == 0.0:
        return 0, 0
    m, ex = math.frexp(v)                        # v = m * 2**ex, 0.5 <= |m| < 1
    n = int(m * (1 << 53))
    return n, ex - 53


# ---------------------------------------------------------------------------
# Slot decode
# ---------------------------------------------------------------------------

def _check_range(offset: int, length: int, slot_bytes: int, label: str) -> None:
    if offset < 0:
        raise ValueError(f"{label} offset must be a non-negative safe integer")
    if length < 0:
        raise ValueError(f"{label} length must be a non-negative safe integer")
    if offset + length > slot_bytes:
        raise ValueError(f"{label} exceeds the canonical expert slot")


def check_layout(layout, H: int, I: int, fmt: str = "q4") -> None:
    """Range rules of validateRange / validateCall for the gate/up fields."""
    if H <= 0 or I <= 0 or layout.slot_bytes <= 0:
        raise ValueError("hidden size, intermediate size and slot bytes must be positive")
    if H % 8:
        raise ValueError(f"{fmt.upper()} expert dimensions must be divisible by 8")
    wb = weight_bytes(I, H, fmt)
    _check_range(layout.gate_weight_offset, wb, layout.slot_bytes, "gate weights")
    _check_range(layout.up_weight_offset, wb, layout.slot_bytes, "up weights")
    _check_range(layout.gate_scale_offset, 4 * I, layout.slot_bytes, "gate scales")
    _check_range(layout.up_scale_offset, 4 * I, layout.slot_bytes, "up scales")
    if layout.down_weight_offset != OFFSET_ABSENT:
        _check_range(layout.down_weight_offset, wb, layout.slot_bytes, "down weights")
    if layout.down_scale_offset != OFFSET_ABSENT:
        _check_range(layout.down_scale_offset, 4 * H, layout.slot_bytes, "down scales")


def weight_bytes(rows: int, K: int, fmt: str) -> int:
    """Bytes of a ``[rows, K]`` weight matrix: two weights per byte (Q4) or one (Q8)."""
    if fmt == "q4":
        return rows * K // 2
    if fmt == "q8":
        return rows * K
    raise ValueError(f"unknown weight format {fmt!r}")


def q8_weights(slot: np.ndarray, offset: int, R: int, C: int) -> np.ndarray:
    """Decode a ``[R, C]`` matrix of signed int8 weights stored row-major at ``offset``."""
    return np.frombuffer(slot, dtype=np.int8, count=R * C, offset=offset).reshape(R, C).copy()


def decode_weights(slot: np.ndarray, offset: int, R: int, C: int, fmt: str) -> np.ndarray:
    return q4_weights(slot, offset, R, C) if fmt == "q4" else q8_weights(slot, offset, R, C)


def q4_weights(slot: np.ndarray, offset: int, I: int, H: int) -> np.ndarray:
    """Decode a ``[I, H]`` matrix of weights ``q - 8`` (int8) from the slot.

    Word ``w`` of row ``i`` is the little-endian uint32 at
    ``offset + 4 * (i * H/8 + w)``; its nibble ``p`` is position ``8w + p``.
    """
    words = np.frombuffer(slot, dtype="<u4", count=I * H // 8, offset=offset).reshape(I, H // 8)
    w = np.empty((I, H), dtype=np.int8)
    for p in range(8):
        q = (words >> np.uint32(4 * p)) & np.uint32(0xF)
        w[:, p::8] = q.astype(np.int8) - np.int8(8)
    return w


def row_scales(slot: np.ndarray, offset: int, I: int) -> np.ndarray:
    return np.frombuffer(slot, dtype="<f4", count=I, offset=offset).astype(np.float32)


# ---------------------------------------------------------------------------
# Exact dot products
# ---------------------------------------------------------------------------

def bf16_integer_parts(xbits: np.ndarray):
    """Write each finite bf16 as ``sign * mag * 2**exp``, integer ``mag`` < 256."""
    b = np.asarray(xbits, dtype=np.uint16).astype(np.int64)
    ef = (b >> 7) & 0xFF
    if np.any(ef == 0xFF):
        raise ValueError("non-finite activations are outside the oracle's contract")
    frac = b & 0x7F
    mag = np.where(ef == 0, frac, frac | 0x80)
    exp = np.where(ef == 0, 1, ef) - 127 - 7
    sign = np.where(b & 0x8000, -1, 1)
    return sign, mag, exp


def f32_integer_parts(x):
    """Write each finite float32 as ``sign * mag * 2**exp``, integer ``mag`` < 2**24."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.int64)
    ef = (b >> 23) & 0xFF
    if np.any(ef == 0xFF):
        raise ValueError("non-finite activations are outside the oracle's contract")
    frac = b & 0x7FFFFF
    mag = np.where(ef == 0, frac, frac | 0x800000)
    exp = np.where(ef == 0, 1, ef) - 127 - 23
    sign = np.where(b & 0x80000000, -1, 1)
    return sign, mag, exp


_LIMB_BITS = 24


def exact_dots(w: np.ndarray, xbits: np.ndarray, xdtype: str = "bf16") -> Tuple[List[List[int]], List[int]]:
    """Exact ``S[i][m] = sum_k w[i, k] * x[m, k]`` as ``num[i][m] * 2**e[m]``.

    Each token's x is scaled by a power of two to integers ``X`` (exact: the
    scale is that token's smallest exponent).  ``|X|`` may be wider than 64
    bits, so it is cut into signed 24-bit limbs.  Each limb product is a
    float64 matrix product in which every product ``w * limb`` (|w| <= 128)
    and every partial sum of at most H <= 2**16 of them is an integer of
    magnitude below 2**47, hence exactly representable: the product is exact whatever
    order the library sums in.  Limbs are recombined in Python integers.
    """
    I, H = w.shape
    if H > (1 << 16):
        raise ValueError("oracle supports H <= 65536")
    if xdtype == "bf16":
        sign, mag, exp = bf16_integer_parts(xbits)
        mag_bits = 8
    elif xdtype == "f32":
        sign, mag, exp = f32_integer_parts(xbits)
        mag_bits = 24
    else:
        raise ValueError(f"unknown activation dtype {xdtype!r}")
    M = xbits.shape[0]
    nz = mag != 0
    exps = [int(exp[m][nz[m]].min()) if np.any(nz[m]) else 0 for m in range(M)]
    shifts = np.where(nz, exp - np.array(exps, dtype=np.int64)[:, None], 0)
    nlimbs = max(1, (int(shifts.max()) + mag_bits + _LIMB_BITS - 1) // _LIMB_BITS)
    mask = (1 << _LIMB_BITS) - 1
    wf = np.asarray(w, dtype=np.float64)
    acc = None
    for l in range(nlimbs):
        # bits [24 l, 24 l + 24) of |X| = mag * 2**shift, with X's sign
        d = shifts - l * _LIMB_BITS
        left = (mag << np.clip(d, 0, _LIMB_BITS - 1)) & mask
        right = np.where(d > -64, mag >> np.clip(-d, 0, 63), 0)
        limb = np.where(d >= _LIMB_BITS, 0, np.where(d >= 0, left, right)) * sign
        r = wf @ np.ascontiguousarray(limb.T, dtype=np.float64)     # [I, M], exact
        part = r.astype(np.int64).astype(object) * (1 << (l * _LIMB_BITS))
        acc = part if acc is None else acc + part
    return acc.tolist(), exps


def scaled_f32(nums: List[List[int]], exps: List[int], scales: np.ndarray) -> np.ndarray:
    """``RN_f32(S[i][m] * scale[i])`` for every row and token -> ``[M, I]``.

    The scale is one F32 multiply after the reduction (page 52,
    ``GATE_UP_SOURCE``), so a zero result has the sign of that IEEE product:
    an exact-zero sum (``+0``, the sum starts from ``+0``) gives the scale's
    sign, a non-zero sum times a signed zero scale gives the sign of the two
    factors together."""
    I = len(nums)
    M = len(exps)
    out = np.empty((M, I), dtype=np.float32)
    for i in range(I):
        s = float(scales[i])
        sn, se = f32_parts(s)
        for m in range(M):
            out[m, i] = f32_round_dyadic(nums[i][m] * sn, exps[m] + se, zero_sign=s if nums[i][m] >= 0 else -s)
    return out


# ---------------------------------------------------------------------------
# SwiGLU tail
# ---------------------------------------------------------------------------

def _exp_f32(v: float) -> np.float32:
    """exp(v) evaluated in double, rounded once to float32 (inf on overflow)."""
    try:
        e = math.exp(v)
    except OverflowError:
        return np.float32(np.inf)
    with np.errstate(over="ignore"):
        return np.float32(e)


def swiglu_tail(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """bf16 output bits of the lane-0 tail for F32 gate and up values."""
    gate = np.asarray(gate, dtype=np.float32)
    up = np.asarray(up, dtype=np.float32)
    gT = bf16_to_f32(f32_to_bf16(gate))
    uT = bf16_to_f32(f32_to_bf16(up))
    flat = gT.reshape(-1)
    e = np.array([_exp_f32(-float(g)) for g in flat], dtype=np.float32).reshape(gT.shape)
    one = np.float32(1.0)
    with np.errstate(over="ignore", under="ignore", divide="ignore"):
        d = one + e                       # F32 add
        sig = one / d                     # F32 divide
    sT = bf16_to_f32(f32_to_bf16(sig))
    siluT = bf16_to_f32(f32_to_bf16(gT * sT))   # F32 product, exact for bf16*bf16
    return f32_to_bf16(siluT * uT)


def swiglu_tail_f32(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """The tail with ``T = float``: every conversion to T is the identity, so
    ``s = 1/(1 + exp(-gate))`` (exp in double, rounded once to F32, as for
    bf16), ``out = (gate * s) * up``, each step an F32 operation."""
    gate = np.asarray(gate, dtype=np.float32)
    up = np.asarray(up, dtype=np.float32)
    flat = gate.reshape(-1)
    e = np.array([_exp_f32(-float(g)) for g in flat], dtype=np.float32).reshape(gate.shape)
    one = np.float32(1.0)
    with np.errstate(over="ignore", under="ignore", divide="ignore", invalid="ignore"):
        d = one + e
        sig = one / d
        silu = gate * sig
        return (silu * up).astype(np.float32)


def _x_rows(x, H: int, xdtype: str) -> np.ndarray:
    if xdtype == "bf16":
        return np.ascontiguousarray(x, dtype=np.uint16).reshape(-1, H)
    if xdtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32).reshape(-1, H)
    raise ValueError(f"unknown activation dtype {xdtype!r}")


# ---------------------------------------------------------------------------
# The two calls
# ---------------------------------------------------------------------------

def expert_gate_up(slot: np.ndarray, layout, xbits: np.ndarray, H: int, I: int, fmt: str = "q4",
                   xdtype: str = "bf16"):
    """Single expert: returns ``(gate f32 [M,I], up f32 [M,I], out [M,I])``; ``out``
    is bf16 bit patterns for bf16 x and float32 values for f32 x."""
    slot = np.ascontiguousarray(slot, dtype=np.uint8).reshape(-1)
    xbits = _x_rows(xbits, H, xdtype)
    check_layout(layout, H, I, fmt)
    if slot.size < layout.slot_bytes:
        raise ValueError("canonical expert slot array is shorter than its layout")
    if xbits.shape[0] < 1:
        raise ValueError("Q4 expert gate/up requires input [M,H] with M >= 1")
    wg = decode_weights(slot, layout.gate_weight_offset, I, H, fmt)
    wu = decode_weights(slot, layout.up_weight_offset, I, H, fmt)
    sg = row_scales(slot, layout.gate_scale_offset, I)
    su = row_scales(slot, layout.up_scale_offset, I)
    gate = scaled_f32(*exact_dots(wg, xbits, xdtype), sg)
    up = scaled_f32(*exact_dots(wu, xbits, xdtype), su)
    return gate, up, (swiglu_tail(gate, up) if xdtype == "bf16" else swiglu_tail_f32(gate, up))


def expert_gate_up_grouped(slots: np.ndarray, slot_stride: int, num_slots: int, layout,
                           xbits: np.ndarray, ids: np.ndarray, H: int, I: int, fmt: str = "q4",
                           xdtype: str = "bf16"):
    """Grouped call over routed slots.

    Returns ``(gate [M,K,I], up [M,K,I], out bits [M,K,I], invalid_count)``.
    Pair ``(t, j)`` uses slot ``ids[t, j]`` and token ``t``; invalid ids give
    zero gate, up and output.
    """
    flat = np.ascontiguousarray(slots, dtype=np.uint8).reshape(-1)
    xbits = _x_rows(xbits, H, xdtype)
    ids = np.asarray(ids, dtype=np.int64)
    M, K = ids.shape
    gate = np.zeros((M, K, I), dtype=np.float32)
    up = np.zeros((M, K, I), dtype=np.float32)
    out = np.zeros((M, K, I), dtype=np.uint16 if xdtype == "bf16" else np.float32)
    invalid = 0
    by_slot: Dict[int, List[Tuple[int, int]]] = {}
    for t in range(M):
        for j in range(K):
            e = int(ids[t, j])
            if 0 <= e < num_slots:
                by_slot.setdefault(e, []).append((t, j))
            else:
                invalid += 1
    for e, pairs in sorted(by_slot.items()):
        slot = flat[e * slot_stride:e * slot_stride + layout.slot_bytes]
        toks = [t for t, _ in pairs]
        g, u, o = expert_gate_up(slot, layout, xbits[toks], H, I, fmt, xdtype)
        for r, (t, j) in enumerate(pairs):
            gate[t, j] = g[r]
            up[t, j] = u[r]
            out[t, j] = o[r]
    return gate, up, out, invalid


# ---------------------------------------------------------------------------
# Down projection and the whole expert (page 52, DOWN_SOURCE and execute)
# ---------------------------------------------------------------------------

def check_down_layout(layout, H: int, I: int, fmt: str = "q4") -> None:
    """validateCall's rules for a call that reads the down fields too."""
    check_layout(layout, H, I, fmt)
    if I % 8:
        raise ValueError(f"{fmt.upper()} expert dimensions must be divisible by 8")
    if layout.down_weight_offset == OFFSET_ABSENT or layout.down_scale_offset == OFFSET_ABSENT:
        raise ValueError("down weights exceeds the canonical expert slot")


def expert_down(slot: np.ndarray, layout, midbits: np.ndarray, H: int, I: int, fmt: str = "q4",
                xdtype: str = "bf16"):
    """Down projection of one slot: returns ``(down f32 [M,H], out bf16 bits [M,H])``.

    Row ``h`` of the down matrix is ``I/8`` words at
    ``down_weight_offset + 4 * (h * I/8 + w)``; nibble ``p`` of word ``w`` is
    input position ``8w + p``.  ``down = RN_f32(S_exact * down_scale[h])`` and
    the output is its bf16 rounding (the kernel's ``T(value)``).
    """
    slot = np.ascontiguousarray(slot, dtype=np.uint8).reshape(-1)
    midbits = _x_rows(midbits, I, xdtype)
    check_down_layout(layout, H, I, fmt)
    if slot.size < layout.slot_bytes:
        raise ValueError("canonical expert slot array is shorter than its layout")
    wd = decode_weights(slot, layout.down_weight_offset, H, I, fmt)
    sd = row_scales(slot, layout.down_scale_offset, H)
    down = scaled_f32(*exact_dots(wd, midbits, xdtype), sd)
    return down, (f32_to_bf16(down) if xdtype == "bf16" else down.copy())


def expert_forward(slot: np.ndarray, layout, xbits: np.ndarray, H: int, I: int, fmt: str = "q4",
                   xdtype: str = "bf16"):
    """The whole expert of one slot, as ``execute`` chains its two kernels:
    returns ``(mid [M,I], out [M,H])`` in the input's dtype."""
    check_down_layout(layout, H, I, fmt)
    _, _, mid = expert_gate_up(slot, layout, xbits, H, I, fmt, xdtype)
    _, out = expert_down(slot, layout, mid, H, I, fmt, xdtype)
    return mid, out


def expert_down_grouped(slots: np.ndarray, slot_stride: int, num_slots: int, layout,
                        midbits: np.ndarray, ids: np.ndarray, H: int, I: int, fmt: str = "q4",
                        xdtype: str = "bf16"):
    """Grouped down projection: pair ``(t, j)`` runs its own input row
    ``mid[t, j, :]`` against slot ``ids[t, j]`` and writes ``out[t, j, :]``.

    Returns ``(down f32 [M,K,H], out bits [M,K,H], invalid_count)``; invalid
    ids give zeros, as in the grouped gate/up call.
    """
    flat = np.ascontiguousarray(slots, dtype=np.uint8).reshape(-1)
    ids = np.asarray(ids, dtype=np.int64)
    M, K = ids.shape
    midbits = _x_rows(midbits, I, xdtype).reshape(M, K, I)
    down = np.zeros((M, K, H), dtype=np.float32)
    out = np.zeros((M, K, H), dtype=np.uint16 if xdtype == "bf16" else np.float32)
    invalid = 0
    by_slot: Dict[int, List[Tuple[int, int]]] = {}
    for t in range(M):
        for j in range(K):
            e = int(ids[t, j])
            if 0 <= e < num_slots:
                by_slot.setdefault(e, []).append((t, j))
            else:
                invalid += 1
    for e, pairs in sorted(by_slot.items()):
        slot = flat[e * slot_stride:e * slot_stride + layout.slot_bytes]
        rows = np.stack([midbits[t, j] for t, j in pairs])
        d, o = expert_down(slot, layout, rows, H, I, fmt, xdtype)
        for r, (t, j) in enumerate(pairs):
            down[t, j] = d[r]
            out[t, j] = o[r]
    return down, out, invalid


def expert_forward_grouped(slots: np.ndarray, slot_stride: int, num_slots: int, layout,
                           xbits: np.ndarray, ids: np.ndarray, H: int, I: int, fmt: str = "q4",
                           xdtype: str = "bf16"):
    """Grouped whole expert: returns ``(mid [M,K,I], out [M,K,H], invalid_count)``."""
    check_down_layout(layout, H, I, fmt)
    _, _, mid, invalid = expert_gate_up_grouped(slots, slot_stride, num_slots, layout, xbits, ids, H, I, fmt,
                                                xdtype)
    _, out, _ = expert_down_grouped(slots, slot_stride, num_slots, layout, mid, ids, H, I, fmt, xdtype)
    return mid, out, invalid
