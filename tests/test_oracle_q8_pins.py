"""Pins of the oracle's Q8 family (page 52 of the @mlx-bun/inference 1.0.0
diff, kernels/glm52/streamed-experts.ts: Q8_GATE_UP_SOURCE, Q8_DOWN_SOURCE,
Glm52CanonicalQ8MetalExecutor): signed int8 weights, one per byte, row-major,
no zero point, the same scale and tail as Q4.  Checked against exact rational
brute force, unit vectors, constant weights and a cross-format identity (a
Q8 slot holding the Q4 slot's weights q - 8 gives the same results)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.exact_helpers import bf16_value, nearest_f32


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _q8_slot(H, I, wg, wu, wd, gs, us, ds):
    """Whole-expert Q8 slot from int8 matrices (gate/up [I,H], down [H,I])."""
    lay = synth.expert_layout(H, I, fmt="q8")
    slot = np.zeros(lay.slot_bytes, np.uint8)
    for off, w in ((lay.gate_weight_offset, wg), (lay.up_weight_offset, wu), (lay.down_weight_offset, wd)):
        b = np.ascontiguousarray(w, dtype=np.int8).view(np.uint8).ravel()
        slot[off:off + b.size] = b
    for off, v in ((lay.gate_scale_offset, gs), (lay.up_scale_offset, us), (lay.down_scale_offset, ds)):
        b = np.asarray(v, "<f4").view(np.uint8)
        slot[off:off + b.size] = b
    return lay, slot


def _rand(rng, H, I, scale=(0.005, 0.02)):
    wg = rng.integers(-128, 128, (I, H))
    wu = rng.integers(-128, 128, (I, H))
    wd = rng.integers(-128, 128, (H, I))
    gs = rng.uniform(*scale, I).astype(np.float32)
    us = rng.uniform(*scale, I).astype(np.float32)
    ds = rng.uniform(*scale, H).astype(np.float32)
    return (wg, wu, wd, gs, us, ds)


def test_q8_one_hot_pins_row_major_signed_bytes():
    rng = np.random.default_rng(51)
    H, I = 64, 16
    wg, wu, wd, gs, us, ds = _rand(rng, H, I, (0.5, 2.0))
    lay, slot = _q8_slot(H, I, wg, wu, wd, gs, us, ds)
    x = np.zeros((H, H), dtype=np.uint16)
    x[np.arange(H), np.arange(H)] = 0x3F80
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I, fmt="q8")
    assert np.array_equal(_bits(g), _bits(np.float32(np.float64(wg.T) * np.float64(gs)[None, :])))
    assert np.array_equal(_bits(u), _bits(np.float32(np.float64(wu.T) * np.float64(us)[None, :])))
    mid = np.zeros((I, I), dtype=np.uint16)
    mid[np.arange(I), np.arange(I)] = 0x3F80
    d, _ = oracle.expert_down(slot, lay, mid, H, I, fmt="q8")
    assert np.array_equal(_bits(d), _bits(np.float32(np.float64(wd.T) * np.float64(ds)[None, :])))


@pytest.mark.parametrize("seed", range(6))
def test_q8_bruteforce_exact_rationals(seed):
    rng = np.random.default_rng(500 + seed)
    H = int(rng.choice([8, 16, 48]))
    I = int(rng.choice([8, 16, 24]))
    M = int(rng.integers(1, 4))
    wg, wu, wd, gs, us, ds = _rand(rng, H, I, (0.001, 0.1))
    lay, slot = _q8_slot(H, I, wg, wu, wd, gs, us, ds)
    x = synth.bf16_normal(rng, (M, H))
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I, fmt="q8")
    mid = synth.bf16_normal(rng, (M, I))
    d, _ = oracle.expert_down(slot, lay, mid, H, I, fmt="q8")
    for m in range(M):
        xv = [bf16_value(int(b)) for b in x[m]]
        mv = [bf16_value(int(b)) for b in mid[m]]
        for i in range(I):
            sg = sum(int(wg[i, k]) * xv[k] for k in range(H))
            su = sum(int(wu[i, k]) * xv[k] for k in range(H))
            assert _bits(g[m, i]) == _bits(nearest_f32(sg * Fraction(float(gs[i])))) or (sg == 0 and g[m, i] == 0)
            assert _bits(u[m, i]) == _bits(nearest_f32(su * Fraction(float(us[i])))) or (su == 0 and u[m, i] == 0)
        for h in range(H):
            sd = sum(int(wd[h, i]) * mv[i] for i in range(I))
            assert _bits(d[m, h]) == _bits(nearest_f32(sd * Fraction(float(ds[h])))) or (sd == 0 and d[m, h] == 0)


def test_q8_slot_with_q4_weights_gives_q4_results():
    """A Q8 slot whose bytes are the Q4 slot's weights q - 8 computes the same
    gate, up, SwiGLU output, down and whole-expert output bit for bit."""
    rng = np.random.default_rng(53)
    H, I, M = 64, 32, 3
    gn, un, dn = rng.integers(0, 16, (I, H)), rng.integers(0, 16, (I, H)), rng.integers(0, 16, (H, I))
    gs = rng.uniform(0.005, 0.02, I).astype(np.float32)
    us = rng.uniform(0.005, 0.02, I).astype(np.float32)
    ds = rng.uniform(0.005, 0.02, H).astype(np.float32)
    lay4 = synth.expert_layout(H, I)
    s4 = synth.write_slot(lay4, H, I, synth.pack_nibbles(gn), synth.pack_nibbles(un), gs, us)
    s4[lay4.down_weight_offset:lay4.down_weight_offset + H * I // 2] = \
        synth.pack_nibbles(dn).astype("<u4").view(np.uint8).ravel()
    s4[lay4.down_scale_offset:lay4.down_scale_offset + 4 * H] = ds.astype("<f4").view(np.uint8)
    lay8, s8 = _q8_slot(H, I, gn - 8, un - 8, dn - 8, gs, us, ds)
    x = synth.bf16_normal(rng, (M, H))
    r4 = oracle.expert_gate_up(s4, lay4, x, H, I)
    r8 = oracle.expert_gate_up(s8, lay8, x, H, I, fmt="q8")
    for a, b in zip(r4, r8):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    f4 = oracle.expert_forward(s4, lay4, x, H, I)
    f8 = oracle.expert_forward(s8, lay8, x, H, I, fmt="q8")
    assert np.array_equal(f4[0], f8[0]) and np.array_equal(f4[1], f8[1])


def test_q8_constant_and_zero_weights():
    rng = np.random.default_rng(54)
    H, I, M = 128, 4, 3
    x = synth.bf16_normal(rng, (M, H))
    sums = [sum(bf16_value(int(b)) for b in x[m]) for m in range(M)]
    for w in (-128, 127, 1, 0):
        W = np.full((I, H), w)
        gs = np.array([0.01, 0.5, 3.0, 1e-3], dtype=np.float32)
        lay, slot = _q8_slot(H, I, W, W, np.zeros((H, I), int), gs, gs, np.ones(H, np.float32))
        g, u, o = oracle.expert_gate_up(slot, lay, x, H, I, fmt="q8")
        for m in range(M):
            for i in range(I):
                want = nearest_f32(Fraction(w) * sums[m] * Fraction(float(gs[i])))
                assert _bits(g[m, i]) == _bits(want) or (w == 0 and g[m, i] == 0.0)
        if w == 0:
            assert np.all(_bits(g) == 0) and np.all(o == 0)


def test_q8_layout_sizes_and_rules():
    H, I = 64, 24
    lay = synth.expert_layout(H, I, fmt="q8")
    assert lay.up_weight_offset - lay.gate_weight_offset >= I * H
    assert oracle.weight_bytes(I, H, "q8") == I * H and oracle.weight_bytes(I, H, "q4") == I * H // 2
    small = synth.contiguous_layout(256, 64)       # sized for Q4: too short for Q8 weights
    with pytest.raises(ValueError, match="exceeds the canonical expert slot"):
        oracle.expert_gate_up(np.zeros(small.slot_bytes, np.uint8), small, np.zeros((1, 256), np.uint16), 256, 64,
                              fmt="q8")
