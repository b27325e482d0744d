"""Pins of the oracle's down projection and whole expert.

The down kernel of page 52 of the @mlx-bun/inference 1.0.0 diff
(kernels/glm52/streamed-experts.ts, ``DOWN_SOURCE``) reads row ``h`` of the
down matrix as ``I/8`` packed words in the gate/up nibble order, multiplies by
the bf16 ``mid`` row, scales by ``down_scale[h]`` in F32 and stores the bf16
rounding; ``Glm52CanonicalMetalExecutor.execute`` chains gate/up and down.
Each test checks the oracle against something other than itself: exact
rational brute force, closed forms, selector matrices, invariants.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.exact_helpers import bf16_value, nearest_f32, unpack_nibble


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _torch_bf16(f32):
    """bf16 bits of float32 values by torch's conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(f32, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _expert_slot(H, I, gn, un, dn, gs, us, ds):
    """A whole-expert slot from nibble arrays (gate/up [I,H], down [H,I]) and scales."""
    lay = synth.expert_layout(H, I)
    slot = synth.write_slot(lay, H, I, synth.pack_nibbles(gn), synth.pack_nibbles(un), gs, us)
    dw = synth.pack_nibbles(dn).astype("<u4")
    slot[lay.down_weight_offset:lay.down_weight_offset + H * I // 2] = dw.view(np.uint8).ravel()
    slot[lay.down_scale_offset:lay.down_scale_offset + 4 * H] = np.asarray(ds, "<f4").view(np.uint8)
    return lay, slot


def _rand_expert(rng, H, I, scale=(0.005, 0.02)):
    gn = rng.integers(0, 16, (I, H))
    un = rng.integers(0, 16, (I, H))
    dn = rng.integers(0, 16, (H, I))
    gs = rng.uniform(*scale, I).astype(np.float32)
    us = rng.uniform(*scale, I).astype(np.float32)
    ds = rng.uniform(*scale, H).astype(np.float32)
    return (gn, un, dn, gs, us, ds), _expert_slot(H, I, gn, un, dn, gs, us, ds)


def test_one_hot_mid_pins_down_row_orientation_and_zero_point():
    rng = np.random.default_rng(31)
    H, I = 24, 64
    (gn, un, dn, gs, us, ds), (lay, slot) = _rand_expert(rng, H, I, (0.5, 2.0))
    mid = np.zeros((I, I), dtype=np.uint16)
    mid[np.arange(I), np.arange(I)] = 0x3F80        # token i is the unit vector e_i
    d, o = oracle.expert_down(slot, lay, mid, H, I)
    want = np.float32(np.float64(dn.T - 8) * np.float64(ds)[None, :])   # [I tokens, H rows]
    assert np.array_equal(_bits(d), _bits(want))
    assert np.array_equal(o, _torch_bf16(want))


@pytest.mark.parametrize("seed", range(8))
def test_down_bruteforce_exact_rationals(seed):
    rng = np.random.default_rng(300 + seed)
    H = int(rng.choice([8, 16, 40]))
    I = int(rng.choice([8, 16, 64]))
    M = int(rng.integers(1, 4))
    dn = rng.integers(0, 16, (H, I))
    ds = (rng.uniform(0.001, 4.0, H) * np.exp2(rng.integers(-10, 10, H))).astype(np.float32)
    z = np.zeros((I, H), dtype=np.int64)
    lay, slot = _expert_slot(H, I, z + 8, z + 8, dn, np.ones(I, np.float32), np.ones(I, np.float32), ds)
    mid = synth.bf16_normal(rng, (M, I))
    mid[rng.random((M, I)) < 0.1] = 0
    d, o = oracle.expert_down(slot, lay, mid, H, I)
    words = synth.pack_nibbles(dn)
    for m in range(M):
        mv = [bf16_value(int(b)) for b in mid[m]]
        for h in range(H):
            s = sum((unpack_nibble(words, h, i) - 8) * mv[i] for i in range(I))
            want = nearest_f32(s * Fraction(float(ds[h])))
            assert _bits(d[m, h]) == _bits(want) or (s == 0 and d[m, h] == 0.0)
    assert np.array_equal(o, _torch_bf16(d))


def test_down_zero_rows_and_zero_input():
    rng = np.random.default_rng(33)
    H, I = 32, 64
    (gn, un, dn, gs, us, ds), _ = _rand_expert(rng, H, I)
    dn8 = dn.copy()
    dn8[::3] = 8
    lay, slot = _expert_slot(H, I, gn, un, dn8, gs, us, ds)
    mid = synth.bf16_normal(rng, (3, I))
    d, o = oracle.expert_down(slot, lay, mid, H, I)
    assert np.all(_bits(d[:, ::3]) == 0) and np.all(o[:, ::3] == 0)
    d0, o0 = oracle.expert_down(slot, lay, np.zeros((2, I), np.uint16), H, I)
    assert np.all(_bits(d0) == 0) and np.all(o0 == 0)


def test_down_power_of_two_scale_is_exact():
    rng = np.random.default_rng(34)
    H, I = 16, 64
    (gn, un, dn, gs, us, ds), (lay, slot) = _rand_expert(rng, H, I)
    mid = synth.bf16_normal(rng, (2, I))
    d, _ = oracle.expert_down(slot, lay, mid, H, I)
    lay2, slot2 = _expert_slot(H, I, gn, un, dn, gs, us, (ds * np.float32(8.0)).astype(np.float32))
    d2, _ = oracle.expert_down(slot2, lay2, mid, H, I)
    assert np.array_equal(_bits(d2), _bits(d * np.float32(8.0)))


def test_forward_with_selector_down_returns_mid_columns():
    """Down row h = e_{sel[h]} (nibble 9 there, 8 elsewhere) with scale 1:
    the whole expert's output column h is mid column sel[h], bit for bit."""
    rng = np.random.default_rng(35)
    H, I, M = 48, 32, 3
    (gn, un, _, gs, us, _), _ = _rand_expert(rng, H, I, (0.05, 0.2))
    sel = rng.integers(0, I, H)
    dn = np.full((H, I), 8)
    dn[np.arange(H), sel] = 9
    lay, slot = _expert_slot(H, I, gn, un, dn, gs, us, np.ones(H, np.float32))
    x = synth.bf16_normal(rng, (M, H))
    mid, out = oracle.expert_forward(slot, lay, x, H, I)
    _, _, mid_gu = oracle.expert_gate_up(slot, lay, x, H, I)
    assert np.array_equal(mid, mid_gu)
    want = mid[:, sel]
    same = (out == want) | (((out | want) & 0x7FFF) == 0)    # +-0 compare equal
    assert np.all(same)


def test_down_grouped_equals_single_calls_and_zero_fills_invalid_ids():
    rng = np.random.default_rng(36)
    H, I, E, M, K = 16, 32, 3, 3, 2
    c = synth.make_config("cfg4", num_slots=E, H=H, I=I, M=M, with_down=True)
    ids = np.array([[0, 2], [1, 7], [2, 2]], dtype=np.int32)
    mid = synth.bf16_normal(rng, (M, K, I))
    d, o, bad = oracle.expert_down_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, mid, ids, H, I)
    assert bad == 1
    for t in range(M):
        for j in range(K):
            e = ids[t, j]
            if 0 <= e < E:
                d1, o1 = oracle.expert_down(c.slots[e], c.layout, mid[t, j][None], H, I)
                assert np.array_equal(_bits(d[t, j]), _bits(d1[0])) and np.array_equal(o[t, j], o1[0])
            else:
                assert np.all(_bits(d[t, j]) == 0) and np.all(o[t, j] == 0)
    x = synth.bf16_normal(rng, (M, H))
    midg, outg, bad2 = oracle.expert_forward_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, x, ids, H, I)
    assert bad2 == 1
    for t, j in ((0, 0), (2, 1)):
        m1, o1 = oracle.expert_forward(c.slots[ids[t, j]], c.layout, x[t][None], H, I)
        assert np.array_equal(midg[t, j], m1[0]) and np.array_equal(outg[t, j], o1[0])


def test_down_layout_rules():
    H, I = 16, 12
    lay = synth.expert_layout(H, I)
    slot = np.zeros(lay.slot_bytes, np.uint8)
    with pytest.raises(ValueError, match="divisible by 8"):
        oracle.expert_down(slot, lay, np.zeros((1, I), np.uint16), H, I)
    lay2 = synth.contiguous_layout(16, 16)
    with pytest.raises(ValueError, match="down"):
        oracle.expert_down(np.zeros(lay2.slot_bytes, np.uint8), lay2, np.zeros((1, 16), np.uint16), 16, 16)
