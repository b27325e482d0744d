"""Pins of the oracle's f32-activation calls (page 52 of the @mlx-bun/inference
1.0.0 diff, kernels/glm52/streamed-experts.ts: validateCall accepts bfloat16 or
float32 input and execute gives the outputs the input's dtype; with T = float
every conversion in the tail is the identity).  Checked against exact rational
brute force, the bf16 path on bf16-representable inputs, rational evaluation
of the F32 tail and closed forms."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.exact_helpers import nearest_f32, unpack_nibble


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _f32_wide(rng, shape, emin=-40, emax=40):
    """float32 values with random 24-bit significands over a wide exponent range, some zeros."""
    m = rng.integers(1 << 23, 1 << 24, shape).astype(np.float64)
    e = rng.integers(emin, emax, shape)
    s = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    v = (s * m * np.exp2(e - 23)).astype(np.float32)
    v[rng.random(shape) < 0.1] = 0
    return v


def test_f32_bf16_representable_inputs_match_the_bf16_path():
    rng = np.random.default_rng(71)
    H, I, M = 256, 24, 3
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    xb = synth.bf16_normal(rng, (M, H))
    xf = oracle.bf16_to_f32(xb)
    g16, u16, _ = oracle.expert_gate_up(slot, lay, xb, H, I)
    g32, u32, _ = oracle.expert_gate_up(slot, lay, xf, H, I, xdtype="f32")
    assert np.array_equal(_bits(g16), _bits(g32)) and np.array_equal(_bits(u16), _bits(u32))


@pytest.mark.parametrize("seed", range(6))
def test_f32_bruteforce_exact_rationals(seed):
    rng = np.random.default_rng(700 + seed)
    H = int(rng.choice([8, 16, 64]))
    I = int(rng.integers(1, 6))
    M = int(rng.integers(1, 4))
    gn, un = rng.integers(0, 16, (I, H)), rng.integers(0, 16, (I, H))
    gs = rng.uniform(0.001, 2.0, I).astype(np.float32)
    us = rng.uniform(0.001, 2.0, I).astype(np.float32)
    lay = synth.contiguous_layout(H, I)
    gw, uw = synth.pack_nibbles(gn), synth.pack_nibbles(un)
    slot = synth.write_slot(lay, H, I, gw, uw, gs, us)
    x = _f32_wide(rng, (M, H))
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I, xdtype="f32")
    for m in range(M):
        xv = [Fraction(float(v)) for v in x[m]]
        for i in range(I):
            sg = sum((unpack_nibble(gw, i, k) - 8) * xv[k] for k in range(H))
            su = sum((unpack_nibble(uw, i, k) - 8) * xv[k] for k in range(H))
            assert _bits(g[m, i]) == _bits(nearest_f32(sg * Fraction(float(gs[i])))) or (sg == 0 and g[m, i] == 0)
            assert _bits(u[m, i]) == _bits(nearest_f32(su * Fraction(float(us[i])))) or (su == 0 and u[m, i] == 0)


def test_f32_subnormal_tokens_bruteforce():
    # f32 tokens of subnormals, alone and next to the smallest normal
    # exponent, scaled up so that the F32 results stay normal
    rng = np.random.default_rng(740)
    H, I, M = 32, 4, 3
    gn, un = rng.integers(0, 16, (I, H)), rng.integers(0, 16, (I, H))
    gs = (rng.uniform(0.5, 2.0, I) * 2.0 ** 120).astype(np.float32)
    us = (rng.uniform(0.5, 2.0, I) * 2.0 ** 120).astype(np.float32)
    lay = synth.contiguous_layout(H, I)
    gw, uw = synth.pack_nibbles(gn), synth.pack_nibbles(un)
    slot = synth.write_slot(lay, H, I, gw, uw, gs, us)
    bits = rng.integers(1, 1 << 23, (M, H)).astype(np.uint32) | (rng.integers(0, 2, (M, H)).astype(np.uint32) << 31)
    bits[1, ::2] |= np.uint32(1 << 23)                # exponent field 1 (2**-126)
    bits[2] = 0
    bits[2, 3] = 0x00000003
    x = bits.view(np.float32)
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I, xdtype="f32")
    for m in range(M):
        xv = [Fraction(float(v)) for v in x[m]]
        for i in range(I):
            sg = sum((unpack_nibble(gw, i, k) - 8) * xv[k] for k in range(H))
            su = sum((unpack_nibble(uw, i, k) - 8) * xv[k] for k in range(H))
            assert _bits(g[m, i]) == _bits(nearest_f32(sg * Fraction(float(gs[i])))) or (sg == 0 and g[m, i] == 0)
            assert _bits(u[m, i]) == _bits(nearest_f32(su * Fraction(float(us[i])))) or (su == 0 and u[m, i] == 0)
    assert np.all(np.abs(g[g != 0]) >= 2.0 ** -126)


def test_f32_tail_against_rational_steps_and_closed_forms():
    rng = np.random.default_rng(73)
    g = np.concatenate([rng.standard_normal(400) * 4, rng.standard_normal(100) * 40,
                        [0.0, -0.0, 88.0, -88.0, -87.5, 100.0, -100.0]]).astype(np.float32)
    u = rng.standard_normal(g.size).astype(np.float32) * 3
    out = oracle.swiglu_tail_f32(g, u)
    for gi, ui, oi in zip(g, u, out):
        gv = float(gi)
        try:
            e = np.float32(math.exp(-gv))          # exp in double, one rounding to F32
        except OverflowError:
            e = np.float32(np.inf)
        if np.isinf(e):
            s = np.float32(0.0)
        else:
            d = nearest_f32(Fraction(1) + Fraction(float(e)))
            s = nearest_f32(Fraction(1) / Fraction(float(d)))
        silu = nearest_f32(Fraction(gv) * Fraction(float(s))) if s != 0 else np.float32(gv * 0.0)
        want = nearest_f32(Fraction(float(silu)) * Fraction(float(ui))) if silu != 0 else np.float32(silu * ui)
        assert _bits(oi) == _bits(want) or (oi == 0 and want == 0), (gi, ui, oi, want)
    z = oracle.swiglu_tail_f32(np.float32([0.0]), np.float32([3.0]))
    assert z[0] == 0.0
    big = oracle.swiglu_tail_f32(np.float32([100.0]), np.float32([0.5]))
    assert big[0] == np.float32(50.0)                # s = 1 exactly
    neg = oracle.swiglu_tail_f32(np.float32([-100.0]), np.float32([2.0]))
    assert neg[0] == 0.0 and math.copysign(1.0, float(neg[0])) < 0   # exp overflows: s = +0


def test_f32_down_and_forward_selector():
    rng = np.random.default_rng(74)
    H, I, M = 40, 32, 2
    lay = synth.expert_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay, scale_range=(0.05, 0.2))
    sel = rng.integers(0, I, H)
    dn = np.full((H, I), 8)
    dn[np.arange(H), sel] = 9
    dw = synth.pack_nibbles(dn).astype("<u4")
    slot[lay.down_weight_offset:lay.down_weight_offset + H * I // 2] = dw.view(np.uint8).ravel()
    slot[lay.down_scale_offset:lay.down_scale_offset + 4 * H] = np.ones(H, "<f4").view(np.uint8)
    x = _f32_wide(rng, (M, H), -4, 4)
    mid, out = oracle.expert_forward(slot, lay, x, H, I, xdtype="f32")
    assert mid.dtype == np.float32 and out.dtype == np.float32
    _, _, mid_gu = oracle.expert_gate_up(slot, lay, x, H, I, xdtype="f32")
    assert np.array_equal(_bits(mid), _bits(mid_gu))
    want = mid[:, sel]
    assert np.all((_bits(out) == _bits(want)) | ((out == 0) & (want == 0)))
    # one-hot f32 mid rows pin the down orientation in the f32 path too
    onehot = np.eye(I, dtype=np.float32)
    d, o = oracle.expert_down(slot, lay, onehot, H, I, xdtype="f32")
    wd = dn.T - 8
    assert np.array_equal(_bits(d), _bits(np.float32(np.float64(wd) * 1.0)))
    assert np.array_equal(_bits(o), _bits(d))
