"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

The oracle follows page 52 of the @mlx-bun/inference 1.0.0 diff
(kernels/glm52/streamed-experts.ts, ``GATE_UP_SOURCE``) and the bf16 rounding
rule of page 54 (kernels/trellis/codebook.ts, ``trellis_bf16``).  Each test
here checks it against something other than itself: exact rational brute
force, closed forms, library conversions, invariants, a hand-worked example.
A plausible slip (nibble order, zero point, a dropped scale, a sign in the
sigmoid, a wrong rounding rule, a transposed operand) fails at least one.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.exact_helpers import bf16_value, nearest_f32, unpack_nibble

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _slot(H, I, gw, uw, gs, us):
    lay = synth.contiguous_layout(H, I)
    return lay, synth.write_slot(lay, H, I, gw, uw, gs, us)


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# --------------------------------------------------------------------------
# bf16 rounding (page 54, trellis_bf16: round to nearest, ties to even)
# --------------------------------------------------------------------------

def _page_bf16(u):
    """The pages' bit formula, for finite inputs."""
    u = u.astype(np.uint64)
    return (((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000) >> 16).astype(np.uint16)


def _all_decision_classes():
    hi = np.arange(1 << 16, dtype=np.uint32)
    lows = np.array([0, 1, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFE, 0xFFFF],
                    dtype=np.uint32)
    u = (hi[:, None] << np.uint32(16)) | lows[None, :]
    return u.reshape(-1)


def test_bf16_rounding_matches_page_formula_on_every_decision_class():
    u = _all_decision_classes()
    u = np.concatenate([u, np.random.default_rng(7).integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)])
    finite = (u & 0x7F800000) != 0x7F800000
    u = u[finite]
    got = oracle.f32_to_bf16(u.view(np.float32))
    want = _page_bf16(u)
    # the page's formula overflows finite values past the largest bf16 into the
    # infinity pattern, which is also IEEE rounding to nearest
    assert np.array_equal(got, want)


def test_bf16_rounding_matches_torch():
    u = _all_decision_classes()
    f = u.view(np.float32)
    finite = np.isfinite(f)
    got = oracle.f32_to_bf16(f[finite])
    want = torch.from_numpy(f[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rounding_special_values():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, 1.00390625, 1.01171875], dtype=np.float32)
    got = oracle.f32_to_bf16(vals)
    assert list(got) == [0x0000, 0x8000, 0x7F80, 0xFF80, 0x3F80, 0x3F80, 0x3F82]
    nan = oracle.f32_to_bf16(np.array([np.nan], dtype=np.float32))
    assert (int(nan[0]) & 0x7FFF) == 0x7FC0


@pytest.mark.slow
def test_bf16_rounding_exhaustive():
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        u = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        u = u[(u & 0x7F800000) != 0x7F800000]
        assert np.array_equal(oracle.f32_to_bf16(u.view(np.float32)), _page_bf16(u))


# --------------------------------------------------------------------------
# float32 rounding of exact dyadic values
# --------------------------------------------------------------------------

def test_round_dyadic_matches_numpy_cast_on_doubles():
    rng = np.random.default_rng(11)
    d = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.integers(-160, 120, 20000)),
        rng.standard_normal(2000) * 1e-44,
    ])
    for v in d:
        n, e = oracle.f32_parts(float(v))
        got = oracle.f32_round_dyadic(n, e)
        assert np.float32(got) == np.float32(v) or (math.isnan(got) and math.isnan(v)), v


def test_round_dyadic_ties_subnormals_overflow():
    # exact ties between f32 neighbours go to the even significand
    one = 1 << 23
    for m in (one, one + 1, one + 2, (1 << 24) - 1):
        n = 2 * m + 1                     # halfway between m and m+1 (ulp units)
        got = oracle.f32_round_dyadic(n, -1 - 23)
        want = (m + (m & 1)) / one
        assert got == want
    # halfway between the two smallest subnormals, and just above
    assert oracle.f32_round_dyadic(3, -150) == 2 * 2.0 ** -149
    assert oracle.f32_round_dyadic(1, -150) == 0.0
    assert oracle.f32_round_dyadic(3, -151) == 2.0 ** -149
    # largest finite float32 and the overflow threshold (half an ulp above)
    fmax = float(np.finfo(np.float32).max)
    assert oracle.f32_round_dyadic((1 << 24) - 1, 104) == fmax
    assert oracle.f32_round_dyadic((1 << 25) - 1, 103) == math.inf
    assert oracle.f32_round_dyadic((1 << 26) - 3, 102) == fmax
    assert oracle.f32_round_dyadic(-((1 << 25) - 1), 103) == -math.inf


# --------------------------------------------------------------------------
# Hand-worked example (values derived by hand in the fixture)
# --------------------------------------------------------------------------

def test_worked_example_fixture():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    H, I = ex["H"], ex["I"]
    gw = np.array([int(w, 16) for w in ex["gate_words"]], dtype=np.uint32).reshape(I, H // 8)
    uw = np.array([int(w, 16) for w in ex["up_words"]], dtype=np.uint32).reshape(I, H // 8)
    lay, slot = _slot(H, I, gw, uw, ex["gate_scales"], ex["up_scales"])
    x = np.array([int(b, 16) for b in ex["x_bits"]], dtype=np.uint16).reshape(1, H)
    g, u, o = oracle.expert_gate_up(slot, lay, x, H, I)
    assert [float(v) for v in g[0]] == ex["gate"]
    assert [float(v) for v in u[0]] == ex["up"]
    assert [int(v) for v in o[0]] == [int(b, 16) for b in ex["out_bits"]]
    assert list(_bits(g[0]) >> 31) == ex["gate_sign_bits"]


# --------------------------------------------------------------------------
# Decode pins: nibble order, zero point, where the scale applies
# --------------------------------------------------------------------------

def test_one_hot_inputs_pin_nibble_order_and_zero_point():
    rng = np.random.default_rng(3)
    H, I = 64, 8
    gn = rng.integers(0, 16, (I, H))
    un = rng.integers(0, 16, (I, H))
    gs = rng.uniform(0.005, 0.02, I).astype(np.float32)
    us = rng.uniform(0.5, 2.0, I).astype(np.float32)
    lay, slot = _slot(H, I, synth.pack_nibbles(gn), synth.pack_nibbles(un), gs, us)
    x = np.zeros((H, H), dtype=np.uint16)
    x[np.arange(H), np.arange(H)] = 0x3F80          # token k is the unit vector e_k
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I)
    want_g = np.float32(np.float64(gn.T - 8) * np.float64(gs)[None, :])
    want_u = np.float32(np.float64(un.T - 8) * np.float64(us)[None, :])
    assert np.array_equal(_bits(g), _bits(want_g))
    assert np.array_equal(_bits(u), _bits(want_u))


def test_constant_nibbles_give_scaled_sum_of_x():
    rng = np.random.default_rng(5)
    H, I, M = 256, 3, 4
    x = synth.bf16_normal(rng, (M, H))
    sums = [sum(bf16_value(int(b)) for b in x[m]) for m in range(M)]
    for nib, w in ((9, 1), (0, -8), (15, 7), (8, 0)):
        words = synth.pack_nibbles(np.full((I, H), nib))
        gs = np.array([0.01, 0.5, 3.0], dtype=np.float32)
        lay, slot = _slot(H, I, words, words, gs, gs)
        g, _, _ = oracle.expert_gate_up(slot, lay, x, H, I)
        for m in range(M):
            for i in range(I):
                want = nearest_f32(Fraction(w) * sums[m] * Fraction(float(gs[i])))
                assert _bits(g[m, i]) == _bits(want) or (w == 0 and g[m, i] == 0.0)


def _bf16_wide(rng, shape):
    """bf16 patterns over a wide exponent range, including subnormals and zeros."""
    sign = rng.integers(0, 2, shape) << 15
    e = rng.integers(0, 255, shape)                # 0 (subnormal) .. 254
    f = rng.integers(0, 128, shape)
    bits = (sign | (e << 7) | f).astype(np.uint16)
    bits[rng.random(shape) < 0.1] = 0
    return bits


@pytest.mark.parametrize("seed", range(12))
def test_bruteforce_exact_rationals(seed):
    rng = np.random.default_rng(100 + seed)
    H = int(rng.choice([8, 16, 64, 256]))
    I = int(rng.integers(1, 9))
    M = int(rng.integers(1, 5))
    gn = rng.integers(0, 16, (I, H))
    un = rng.integers(0, 16, (I, H))
    gs = (rng.uniform(0.001, 4.0, I) * np.exp2(rng.integers(-20, 20, I))).astype(np.float32)
    us = (rng.uniform(0.001, 4.0, I) * np.exp2(rng.integers(-20, 20, I))).astype(np.float32)
    gw, uw = synth.pack_nibbles(gn), synth.pack_nibbles(un)
    lay, slot = _slot(H, I, gw, uw, gs, us)
    if seed % 3 == 0:
        x = synth.bf16_normal(rng, (M, H))
    else:
        x = _bf16_wide(rng, (M, H))                # spans up to ~2**254: many limbs
        # keep products finite in f32 after the scale: clamp the exponent field
        x = np.where(((x >> 7) & 0xFF) > 200, x & 0x807F | (200 << 7), x).astype(np.uint16)
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I)
    for m in range(M):
        xv = [bf16_value(int(b)) for b in x[m]]
        for i in range(I):
            sg = sum((unpack_nibble(gw, i, k) - 8) * xv[k] for k in range(H))
            su = sum((unpack_nibble(uw, i, k) - 8) * xv[k] for k in range(H))
            wg = nearest_f32(sg * Fraction(float(gs[i])))
            wu = nearest_f32(su * Fraction(float(us[i])))
            assert _bits(g[m, i]) == _bits(wg) or (sg == 0 and g[m, i] == 0.0)
            assert _bits(u[m, i]) == _bits(wu) or (su == 0 and u[m, i] == 0.0)


def test_subnormal_tokens_bruteforce():
    # tokens made of subnormal bf16 values, alone and next to the smallest
    # normal exponent, with scales that keep the F32 results normal: an
    # exponent slip at the subnormal boundary changes the result by 2x
    rng = np.random.default_rng(140)
    H, I, M = 64, 5, 3
    gn, un = rng.integers(0, 16, (I, H)), rng.integers(0, 16, (I, H))
    gs = (rng.uniform(0.5, 2.0, I) * 2.0 ** 110).astype(np.float32)
    us = (rng.uniform(0.5, 2.0, I) * 2.0 ** 110).astype(np.float32)
    gw, uw = synth.pack_nibbles(gn), synth.pack_nibbles(un)
    lay, slot = _slot(H, I, gw, uw, gs, us)
    sign = (rng.integers(0, 2, (M, H)) << 15).astype(np.uint16)
    x = (rng.integers(1, 0x80, (M, H)).astype(np.uint16) | sign)   # exponent field 0
    x[1, ::2] |= np.uint16(1 << 7)                                  # exponent field 1 (2**-126)
    x[2] = 0
    x[2, 7] = 0x0005
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I)
    for m in range(M):
        xv = [bf16_value(int(b)) for b in x[m]]
        for i in range(I):
            sg = sum((unpack_nibble(gw, i, k) - 8) * xv[k] for k in range(H))
            su = sum((unpack_nibble(uw, i, k) - 8) * xv[k] for k in range(H))
            assert _bits(g[m, i]) == _bits(nearest_f32(sg * Fraction(float(gs[i])))) or (sg == 0 and g[m, i] == 0)
            assert _bits(u[m, i]) == _bits(nearest_f32(su * Fraction(float(us[i])))) or (su == 0 and u[m, i] == 0)
    assert np.all(np.abs(g[g != 0]) >= 2.0 ** -126)


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def _random_expert(seed, H=128, I=16, M=3):
    rng = np.random.default_rng(seed)
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    x = synth.bf16_normal(rng, (M, H))
    return rng, lay, slot, x, H, I


def test_all_eight_rows_and_zero_input_give_exact_zeros():
    rng, lay, slot, x, H, I = _random_expert(21)
    words = np.full((I, H // 8), 0x88888888, dtype=np.uint32)
    scales = np.full(I, 0.01, dtype=np.float32)
    lay2, slot2 = _slot(H, I, words, words, scales, scales)
    g, u, o = oracle.expert_gate_up(slot2, lay2, x, H, I)
    assert np.all(_bits(g) == 0) and np.all(_bits(u) == 0)
    assert np.all((o & 0x7FFF) == 0)
    z = np.zeros_like(x)
    g, u, o = oracle.expert_gate_up(slot, lay, z, H, I)
    assert np.all(_bits(g) == 0) and np.all(_bits(u) == 0) and np.all(o == 0)


def _with_scales(slot, lay, I, gmul=1.0, umul=1.0):
    s = slot.copy()
    gs = np.frombuffer(s, "<f4", I, lay.gate_scale_offset).copy() * np.float32(gmul)
    us = np.frombuffer(s, "<f4", I, lay.up_scale_offset).copy() * np.float32(umul)
    s[lay.gate_scale_offset:lay.gate_scale_offset + 4 * I] = gs.astype("<f4").view(np.uint8)
    s[lay.up_scale_offset:lay.up_scale_offset + 4 * I] = us.astype("<f4").view(np.uint8)
    return s


def test_power_of_two_scale_is_exact():
    rng, lay, slot, x, H, I = _random_expert(22)
    g, u, o = oracle.expert_gate_up(slot, lay, x, H, I)
    for j in (-3, 1, 5):
        g2, u2, _ = oracle.expert_gate_up(_with_scales(slot, lay, I, 2.0 ** j, 2.0 ** j), lay, x, H, I)
        assert np.array_equal(g2, g * np.float32(2.0 ** j))
        assert np.array_equal(u2, u * np.float32(2.0 ** j))
    _, _, o2 = oracle.expert_gate_up(_with_scales(slot, lay, I, 1.0, 2.0), lay, x, H, I)
    assert np.array_equal(oracle.bf16_to_f32(o2), oracle.bf16_to_f32(o) * np.float32(2.0))


def test_general_scale_factor_within_one_rounding():
    rng, lay, slot, x, H, I = _random_expert(23)
    g, _, _ = oracle.expert_gate_up(slot, lay, x, H, I)
    c = 1.337
    g2, _, _ = oracle.expert_gate_up(_with_scales(slot, lay, I, c, 1.0), lay, x, H, I)
    # (S * RN(s*c)) vs c * RN(S*s): both within ~2 ulps of S*s*c
    ratio = np.float64(g2) / (np.float64(g) * c)
    assert np.all(np.abs(ratio - 1.0) < 4 * 2.0 ** -24)


def test_negated_scales_negate_gate_and_up_bit_for_bit():
    # RN(-v) = -RN(v), and a zero result takes the sign of the IEEE product
    rng, lay, slot, x, H, I = _random_expert(27)
    x[0] = 0                                           # exact-zero sums: +0 * s
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I)
    g2, u2, _ = oracle.expert_gate_up(_with_scales(slot, lay, I, -1.0, -1.0), lay, x, H, I)
    assert np.array_equal(_bits(g2), _bits(-g)) and np.array_equal(_bits(u2), _bits(-u))
    assert np.all(_bits(g2[0]) == 0x80000000)


_F32_OVERFLOW = Fraction(2) ** 128 - Fraction(2) ** 103     # fmax + half an ulp: ties go to infinity


def _ieee_scaled(S, s):
    """F32 value of ``S * s`` for an exact sum ``S`` and an F32 scale ``s``:
    zeros from numpy's float32 multiply (which fixes their sign), infinities
    beyond the overflow threshold, else the nearest float32."""
    if S == 0 or s == 0:
        return np.float32(np.sign(float(S))) * np.float32(s)
    v = S * Fraction(float(s))
    if abs(v) >= _F32_OVERFLOW:
        return np.float32(math.copysign(math.inf, v))
    r = nearest_f32(v)
    return np.float32(math.copysign(0.0, v)) if r == 0 else r


def test_signed_zero_subnormal_and_huge_scales():
    H, I, M = 64, 10, 4
    rng = np.random.default_rng(28)
    gn = rng.integers(0, 16, (I, H))
    un = rng.integers(0, 16, (I, H))
    gs = np.array([0.0, -0.0, 1e-45, -3e-39, 2.0 ** -126, 1e38, -1e38, 0.75, -0.01, 3.4e38], dtype=np.float32)
    us = gs[::-1].copy()
    gw, uw = synth.pack_nibbles(gn), synth.pack_nibbles(un)
    lay, slot = _slot(H, I, gw, uw, gs, us)
    x = synth.bf16_normal(rng, (M, H))
    x[1] = 0                                           # exact-zero sums
    x[2, :8] = 0x7149                                  # ~1e30: products far beyond F32
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I)
    for m in range(M):
        xv = [bf16_value(int(b)) for b in x[m]]
        for i in range(I):
            sg = sum((unpack_nibble(gw, i, k) - 8) * xv[k] for k in range(H))
            su = sum((unpack_nibble(uw, i, k) - 8) * xv[k] for k in range(H))
            assert _bits(g[m, i]) == _bits(_ieee_scaled(sg, gs[i])), (m, i)
            assert _bits(u[m, i]) == _bits(_ieee_scaled(su, us[i])), (m, i)
    assert np.any(np.isinf(g)) and np.any(_bits(g) == 0x80000000) and np.any((_bits(g) & 0x7F800000) == 0)


def test_negated_input_negates_gate_and_up():
    rng, lay, slot, x, H, I = _random_expert(24)
    g, u, _ = oracle.expert_gate_up(slot, lay, x, H, I)
    g2, u2, _ = oracle.expert_gate_up(slot, lay, (x ^ 0x8000).astype(np.uint16), H, I)
    assert np.array_equal(g2, -g) and np.array_equal(u2, -u)


def test_row_permutation_is_equivariant():
    rng, lay, slot, x, H, I = _random_expert(25)
    g, u, o = oracle.expert_gate_up(slot, lay, x, H, I)
    perm = rng.permutation(I)
    gw = np.frombuffer(slot, "<u4", I * H // 8, lay.gate_weight_offset).reshape(I, H // 8)[perm]
    uw = np.frombuffer(slot, "<u4", I * H // 8, lay.up_weight_offset).reshape(I, H // 8)[perm]
    gs = np.frombuffer(slot, "<f4", I, lay.gate_scale_offset)[perm]
    us = np.frombuffer(slot, "<f4", I, lay.up_scale_offset)[perm]
    lay2, slot2 = _slot(H, I, gw, uw, gs, us)
    g2, u2, o2 = oracle.expert_gate_up(slot2, lay2, x, H, I)
    assert np.array_equal(g2, g[:, perm]) and np.array_equal(o2, o[:, perm])


def test_token_order_is_equivariant():
    rng, lay, slot, x, H, I = _random_expert(26, M=5)
    g, u, o = oracle.expert_gate_up(slot, lay, x, H, I)
    g2, u2, o2 = oracle.expert_gate_up(slot, lay, x[::-1].copy(), H, I)
    assert np.array_equal(g2, g[::-1]) and np.array_equal(o2, o[::-1])


# --------------------------------------------------------------------------
# SwiGLU tail
# --------------------------------------------------------------------------

def test_tail_closed_forms():
    up = np.array([3.0, -2.5, 7.0, 1.0], dtype=np.float32)
    o = oracle.swiglu_tail(np.zeros(4, np.float32), up)
    assert np.all((o & 0x7FFF) == 0)                       # silu(0) = 0
    o = oracle.swiglu_tail(np.full(4, 100.0, np.float32), up)
    assert np.array_equal(oracle.bf16_to_f32(o), np.float32(100.0) * up)   # sigmoid -> 1
    o = oracle.swiglu_tail(np.full(4, -89.0, np.float32), up)              # exp overflows f32
    assert np.all((o & 0x7FFF) == 0)
    o = oracle.swiglu_tail(np.array([-89.0], np.float32), np.array([1.0], np.float32))
    assert int(o[0]) == 0x8000                             # (-89) * 0 = -0


def test_tail_sigmoid_exhaustive_over_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    g = oracle.bf16_to_f32(bits)
    keep = np.isfinite(g)
    g = g[keep]
    o = oracle.swiglu_tail(g, np.ones_like(g))              # out = bf16(g * bf16(sigmoid(g)))
    got = oracle.bf16_to_f32(o).astype(np.float64)
    gd = g.astype(np.float64)
    with np.errstate(over="ignore"):
        exact = gd / (1.0 + np.exp(-gd))
    tol = np.abs(exact) * 2.0 ** -7 + 2.0 ** -133           # 1 bf16 subnormal step
    tol = np.where(gd < -80.0, 1e-34, tol)                  # F32 sigmoid underflow band
    assert np.all(np.abs(got - exact) <= tol)
    # sign follows g except where the product underflows to zero
    nz = got != 0
    assert np.all(np.sign(got[nz]) == np.sign(gd[nz]))


def test_tail_rounding_points_against_rationals():
    """Spot checks: every intermediate rounded as the kernel's comment says."""
    rng = np.random.default_rng(31)
    gate = (rng.standard_normal(400) * 4).astype(np.float32)
    up = (rng.standard_normal(400) * 4).astype(np.float32)
    o = oracle.swiglu_tail(gate, up)
    for gv, uv, ov in zip(gate, up, o):
        gT = Fraction(float(oracle.bf16_to_f32(oracle.f32_to_bf16(np.float32(gv)))))
        uT = Fraction(float(oracle.bf16_to_f32(oracle.f32_to_bf16(np.float32(uv)))))
        e = np.float32(math.exp(-float(gT)))
        d = np.float32(1.0) + e
        sig = np.float32(1.0) / d
        sT = Fraction(float(oracle.bf16_to_f32(oracle.f32_to_bf16(sig))))
        # the two products are exact in f32; round them to bf16 via the torch conversion
        silu = torch.tensor(float(gT * sT), dtype=torch.float32).to(torch.bfloat16).float().item()
        out = torch.tensor(float(Fraction(silu) * uT), dtype=torch.float32).to(torch.bfloat16)
        assert int(out.view(torch.int16).item()) & 0xFFFF == int(ov)


# --------------------------------------------------------------------------
# Grouped call
# --------------------------------------------------------------------------

def test_grouped_equals_single_calls_and_zero_fills_invalid_ids():
    rng = np.random.default_rng(41)
    H, I, E, M, K = 64, 12, 5, 6, 3
    lay = synth.contiguous_layout(H, I)
    slots = np.zeros((E, lay.slot_bytes), np.uint8)
    for e in range(E):
        synth.fill_slot(rng, H, I, lay, out=slots[e])
    x = synth.bf16_normal(rng, (M, H))
    ids = rng.integers(0, E, (M, K)).astype(np.int32)
    ids[0, 0] = ids[0, 1]          # duplicate routing is computed twice
    ids[2, 1] = E                  # out of range
    ids[4, 2] = -1
    g, u, o, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert bad == 2
    for t in range(M):
        for j in range(K):
            e = int(ids[t, j])
            if 0 <= e < E:
                gs, us, os_ = oracle.expert_gate_up(slots[e], lay, x[t:t + 1], H, I)
                assert np.array_equal(g[t, j], gs[0]) and np.array_equal(o[t, j], os_[0])
            else:
                assert np.all(g[t, j] == 0) and np.all(o[t, j] == 0)


def test_layout_rules():
    lay = synth.contiguous_layout(64, 8)
    with pytest.raises(ValueError, match="divisible by 8"):
        oracle.check_layout(lay, 60, 8)
    from dataclasses import replace
    bad = replace(lay, up_scale_offset=lay.slot_bytes - 8)
    with pytest.raises(ValueError, match="up scales exceeds the canonical expert slot"):
        oracle.check_layout(bad, 64, 8)


# --------------------------------------------------------------------------
# Stored oracle outputs (regression anchor, written by tests/golden/make_golden.py)
# --------------------------------------------------------------------------

def test_cfg1_golden_is_reproduced():
    with open(os.path.join(GOLDEN, "cfg1_oracle.json")) as f:
        gold = json.load(f)
    c = synth.make_config("cfg1")
    assert synth.sha256_hex(c.slots) == gold["slot_sha256"]
    assert synth.sha256_hex(c.x) == gold["x_sha256"]
    g, u, o = oracle.expert_gate_up(c.slots[0], c.layout, c.x, c.H, c.I)
    assert [int(v) for v in _bits(g).ravel()] == gold["gate_f32_bits"]
    assert [int(v) for v in _bits(u).ravel()] == gold["up_f32_bits"]
    assert [int(v) for v in o.ravel()] == gold["out_bf16_bits"]
