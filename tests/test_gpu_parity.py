"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Covers the five workloads at full size, ragged shapes that reach every kernel
variant (column tiles NT=1/2/3, row split RT=1/2/4, 16-byte and 4-byte weight
loads, partial K-steps and chunks, ragged row tails, several token groups),
grouped-routing edge cases, special inputs, determinism and batch invariance.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import check_parity, run_grouped, run_single, say, t1_violations

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import quantized_moe_expert_q4_amd as q4
    q4.load()   # raises if the HIP library is missing: there is no fallback
    yield


def _single_case(c, label, exact=True):
    say(f"[{label}] single H={c.H} I={c.I} M={c.x.shape[0]}")
    out, g, u = run_single(c.slots[0], c.layout, c.x, c.H, c.I)
    gr, ur, orf = oracle.expert_gate_up(c.slots[0], c.layout, c.x, c.H, c.I)
    return check_parity(out, g, u, gr, ur, orf, label, require_exact_gate_up=exact)


def test_cfg1_matches_stored_oracle_bits():
    with open(os.path.join(GOLDEN, "cfg1_oracle.json")) as f:
        gold = json.load(f)
    c = synth.make_config("cfg1")
    say("[cfg1] H=256 I=128 M=1 vs tests/golden/cfg1_oracle.json")
    out, g, u = run_single(c.slots[0], c.layout, c.x, c.H, c.I)
    assert [int(v) for v in g.view(np.uint32).ravel()] == gold["gate_f32_bits"]
    assert [int(v) for v in u.view(np.uint32).ravel()] == gold["up_f32_bits"]
    assert [int(v) for v in out.ravel()] == gold["out_bf16_bits"]


def test_cfg2_decode_m1():
    _single_case(synth.make_config("cfg2"), "cfg2")


def test_cfg3_verify_m8():
    _single_case(synth.make_config("cfg3"), "cfg3")


@pytest.mark.parametrize("M", [1, 4, 16, 32])
def test_cfg5_large_expert_with_outliers(M):
    _single_case(synth.make_config("cfg5", M=M), f"cfg5 M={M}")


def test_cfg4_routed_step():
    c = synth.make_config("cfg4")
    say("[cfg4] grouped 64 slots H=6144 I=2048 M=32 K=8")
    (out, g, u), invalid = run_grouped(c.slots, c.layout, c.x, c.ids, c.H, c.I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, c.x, c.ids,
                                                     c.H, c.I)
    assert invalid == bad == 0
    check_parity(out, g, u, gr, ur, orf, "cfg4")


# (H, I, M): H % 32 != 0 (4-byte loads), H % 128 != 0 (partial K-step),
# H > chunk (several LDS chunks), I % 16 != 0, M across token-group sizes.
RAGGED = [
    (8, 1, 1), (8, 16, 3), (24, 7, 2), (136, 33, 5), (264, 18, 6), (1000, 70, 6),
    (4104, 130, 9), (4128, 17, 17), (256, 128, 40), (2048, 100, 64), (1544, 40, 2),
    (3080, 24, 8), (512, 300, 1),
]


@pytest.mark.parametrize("H,I,M", RAGGED)
def test_ragged_shapes(H, I, M):
    rng = np.random.default_rng(1000 + H + 7 * I + 13 * M)
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    x = synth.bf16_normal(rng, (M, H))
    say(f"[ragged H={H} I={I} M={M}]")
    out, g, u = run_single(slot, lay, x, H, I)
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x, H, I)
    check_parity(out, g, u, gr, ur, orf, f"ragged H={H} I={I} M={M}")


@pytest.mark.parametrize("E,I,M,K", [(64, 512, 4, 2), (64, 256, 3, 2), (32, 512, 2, 1), (3, 40, 9, 3)])
def test_grouped_row_splits(E, I, M, K):
    """Slot counts and row counts that select every row split of the kernel."""
    H = 256
    rng = np.random.default_rng(E * 100 + I + M)
    lay = synth.contiguous_layout(H, I)
    slots = np.zeros((E, lay.slot_bytes), np.uint8)
    for e in range(E):
        synth.fill_slot(rng, H, I, lay, out=slots[e])
    x = synth.bf16_normal(rng, (M, H))
    ids = synth.top_k_routing(rng, M, K, E)
    say(f"[grouped E={E} I={I} M={M} K={K}]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert invalid == bad
    check_parity(out, g, u, gr, ur, orf, f"grouped E={E} I={I} M={M} K={K}")


def test_grouped_edge_cases():
    """Invalid ids, duplicates, unused slots, a slot with more than 8 tokens."""
    H, I, E, M, K = 520, 50, 6, 20, 3
    rng = np.random.default_rng(77)
    lay = synth.contiguous_layout(H, I)
    stride = lay.slot_bytes + 4096             # slots spaced wider than their layout
    slots = np.zeros((E, stride), np.uint8)
    for e in range(E):
        synth.fill_slot(rng, H, I, lay, out=slots[e, :lay.slot_bytes])
    x = synth.bf16_normal(rng, (M, H))
    ids = rng.integers(0, 3, (M, K)).astype(np.int32)   # slots 3..5 unused; slot 0..2 get ~20 pairs
    ids[1, 0] = ids[1, 1] = 2                          # duplicate pair
    ids[3, 2] = E
    ids[7, 0] = -5
    ids[19, 2] = 1 << 30
    say("[grouped edge cases]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, stride, E, lay, x, ids, H, I)
    assert bad == 3 and invalid == 3
    check_parity(out, g, u, gr, ur, orf, "grouped edge cases")


def test_grouped_many_invalid_ids_batch_kernel():
    """Hundreds of invalid ids on one work-group of the batch kernel (two
    slots of one 16-row tile each: two work-groups), past one zero-fill batch
    of 64 pairs: every invalid pair's outputs are zeros, the count is exact."""
    H, I, E, M, K = 256, 16, 2, 500, 4
    rng = np.random.default_rng(78)
    lay = synth.contiguous_layout(H, I)
    slots = np.zeros((E, lay.slot_bytes), np.uint8)
    for e in range(E):
        synth.fill_slot(rng, H, I, lay, out=slots[e])
    x = synth.bf16_normal(rng, (M, H))
    ids = rng.integers(0, E, (M, K)).astype(np.int32)
    bad_mask = rng.random((M, K)) < 0.5
    ids[bad_mask] = np.where(rng.random(int(bad_mask.sum())) < 0.5, -1, E + 7).astype(np.int32)
    say(f"[grouped many invalid ids: {int(bad_mask.sum())} of {M * K}]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert bad == invalid == int(bad_mask.sum())
    check_parity(out, g, u, gr, ur, orf, "grouped many invalid ids")


def test_field_order_and_padding_in_slot():
    """Fields in another order with gaps: only the offsets matter."""
    H, I, M = 384, 24, 3
    rng = np.random.default_rng(5)
    wb = I * H // 2
    lay = synth.SlotLayout(slot_bytes=8192 + 2 * wb + 4096, up_weight_offset=4096, gate_weight_offset=4096 + wb + 48,
                           up_scale_offset=64, gate_scale_offset=1024)
    slot = np.zeros(lay.slot_bytes, np.uint8)
    gw = rng.integers(0, 1 << 32, (I, H // 8), dtype=np.uint64).astype(np.uint32)
    uw = rng.integers(0, 1 << 32, (I, H // 8), dtype=np.uint64).astype(np.uint32)
    synth.write_slot(lay, H, I, gw, uw, rng.uniform(0.01, 0.02, I), rng.uniform(0.01, 0.02, I), out=slot)
    x = synth.bf16_normal(rng, (M, H))
    out, g, u = run_single(slot, lay, x, H, I)
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x, H, I)
    check_parity(out, g, u, gr, ur, orf, "reordered fields")


def _wide_bits(rng, shape, max_field=200):
    sign = rng.integers(0, 2, shape) << 15
    e = rng.integers(0, max_field + 1, shape)
    f = rng.integers(0, 128, shape)
    b = (sign | (e << 7) | f).astype(np.uint16)
    b[rng.random(shape) < 0.05] = 0
    return b


def test_wide_exponent_range_within_certified_bound():
    """Entries far below a token's largest are rounded to its 2^-38 grid."""
    H, I, M = 512, 32, 4
    rng = np.random.default_rng(9)
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    x = _wide_bits(rng, (M, H))
    x[0] = synth.bf16_normal(rng, (1, H))[0]          # one ordinary token: exact
    out, g, u = run_single(slot, lay, x, H, I)
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x, H, I)
    gs = np.frombuffer(slot, "<f4", I, lay.gate_scale_offset).astype(np.float64)
    etop1 = np.maximum((np.max(x & 0x7FFF, axis=1) >> 7) & 0xFF, 1).astype(np.float64)
    # per token: |error of the sum| <= sum_k |w_k| * 2^(etop1 - 173) <= 8 H 2^(etop1-173)
    bound = 8 * H * np.exp2(etop1 - 173)[:, None] * gs[None, :]
    err = np.abs(g.astype(np.float64) - gr.astype(np.float64))
    ok = err <= 1e-5 * np.abs(gr) + 1e-6 + bound * (1 + 1e-6) + np.abs(gr) * 2.0 ** -23
    t1 = t1_violations(g, gr)
    say(f"[wide exponents] max err/bound = {float(np.max(err / (bound + 1e-300))):.3g}; "
        f"T1 violations {t1}/{g.size}")
    assert ok.all()
    # on these inputs (random exponents, no cancellation built in) the
    # rounded small entries stay inside plain T1 as well
    assert t1 == 0
    assert np.array_equal(g[0].view(np.uint32), gr[0].view(np.uint32))


def test_entries_below_the_exact_window_follow_the_stated_bound():
    """The limit of the exact window, shown on purpose.  A token with one
    entry of 2^40 and the rest near 2^-10 spans 50 binades; its entries more
    than 38 binades below the largest are rounded to the 2^(e_top - 38) grid
    (those more than 46 below, as here, to zero).  Rows whose weight at the
    huge entry is zero (nibble 8) then lose their whole true sum: the result
    stays within the stated bound but T1 does not hold for them.  The
    ordinary token next to it stays bit-exact."""
    H, I, M = 512, 32, 2
    rng = np.random.default_rng(21)
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    words = np.frombuffer(slot, "<u4").copy()
    for off in (lay.gate_weight_offset, lay.up_weight_offset):
        rows = words[off // 4: off // 4 + I * H // 8].reshape(I, H // 8)
        rows[:, 0] = (rows[:, 0] & ~np.uint32(0xF)) | np.uint32(8)     # weight 0 at k = 0
    slot = words.view(np.uint8)
    x = synth.bf16_normal(rng, (M, H))
    small = (np.exp2(rng.uniform(-12, -8, H)) * np.where(rng.random(H) < 0.5, -1.0, 1.0)).astype(np.float32)
    x[1] = (small.view(np.uint32) >> 16).astype(np.uint16)
    x[1, 0] = (127 + 40) << 7                                         # 2^40
    out, g, u = run_single(slot, lay, x, H, I)
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x, H, I)
    gs = np.frombuffer(slot, "<f4", I, lay.gate_scale_offset).astype(np.float64)
    etop1 = np.maximum((np.max(x & 0x7FFF, axis=1) >> 7) & 0xFF, 1).astype(np.float64)
    bound = 8 * H * np.exp2(etop1 - 173)[:, None] * gs[None, :]
    err = np.abs(g.astype(np.float64) - gr.astype(np.float64))
    t1 = t1_violations(g[1], gr[1])
    say(f"[below the window] token 1: max err {float(err[1].max()):.3g}, bound {float(bound[1].max()):.3g}, "
        f"T1 violations {t1}/{I}")
    assert (err <= bound * (1 + 1e-6) + np.abs(gr) * 2.0 ** -23 + 1e-30).all()
    assert np.array_equal(g[0].view(np.uint32), gr[0].view(np.uint32))
    assert np.array_equal(u[0].view(np.uint32), ur[0].view(np.uint32))


def test_nonfinite_token_gives_nan_rows_only():
    H, I, M = 256, 20, 3
    rng = np.random.default_rng(11)
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    x = synth.bf16_normal(rng, (M, H))
    x[1, 17] = 0x7F80                                  # +Inf
    out, g, u = run_single(slot, lay, x, H, I)
    assert np.all(np.isnan(g[1])) and np.all(np.isnan(u[1]))
    assert np.all((out[1] & 0x7FFF) > 0x7F80)          # NaN
    keep = [0, 2]
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x[keep], H, I)
    check_parity(out[keep], g[keep], u[keep], gr, ur, orf, "finite tokens next to an Inf token")


def test_zero_token_and_all_eight_rows():
    H, I, M = 256, 40, 2
    rng = np.random.default_rng(12)
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay, zero_row_fraction=0.25)
    x = synth.bf16_normal(rng, (M, H))
    x[1] = 0
    out, g, u = run_single(slot, lay, x, H, I)
    assert np.all(g[1].view(np.uint32) == 0) and np.all(out[1] == 0)
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x, H, I)
    check_parity(out, g, u, gr, ur, orf, "zero token / all-8 rows")


@pytest.mark.parametrize("H,M", [(4096, 3), (1024, 6), (264, 2), (7168, 8)])
def test_subnormal_and_sparse_tokens(H, M):
    """Tokens of zeros, signed zeros, subnormals and lone values: the largest
    magnitude and the smallest non-zero exponent each kernel derives per token
    (its digit count and split exponent) must give the oracle's exact bits.
    Shapes reach the resident kernel's wave and per-lane range paths and the
    batch kernel."""
    I = 48
    rng = np.random.default_rng(H + 13 * M)
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    x = synth.bf16_normal(rng, (M, H))
    x[0] = 0x8000                                      # negative zeros ...
    x[0, 5] = 0x0001                                   # ... and one subnormal
    mag = rng.integers(0, 0x80, H).astype(np.uint16)   # subnormal magnitudes and zeros
    x[1] = mag | (rng.integers(0, 2, H).astype(np.uint16) << 15)
    if M > 2:
        x[2, rng.integers(0, H, 7)] = 0x0003           # a normal token with subnormals in it
    if M > 3:
        x[3] = 0
        x[3, H - 1] = 0xC780                           # one value, -65536
    say(f"[subnormal/sparse tokens] H={H} M={M}")
    out, g, u = run_single(slot, lay, x, H, I)
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x, H, I)
    check_parity(out, g, u, gr, ur, orf, f"subnormal/sparse tokens H={H} M={M}")


def test_determinism_and_batch_invariance():
    c = synth.make_config("cfg3")
    say("[invariance] cfg3 twice, per-token M=1 calls, grouped with one slot")
    o1, g1, u1 = run_single(c.slots[0], c.layout, c.x, c.H, c.I)
    o2, g2, u2 = run_single(c.slots[0], c.layout, c.x, c.H, c.I)
    assert np.array_equal(o1, o2) and np.array_equal(g1.view(np.uint32), g2.view(np.uint32))
    for t in range(c.M):
        ot, gt, ut = run_single(c.slots[0], c.layout, c.x[t:t + 1], c.H, c.I)
        assert np.array_equal(ot[0], o1[t]) and np.array_equal(gt[0].view(np.uint32), g1[t].view(np.uint32))
    ids = np.zeros((c.M, 1), np.int32)
    (og, gg, ug), invalid = run_grouped(c.slots, c.layout, c.x, ids, c.H, c.I)
    assert invalid == 0
    assert np.array_equal(og[:, 0], o1) and np.array_equal(gg[:, 0].view(np.uint32), g1.view(np.uint32))


DIGIT_PATHS = [
    (7168, 96, 8, False),   # batch kernel, three column tiles, K-chunks, four digits
    (7168, 64, 4, True),    # batch kernel, two column tiles, six digits
    (8832, 40, 2, False),   # batch kernel, one column tile (too long for resident digits)
    (4096, 80, 8, True),    # resident digits, two column tiles, six digits: two passes
    (2048, 40, 4, True),    # resident, two column tiles, six digits, one pass
    (1024, 48, 5, False),   # resident, two column tiles, four digits
    (2048, 40, 2, True),    # resident, one column tile, six digits
]


@pytest.mark.parametrize("H,I,M,wide", DIGIT_PATHS)
def test_digit_count_paths(H, I, M, wide):
    """Calls whose tokens all have their values within 22 binades of the
    token's largest (four digits per value) and calls sent back to six digits
    by one token whose values span more binades, through every kernel and
    column-tile count that the width and H select."""
    rng = np.random.default_rng(H + I + M + int(wide))
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    x = synth.bf16_normal(rng, (M, H))
    if wide:
        t = min(3, M - 1)
        x[t, 5] = 0x461C                                 # 9984
        x[t, 6] = 0x3300                                 # 2^-25: 38 binades below it
    say(f"[digit paths H={H} I={I} M={M} wide={wide}]")
    out, g, u = run_single(slot, lay, x, H, I)
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x, H, I)
    check_parity(out, g, u, gr, ur, orf, f"digit paths H={H} M={M} wide={wide}")
