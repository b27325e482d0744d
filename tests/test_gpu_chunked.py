"""GPU parity of the chunked kernel (routed calls with a few rows per slot
whose digits do not all fit LDS for the launch) against the oracle.

Grouped calls with bf16 activations and Q4 weights go to this kernel when
the resident kernel cannot hold their rows and the routed pairs per slot
average at most six (two column tiles; one for a down projection of one row
per slot); single-expert calls of up to eight tokens that the resident
kernel cannot hold go there too.  The shapes below reach: one and two column
tiles; the whole K in LDS and K cut into two-buffer chunks (with a short last
chunk and padding steps); several rounds per segment and several segments
per work-group; slots with more pairs than one pass holds (work cut by
cost); calls over more slots than the pass counts cover; rounds of a few
tiles shared by many waves through the fix-up slots; four- and six-digit rows
in one group; invalid and duplicate ids; rows whose bytes are not 16-byte
aligned; ragged tiles; and the down projection, single and grouped.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_moe_expert_q4_amd as q4
from tests.gpu_helpers import (check_down_parity, check_parity, run_down_grouped, run_down_single, run_grouped,
                               run_single, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    q4.load()   # raises if the HIP library is missing: there is no fallback
    yield


def _pool(rng, E, H, I, down=False):
    lay = synth.expert_layout(H, I) if down else synth.contiguous_layout(H, I)
    slots = np.zeros((E, lay.slot_bytes), np.uint8)
    for e in range(E):
        synth.fill_slot(rng, H, I, lay, out=slots[e])
    return lay, slots


def _wide(x, rows):
    """Rows given a 9984 entry next to a 2^-25 one: six digits per value."""
    x = x.copy()
    for t in rows:
        x[t, 5] = 0x461C
        x[t, 6] = 0x3300
    return x


# (E, H, I, M, K, wide rows, label)
GROUPED = [
    (24, 2048, 520, 12, 2, (), "one column tile, ragged tiles, tiny ranges (fix-ups)"),
    (8, 6144, 2048, 32, 1, (), "two column tiles, four pairs per slot, K in three chunks"),
    (16, 4104, 200, 20, 3, (), "rows not 16-byte aligned, padding steps, short last chunk"),
    (8, 3072, 256, 10, 4, (1, 7), "six-digit groups: several groups per slot"),
    (40, 512, 2048, 40, 5, (), "several rounds per segment"),
    (160, 512, 2048, 160, 1, (), "several segments per work-group, one pair per slot"),
    (2100, 256, 16, 20, 2, (), "more slots than the pair counts cover"),
]


@pytest.mark.parametrize("E,H,I,M,K,wide,label", GROUPED, ids=[g[-1] for g in GROUPED])
def test_chunked_grouped(E, H, I, M, K, wide, label):
    rng = np.random.default_rng(E * 1000 + H + I + M + K)
    lay, slots = _pool(rng, E, H, I)
    x = _wide(synth.bf16_normal(rng, (M, H)), wide)
    ids = synth.top_k_routing(rng, M, K, E)
    say(f"[chunked grouped E={E} H={H} I={I} M={M} K={K} wide={list(wide)}]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert invalid == bad == 0
    check_parity(out, g, u, gr, ur, orf, f"chunked grouped {label}")


def test_chunked_skewed_routing_invalid_and_duplicate_ids():
    """Most pairs on two slots (several groups there), unrouted slots, a token
    routed twice to one slot, and ids outside [0, E)."""
    E, H, I, M, K = 16, 1536, 96, 24, 3
    rng = np.random.default_rng(4242)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    ids = np.where(rng.random((M, K)) < 0.7, rng.integers(3, 5, (M, K)), rng.integers(0, E, (M, K))).astype(np.int32)
    ids[2, 0] = ids[2, 1] = 4
    ids[5, 2] = E
    ids[9, 0] = -1
    ids[23, 1] = 1 << 30
    say(f"[chunked skewed E={E} H={H} I={I} M={M} K={K}]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert bad == 3 and invalid == 3
    check_parity(out, g, u, gr, ur, orf, "chunked skewed routing")


def test_chunked_slot_with_more_passes_than_counted():
    """1800 of 2400 pairs on one slot (more than 255 passes of 7): the pass
    counts are turned off, every slot takes one pass and the hot slot's pairs
    run in 258 token groups over its tiles."""
    E, H, I, M, K = 400, 256, 16, 300, 8
    rng = np.random.default_rng(1800)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    ids = rng.integers(1, E, size=(M, K)).astype(np.int32)
    ids[:, :6] = 0
    say(f"[chunked hot slot E={E} H={H} I={I} M={M} K={K}]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert invalid == bad == 0
    check_parity(out, g, u, gr, ur, orf, "chunked slot with more passes than counted")


@pytest.mark.parametrize("hot", [1785, 1786])
def test_chunked_pass_count_limit(hot):
    """A slot with 1785 pairs (255 passes of 7, the most one byte of the pass
    table holds: counted) or 1786 (256 passes: the counts are turned off)."""
    E, H, I, M, K = 300, 256, 16, 300, 6
    rng = np.random.default_rng(hot)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    ids = rng.integers(1, E, size=(M, K)).astype(np.int32)
    flat = ids.reshape(-1)
    flat[:hot] = 0
    say(f"[chunked pass count limit: {hot} pairs on one slot]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert invalid == bad == 0
    check_parity(out, g, u, gr, ur, orf, f"chunked pass count limit {hot}")


@pytest.mark.parametrize("E", [2048, 2049])
def test_chunked_slot_count_limit(E):
    """Sparse routing over 2048 slots (the most the pass table covers) and over
    2049 (one pass per slot, no counts)."""
    H, I, M, K = 256, 16, 40, 8
    rng = np.random.default_rng(E)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    ids = synth.top_k_routing(rng, M, K, E)
    ids[0, 0] = E - 1
    say(f"[chunked slot count limit E={E}]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert invalid == bad == 0
    check_parity(out, g, u, gr, ur, orf, f"chunked slot count limit E={E}")


def test_chunked_all_ids_invalid():
    """Every id out of range: no slot is streamed, every pair is zero and counted."""
    E, H, I, M, K = 16, 512, 48, 20, 4
    rng = np.random.default_rng(404)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    ids = np.where(rng.random((M, K)) < 0.5, -1 - rng.integers(0, 5, (M, K)), E + rng.integers(0, 5, (M, K)))
    ids = ids.astype(np.int32)
    say(f"[chunked all ids invalid E={E} M={M} K={K}]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert invalid == bad == M * K
    check_parity(out, g, u, gr, ur, orf, "chunked all ids invalid")


def test_chunked_invalid_ids_before_and_past_the_id_registers():
    """Invalid ids among the first 2048 pairs (marked at the start from the ids
    held in registers) and past them (read again at the end): 2400 pairs of
    400 tokens over 600 slots, four per slot on average."""
    E, H, I, M, K = 600, 512, 48, 400, 6
    rng = np.random.default_rng(6006)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    ids = synth.top_k_routing(rng, M, K, E)
    flat = ids.reshape(-1)
    for p, v in [(0, -1), (7, E), (511, -9), (1024, E + 1), (2047, -1), (2048, E), (2222, -3), (2399, 1 << 24)]:
        flat[p] = v
    say(f"[chunked invalid ids E={E} H={H} I={I} M={M} K={K}]")
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, lay.slot_bytes, E, lay, x, ids, H, I)
    assert bad == 8 and invalid == 8
    check_parity(out, g, u, gr, ur, orf, "chunked invalid ids before and past the id registers")


@pytest.mark.parametrize("H,I,M,wide", [(7168, 512, 3, True), (16384, 64, 5, False), (12288, 48, 8, False),
                                         (7168, 264, 8, "all")])
def test_chunked_single_expert(H, I, M, wide):
    """Single-expert calls of up to eight tokens whose digits exceed the
    resident kernel's LDS (eight six-digit tokens: two groups per pass)."""
    rng = np.random.default_rng(H + I + M)
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    x = _wide(synth.bf16_normal(rng, (M, H)), tuple(range(M)) if wide == "all" else ((0,) if wide else ()))
    say(f"[chunked single H={H} I={I} M={M} wide={wide}]")
    out, g, u = run_single(slot, lay, x, H, I)
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x, H, I)
    check_parity(out, g, u, gr, ur, orf, f"chunked single H={H} I={I} M={M}")


@pytest.mark.parametrize("E,H,I,wide", [(20, 4096, 1536, False), (12, 520, 2048, True), (40, 264, 8192, False),
                                        (120, 4096, 64, True)])
def test_chunked_down_grouped(E, H, I, wide):
    """The grouped down projection with one routed row per slot (the down
    step of one token routed to E experts): H output rows, I inputs.  The
    last case gives each work-group about 60 tiles: segments longer than
    the 48 tiles of gate/up calls."""
    rng = np.random.default_rng(E + H + I)
    lay, slots = _pool(rng, E, H, I, down=True)
    ids = np.arange(E, dtype=np.int32).reshape(1, E)
    mid = synth.bf16_normal(rng, (1, E, I))
    if wide:
        mid[0, 3, 5] = 0x461C
        mid[0, 3, 6] = 0x3300
    say(f"[chunked down grouped E={E} H={H} I={I}]")
    (out, d), invalid = run_down_grouped(slots, lay, mid, ids, H, I)
    d_ref, o_ref, bad = oracle.expert_down_grouped(slots, lay.slot_bytes, E, lay, mid, ids, H, I)
    assert invalid == bad == 0
    check_down_parity(out, d, d_ref, o_ref, f"chunked down grouped E={E} H={H} I={I}")


def test_chunked_down_single():
    """A single-slot down call whose reduction is too long for the resident
    kernel's LDS."""
    H, I, M = 72, 16384, 5
    rng = np.random.default_rng(515)
    lay = synth.expert_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    mid = synth.bf16_normal(rng, (M, I))
    say(f"[chunked down single H={H} I={I} M={M}]")
    out, d = run_down_single(slot, lay, mid, H, I)
    d_ref, o_ref = oracle.expert_down(slot, lay, mid, H, I)
    check_down_parity(out, d, d_ref, o_ref, "chunked down single")
