"""GPU parity of grouped calls with one or two tokens (the decode kernel).

The cases cover the full-size slot pool the benchmark times (every output
checked, also at eight tokens), sparse routing, two tokens sharing or
splitting slots, a token routed twice to one slot, invalid ids, hidden sizes
whose K-steps split unevenly between waves, many one-tile slots, a pool of
1500 small slots, and a workspace reused across calls.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import check_parity, poisoned, run_grouped, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import quantized_moe_expert_q4_amd as q4
    q4.load()
    yield


def _pool(rng, E, H, I, stride_pad=0):
    lay = synth.contiguous_layout(H, I)
    slots = np.zeros((E, lay.slot_bytes + stride_pad), np.uint8)
    for e in range(E):
        synth.fill_slot(rng, H, I, lay, out=slots[e, :lay.slot_bytes])
    return lay, slots


def _check(slots, lay, x, ids, H, I, label, ws=None):
    (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I, ws=ws)
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, slots.shape[1], slots.shape[0], lay, x, ids, H, I)
    assert invalid == bad, label
    check_parity(out, g, u, gr, ur, orf, label)


@pytest.mark.parametrize("M", [1, 8])
def test_benchmark_pool_full_size(M):
    """The exact launch the benchmark times: 171 slots (eight distinct
    contents), H=4096, I=1536, every slot routed by every token."""
    import torch
    import bench
    import quantized_moe_expert_q4_amd as q4
    from quantized_moe_expert_q4_amd.device import aligned_empty, bf16_bits, upload_bf16_bits
    lay, contents, x8 = bench.make_pool_host()
    pool = bench.Pool(lay, contents, x8)
    E, H, I = bench.POOL_SLOTS, bench.H, bench.I
    x = x8[:M]
    ids = np.tile(np.arange(E, dtype=np.int32), (M, 1))
    say(f"[benchmark pool M={M}] {E} slots H={H} I={I}")
    out = poisoned((M, E, I), torch.bfloat16)
    g = poisoned((M, E, I), torch.float32)
    u = poisoned((M, E, I), torch.float32)
    wsb = q4.grouped_workspace_bytes(M, E, E)
    ws = aligned_empty(wsb, 256)
    ws.fill_(0xAB)
    idt = torch.from_numpy(ids).cuda()
    xd = upload_bf16_bits(x)
    for rep in range(2):  # the second call reuses the workspace as the benchmark does
        out.zero_()
        q4.expert_gate_up_grouped(pool.slots, pool.stride, E, lay, xd, M, idt, E, H, I, out, ws, wsb, g, u)
        torch.cuda.synchronize()
        ob, gb, ub = bf16_bits(out), g.cpu().numpy(), u.cpu().numpy()
        ref = [oracle.expert_gate_up(contents[c], lay, x, H, I) for c in range(bench.DISTINCT_CONTENTS)] if rep == 0 else ref
        sel = np.arange(E) % bench.DISTINCT_CONTENTS
        gr = np.stack([ref[c][0] for c in sel], axis=1)
        ur = np.stack([ref[c][1] for c in sel], axis=1)
        orf = np.stack([ref[c][2] for c in sel], axis=1)
        check_parity(ob, gb, ub, gr, ur, orf, f"benchmark pool M={M} call {rep}")


CASES = [
    # E, M, K, H, I, routing
    (64, 1, 8, 2048, 384, "topk"),       # sparse: 8 of 64 slots streamed
    (48, 2, 6, 2048, 512, "topk"),       # two tokens: slots with one or both
    (12, 1, 12, 7168, 256, "perm"),      # every slot, permuted; 56 K-steps split 6/8 between waves
    (40, 2, 20, 256, 100, "topk"),       # two K-steps: waves with empty ranges
    (700, 1, 700, 256, 16, "perm"),      # one tile per slot, more tiles than work-groups
    (1, 2, 1, 4096, 1536, "perm"),       # one slot, both tokens
    (1500, 1, 40, 256, 32, "topk"),      # a large pool, few routed slots
    (64, 8, 8, 1024, 200, "topk"),       # verify width: two column tiles, sparse slots
    (16, 5, 16, 512, 64, "perm"),        # five tokens on every slot
    (300, 8, 300, 256, 16, "perm"),      # 2400 pairs: routing windows past the id registers
    (3, 3, 3, 4096, 48, "perm"),         # three tokens, three slots
]


@pytest.mark.parametrize("E,M,K,H,I,kind", CASES)
def test_decode_routing(E, M, K, H, I, kind):
    rng = np.random.default_rng(E * 7 + M * 3 + H + I)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    if kind == "topk":
        ids = synth.top_k_routing(rng, M, K, E)
    else:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(M)]).astype(np.int32)
    label = f"decode E={E} M={M} K={K} H={H} I={I} {kind}"
    say(f"[{label}]")
    _check(slots, lay, x, ids, H, I, label)


def test_decode_duplicates_and_invalid_ids():
    """A token routed twice to one slot gets the result in both pairs; invalid
    ids zero their pairs and are counted."""
    E, M, K, H, I = 7, 2, 5, 1024, 200
    rng = np.random.default_rng(4242)
    lay, slots = _pool(rng, E, H, I, stride_pad=4096)
    x = synth.bf16_normal(rng, (M, H))
    ids = np.array([[3, 1, 3, 6, -1],
                    [3, 3, 3, E, 0]], np.int32)
    say("[decode duplicates and invalid ids]")
    _check(slots, lay, x, ids, H, I, "decode duplicates and invalid ids")


def test_invalid_ids_before_and_past_the_id_registers():
    """Invalid ids among the first 2048 pairs (marked at the start from the
    ids held in registers) and past them (read again at the end), in one call
    of eight tokens: every such pair is zero and counted."""
    E, M, K, H, I = 300, 8, 300, 256, 16
    rng = np.random.default_rng(2048)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(M)]).astype(np.int32)
    flat = ids.reshape(-1)
    for p, v in [(0, -1), (5, E), (511, -7), (512, E + 3), (2047, -1), (2048, E), (2300, -2), (2399, 1 << 20)]:
        flat[p] = v
    say("[invalid ids before and past the id registers]")
    _check(slots, lay, x, ids, H, I, "invalid ids before and past the id registers")


@pytest.mark.parametrize("M", [2, 5])
def test_token_routed_three_times_to_one_slot(M):
    """A token routed an odd number (3) of times to one slot while every other
    token of the slot's group has a single pair there: each of the three
    pairs gets the result (regression: the third match once undid the
    several-pairs flag, and only the last pair was written)."""
    E, K, H, I = 6, 3, 1024, 200
    rng = np.random.default_rng(77 + M)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    ids = np.array([[(t + j) % E for j in range(K)] for t in range(M)], np.int32)
    ids[0] = [5, 1, 0]
    ids[1] = [5, 5, 5]
    label = f"token routed three times, M={M}"
    say(f"[{label}]")
    _check(slots, lay, x, ids, H, I, label)


def test_verify_width_many_pairs_on_one_slot():
    """Eight tokens each routed several times to one slot: more pairs than one
    pass over the slot finishes, duplicates, and an unrouted slot."""
    E, M, K, H, I = 3, 8, 5, 2048, 96
    rng = np.random.default_rng(515)
    lay, slots = _pool(rng, E, H, I)
    x = synth.bf16_normal(rng, (M, H))
    ids = np.full((M, K), 1, np.int32)
    ids[:, 4] = 0
    ids[2, 1] = 0
    ids[5, 3] = -7
    say("[verify width, many pairs on one slot]")
    _check(slots, lay, x, ids, H, I, "verify width many pairs")


def test_decode_workspace_reuse():
    """Three calls with different routing through one workspace."""
    import torch
    import quantized_moe_expert_q4_amd as q4
    from quantized_moe_expert_q4_amd.device import aligned_empty, upload_slots
    E, M, K, H, I = 32, 1, 6, 2048, 512
    rng = np.random.default_rng(99)
    lay, slots = _pool(rng, E, H, I)
    dev = upload_slots(slots)
    ws = aligned_empty(q4.grouped_workspace_bytes(M, K, E), 256)
    ws.fill_(0x5A)
    for call in range(3):
        x = synth.bf16_normal(rng, (M, H))
        ids = synth.top_k_routing(rng, M, K, E)
        (out, g, u), invalid = run_grouped(slots, lay, x, ids, H, I, ws=ws, slots=dev)
        gr, ur, orf, bad = oracle.expert_gate_up_grouped(slots, slots.shape[1], E, lay, x, ids, H, I)
        assert invalid == bad
        check_parity(out, g, u, gr, ur, orf, f"workspace reuse call {call}")
