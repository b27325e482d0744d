"""The grouped call on the library's static scratch (no device allocation)
against the grouped call with a caller-provided workspace, through the C ABI:
bit-identical outputs and the same out-of-range id count, on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
contents, so the second call's count must be its own)."""
import numpy as np
import pytest
import torch

import synth
import quantized_moe_expert_q4_amd as q4
from quantized_moe_expert_q4_amd.device import aligned_empty, bf16_bits, upload_bf16_bits, upload_slots
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    q4.load()   # raises if the HIP library is missing: there is no fallback
    yield


def _case(E, H, I, M, K, seed, n_invalid):
    rng = np.random.default_rng(seed)
    lay = synth.contiguous_layout(H, I)
    slots = np.zeros((E, lay.slot_bytes), np.uint8)
    for e in range(E):
        synth.fill_slot(rng, H, I, lay, out=slots[e])
    x = synth.bf16_normal(rng, (M, H))
    ids = synth.top_k_routing(rng, M, K, E).astype(np.int32)
    flat = ids.reshape(-1)
    pos = rng.choice(flat.size, n_invalid, replace=False)
    flat[pos[0::2]] = E + 3
    flat[pos[1::2]] = -1
    return lay, slots, x, ids


def _both(lay, slots, x, ids, H, I):
    E = slots.shape[0]
    M, K = ids.shape
    d_slots = upload_slots(slots)
    xd = upload_bf16_bits(x)
    idt = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
    ref = torch.full((M, K, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, K, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    wsb = q4.grouped_workspace_bytes(M, K, E)
    ws = aligned_empty(wsb, 256)
    ws.fill_(0xAB)
    q4.expert_gate_up_grouped(d_slots, lay.slot_bytes, E, lay, xd, M, idt, K, H, I, ref, ws, wsb)
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    q4.expert_gate_up_grouped_noalloc(d_slots, lay.slot_bytes, E, lay, xd, M, idt, K, H, I, out, cnt)
    torch.cuda.synchronize()
    ref_cnt = int(ws[:4].cpu().numpy().view(np.int32)[0])
    return bf16_bits(ref), bf16_bits(out), ref_cnt, int(cnt.item())


@pytest.mark.parametrize("first,second", [
    # (E, H, I, M, K, seed, invalid ids): resident widths, then a smaller call
    ((24, 1024, 200, 6, 4, 31, 3), (5, 256, 40, 2, 2, 32, 0)),
    # the batch kernel (more than eight tokens on a slot), then a smaller call
    ((6, 512, 72, 20, 3, 33, 4), (3, 264, 18, 3, 1, 34, 1)),
])
def test_noalloc_matches_workspace_call_twice(first, second):
    for n, (E, H, I, M, K, seed, bad) in enumerate((first, second)):
        say(f"[no-alloc call {n}] E={E} H={H} I={I} M={M} K={K} invalid={bad}")
        lay, slots, x, ids = _case(E, H, I, M, K, seed, bad)
        ref, out, ref_cnt, cnt = _both(lay, slots, x, ids, H, I)
        assert ref_cnt == bad
        assert cnt == bad
        assert np.array_equal(out, ref)


def test_noalloc_without_count_output():
    lay, slots, x, ids = _case(4, 256, 24, 2, 2, 35, 1)
    E, (M, K), H, I = slots.shape[0], ids.shape, 256, 24
    d_slots = upload_slots(slots)
    out = torch.zeros((M, K, I), dtype=torch.bfloat16, device="cuda")
    q4.expert_gate_up_grouped_noalloc(d_slots, lay.slot_bytes, E, lay, upload_bf16_bits(x), M,
                                      torch.from_numpy(ids).cuda(), K, H, I, out, None)
    torch.cuda.synchronize()
    ref, out2, _, _ = _both(lay, slots, x, ids, H, I)
    assert np.array_equal(bf16_bits(out), ref)
