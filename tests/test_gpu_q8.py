"""GPU parity of the Q8 family (signed int8 weights; page 52 Q8_GATE_UP_SOURCE,
Q8_DOWN_SOURCE, Glm52CanonicalQ8MetalExecutor) against the oracle, through
the C ABI's q8_ entry points: the five workload shapes with int8 weights,
ragged shapes that reach both kernels, 16-byte and 4-byte loads (H % 16),
partial K-steps, four- and six-digit activations, grouped routing with
invalid ids and duplicates, the down projection and the whole expert."""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_moe_expert_q4_amd as q4
from quantized_moe_expert_q4_amd.device import aligned_empty, bf16_bits, upload_bf16_bits, upload_slots
from tests.gpu_helpers import (check_down_parity, check_parity, poisoned, run_down_grouped, run_down_single, run_grouped,
                               run_single, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    q4.load()   # raises if the HIP library is missing: there is no fallback
    yield


def _single(c, label):
    say(f"[{label}] q8 single H={c.H} I={c.I} M={c.x.shape[0]}")
    out, g, u = run_single(c.slots[0], c.layout, c.x, c.H, c.I, fmt="q8")
    gr, ur, orf = oracle.expert_gate_up(c.slots[0], c.layout, c.x, c.H, c.I, fmt="q8")
    check_parity(out, g, u, gr, ur, orf, label)


@pytest.mark.parametrize("cfg,M", [("cfg1", None), ("cfg2", None), ("cfg3", None), ("cfg5", 1), ("cfg5", 4),
                                   ("cfg5", 16)])
def test_q8_configs(cfg, M):
    _single(synth.make_config(cfg, M=M, fmt="q8"), f"q8 {cfg} M={M}")


Q8_RAGGED = [(8, 1, 1), (24, 7, 2), (136, 33, 5), (1000, 70, 6), (4104, 130, 9), (2048, 100, 40), (8704, 20, 2),
             (7168, 64, 8), (520, 300, 1)]


@pytest.mark.parametrize("H,I,M", Q8_RAGGED)
def test_q8_ragged(H, I, M):
    c = synth.make_config("cfg2", H=H, I=I, M=M, seed=H + 7 * I + M, fmt="q8")
    _single(c, f"q8 ragged H={H} I={I} M={M}")


def test_q8_cfg5_outliers_batch_width():
    c = synth.make_config("cfg5", M=32, fmt="q8")
    _single(c, "q8 cfg5 M=32")


def test_q8_grouped_routed_step_and_edges():
    c = synth.make_config("cfg4", fmt="q8", num_slots=16, H=1024, I=512, M=12)
    say("[q8 grouped 16 slots H=1024 I=512 M=12 K=8]")
    (out, g, u), invalid = run_grouped(c.slots, c.layout, c.x, c.ids, c.H, c.I, fmt="q8")
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, c.x, c.ids,
                                                     c.H, c.I, fmt="q8")
    assert invalid == bad == 0
    check_parity(out, g, u, gr, ur, orf, "q8 grouped")
    ids = c.ids[:3, :4].copy()
    ids[0, 1] = -3
    ids[1, 2] = 99
    ids[2] = [5, 5, 5, 1]
    say("[q8 grouped edge ids]")
    (out, g, u), invalid = run_grouped(c.slots, c.layout, c.x[:3], ids, c.H, c.I, fmt="q8")
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, c.x[:3], ids,
                                                     c.H, c.I, fmt="q8")
    assert invalid == bad == 2
    check_parity(out, g, u, gr, ur, orf, "q8 grouped edge ids")


@pytest.mark.parametrize("H,I,M", [(24, 16, 2), (4096, 1536, 1), (520, 264, 17), (136, 4104, 9)])
def test_q8_down(H, I, M):
    rng = np.random.default_rng(H + I + M)
    lay = synth.expert_layout(H, I, fmt="q8")
    slot = synth.fill_slot(rng, H, I, lay, fmt="q8")
    mid = synth.bf16_normal(rng, (M, I))
    label = f"q8 down H={H} I={I} M={M}"
    say(f"[{label}]")
    out, d = run_down_single(slot, lay, mid, H, I, fmt="q8")
    d_ref, o_ref = oracle.expert_down(slot, lay, mid, H, I, fmt="q8")
    check_down_parity(out, d, d_ref, o_ref, label)


@pytest.mark.parametrize("M,K,E", [(1, 8, 12), (5, 3, 4)])
def test_q8_forward_grouped(M, K, E):
    c = synth.make_config("cfg4", num_slots=E, H=1024, I=512, M=M, with_down=True, fmt="q8")
    label = f"q8 forward grouped M={M} K={c.K} E={E}"
    say(f"[{label}]")
    Mk, Kk = c.ids.shape
    slots = upload_slots(c.slots)
    x = upload_bf16_bits(c.x)
    idt = torch.from_numpy(np.ascontiguousarray(c.ids, dtype=np.int32)).cuda()
    mid = poisoned((Mk, Kk, c.I), torch.bfloat16)
    out = poisoned((Mk, Kk, c.H), torch.bfloat16)
    wsb = q4.grouped_workspace_bytes(Mk, Kk, c.num_slots)
    ws = aligned_empty(wsb, 256)
    q4.expert_forward_grouped(slots, c.slot_stride, c.num_slots, c.layout, x, Mk, idt, Kk, c.H, c.I, mid, out, ws,
                              wsb, fmt="q8")
    torch.cuda.synchronize()
    mid_ref, out_ref, bad = oracle.expert_forward_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, c.x, c.ids,
                                                          c.H, c.I, fmt="q8")
    assert bad == 0
    assert np.array_equal(bf16_bits(mid), mid_ref), label
    assert np.array_equal(bf16_bits(out), out_ref), label


def test_q8_forward_single_and_down_grouped():
    c = synth.make_config("cfg3", with_down=True, fmt="q8")
    say("[q8 forward cfg3]")
    slot = upload_slots(c.slots[:1])
    x = upload_bf16_bits(c.x)
    mid = poisoned((8, c.I), torch.bfloat16)
    out = poisoned((8, c.H), torch.bfloat16)
    q4.expert_forward(slot, c.layout, x, 8, c.H, c.I, mid, out, fmt="q8")
    torch.cuda.synchronize()
    mid_ref, out_ref = oracle.expert_forward(c.slots[0], c.layout, c.x, c.H, c.I, fmt="q8")
    assert np.array_equal(bf16_bits(mid), mid_ref) and np.array_equal(bf16_bits(out), out_ref)
    rng = np.random.default_rng(61)
    cg = synth.make_config("cfg4", num_slots=5, H=264, I=136, M=3, with_down=True, fmt="q8")
    ids = np.array([[0, 4], [7, 2], [2, 2]], dtype=np.int32)
    midg = synth.bf16_normal(rng, (3, 2, 136))
    say("[q8 down grouped]")
    (o, d), invalid = run_down_grouped(cg.slots, cg.layout, midg, ids, 264, 136, fmt="q8")
    d_ref, o_ref, bad = oracle.expert_down_grouped(cg.slots, cg.slot_stride, cg.num_slots, cg.layout, midg, ids,
                                                   264, 136, fmt="q8")
    assert invalid == bad == 1
    check_down_parity(o, d, d_ref, o_ref, "q8 down grouped")
