"""GPU parity of the down projection and the whole expert against the oracle.

The down kernels are the gate/up kernels in their down mode (32-row tiles,
each half rounded to bf16 on its own; page 52 DOWN_SOURCE), called through the
C ABI: single slot, grouped (one input row per routed pair), and the whole
expert (gate/up then down, page 52 Glm52CanonicalMetalExecutor.execute).
Shapes reach both kernels (resident for up to eight tokens, batch beyond),
16-byte and 4-byte weight loads (I % 32), partial K-steps (I % 128), ragged
32-row tiles (H % 32, H < 16), four- and six-digit activations.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_moe_expert_q4_amd as q4
from quantized_moe_expert_q4_amd.device import aligned_empty, bf16_bits, upload_bf16_bits, upload_slots
from tests.gpu_helpers import check_down_parity, poisoned, run_down_grouped, run_down_single, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    q4.load()   # raises if the HIP library is missing: there is no fallback
    yield


def _wide_mid(rng, shape):
    """bf16 values spread over ~60 binades (forces six digits per value)."""
    x = synth.bf16_normal(rng, shape).astype(np.int64)
    e = (x >> 7) & 0xFF
    e = np.clip(e + rng.integers(-30, 30, shape), 1, 200)
    return ((x & 0x807F) | (e << 7)).astype(np.uint16)


# (H, I, M, wide): rows H (any multiple of 8), reduction I % 8 == 0
DOWN_SHAPES = [
    (8, 8, 1, False), (24, 16, 2, False), (40, 136, 3, True), (264, 1000, 6, False),
    (136, 4104, 9, False), (48, 2048, 40, True), (4096, 1536, 1, False), (4096, 1536, 8, True),
    (520, 264, 17, False), (7168, 4096, 2, True),
]


@pytest.mark.parametrize("H,I,M,wide", DOWN_SHAPES)
def test_down_single_shapes(H, I, M, wide):
    rng = np.random.default_rng(H * 7 + I * 3 + M)
    lay = synth.expert_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    mid = _wide_mid(rng, (M, I)) if wide else synth.bf16_normal(rng, (M, I))
    label = f"down H={H} I={I} M={M} wide={wide}"
    say(f"[{label}]")
    out, d = run_down_single(slot, lay, mid, H, I)
    d_ref, o_ref = oracle.expert_down(slot, lay, mid, H, I)
    check_down_parity(out, d, d_ref, o_ref, label)


def _forward(c):
    M = c.x.shape[0]
    slot = upload_slots(c.slots[:1])
    x = upload_bf16_bits(c.x)
    mid = poisoned((M, c.I), torch.bfloat16)
    out = poisoned((M, c.H), torch.bfloat16)
    q4.expert_forward(slot, c.layout, x, M, c.H, c.I, mid, out)
    torch.cuda.synchronize()
    return bf16_bits(mid), bf16_bits(out)


@pytest.mark.parametrize("cfg,M", [("cfg1", None), ("cfg2", None), ("cfg3", None), ("cfg5", 1), ("cfg5", 4)])
def test_forward_single_expert_configs(cfg, M):
    c = synth.make_config(cfg, M=M, with_down=True)
    label = f"forward {cfg} H={c.H} I={c.I} M={c.x.shape[0]}"
    say(f"[{label}]")
    mid, out = _forward(c)
    mid_ref, out_ref = oracle.expert_forward(c.slots[0], c.layout, c.x, c.H, c.I)
    n_mid = int(np.sum(mid == mid_ref))
    n_out = int(np.sum(out == out_ref))
    say(f"[{label}] bit-exact mid={n_mid}/{mid.size} out={n_out}/{out.size}")
    assert n_mid == mid.size and n_out == out.size, label


def test_down_grouped_edge_cases():
    rng = np.random.default_rng(41)
    H, I, E = 520, 264, 6
    c = synth.make_config("cfg4", num_slots=E, H=H, I=I, M=4, with_down=True)
    ids = np.array([[0, 5, -1], [2, 2, 9], [5, 1, 3], [4, 0, 2]], dtype=np.int32)   # invalid, duplicates
    M, K = ids.shape
    for wide in (False, True):
        mid = _wide_mid(rng, (M, K, I)) if wide else synth.bf16_normal(rng, (M, K, I))
        say(f"[down grouped edge wide={wide}]")
        (out, d), invalid = run_down_grouped(c.slots, c.layout, mid, ids, H, I)
        d_ref, o_ref, bad = oracle.expert_down_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, mid, ids,
                                                       H, I)
        assert invalid == bad == 2
        check_down_parity(out, d, d_ref, o_ref, f"down grouped edge wide={wide}")


def _forward_grouped(c, slots=None):
    M, K = c.ids.shape
    if slots is None:
        slots = upload_slots(c.slots)
    x = upload_bf16_bits(c.x)
    idt = torch.from_numpy(np.ascontiguousarray(c.ids, dtype=np.int32)).cuda()
    mid = poisoned((M, K, c.I), torch.bfloat16)
    out = poisoned((M, K, c.H), torch.bfloat16)
    wsb = q4.grouped_workspace_bytes(M, K, c.num_slots)
    ws = aligned_empty(wsb, 256)
    q4.expert_forward_grouped(slots, c.slot_stride, c.num_slots, c.layout, x, M, idt, K, c.H, c.I, mid, out, ws,
                              wsb)
    torch.cuda.synchronize()
    return bf16_bits(mid), bf16_bits(out), int(ws[:4].cpu().numpy().view(np.int32)[0])


@pytest.mark.parametrize("M,K,E", [(1, 8, 16), (3, 4, 5), (12, 2, 3)])
def test_forward_grouped_decode_and_verify_widths(M, K, E):
    c = synth.make_config("cfg4", num_slots=E, H=1024, I=512, M=M, with_down=True)
    label = f"forward grouped H=1024 I=512 M={M} K={c.K} E={E}"
    say(f"[{label}]")
    mid, out, invalid = _forward_grouped(c)
    mid_ref, out_ref, bad = oracle.expert_forward_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, c.x,
                                                          c.ids, c.H, c.I)
    assert invalid == bad == 0
    assert np.array_equal(mid, mid_ref), label
    assert np.array_equal(out, out_ref), label


def test_forward_grouped_routed_step_full_size():
    """The routed MoE step at its full size: 64 whole-expert slots of H=6144,
    I=2048, 32 tokens, top-8 routing; every mid and output element checked."""
    c = synth.make_config("cfg4", with_down=True)
    label = "forward grouped cfg4 64 slots H=6144 I=2048 M=32 K=8"
    say(f"[{label}]")
    mid, out, invalid = _forward_grouped(c)
    mid_ref, out_ref, bad = oracle.expert_forward_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, c.x,
                                                          c.ids, c.H, c.I)
    assert invalid == bad == 0
    n_mid, n_out = int(np.sum(mid == mid_ref)), int(np.sum(out == out_ref))
    say(f"[{label}] bit-exact mid={n_mid}/{mid.size} out={n_out}/{out.size}")
    assert n_mid == mid.size and n_out == out.size


def test_down_batch_invariance():
    """A token's down output is bitwise the same alone, in a batch of 8
    (resident kernel) and in a batch of 40 (batch kernel)."""
    rng = np.random.default_rng(43)
    H, I = 1032, 776
    lay = synth.expert_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    mid = _wide_mid(rng, (40, I))
    mid[:20] = synth.bf16_normal(rng, (20, I))
    outs = {}
    for M in (1, 8, 40):
        say(f"[down invariance M={M}]")
        outs[M] = run_down_single(slot, lay, mid[:M], H, I)
    for M in (8, 40):
        assert np.array_equal(outs[M][0][:1], outs[1][0])
        assert np.array_equal(outs[M][1][:1].view(np.uint32), outs[1][1].view(np.uint32))
    assert np.array_equal(outs[40][0][:8], outs[8][0])
