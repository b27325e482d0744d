"""GPU parity of f32 activations (page 52: validateCall accepts float32 input,
execute returns outputs in the input's dtype; T = float tail) against the
oracle, through the C ABI's _f32 entry points: the workload shapes with f32
x (the large shape with 1% of x at +-1e4), ragged shapes through both
kernels and both load widths, wide exponent ranges within the exact window,
scales that drive results to subnormals and to overflow, grouped routing with
invalid ids and duplicates, the down projection and the whole expert (Q4 and
Q8).  F32 gate/up/down values must be bit-exact; f32 outputs must equal the
oracle's tail on the GPU's own gate/up and the oracle's output."""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_moe_expert_q4_amd as q4
from quantized_moe_expert_q4_amd.device import aligned_empty, upload_slots
from tests.gpu_helpers import poisoned, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    q4.load()   # raises if the HIP library is missing: there is no fallback
    yield


def _same(a, b):
    """Bitwise equal float32 arrays, +0 == -0 and NaN == NaN."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return (a.view(np.uint32) == b.view(np.uint32)) | ((a == 0) & (b == 0)) | (np.isnan(a) & np.isnan(b))


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def _single(slot_np, lay, x, H, I, fmt="q4", label=""):
    M = x.shape[0]
    slot = upload_slots(slot_np.reshape(1, -1))
    out = poisoned((M, I), torch.float32)
    g = poisoned((M, I), torch.float32)
    u = poisoned((M, I), torch.float32)
    q4.expert_gate_up(slot, lay, _dev(x), M, H, I, out, g, u, fmt=fmt, xdtype="f32")
    torch.cuda.synchronize()
    o, g, u = out.cpu().numpy(), g.cpu().numpy(), u.cpu().numpy()
    gr, ur, orf = oracle.expert_gate_up(slot_np, lay, x, H, I, fmt=fmt, xdtype="f32")
    ng, nu = int(_same(g, gr).sum()), int(_same(u, ur).sum())
    tail = oracle.swiglu_tail_f32(g, u)
    nt, no = int(_same(o, tail).sum()), int(_same(o, orf).sum())
    say(f"[{label}] n={g.size} bit-exact gate={ng} up={nu} out-vs-tail(gpu gate/up)={nt} out={no}")
    assert ng == nu == nt == no == g.size, label


@pytest.mark.parametrize("cfg,M", [("cfg1", None), ("cfg2", None), ("cfg3", None), ("cfg5", 1), ("cfg5", 4),
                                   ("cfg5", 16)])
def test_f32_configs(cfg, M):
    c = synth.make_config(cfg, M=M)
    rng = np.random.default_rng(900 + c.x.shape[0])
    x = synth.f32_normal(rng, c.x.shape)
    if cfg == "cfg5":
        x = synth.add_outliers_f32(rng, x, 0.01)
    _single(c.slots[0], c.layout, x, c.H, c.I, label=f"f32 {cfg} M={c.x.shape[0]}")


F32_RAGGED = [(8, 1, 1), (24, 7, 2), (136, 33, 3), (1000, 70, 5), (4104, 130, 9), (2048, 100, 40), (512, 300, 8),
              (7168, 64, 2)]


@pytest.mark.parametrize("H,I,M", F32_RAGGED)
def test_f32_ragged(H, I, M):
    rng = np.random.default_rng(H + 3 * I + M)
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    x = synth.f32_normal(rng, (M, H))
    _single(slot, lay, x, H, I, label=f"f32 ragged H={H} I={I} M={M}")


def test_f32_wide_exponents_and_q8():
    rng = np.random.default_rng(91)
    H, I, M = 520, 48, 3
    m = rng.integers(1 << 23, 1 << 24, (M, H)).astype(np.float64)
    e = rng.integers(-20, 18, (M, H))           # within the 38-binade exact window
    x = (np.where(rng.random((M, H)) < 0.5, -1, 1) * m * np.exp2(e - 23)).astype(np.float32)
    x[rng.random((M, H)) < 0.05] = 0
    lay = synth.contiguous_layout(H, I)
    _single(synth.fill_slot(rng, H, I, lay), lay, x, H, I, label="f32 wide exponents")
    lay8 = synth.contiguous_layout(H, I, fmt="q8")
    _single(synth.fill_slot(rng, H, I, lay8, fmt="q8"), lay8, x, H, I, fmt="q8", label="f32 wide exponents q8")


def test_f32_subnormal_and_overflowing_results():
    rng = np.random.default_rng(92)
    H, I, M = 256, 32, 2
    lay = synth.contiguous_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    gs = np.exp2(rng.integers(-150, -120, I)).astype(np.float32) * np.float32(1.37)
    us = np.full(I, 3e37, np.float32)
    slot[lay.gate_scale_offset:lay.gate_scale_offset + 4 * I] = gs.astype("<f4").view(np.uint8)
    slot[lay.up_scale_offset:lay.up_scale_offset + 4 * I] = us.astype("<f4").view(np.uint8)
    x = synth.f32_normal(rng, (M, H)) * np.float32(8.0)
    _single(slot, lay, x, H, I, label="f32 subnormal gate, overflowing up")


def test_f32_grouped_edges():
    c = synth.make_config("cfg4", num_slots=6, H=520, I=264, M=4)
    rng = np.random.default_rng(93)
    x = synth.f32_normal(rng, (4, 520))
    ids = np.array([[0, 5, -1], [2, 2, 9], [5, 1, 3], [2, 2, 2]], dtype=np.int32)
    M, K = ids.shape
    slots = upload_slots(c.slots)
    idt = torch.from_numpy(ids).cuda()
    out = poisoned((M, K, c.I), torch.float32)
    g = poisoned((M, K, c.I), torch.float32)
    u = poisoned((M, K, c.I), torch.float32)
    wsb = q4.grouped_workspace_bytes(M, K, c.num_slots)
    ws = aligned_empty(wsb, 256)
    q4.expert_gate_up_grouped(slots, c.slot_stride, c.num_slots, c.layout, _dev(x), M, idt, K, c.H, c.I, out, ws,
                              wsb, g, u, xdtype="f32")
    torch.cuda.synchronize()
    gr, ur, orf, bad = oracle.expert_gate_up_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, x, ids, c.H,
                                                     c.I, xdtype="f32")
    assert int(ws[:4].cpu().numpy().view(np.int32)[0]) == bad == 2
    assert _same(g.cpu().numpy(), gr).all() and _same(u.cpu().numpy(), ur).all()
    assert _same(out.cpu().numpy(), orf).all()


@pytest.mark.parametrize("fmt", ["q4", "q8"])
def test_f32_down_and_whole_expert(fmt):
    rng = np.random.default_rng(94)
    for H, I, M in ((264, 136, 2), (1024, 512, 9)):
        lay = synth.expert_layout(H, I, fmt=fmt)
        slot_np = synth.fill_slot(rng, H, I, lay, fmt=fmt)
        slot = upload_slots(slot_np.reshape(1, -1))
        mid = synth.f32_normal(rng, (M, I))
        out = poisoned((M, H), torch.float32)
        d = poisoned((M, H), torch.float32)
        q4.expert_down(slot, lay, _dev(mid), M, H, I, out, d, fmt=fmt, xdtype="f32")
        x = synth.f32_normal(rng, (M, H))
        midg = poisoned((M, I), torch.float32)
        outg = poisoned((M, H), torch.float32)
        q4.expert_forward(slot, lay, _dev(x), M, H, I, midg, outg, fmt=fmt, xdtype="f32")
        torch.cuda.synchronize()
        d_ref, o_ref = oracle.expert_down(slot_np, lay, mid, H, I, fmt=fmt, xdtype="f32")
        m_ref, f_ref = oracle.expert_forward(slot_np, lay, x, H, I, fmt=fmt, xdtype="f32")
        say(f"[f32 {fmt} down/forward H={H} I={I} M={M}]")
        assert _same(d.cpu().numpy(), d_ref).all() and _same(out.cpu().numpy(), o_ref).all()
        assert _same(midg.cpu().numpy(), m_ref).all() and _same(outg.cpu().numpy(), f_ref).all()


def test_f32_forward_grouped():
    c = synth.make_config("cfg4", num_slots=10, H=1024, I=512, M=2, with_down=True)
    rng = np.random.default_rng(95)
    x = synth.f32_normal(rng, (2, 1024))
    M, K = c.ids.shape
    slots = upload_slots(c.slots)
    idt = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32)).cuda()
    mid = poisoned((M, K, c.I), torch.float32)
    out = poisoned((M, K, c.H), torch.float32)
    wsb = q4.grouped_workspace_bytes(M, K, c.num_slots)
    ws = aligned_empty(wsb, 256)
    q4.expert_forward_grouped(slots, c.slot_stride, c.num_slots, c.layout, _dev(x), M, idt, K, c.H, c.I, mid, out,
                              ws, wsb, xdtype="f32")
    torch.cuda.synchronize()
    m_ref, o_ref, bad = oracle.expert_forward_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, x, c.ids, c.H,
                                                      c.I, xdtype="f32")
    assert bad == 0
    assert _same(mid.cpu().numpy(), m_ref).all() and _same(out.cpu().numpy(), o_ref).all()
