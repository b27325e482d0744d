"""GPU parity on row scales of every sign and size.

The scale is one F32 multiply after the reduction (page 52 of the
@mlx-bun/inference 1.0.0 diff, kernels/glm52/streamed-experts.ts,
``GATE_UP_SOURCE`` and ``DOWN_SOURCE``), so every IEEE rule of a product
applies to the rounded result: negative scales, signed zero scales (a zero
whose sign is that of the two factors), subnormal scales and results, and
products beyond the F32 range (infinities, and the NaN of the tail for an
infinite negative gate).  Each case runs through the four-digit, six-digit
and eight-digit (f32) roundings of both kernels, Q4 and Q8, gate/up and down,
and requires the oracle's bits exactly: signed zeros are told apart and only
NaN payloads may differ.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_moe_expert_q4_amd as q4
from quantized_moe_expert_q4_amd.device import upload_slots
from tests.gpu_helpers import poisoned, run_down_single, run_single, say

pytestmark = pytest.mark.gpu

SPECIAL_SCALES = np.array([0.0, -0.0, 1e-45, -3e-39, 2.0 ** -126, 1e38, -1e38, 0.75, -0.01, 3.4e38,
                           -(2.0 ** -140), 1.5e-5], dtype=np.float32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    q4.load()   # raises if the HIP library is missing: there is no fallback
    yield


def _scales(rng, n):
    """Random signs and magnitudes, every third row one of the special scales."""
    s = (rng.uniform(0.005, 0.02, n) * np.where(rng.random(n) < 0.5, -1.0, 1.0)).astype(np.float32)
    k = np.arange(0, n, 3)
    s[k] = SPECIAL_SCALES[(k // 3 + int(rng.integers(0, len(SPECIAL_SCALES)))) % len(SPECIAL_SCALES)]
    return s


def _put(slot, off, s):
    slot[off:off + 4 * s.size] = s.astype("<f4").view(np.uint8)


def _same_f32(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))


def _same_bf16(a, b):
    a = np.asarray(a, np.uint16)
    b = np.asarray(b, np.uint16)
    nan = lambda v: (v & 0x7FFF) > 0x7F80
    return (a == b) | (nan(a) & nan(b))


def _tokens(rng, M, H, wide, xdtype):
    """Normal tokens; one token of zeros (exact-zero sums); one token scaled
    up by 2^90 (products far beyond F32); with ``wide`` one token spanning 38
    binades (six digits per value)."""
    x = synth.bf16_normal(rng, (M, H))
    if M > 1:
        x[1] = 0
    if M > 2:
        e = (x[2].astype(np.int64) >> 7) & 0xFF
        x[2] = np.where(e > 0, (x[2] & 0x807F) | (np.minimum(e + 90, 254) << 7), x[2]).astype(np.uint16)
    if wide:
        t = M - 1 if M != 2 else 0
        x[t, 5] = 0x461C                                 # 9984
        x[t, 6] = 0x3300                                 # 2^-25: 38 binades below it
    return oracle.bf16_to_f32(x) if xdtype == "f32" else x


# (H, I, M, wide): resident kernel with one and two column tiles, four and six
# digits, and the batch kernel
CASES = [(256, 72, 1, False), (2048, 72, 2, True), (1024, 96, 8, False), (4096, 80, 8, True),
         (264, 100, 16, False), (512, 64, 24, True),
         # digits beyond the resident kernel's LDS: the chunked kernel (q4/bf16); the
         # six-digit token (the last) is not the 2^90 one (token 2), whose entries
         # all lie within 38 binades of its largest
         (12288, 80, 4, True), (12288, 80, 5, False)]


@pytest.mark.parametrize("H,I,M,wide", CASES)
@pytest.mark.parametrize("fmt,xdtype", [("q4", "bf16"), ("q8", "bf16"), ("q4", "f32")])
def test_gate_up_scales(H, I, M, wide, fmt, xdtype):
    rng = np.random.default_rng(H + 3 * I + 5 * M + int(wide) + (7 if fmt == "q8" else 0) + (11 if xdtype == "f32" else 0))
    lay = synth.contiguous_layout(H, I, fmt=fmt)
    slot = synth.fill_slot(rng, H, I, lay, fmt=fmt)
    _put(slot, lay.gate_scale_offset, _scales(rng, I))
    _put(slot, lay.up_scale_offset, _scales(rng, I))
    x = _tokens(rng, M, H, wide, xdtype)
    label = f"scales {fmt}/{xdtype} H={H} I={I} M={M} wide={wide}"
    say(f"[{label}]")
    gr, ur, orf = oracle.expert_gate_up(slot, lay, x, H, I, fmt=fmt, xdtype=xdtype)
    if xdtype == "bf16":
        out, g, u = run_single(slot, lay, x, H, I, fmt=fmt)
        same_out = _same_bf16(out, orf)
    else:
        dev = upload_slots(slot.reshape(1, -1))
        xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
        o = poisoned((M, I), torch.float32)
        gt = poisoned((M, I), torch.float32)
        ut = poisoned((M, I), torch.float32)
        q4.expert_gate_up(dev, lay, xt, M, H, I, o, gt, ut, fmt=fmt, xdtype="f32")
        torch.cuda.synchronize()
        out, g, u = o.cpu().numpy(), gt.cpu().numpy(), ut.cpu().numpy()
        same_out = _same_f32(out, orf)
    ng, nu, no = int(_same_f32(g, gr).sum()), int(_same_f32(u, ur).sum()), int(same_out.sum())
    say(f"[{label}] n={g.size} bit-exact gate={ng} up={nu} out={no}; "
        f"inf={int(np.isinf(gr).sum())} signed zeros={int((np.asarray(gr).view(np.uint32) == 0x80000000).sum())}")
    assert ng == nu == no == g.size, label
    assert np.any(np.asarray(gr).view(np.uint32) == 0x80000000), label


DOWN_CASES = [(256, 128, 1, False), (520, 264, 3, True), (128, 1024, 8, False), (264, 512, 17, True),
              (72, 16384, 5, True)]    # a reduction beyond the resident kernel's LDS: the chunked kernel


@pytest.mark.parametrize("H,I,M,wide", DOWN_CASES)
@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_down_scales(H, I, M, wide, xdtype):
    rng = np.random.default_rng(H + 3 * I + 5 * M + int(wide) + (11 if xdtype == "f32" else 0))
    lay = synth.expert_layout(H, I)
    slot = synth.fill_slot(rng, H, I, lay)
    _put(slot, lay.down_scale_offset, _scales(rng, H))
    mid = _tokens(rng, M, I, wide, xdtype)
    label = f"down scales {xdtype} H={H} I={I} M={M} wide={wide}"
    say(f"[{label}]")
    d_ref, o_ref = oracle.expert_down(slot, lay, mid, H, I, xdtype=xdtype)
    if xdtype == "bf16":
        out, d = run_down_single(slot, lay, mid, H, I)
        same_out = _same_bf16(out, o_ref)
    else:
        dev = upload_slots(slot.reshape(1, -1))
        mt = torch.from_numpy(np.ascontiguousarray(mid, np.float32)).cuda()
        o = poisoned((M, H), torch.float32)
        dt = poisoned((M, H), torch.float32)
        q4.expert_down(dev, lay, mt, M, H, I, o, dt, xdtype="f32")
        torch.cuda.synchronize()
        out, d = o.cpu().numpy(), dt.cpu().numpy()
        same_out = _same_f32(out, o_ref)
    nd, no = int(_same_f32(d, d_ref).sum()), int(same_out.sum())
    say(f"[{label}] n={d.size} bit-exact down={nd} out={no}")
    assert nd == no == d.size, label
