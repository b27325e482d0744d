"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare it with the oracle under the stated tolerances.

T1 (F32 gate/up before their bf16 rounding): |g - g_ref| <= 1e-5 |g_ref| + 1e-6.
T2 (bf16 output): distance in ordered bf16 keys (+0 and -0 equal, two values
both below 2^-100 in magnitude equal) between the GPU output and the oracle's
tail evaluated on the GPU's own F32 gate/up is at most 1.
"""
import sys

import numpy as np
import torch

import oracle
import quantized_moe_expert_q4_amd as q4
from quantized_moe_expert_q4_amd.device import aligned_empty, bf16_bits, upload_bf16_bits, upload_slots


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def poisoned(shape, dtype):
    """An output buffer filled with NaN, so that an element the kernels leave
    unwritten fails the comparison instead of passing as a stale zero."""
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def run_single(slot_np, layout, xbits, H, I, probes=True, fmt="q4"):
    M = xbits.shape[0]
    slot = upload_slots(slot_np.reshape(1, -1))
    x = upload_bf16_bits(xbits)
    out = poisoned((M, I), torch.bfloat16)
    g = poisoned((M, I), torch.float32) if probes else None
    u = poisoned((M, I), torch.float32) if probes else None
    q4.expert_gate_up(slot, layout, x, M, H, I, out, g, u, fmt=fmt)
    torch.cuda.synchronize()
    res = [bf16_bits(out)]
    if probes:
        res += [g.cpu().numpy(), u.cpu().numpy()]
    return res


def run_grouped(slots_np, layout, xbits, ids, H, I, probes=True, ws_fill=None, ws=None, slots=None, fmt="q4"):
    """One grouped call.  `ws` reuses a workspace (left as the last call left
    it); otherwise a new one filled with `ws_fill` (default 0xAB).  `slots`
    passes slots already on the device (then `slots_np` gives only the shape)."""
    M, K = ids.shape
    E = slots_np.shape[0]
    if slots is None:
        slots = upload_slots(slots_np)
    x = upload_bf16_bits(xbits)
    idt = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    out = poisoned((M, K, I), torch.bfloat16)
    g = poisoned((M, K, I), torch.float32) if probes else None
    u = poisoned((M, K, I), torch.float32) if probes else None
    wsb = q4.grouped_workspace_bytes(M, K, E)
    if ws is None:
        ws = aligned_empty(wsb, 256)
        ws.fill_(0xAB if ws_fill is None else ws_fill)
    q4.expert_gate_up_grouped(slots, slots_np.shape[1], E, layout, x, M, idt, K, H, I, out, ws, wsb, g, u, fmt=fmt)
    torch.cuda.synchronize()
    invalid = int(ws[:4].cpu().numpy().view(np.int32)[0])
    res = [bf16_bits(out)]
    if probes:
        res += [g.cpu().numpy(), u.cpu().numpy()]
    return res, invalid


def t1_violations(g, g_ref):
    g = np.asarray(g, np.float64)
    r = np.asarray(g_ref, np.float64)
    bad = ~(np.abs(g - r) <= 1e-5 * np.abs(r) + 1e-6)
    return int(bad.sum())


def bf16_key(bits):
    b = np.asarray(bits, dtype=np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_dist(a, b):
    d = np.abs(bf16_key(a) - bf16_key(b))
    va = np.abs(oracle.bf16_to_f32(a).astype(np.float64))
    vb = np.abs(oracle.bf16_to_f32(b).astype(np.float64))
    tiny = (va < 2.0 ** -100) & (vb < 2.0 ** -100)
    return np.where(tiny, 0, d)


def check_parity(out, g, u, g_ref, u_ref, out_ref, label, require_exact_gate_up=True):
    """Assert T1 and T2; report (and by default require) bit-exact gate/up."""
    n = out.size
    t1g, t1u = t1_violations(g, g_ref), t1_violations(u, u_ref)
    tail = oracle.swiglu_tail(g, u)
    t2 = bf16_dist(out, tail)
    e2e = bf16_dist(out, out_ref)
    exact_g = int(np.sum(g.view(np.uint32) == np.asarray(g_ref, np.float32).view(np.uint32)))
    exact_u = int(np.sum(u.view(np.uint32) == np.asarray(u_ref, np.float32).view(np.uint32)))
    exact_o = int(np.sum(out == out_ref))
    say(f"[{label}] n={n} T1 fail gate={t1g} up={t1u}; T2 max={int(t2.max())}; end-to-end max={int(e2e.max())}; "
        f"bit-exact gate={exact_g}/{n} up={exact_u}/{n} out={exact_o}/{n}")
    assert t1g == 0 and t1u == 0, label
    assert int(t2.max()) <= 1, label
    assert int(e2e.max()) <= 1, label
    if require_exact_gate_up:
        assert exact_g == n and exact_u == n, label
    return dict(n=n, exact_gate=exact_g, exact_up=exact_u, exact_out=exact_o, t2_max=int(t2.max()),
                e2e_max=int(e2e.max()))


def run_down_single(slot_np, layout, midbits, H, I, fmt="q4"):
    """One single-slot down call: returns (out bf16 bits [M,H], F32 probe [M,H])."""
    M = midbits.shape[0]
    slot = upload_slots(slot_np.reshape(1, -1))
    mid = upload_bf16_bits(midbits)
    out = poisoned((M, H), torch.bfloat16)
    d = poisoned((M, H), torch.float32)
    q4.expert_down(slot, layout, mid, M, H, I, out, d, fmt=fmt)
    torch.cuda.synchronize()
    return bf16_bits(out), d.cpu().numpy()


def run_down_grouped(slots_np, layout, midbits, ids, H, I, slots=None, fmt="q4"):
    """One grouped down call on mid [M,K,I]: returns ((out [M,K,H], probe), invalid count)."""
    M, K = ids.shape
    E = slots_np.shape[0]
    if slots is None:
        slots = upload_slots(slots_np)
    mid = upload_bf16_bits(np.ascontiguousarray(midbits).reshape(M, K, I))
    idt = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    out = poisoned((M, K, H), torch.bfloat16)
    d = poisoned((M, K, H), torch.float32)
    wsb = q4.grouped_workspace_bytes(M, K, E)
    ws = aligned_empty(wsb, 256)
    ws.fill_(0xAB)
    q4.expert_down_grouped(slots, slots_np.shape[1], E, layout, mid, M, idt, K, H, I, out, ws, wsb, d, fmt=fmt)
    torch.cuda.synchronize()
    invalid = int(ws[:4].cpu().numpy().view(np.int32)[0])
    return (bf16_bits(out), d.cpu().numpy()), invalid


def check_down_parity(out, d, d_ref, out_ref, label):
    """T1 on the F32 values before rounding, the bf16 output within one ulp of
    the oracle's; both are also required to be bit-exact (exact sums)."""
    n = out.size
    t1 = t1_violations(d, d_ref)
    e2e = bf16_dist(out, out_ref)
    exact_d = int(np.sum(d.view(np.uint32) == np.asarray(d_ref, np.float32).view(np.uint32)))
    exact_o = int(np.sum(out == out_ref))
    say(f"[{label}] n={n} T1 fail={t1}; out max dist={int(e2e.max()) if n else 0}; "
        f"bit-exact down={exact_d}/{n} out={exact_o}/{n}")
    assert t1 == 0, label
    assert n == 0 or int(e2e.max()) <= 1, label
    assert exact_d == n and exact_o == n, label
