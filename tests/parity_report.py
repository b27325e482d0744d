"""Per-workload parity statistics of the HIP path against the oracle.

Runs the five workloads (the large expert at M = 1, 4, 16 and 32), the
benchmark's 171-slot pool at M = 1 and M = 8, the down projection, Q8 weights
and f32 activations on the decode shape through the C ABI, compares each
element with the oracle and writes ``profiles/parity_stats.json`` (with the
sha256 of the kernel sources it ran on; a path given as the first argument
replaces that file name).  Statistics per workload: element
count, T1 violations (F32 gate/up within 1e-5 relative plus 1e-6 absolute of
the oracle), the largest relative F32 error, bit-exact counts, T2 (bf16 output
against the oracle's tail on the GPU's own F32 values, in ordered bf16 keys)
and the end-to-end bf16 distance.  Needs a GPU:
``python tests/parity_report.py``.
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from tests.gpu_helpers import (bf16_dist, run_down_single, run_grouped, run_single, say,  # noqa: E402
                               t1_violations)

OUT = os.path.join(ROOT, "profiles", "parity_stats.json")


def _rel(a, r):
    a = np.asarray(a, np.float64)
    r = np.asarray(r, np.float64)
    d = np.abs(a - r)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(d == 0, 0.0, d / np.abs(r))
    return float(np.max(rel)) if rel.size else 0.0


def _exact(a, r):
    return int(np.sum(np.asarray(a, np.float32).view(np.uint32) == np.asarray(r, np.float32).view(np.uint32)))


def gate_up_stats(out, g, u, gr, ur, orf):
    tail = oracle.swiglu_tail(g, u)
    n = int(out.size)
    return {"n": n, "t1_fail_gate": t1_violations(g, gr), "t1_fail_up": t1_violations(u, ur),
            "max_rel_err_gate": _rel(g, gr), "max_rel_err_up": _rel(u, ur),
            "exact_gate": _exact(g, gr), "exact_up": _exact(u, ur), "exact_out": int(np.sum(out == orf)),
            "t2_max": int(bf16_dist(out, tail).max()) if n else 0,
            "e2e_max": int(bf16_dist(out, orf).max()) if n else 0}


def down_stats(out, d, dr, orf):
    n = int(out.size)
    return {"n": n, "t1_fail_down": t1_violations(d, dr), "max_rel_err_down": _rel(d, dr),
            "exact_down": _exact(d, dr), "exact_out": int(np.sum(out == orf)),
            "e2e_max": int(bf16_dist(out, orf).max()) if n else 0}


def single(c, fmt="q4"):
    out, g, u = run_single(c.slots[0], c.layout, c.x, c.H, c.I, fmt=fmt)
    gr, ur, orf = oracle.expert_gate_up(c.slots[0], c.layout, c.x, c.H, c.I, fmt=fmt)
    return gate_up_stats(out, g, u, gr, ur, orf)


def f32_single(c):
    import torch
    import quantized_moe_expert_q4_amd as q4
    from quantized_moe_expert_q4_amd.device import upload_slots
    rng = np.random.default_rng(900 + c.x.shape[0])
    x = synth.f32_normal(rng, c.x.shape)
    M = x.shape[0]
    slot = upload_slots(c.slots[0].reshape(1, -1))
    out = torch.empty((M, c.I), dtype=torch.float32, device="cuda")
    g = torch.empty_like(out)
    u = torch.empty_like(out)
    q4.expert_gate_up(slot, c.layout, torch.from_numpy(x).cuda(), M, c.H, c.I, out, g, u, xdtype="f32")
    torch.cuda.synchronize()
    o, g, u = out.cpu().numpy(), g.cpu().numpy(), u.cpu().numpy()
    gr, ur, orf = oracle.expert_gate_up(c.slots[0], c.layout, x, c.H, c.I, xdtype="f32")
    tail = oracle.swiglu_tail_f32(g, u)
    n = int(o.size)
    return {"n": n, "t1_fail_gate": t1_violations(g, gr), "t1_fail_up": t1_violations(u, ur),
            "max_rel_err_gate": _rel(g, gr), "max_rel_err_up": _rel(u, ur), "exact_gate": _exact(g, gr),
            "exact_up": _exact(u, ur), "exact_out": _exact(o, orf), "out_equals_tail_of_gpu_gate_up": _exact(o, tail)}


def bench_pool(M):
    import bench
    lay, contents, x8 = bench.make_pool_host()
    pool = bench.Pool(lay, contents, x8)
    E = bench.POOL_SLOTS
    ids = np.tile(np.arange(E, dtype=np.int32), (M, 1))
    (out, g, u), invalid = run_grouped(_Shape(E, lay.slot_bytes), lay, x8[:M], ids, bench.H, bench.I,
                                       slots=pool.slots)
    ref = [oracle.expert_gate_up(contents[c], lay, x8[:M], bench.H, bench.I) for c in range(bench.DISTINCT_CONTENTS)]
    sel = np.arange(E) % bench.DISTINCT_CONTENTS
    gr = np.stack([ref[c][0] for c in sel], axis=1)
    ur = np.stack([ref[c][1] for c in sel], axis=1)
    orf = np.stack([ref[c][2] for c in sel], axis=1)
    s = gate_up_stats(out, g, u, gr, ur, orf)
    s["invalid"] = invalid
    return s


class _Shape:
    """Stands in for the host slot array when the slots are already on the device."""

    def __init__(self, E, stride):
        self.shape = (E, stride)


def main():
    import torch
    if not torch.cuda.is_available():
        print("parity_report.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import bench
    import quantized_moe_expert_q4_amd as q4
    q4.load()
    res = {}

    def run(name, fn):
        t0 = time.time()
        say(f"[{name}] ...")
        res[name] = fn()
        say(f"[{name}] {json.dumps(res[name])} ({time.time() - t0:.1f} s)")

    run("cfg1 H=256 I=128 M=1", lambda: single(synth.make_config("cfg1")))
    run("cfg2 H=4096 I=1536 M=1", lambda: single(synth.make_config("cfg2")))
    run("cfg3 H=4096 I=1536 M=8", lambda: single(synth.make_config("cfg3")))

    def cfg4():
        c = synth.make_config("cfg4")
        (out, g, u), invalid = run_grouped(c.slots, c.layout, c.x, c.ids, c.H, c.I)
        gr, ur, orf, bad = oracle.expert_gate_up_grouped(c.slots, c.slot_stride, c.num_slots, c.layout, c.x, c.ids,
                                                         c.H, c.I)
        s = gate_up_stats(out, g, u, gr, ur, orf)
        s["invalid"], s["invalid_oracle"] = invalid, bad
        return s
    run("cfg4 routed 64x(H=6144 I=2048) M=32 K=8", cfg4)
    for M in (1, 4, 16, 32):
        run(f"cfg5 H=7168 I=4096 M={M}", lambda M=M: single(synth.make_config("cfg5", M=M)))
    for M in (1, 8):
        run(f"bench pool 171x(H=4096 I=1536) M={M}", lambda M=M: bench_pool(M))

    def down(M):
        c = synth.make_config("cfg2", with_down=True)
        rng = np.random.default_rng(700 + M)
        mid = synth.bf16_normal(rng, (M, c.I))
        out, d = run_down_single(c.slots[0], c.layout, mid, c.H, c.I)
        dr, orf = oracle.expert_down(c.slots[0], c.layout, mid, c.H, c.I)
        return down_stats(out, d, dr, orf)
    run("down H=4096 I=1536 M=1", lambda: down(1))
    run("down H=4096 I=1536 M=8", lambda: down(8))
    run("q8 cfg2 H=4096 I=1536 M=1", lambda: single(synth.make_config("cfg2", fmt="q8"), fmt="q8"))
    run("f32 x cfg3 H=4096 I=1536 M=8", lambda: f32_single(synth.make_config("cfg3")))

    doc = {"kernel_sha256": bench.kernel_sha(),
           "tolerance": {"T1": "|g - g_ref| <= 1e-5 |g_ref| + 1e-6 on the F32 gate/up (down) before bf16 rounding",
                         "T2": "ordered-bf16-key distance <= 1 between the output and the oracle's tail on the "
                               "GPU's own F32 gate/up"},
           "workloads": res}
    out_path = sys.argv[1] if len(sys.argv) > 1 else OUT
    with open(out_path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    bad = [k for k, v in res.items() if v.get("t1_fail_gate", 0) or v.get("t1_fail_up", 0) or
           v.get("t1_fail_down", 0) or v.get("t2_max", 0) > 1 or v.get("e2e_max", 0) > 1]
    say(f"wrote {out_path}; workloads outside tolerance: {bad}")
    sys.exit(1 if bad else 0)


if __name__ == "__main__":
    main()
