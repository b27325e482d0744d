"""Weight-stream benchmark of the Q4 expert gate/up + SwiGLU path on one MI355X.

Headline workload (the decode-matvec expert shape H=4096, I=1536, M=1): a pool
of 171 distinct expert slots of that shape (171 * 6,303,744 B = 1.08 GB, larger
than the 256 MB Infinity Cache, so every step streams its weights from HBM).
One step is one grouped call routing the token to every slot of the pool: the
routing, activation split, weight stream, exact accumulation, scale and
SwiGLU tail of every slot, in one launch.  ``value`` is algorithmic weight
bytes (packed gate and up nibbles plus their F32 row scales) per second, the
median of five repetitions of ``--steps`` timed steps (after SETTLE_S seconds
of untimed steps, in which the GPU's clocks settle, and ``--warmup`` untimed
steps); ``m8`` is the same pool with eight tokens on every slot (the verify
width).

``shapes`` holds the other measured workloads, each the median of five
repetitions: single-expert launches and top-8 decode steps captured in HIP
graphs (device time, no host gaps), the one-GPU share of an expert-parallel
routed step, the large expert shape H=7168, I=4096 at M = 1, 4, 8, 16, 32, the
routed 64-expert step, the down projection, the whole expert, f32 activations
and Q8 weights.

``roofline`` prices the gate/up kernel against MI355X's 8 TB/s HBM peak and
against a read-only kernel with the same access on this device
(``stream_ceiling``).  ``traffic`` comes from the committed rocprofv3 counter
summary (profiles/traffic_gate_up_pool.json) when that summary was taken on
the current kernel source, else null.

``cpu_baseline`` times the CPU oracle (test infrastructure, exact arithmetic)
on a bounded sample of the same workload, on one core and on every core the
process may use (row-partitioned over processes), before the GPU is touched.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
POOL_SLOTS = 171
DISTINCT_CONTENTS = 8
H, I = 4096, 1536
SEED = 102
REPS = 5
SETTLE_S = 0.3      # seconds of untimed steps before each leg is timed (see settle)
CSRC = os.path.join(ROOT, "quantized_moe_expert_q4_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_pool.json")
PARITY_FILE = os.path.join(ROOT, "profiles", "parity_stats.json")
LARGE_H, LARGE_I, LARGE_SLOTS = 7168, 4096, 37
EXPERT_SLOTS = 114
Q8_SLOTS = 86
SEEDS = {"pool": SEED, "expert_pool": SEED + 1000, "f32_x": SEED + 2000, "q8_pool": SEED + 3000,
         "decode_routing": SEED + 4000, "ep_routing": SEED + 5000, "large": 105, "routed": 104}


# the sources of the gate/up and down kernels and their launchers (a change in
# any of them invalidates stored counters and parity statistics)
KERNEL_SOURCES = ["q4moe_device.h", "q4moe_launch.h", "q4moe_resident.hip", "q4moe_batch.hip", "q4moe_chunked.hip",
                  "q4moe_sigmoid.hip"]


def kernel_sha() -> str:
    """sha256 over the kernel sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def sha256_hex(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def make_pool_host():
    import synth
    lay = synth.contiguous_layout(H, I)
    rng = np.random.default_rng(SEED)
    contents = np.zeros((DISTINCT_CONTENTS, lay.slot_bytes), np.uint8)
    for d in range(DISTINCT_CONTENTS):
        synth.fill_slot(rng, H, I, lay, out=contents[d])
    x = synth.bf16_normal(rng, (8, H))
    return lay, contents, x


def weight_bytes_per_slot(H_: int = H, I_: int = I) -> int:
    return 2 * (I_ * H_ // 2) + 2 * 4 * I_


def down_bytes_per_slot(H_: int = H, I_: int = I) -> int:
    return H_ * I_ // 2 + 4 * H_


def kernel_label(M: int, H_: int, per_slot: int = None) -> str:
    """The gate/up kernel the library launches for a call whose slots see up
    to M tokens, `per_slot` routed pairs per slot on average (grouped calls;
    None for a single expert): the selection rule of q4moe_resident.hip --
    resident digits for up to eight tokens when their digits fit LDS, else the
    chunked kernel for a few rows per slot, else the batch kernel."""
    nt = 1 if M <= 2 else 2
    steps = ((H_ + 255) // 256 + 3) // 4 * 4
    fits = M <= 8 and M * ((H_ // 8 + 1) // 2) * 2 <= 8 * 512 and steps * 4096 * nt + 7 * nt * 1024 <= 144 * 1024
    if fits:
        return "q4::resident_kernel"
    if (per_slot if per_slot is not None else M) <= (6 if per_slot is not None else 8):
        return "q4::chunked_kernel"
    return "q4::batch_kernel"


def large_shape_host(M: int):
    """The large expert shape (H=7168, I=4096): its seeded slot (1% all-8 rows
    per matrix) and M tokens of N(0,1) bf16 with 1% of entries at +-9984."""
    import synth
    c = synth.make_config("cfg5", M=M)
    return c.layout, c.slots[:1], c.x


def expert_pool_host():
    """Whole-expert slots of the decode shape (gate, up and down fields)."""
    import synth
    lay = synth.expert_layout(H, I)
    rng = np.random.default_rng(SEEDS["expert_pool"])
    contents = np.zeros((DISTINCT_CONTENTS, lay.slot_bytes), np.uint8)
    for d in range(DISTINCT_CONTENTS):
        synth.fill_slot(rng, H, I, lay, out=contents[d])
    x = synth.bf16_normal(rng, (8, H))
    return lay, contents, x


class Pool:
    """``nslots`` device slots of one shape, filled round-robin from ``contents``."""

    def __init__(self, lay, contents, x, nslots: int = POOL_SLOTS, H_: int = H, I_: int = I, fmt: str = "q4",
                 xdtype: str = "bf16"):
        import torch
        from quantized_moe_expert_q4_amd.device import aligned_empty, upload_bf16_bits
        self.torch = torch
        self.lay = lay
        self.fmt, self.xdtype = fmt, xdtype
        self.H, self.I, self.nslots = H_, I_, nslots
        self.stride = lay.slot_bytes
        self.slots = aligned_empty(nslots * self.stride)
        for d in range(contents.shape[0]):
            dev = torch.from_numpy(contents[d]).cuda()
            for s in range(d, nslots, contents.shape[0]):
                self.slots[s * self.stride:(s + 1) * self.stride].copy_(dev)
            del dev
        self.x = upload_bf16_bits(x) if xdtype == "bf16" else torch.from_numpy(x).cuda()
        torch.cuda.synchronize()

    def slot_bytes(self) -> int:
        return weight_bytes_per_slot(self.H, self.I) if self.fmt == "q4" else 2 * self.H * self.I + 8 * self.I

    def bytes_per_step(self) -> int:
        return self.nslots * self.slot_bytes()

    def step_fn(self, M: int, stream=None):
        """One grouped call routing each of M tokens to every slot."""
        ids = self.torch.arange(self.nslots, dtype=self.torch.int32, device="cuda").repeat(M, 1).contiguous()
        return self.routed_fn(ids, stream)

    def routed_fn(self, ids, stream=None):
        """One grouped call with the given ids [M, K] (x rows 0..M-1)."""
        import quantized_moe_expert_q4_amd as q4
        from quantized_moe_expert_q4_amd.device import aligned_empty
        torch = self.torch
        M, K = ids.shape
        x = self.x[:M].contiguous()
        odt = torch.bfloat16 if self.xdtype == "bf16" else torch.float32
        out = torch.empty((M, K, self.I), dtype=odt, device="cuda")
        wsb = q4.grouped_workspace_bytes(M, K, self.nslots)
        ws = aligned_empty(wsb, 256)

        def step():
            q4.expert_gate_up_grouped(self.slots, self.stride, self.nslots, self.lay, x, M, ids, K, self.H, self.I,
                                      out, ws, wsb, stream=stream, fmt=self.fmt, xdtype=self.xdtype)
        return step

    def single_fn(self, slot_index: int, stream=None):
        """One single-expert launch on one slot (M=1)."""
        import quantized_moe_expert_q4_amd as q4
        x = self.x[:1].contiguous()
        out = self.torch.empty((1, self.I), dtype=self.torch.bfloat16, device="cuda")
        ptr = self.slots.data_ptr() + slot_index * self.stride

        def step():
            q4.expert_gate_up(ptr, self.lay, x, 1, self.H, self.I, out, stream=stream)
        return step

    def down_fn(self, stream=None):
        """One grouped down call: the token's own mid row on every slot (the
        gate/up + SwiGLU output of that token on each slot, made once)."""
        import quantized_moe_expert_q4_amd as q4
        from quantized_moe_expert_q4_amd.device import aligned_empty
        torch = self.torch
        n = self.nslots
        ids = torch.arange(n, dtype=torch.int32, device="cuda").reshape(1, n).contiguous()
        x = self.x[:1].contiguous()
        mid = torch.empty((1, n, self.I), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((1, n, self.H), dtype=torch.bfloat16, device="cuda")
        wsb = q4.grouped_workspace_bytes(1, n, n)
        ws = aligned_empty(wsb, 256)
        q4.expert_gate_up_grouped(self.slots, self.stride, n, self.lay, x, 1, ids, n, self.H, self.I, mid, ws, wsb,
                                  stream=stream)

        def step():
            q4.expert_down_grouped(self.slots, self.stride, n, self.lay, mid, 1, ids, n, self.H, self.I, out, ws,
                                   wsb, stream=stream)
        return step

    def forward_fn(self, stream=None):
        """One grouped whole-expert call (gate/up then down) routing the token to every slot."""
        import quantized_moe_expert_q4_amd as q4
        from quantized_moe_expert_q4_amd.device import aligned_empty
        torch = self.torch
        n = self.nslots
        ids = torch.arange(n, dtype=torch.int32, device="cuda").reshape(1, n).contiguous()
        x = self.x[:1].contiguous()
        mid = torch.empty((1, n, self.I), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((1, n, self.H), dtype=torch.bfloat16, device="cuda")
        wsb = q4.grouped_workspace_bytes(1, n, n)
        ws = aligned_empty(wsb, 256)

        def step():
            q4.expert_forward_grouped(self.slots, self.stride, n, self.lay, x, 1, ids, n, self.H, self.I, mid, out,
                                      ws, wsb, stream=stream)
        return step


def settle(step):
    """Untimed steps for SETTLE_S seconds of wall time: the GPU's clocks ramp
    up over tens of milliseconds of load (a leg's repetitions kept speeding up
    without this), so each leg's first repetition starts from the steady
    state a serving loop runs at."""
    import time
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(10):
            step()
        torch.cuda.synchronize()


def time_steps(step, steps: int, warmup: int):
    """Seconds for `steps` calls of step() on the current stream (HIP events on
    that stream, which is the one the library launches on)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1000.0


def timed(step, steps: int, warmup: int, reps: int = REPS):
    """Median over `reps` repetitions of the mean seconds per step (after the
    clock-settling steps, then `warmup` untimed steps)."""
    settle(step)
    per = [time_steps(step, steps, warmup if r == 0 else 1) / steps for r in range(reps)]
    return statistics.median(per), per


def graph_timed(calls, reps: int = REPS, replays: int = 5):
    """Capture the calls (one pass) into a HIP graph, then time replays:
    median over `reps` of the mean seconds per pass.  Each call runs once
    eagerly before capture (one-time initialisation stays out of the graph)."""
    import torch
    for c in calls:
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    settle(g.replay)
    stream = torch.cuda.current_stream()
    per = []
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(replays):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        per.append(start.elapsed_time(end) / 1000.0 / replays)
    del g
    return statistics.median(per), per


def leg(nbytes: float, sec: float, per, workload: str, kernel: str, rows: float = None, **extra):
    v = nbytes / sec / 1e9
    d = {"value": round(v, 2), "unit": "GB/s", "pct_hbm_peak": round(100 * v / HBM_PEAK_GBS, 2),
         "ms_per_step": round(sec * 1e3, 4), "reps_GBps": [round(nbytes / p / 1e9, 1) for p in per],
         "workload": workload, "kernel": kernel}
    if rows is not None:
        d["rows_per_s"] = round(rows / sec, 1)
    d.update(extra)
    return d


STREAM_VARIANTS = [("tile_w8_d2", 0, 8, 2), ("tile_w8_d4", 0, 8, 4), ("line_w8_d1", 3, 8, 1),
                   ("line_w8_d2", 3, 8, 2), ("linear_w8_d2", 1, 8, 2), ("tile_nt_w8_d2", 4, 8, 2),
                   ("line_nt_w8_d1", 7, 8, 1), ("line_nt_w8_d2", 7, 8, 2), ("line_nt_w8_d4", 7, 8, 4),
                   ("linear_nt_w8_d2", 5, 8, 2), ("line_nt_w16_d2", 7, 16, 2)]


def stream_ceiling(pool, steps: int, warmup: int):
    """Read-only streaming kernel over the pool's gate and up weights (no
    arithmetic): the rate this access pattern reaches on this device."""
    import torch
    import quantized_moe_expert_q4_amd as q4
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lay = pool.lay
    nbytes = pool.nslots * 2 * pool.I * (pool.H // 2)
    res = {}
    for name, pattern, waves, depth in STREAM_VARIANTS:
        def step():
            q4.stream_read(pool.slots, pool.stride, pool.nslots, lay.gate_weight_offset, lay.up_weight_offset,
                           pool.I, pool.H // 2, sink, pattern, waves, depth)
        sec, _ = timed(step, steps, warmup, reps=3)
        res[name] = round(nbytes / sec / 1e9, 1)
    best = max(res, key=res.get)
    return {"best_GBps": res[best], "best_variant": best, "variants_GBps": res, "bytes_per_launch": nbytes,
            "kernel": "q4::stream_read_kernel: the pool's gate and up weights read once, no arithmetic "
                      "(tile = 16-row x 128-byte steps, 4 lanes per row; line = the same with 8 lanes per row, whole "
                      "128-byte lines per load instruction; linear = lane-linear 1 KiB runs; nt = non-temporal load "
                      "hint; "
                      "w = waves per CU, d = steps in flight per wave; median of 3 repetitions)"}


# ---- CPU baseline (the oracle; run before the GPU is touched) ----

def _cpu_worker(args):
    """Oracle passes over whole pool slots at M=1 for ~budget seconds (one process, one BLAS thread)."""
    budget, start = args
    import oracle
    from threadpoolctl import threadpool_limits
    lay, contents, x8 = make_pool_host()
    n = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget:
            oracle.expert_gate_up(contents[(start + n) % DISTINCT_CONTENTS], lay, x8[:1], H, I)
            n += 1
        dt = time.perf_counter() - t0
    return n, dt


def usable_cores() -> int:
    """Cores this process may use: its CPU affinity, capped by the thread
    budget the environment sets (OMP_NUM_THREADS)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(budget_s: float):
    """The exact oracle on whole pool slots at M=1: one process, then one
    process per usable core (slots partitioned over processes)."""
    import multiprocessing as mp
    n1, dt1 = _cpu_worker((budget_s / 2, 0))
    single = n1 * weight_bytes_per_slot() / dt1 / 1e9
    cores = usable_cores()
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as p:
        res = p.map(_cpu_worker, [(budget_s / 2, i) for i in range(cores)])
    wall = time.perf_counter() - t0
    passes = sum(n for n, _ in res)
    span = max(dt for _, dt in res)
    allc = passes * weight_bytes_per_slot() / span / 1e9
    return {"value": round(allc, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "single_core_value": round(single, 4),
            "sample": f"exact oracle, gate/up+SwiGLU of whole H={H} I={I} pool slots at M=1: {n1} passes on one "
                      f"core in {dt1:.1f} s; {passes} passes over {cores} processes (one BLAS thread each) in "
                      f"{span:.1f} s ({wall:.1f} s wall)",
            "cpu": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def load_traffic(bytes_per_launch: float):
    """HBM bytes per launch of the timed kernel (FETCH_SIZE + WRITE_SIZE, each
    scaled by what the counter reads for a plain copy of known size), from the
    committed counter summary; None when the kernels changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_sha256") != kernel_sha():
        return None, {"stale": True, "source": os.path.relpath(TRAFFIC_FILE, ROOT)}
    detail = {"fetch_bytes": t["fetch_bytes_per_launch"], "write_bytes": t["write_bytes_per_launch"],
              "fetch_over_algorithmic": round(t["fetch_bytes_per_launch"] / bytes_per_launch, 4),
              "source": os.path.relpath(TRAFFIC_FILE, ROOT)}
    return t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"], detail


def load_parity():
    """Per-workload parity statistics of the GPU path against the oracle, from
    the committed report (tests/parity_report.py) when it was taken on the
    current kernel source."""
    if not os.path.exists(PARITY_FILE):
        return None
    with open(PARITY_FILE) as f:
        p = json.load(f)
    if p.get("kernel_sha256") != kernel_sha():
        return {"stale": True, "source": os.path.relpath(PARITY_FILE, ROOT)}
    p["source"] = os.path.relpath(PARITY_FILE, ROOT)
    return p


def inputs_info(lay, contents, x8):
    return {"seeds": SEEDS, "generator": "numpy PCG64 (synth/generators.py)",
            "pool_contents_sha256": [sha256_hex(c) for c in contents], "x_sha256": sha256_hex(x8),
            "layout": {"slot_bytes": lay.slot_bytes, "gate_w": lay.gate_weight_offset, "up_w": lay.up_weight_offset,
                       "gate_s": lay.gate_scale_offset, "up_s": lay.up_scale_offset}}


# ---- legs ----

def pool_legs(args, lay, contents, x8, legs, out):
    import torch
    pool = Pool(lay, contents, x8)
    res = {}
    for M in (1, 8):
        name = f"m{M}"
        if name in legs:
            sec, per = timed(pool.step_fn(M), args.steps, args.warmup)
            res[name] = (sec, per)
    if "stream" in legs:
        out["stream_ceiling"] = stream_ceiling(pool, args.steps, args.warmup)
    shapes = out.setdefault("shapes", {})
    if "single" in legs:
        # one single-expert launch per pool slot (cold), captured in a graph
        calls = [pool.single_fn(s) for s in range(POOL_SLOTS)]
        sec, per = graph_timed(calls)
        nb = POOL_SLOTS * weight_bytes_per_slot()
        shapes["single_expert_launches"] = leg(
            nb, sec, per, f"{POOL_SLOTS} back-to-back single-expert launches H={H} I={I} M=1 (one per cold pool "
            f"slot, {weight_bytes_per_slot()} B each), captured in one HIP graph", kernel_label(1, H),
            rows=POOL_SLOTS * I, us_per_launch=round(sec / POOL_SLOTS * 1e6, 3))
    if "decode" in legs:
        # top-8 decode steps over rotating cold slots: step i routes to slots 8i..8i+7 (mod pool)
        nsteps = POOL_SLOTS // 8
        for M in (1, 8):
            rng = np.random.default_rng(SEEDS["decode_routing"] + M)
            calls = []
            distinct = 0
            for i in range(nsteps):
                if M == 1:
                    ids = np.arange(8 * i, 8 * i + 8, dtype=np.int32)[None, :] % POOL_SLOTS
                else:
                    # eight tokens, each top-8 of a 64-slot window that moves on every step
                    win = (64 * i + np.arange(64)) % POOL_SLOTS
                    ids = np.stack([rng.choice(win, 8, replace=False) for _ in range(M)]).astype(np.int32)
                calls.append(pool.routed_fn(torch.from_numpy(ids).cuda()))
                distinct += len(np.unique(ids))
            sec, per = graph_timed(calls)
            nb = distinct * weight_bytes_per_slot()
            shapes[f"decode_top8_m{M}"] = leg(
                nb / nsteps, sec / nsteps, [p / nsteps for p in per],
                f"grouped call, M={M}, top-8 routing over a {POOL_SLOTS}-slot cold pool of H={H} I={I} slots "
                f"({distinct / nsteps:.1f} distinct slots, {nb / nsteps / 1e6:.1f} MB per step; {nsteps} steps on "
                f"rotating slots captured in one HIP graph)", kernel_label(M, H), rows=M * 8 * I,
                us_per_step=round(sec / nsteps * 1e6, 2))
    del pool
    torch.cuda.empty_cache()
    return res


def large_legs(args, legs, shapes):
    import torch
    for M in (1, 4, 8, 16, 32):
        name = f"large_m{M}"
        if name not in legs:
            continue
        llay, lcontents, lx = large_shape_host(M)
        pool = Pool(llay, lcontents, lx, LARGE_SLOTS, LARGE_H, LARGE_I)
        sec, per = timed(pool.step_fn(M), args.steps, args.warmup)
        shapes[f"large_pool_m{M}"] = leg(
            pool.bytes_per_step(), sec, per,
            f"H={LARGE_H} I={LARGE_I}, M={M} (x with 1% of entries at +-9984), {LARGE_SLOTS}-slot cold pool "
            f"({pool.bytes_per_step() / 1e9:.3f} GB per step), one grouped launch per step",
            kernel_label(M, LARGE_H, per_slot=M), rows=M * LARGE_SLOTS * LARGE_I)
        del pool
        torch.cuda.empty_cache()


def routed_legs(args, legs, shapes):
    import torch
    import synth
    if not ({"routed", "ep_share"} & set(legs)):
        return
    c = synth.make_config("cfg4")
    pool = Pool(c.layout, c.slots, c.x, c.num_slots, c.H, c.I)
    if "routed" in legs:
        ids = torch.from_numpy(c.ids).cuda()
        sec, per = timed(pool.routed_fn(ids), args.steps, args.warmup)
        touched = len(np.unique(c.ids))
        nb = touched * weight_bytes_per_slot(c.H, c.I)
        shapes["routed_step_m32_top8"] = leg(
            nb, sec, per, f"{c.num_slots} experts of H={c.H} I={c.I}, M={c.M} tokens, top-{c.K} routing ({touched} "
            f"slots touched, {nb / 1e9:.3f} GB per step), one grouped launch per step", kernel_label(c.M, c.H, per_slot=-(-c.M * c.K // c.num_slots)),
            rows=c.M * c.K * c.I)
    if "ep_share" in legs:
        # one GPU's share of the routed step under 8-way expert parallelism: 8
        # local experts and the 32 routed pairs they receive (K = 1 each);
        # steps rotate over the 64 slots so each step's 8 experts are cold
        rng = np.random.default_rng(SEEDS["ep_routing"])
        calls = []
        distinct = 0
        for i in range(8):
            ids = (8 * i + rng.integers(0, 8, size=(32, 1))).astype(np.int32)
            calls.append(pool.routed_fn(torch.from_numpy(ids).cuda()))
            distinct += len(np.unique(ids))
        sec, per = graph_timed(calls)
        n = len(calls)
        nb = distinct * weight_bytes_per_slot(c.H, c.I) / n
        shapes["ep_share_8slots_32pairs"] = leg(
            nb, sec / n, [p / n for p in per],
            f"one GPU's expert-parallel share of the routed step: 32 routed token rows (K=1) over 8 local "
            f"experts of H={c.H} I={c.I} ({nb / 1e6:.1f} MB per step; {n} steps on rotating slots of the "
            f"{c.num_slots}-slot pool, captured in one HIP graph)", kernel_label(32, c.H, per_slot=-(-32 // c.num_slots)), rows=32 * c.I,
            us_per_step=round(sec / n * 1e6, 2))
    del pool
    torch.cuda.empty_cache()


def expert_legs(args, legs, shapes):
    import torch
    if not ({"down", "forward"} & set(legs)):
        return
    elay, econtents, ex = expert_pool_host()
    pool = Pool(elay, econtents, ex, EXPERT_SLOTS, H, I)
    if "down" in legs:
        sec, per = timed(pool.down_fn(), args.steps, args.warmup)
        nb = EXPERT_SLOTS * down_bytes_per_slot()
        shapes["down_pool_m1"] = leg(
            nb, sec, per, f"down projection H={H} I={I}, one token's mid row per slot on a {EXPERT_SLOTS}-slot cold "
            f"pool of whole-expert slots ({nb / 1e9:.3f} GB of down weights+scales per step), one grouped launch",
            "q4::chunked_kernel (down mode)", rows=EXPERT_SLOTS * H)
    if "forward" in legs:
        sec, per = timed(pool.forward_fn(), args.steps, args.warmup)
        nb = EXPERT_SLOTS * (weight_bytes_per_slot() + down_bytes_per_slot())
        shapes["forward_pool_m1"] = leg(
            nb, sec, per, f"whole expert (gate/up+SwiGLU then down) H={H} I={I}, one token routed to every slot of "
            f"a {EXPERT_SLOTS}-slot cold pool ({nb / 1e9:.3f} GB per step), two launches per step",
            "q4::resident_kernel then q4::chunked_kernel (down mode)")
    del pool
    torch.cuda.empty_cache()


def format_legs(args, lay, contents, x8, legs, shapes):
    import torch
    import synth
    if "f32_m1" in legs:
        rng = np.random.default_rng(SEEDS["f32_x"])
        pool = Pool(lay, contents, rng.standard_normal((8, H), dtype=np.float32), xdtype="f32")
        sec, per = timed(pool.step_fn(1), args.steps, args.warmup)
        shapes["f32_pool_m1"] = leg(
            pool.bytes_per_step(), sec, per, f"f32 activations and outputs, H={H} I={I}, M=1, the {POOL_SLOTS}-slot "
            f"cold pool, one grouped launch per step", "q4::resident_kernel (f32 x)", rows=POOL_SLOTS * I)
        del pool
        torch.cuda.empty_cache()
    if "q8_m1" in legs:
        qlay = synth.contiguous_layout(H, I, fmt="q8")
        rng = np.random.default_rng(SEEDS["q8_pool"])
        qcontents = np.zeros((DISTINCT_CONTENTS, qlay.slot_bytes), np.uint8)
        for d in range(DISTINCT_CONTENTS):
            synth.fill_slot(rng, H, I, qlay, out=qcontents[d], fmt="q8")
        pool = Pool(qlay, qcontents, x8, Q8_SLOTS, H, I, fmt="q8")
        sec, per = timed(pool.step_fn(1), args.steps, args.warmup)
        shapes["q8_pool_m1"] = leg(
            pool.bytes_per_step(), sec, per, f"Q8 (int8) expert gate/up+SwiGLU, H={H} I={I}, M=1, {Q8_SLOTS}-slot "
            f"cold pool ({pool.bytes_per_step() / 1e9:.3f} GB per step), one grouped launch per step",
            "q4::resident_kernel (int8 weights)", rows=Q8_SLOTS * I)
        del pool
        torch.cuda.empty_cache()


ALL_LEGS = ["m1", "m8", "stream", "single", "decode", "large_m1", "large_m4", "large_m8", "large_m16", "large_m32",
            "routed", "ep_share", "down", "forward", "f32_m1", "q8_m1"]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps per repetition (five repetitions per leg)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=16.0, help="seconds of CPU-oracle work (half on one core)")
    ap.add_argument("--no-shapes", action="store_true", help="only the headline pool legs and the stream ceiling")
    ap.add_argument("--only", choices=ALL_LEGS + ["copy"], default=None,
                    help="run one leg only (for profiling); 'copy' times a plain 1 GiB device copy, "
                         "the reference for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE to bytes")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X (no multi-GPU leg)", file=sys.stderr)
        sys.exit(2)

    lay, contents, x8 = make_pool_host()
    out = {}
    # the CPU baseline runs first: its worker processes fork before the GPU is initialised
    cpu = None
    if not args.no_cpu and args.only is None:
        cpu = cpu_baseline(args.cpu_budget)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import quantized_moe_expert_q4_amd as q4
    q4.load()

    if args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        t = time_steps(lambda: dst.copy_(src), args.steps, args.warmup)
        print(json.dumps({"copy_bytes": 1 << 30, "steps": args.steps,
                          "GBps_read_plus_write": round(2 * (1 << 30) * args.steps / t / 1e9, 1)}), flush=True)
        return

    if args.only:
        legs = [args.only]
    elif args.no_shapes:
        legs = ["m1", "m8", "stream"]
    else:
        legs = ALL_LEGS
    res = pool_legs(args, lay, contents, x8, legs, out)
    shapes = out.setdefault("shapes", {})
    large_legs(args, legs, shapes)
    routed_legs(args, legs, shapes)
    expert_legs(args, legs, shapes)
    format_legs(args, lay, contents, x8, legs, shapes)

    bytes_step = POOL_SLOTS * weight_bytes_per_slot()
    if not res:
        # shape legs only (profiling runs)
        print(json.dumps(out), flush=True)
        return
    primary = "m1" if "m1" in res else "m8"
    M = 1 if primary == "m1" else 8
    sec, per = res[primary]
    value = bytes_step / sec / 1e9
    line = {
        "metric": "achieved weight GB/s (% of HBM peak) for Q4 gate/up SwiGLU at M=1 and M=8",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4 weights x bf16 activations, exact int32 matrix-core accumulation, f32 scale, bf16 out",
        "data": "synthetic (seeded uniform nibbles, U[0.005,0.02] f32 scales, N(0,1) bf16 x)",
        "config": {"workload": f"expert gate/up+SwiGLU, H={H} I={I}, M={M}, {POOL_SLOTS}-slot cold pool "
                               f"({bytes_step / 1e9:.3f} GB of weights+scales per step), one grouped launch per step",
                   "H": H, "I": I, "M": M, "slots": POOL_SLOTS, "bytes_per_step": bytes_step,
                   "repetitions": REPS, "statistic": "median of the repetitions' mean step time",
                   "clock_settle_s": SETTLE_S},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "rows_per_s": round(M * POOL_SLOTS * I / sec, 1),
        "reps_GBps": [round(bytes_step / p / 1e9, 1) for p in per],
    }
    if "m8" in res and primary != "m8":
        s8, p8 = res["m8"]
        line["m8"] = leg(bytes_step, s8, p8, f"the same pool with eight tokens on every slot (H={H} I={I}, M=8)",
                         kernel_label(8, H), rows=8 * POOL_SLOTS * I)
    # One step is one launch of the gate/up kernel; HIP events bracket the
    # launches on their own stream, so the per-launch mean is the step time.
    traffic, traffic_detail = load_traffic(bytes_step) if M == 1 else (None, None)
    ceiling = out.get("stream_ceiling")
    line["roofline"] = {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic,
                        "traffic_detail": traffic_detail,
                        "kernel": kernel_label(M, H) + " (grouped call, M=%d)" % M,
                        "algorithmic_bytes_per_launch": bytes_step,
                        "stream_ceiling": ceiling,
                        "frac_of_stream_ceiling": round(value / ceiling["best_GBps"], 4) if ceiling else None}
    if shapes:
        line["shapes"] = shapes
    line["inputs"] = inputs_info(lay, contents, x8)
    line["parity"] = load_parity()
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
