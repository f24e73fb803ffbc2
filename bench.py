"""Benchmark of the composite multi-LoRA apply on one MI355X.

One step = one pass of the whole path over one batch: the mapping stage
(tcl_plan_map's kernel: validation, canonical slots, counting sort by adapter
id, token index, work list) followed by the fused apply (shrink + expand) of
every module of the workload.  Inputs are synthetic, drawn by
tenant_composite_lora_amd.workloads, and resident in HBM before timing starts.
Each step uses the next of R replicas of {adapter pools, x, y} so that the
working set of consecutive steps exceeds the 256 MB Infinity Cache and the
adapter bytes really come from HBM.

Default workload (the headline line): the retained-rank mixed batch, the
largest configuration: 4096 prefill + 128 decode tokens, each a composite of
1-4 adapters drawn Zipf(1.2) from 256 adapters stored at rank 32 (bf16) with
per-(adapter, module) effective ranks k in 1..32, on an 8192 -> 8192 and an
8192 -> 28672 projection.  The decode configurations (32 tokens on one
4096 -> 4096 projection; 64 tokens on the seven Llama-3-8B projections) and
the sparse prefill (8 requests x 256 tokens, gated) are measured in the same
run and reported under config.nested.

Exactly --steps steps are timed (one HIP graph), after --warmup untimed ones.
The oracle is timed on the host's cores (at most 16) before the GPU work.

Prints one JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--no-nested] [--eager]

``--scheduler`` times the host-side LAG batch choice and BAM slot assignment
on a synthetic request stream (no GPU).

``--producer`` times the retained-rank producer instead (LoRAForge, approach
(2) and (3)): balanced factors of a whole Llama-3.1-8B fleet of 35 adapters x
32 layers x 7 projections (its Figure 1: 7840 LoRA matrices), rank 16, then
LoRAForge-S ranks for the LoRAForge-U budget at d = 4 with floor 1 (at
rank 16, d = 12 keeps one direction per module and the floors spend it all).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "composite-LoRA apply tokens/s + achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20


def algorithmic_bytes(wl) -> int:
    """Bytes the method must move for one step: every touched adapter's
    retained rows of A and B once, x once, y read and written once, and the
    16-byte tuple records of the plan once."""
    c = wl.composites
    used = np.unique(c.pair_adapter[:c.n_pairs]) if c.n_pairs else np.zeros(0, np.int64)
    # only adapters that own at least one tuple count
    owner_tokens = np.diff(c.group_tok_ptr)
    pair_tokens = np.repeat(owner_tokens, np.diff(c.group_pair_ptr))
    used = np.unique(c.pair_adapter[pair_tokens > 0]) if c.n_pairs else used
    T = c.n_tokens
    total = 0
    for mi, m in enumerate(wl.modules):
        e_w = 2 if m.A_t.dtype == np.uint16 else 4
        e_x = 2 if wl.x[mi].dtype == np.uint16 else 4
        k = np.full(m.A_t.shape[0], m.r_max) if m.k is None else m.k
        total += int(np.sum(k[used])) * (m.d_in + m.d_out) * e_w
        total += T * m.d_in * e_x + 2 * T * m.d_out * 4
    total += c.n_tuples() * 16
    return total


def kernel_bytes(wl) -> dict:
    """Algorithmic bytes of each kernel of the step (their sum is the step's
    algorithmic bytes): shrink reads the touched adapters' retained A rows and
    x; expand reads their retained B rows and reads and writes y; the mapping
    stage reads the composite table and writes 16-byte tuple records."""
    c = wl.composites
    owner_tokens = np.diff(c.group_tok_ptr)
    pair_tokens = np.repeat(owner_tokens, np.diff(c.group_pair_ptr))
    used = np.unique(c.pair_adapter[pair_tokens > 0]) if c.n_pairs else np.zeros(0, np.int64)
    T = c.n_tokens
    out = {"shrink": 0, "expand": 0, "plan": c.n_tuples() * 16}
    for mi, m in enumerate(wl.modules):
        e_w = 2 if m.A_t.dtype == np.uint16 else 4
        e_x = 2 if wl.x[mi].dtype == np.uint16 else 4
        k = np.full(m.A_t.shape[0], m.r_max) if m.k is None else m.k
        ranks = int(np.sum(k[used]))
        out["shrink"] += ranks * m.d_in * e_w + T * m.d_in * e_x
        out["expand"] += ranks * m.d_out * e_w + 2 * T * m.d_out * 4
    return out


# HIP sources each kernel is built from: a stored counter summary is only
# valid while these are unchanged
KERNEL_SOURCES = {k: ("plan.hip", "plan_core.hpp", "tcl_internal.hpp")
                  for k in ("plan_kernel", "tile_order_count",
                            "plan_m_local", "plan_m_scan", "plan_m_scatter")}
KERNEL_SOURCES.update({k: ("tile.hip", "kern_common.hpp", "tcl_internal.hpp")
                       for k in ("tile_prep", "expand_tile")})
KERNEL_SOURCES.update({k: ("pack.hip", "kern_common.hpp", "tcl_internal.hpp")
                       for k in ("pack_offsets_kernel", "pack_b_kernel")})
KERNEL_SOURCES.update({k: ("gate.hip", "tcl_internal.hpp")
                       for k in ("gate_count_kernel", "gate_scan_kernel", "gate_topk_kernel")})
# the producer's four kernels are summarised per fleet under the entry point's name
KERNEL_SOURCES["tcl_factor_balanced"] = ("factor.hip", "tcl_internal.hpp")
FACTOR_KERNELS = ("tsqr_leaf", "gram_kernel", "factor_core", "factor_out")
PRODUCER_WORKLOAD = "llama31_8b_fleet_35x32x7_r16"
APPLY_SOURCES = ("apply.hip", "kern_common.hpp", "plan_core.hpp", "tcl_internal.hpp")
# library kernels the counter summary keeps apart (whole identifiers of the
# demangled names)
PMC_KERNELS = ("plan_shrink", "shrink_mfma", "shrink_mfma_pair", "shrink_valu", "expand_kernel",
               "tile_prep", "expand_tile", "tile_order_count",
               "pack_offsets_kernel", "pack_b_kernel", "plan_kernel", "plan_m_local",
               "plan_m_scan", "plan_m_scatter", "gate_count_kernel", "gate_scan_kernel",
               "gate_topk_kernel")


def kernel_source_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tenant_composite_lora_amd", "csrc")
    for name in KERNEL_SOURCES.get(kernel, APPLY_SOURCES):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` ("a+b": the sum over kernels launched
    back to back) from the committed rocprofv3 counter summary
    (profiles/pmc_traffic.txt), or None when any part has no entry for this
    workload or its sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    total = 0.0
    for k in kernel.split("+"):
        ent = rec.get("entries", {}).get(f"{workload}:{k}")
        if not ent or ent.get("source_hash") != kernel_source_hash(k):
            return None
        total += ent.get("hbm_bytes_per_launch")
    return total


def pmc_summary(fetch_csv: str, write_csv: str, workload: str, into: str = None) -> dict:
    """HBM traffic per launch of each library kernel from two rocprofv3 --pmc
    runs of the same bench command (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch).  Each counter is scaled by what it reads for the 256 MiB
    calibration copy of that run (the largest __amd_rocclr_copyBuffer
    dispatch): factor = 256 MiB / measured.  Entries are merged into the
    summary `into` when it exists."""
    import csv
    import collections
    import re
    calib = 256 << 20

    def load(path):
        per = collections.defaultdict(list)
        biggest_copy = 0.0
        for r in csv.DictReader(open(path)):
            v = float(r["Counter_Value"]) * 1024.0
            name = r["Kernel_Name"]
            if name.startswith("__amd_rocclr_copyBuffer"):
                biggest_copy = max(biggest_copy, v)
            if any(k in name for k in FACTOR_KERNELS):
                per["tcl_factor_balanced"].append(v)
                continue
            for short in PMC_KERNELS:
                if re.search(r"(?<![A-Za-z0-9_])" + short + r"(?![A-Za-z0-9_])", name):
                    per[short].append(v)
                    break
        return per, calib / biggest_copy

    f, ff = load(fetch_csv)
    w, fw = load(write_csv)
    out = {"units": "bytes per kernel launch; FETCH_SIZE and WRITE_SIZE (KiB per dispatch) "
                    "scaled by the 256 MiB copy calibration of the same run",
           "entries": {}}
    if into and os.path.exists(into):
        out = json.load(open(into))
    for k in sorted(set(f) | set(w)):
        # the producer: one "launch" is one fleet, 4 shapes x 4 kernels
        per_launch = 16 if k == "tcl_factor_balanced" else 1
        fb = sum(f[k]) / len(f[k]) * per_launch * ff if f.get(k) else 0.0
        wb = sum(w[k]) / len(w[k]) * per_launch * fw if w.get(k) else 0.0
        out["entries"][f"{workload}:{k}"] = {
            "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
            "hbm_bytes_per_launch": fb + wb, "launches": len(f.get(k, [])) // per_launch,
            "fetch_factor": ff, "write_factor": fw, "source_hash": kernel_source_hash(k)}
    return out


def algorithmic_flops(wl) -> int:
    c = wl.composites
    owner_tokens = np.diff(c.group_tok_ptr)
    pair_tokens = np.repeat(owner_tokens, np.diff(c.group_pair_ptr))
    total = 0
    for m in wl.modules:
        k = np.full(m.A_t.shape[0], m.r_max) if m.k is None else m.k
        total += int(np.sum(pair_tokens * k[c.pair_adapter])) * 2 * (m.d_in + m.d_out)
    return total


def host_cores() -> int:
    """Cores this process may run on, capped at 16 (one GPU's share of the
    host on the GPU machines, whatever the machine reports)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_CPU_WL = None


def _oracle_rows(lo_hi):
    """One worker's share of the oracle: tokens [lo, hi) of every module of
    the workload inherited from the parent process (one BLAS thread)."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    wl = _CPU_WL
    c = wl.composites
    lo, hi = lo_hi
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for mi, m in enumerate(wl.modules):
            O.apply_rows(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                         m.A_t, m.B_t, m.k, wl.x[mi], wl.y_base[mi], range(lo, hi))
    return time.perf_counter() - t0


def cpu_baseline(wl, budget_s: float = 12.0, cores: int = 0) -> dict:
    """The fp64 oracle timed on this host's cores: the mapping stage once,
    then the whole batch's apply (every module) split into contiguous token
    ranges, one per worker process (one BLAS thread each), repeated until
    ``budget_s`` seconds of wall time.  Workers are forked before anything
    touches the GPU and inherit the workload."""
    global _CPU_WL
    import multiprocessing as mp

    import oracle as O
    c = wl.composites
    n = cores or host_cores()
    _CPU_WL = wl
    T = c.n_tokens
    bounds = [(T * i // n, T * (i + 1) // n) for i in range(n)]
    ctx = mp.get_context("fork")
    reps, wall = 0, 0.0
    with ctx.Pool(n) as pool:
        while wall < budget_s and reps < 100000:
            t0 = time.perf_counter()
            O.plan(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha)
            pool.map(_oracle_rows, bounds, chunksize=1)
            wall += time.perf_counter() - t0
            reps += 1
    _CPU_WL = None
    return {"value": T * reps / wall, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"whole batch ({T} tokens, all {len(wl.modules)} modules; mapping stage "
                      f"on one core, apply split into {n} contiguous token ranges) repeated "
                      f"{reps}x, {wall:.1f} s wall, fp64 numpy, {n} processes x 1 BLAS thread"}


PRODUCER_METRIC = "retained-rank fleet factor construction, LoRA matrices/s"


def producer_alg(classes, r):
    """Algorithmic bytes and flops of one fleet: every factor read once and
    every output written once (bf16), sigma written; QR 2 d_out r^2, Gram
    2 d_in r^2, outputs 2 r^2 (d_out + d_in) flops per module."""
    b = f = 0
    for M, d_out, d_in in classes:
        b += M * (2 * r * (d_out + d_in) * 2 + 4 * r)
        f += M * (2 * d_out * r * r + 2 * d_in * r * r + 2 * r * r * (d_out + d_in))
    return b, f


def producer_cpu_baseline(classes, r, budget_s: float = 12.0) -> dict:
    """The fp64 oracle's factor construction on this host, one module of each
    shape class in turn (fresh inputs from the same recipe), until
    ``budget_s`` seconds of work; scaled to modules per second."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    from tenant_composite_lora_amd import workloads as W
    ins = [W.factor_batch(90 + i, 1, r, d_out, d_in) for i, (_, d_out, d_in) in enumerate(classes)]
    n, t_used = 0, 0.0
    with threadpool_limits(limits=1):
        while t_used < budget_s and n < 100000:
            Bt, At = ins[n % len(ins)]
            t0 = time.perf_counter()
            O.factor_balanced(Bt[0], At[0])
            t_used += time.perf_counter() - t0
            n += 1
    return {"value": n / t_used, "unit": "LoRA matrices/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} modules cycling through the {len(classes)} projection shapes "
                      f"(equal counts; the fleet has 2:2:2:1), {t_used:.1f} s, fp64 numpy, "
                      f"1 BLAS thread"}


def producer_main(args):
    import torch

    from tenant_composite_lora_amd import tclora
    from tenant_composite_lora_amd import workloads as W
    import ctypes

    dev = torch.device("cuda:0")
    r, nA, nL = W.FLEET_RANK, W.FLEET_ADAPTERS, W.FLEET_LAYERS
    shapes = {}
    for name, d_in, d_out in W.LLAMA31_8B_PROJ:
        shapes.setdefault((d_out, d_in), []).append(name)
    classes = [(nA * nL * len(v), d_out, d_in) for (d_out, d_in), v in shapes.items()]
    print(f"[bench] generating the fleet: {classes}", file=sys.stderr, flush=True)
    L = tclora.lib()
    st = torch.cuda.Stream(device=dev)
    bufs = []
    for i, (M, d_out, d_in) in enumerate(classes):
        Bt, At = W.factor_batch_torch(100 + i, M, r, d_out, d_in, dev)
        nb = ctypes.c_size_t()
        tclora.check(L.tcl_factor_workspace_bytes(M, d_out, d_in, r, ctypes.byref(nb)))
        bufs.append(dict(M=M, d_out=d_out, d_in=d_in, Bt=Bt, At=At, Ft=torch.empty_like(Bt),
                         T=torch.empty_like(At),
                         sg=torch.empty(M, r, dtype=torch.float32, device=dev),
                         ws=torch.empty(nb.value, dtype=torch.uint8, device=dev), nb=nb.value))
    torch.cuda.synchronize()
    sp = int(st.cuda_stream)
    # the four shape batches are independent: each runs on a stream of its
    # own (default priority), forked from and joined to `st` by events, so a
    # latency-bound kernel of one batch overlaps the others' streaming ones
    side = [torch.cuda.Stream(device=dev) for _ in bufs] if not args.one_stream else []
    fork, joins = torch.cuda.Event(), [torch.cuda.Event() for _ in bufs]

    def factor_fleet():
        if side:
            fork.record(st)
        for i, b in enumerate(bufs):
            if side:
                side[i].wait_event(fork)
            tclora.check(L.tcl_factor_balanced(b["Bt"].data_ptr(), b["At"].data_ptr(), b["M"],
                                               b["d_out"], b["d_in"], r, b["Ft"].data_ptr(),
                                               b["T"].data_ptr(), b["sg"].data_ptr(),
                                               b["ws"].data_ptr(), b["nb"],
                                               int(side[i].cuda_stream) if side else sp))
            if side:
                joins[i].record(side[i])
        for e in joins if side else []:
            st.wait_event(e)

    costs = np.concatenate([np.full(b["M"], b["d_out"] + b["d_in"], np.int64) for b in bufs])
    ranks = np.full(len(costs), r, np.int32)
    floors = np.ones(len(costs), np.int32)
    _, budget = tclora.rank_uniform(ranks, costs, 4)
    sig_host = torch.empty(len(costs), r, dtype=torch.float32, pin_memory=True)

    def allocate():
        off = 0
        for b in bufs:
            sig_host[off:off + b["M"]].copy_(b["sg"], non_blocking=True)
            off += b["M"]
        st.synchronize()
        return tclora.rank_spectral(sig_host.numpy().astype(np.float64), ranks, costs, floors,
                                    budget)

    K, Wu = max(1, args.steps), max(0, args.warmup)
    with torch.cuda.stream(st):
        for _ in range(Wu):
            factor_fleet()
            allocate()
        st.synchronize()
        # GPU part alone, events on the stream the kernels run on
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(K):
            factor_fleet()
        e1.record(st)
        e1.synchronize()
        gpu_ms = e0.elapsed_time(e1) / K
        # the allocation on the host (sigma copied out, LoRAForge-S), alone
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            k = allocate()
        alloc_ms = (time.perf_counter() - t0) / K * 1e3
    step_s = gpu_ms * 1e-3
    n_mod = int(sum(b["M"] for b in bufs))
    B_alg, F_alg = producer_alg(classes, r)
    achieved = B_alg / (gpu_ms * 1e-3) / 1e9
    out = {
        "metric": PRODUCER_METRIC,
        "value": n_mod / step_s,
        "unit": "LoRA matrices/s",
        "n_gpus": 1, "steps": K, "warmup": Wu,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": PRODUCER_WORKLOAD,
            "modules": n_mod, "rank": r,
            "classes": [{"modules": M, "d_out": d_out, "d_in": d_in} for M, d_out, d_in in classes],
            "factor_gpu_ms": gpu_ms,
            "allocation_host_ms": alloc_ms,
            "allocation": "LoRAForge-S on the host (native, fp64), LoRAForge-U budget at d = 4, "
                          "floor 1; sigma copied out first; not in value",
            "alg_bytes_per_step": B_alg, "alg_flops_per_step": F_alg,
            "budget_params": budget, "kept_params": int((k.astype(np.int64) * costs).sum()),
            "mean_kept_rank": float(k.mean()),
            "compute": "QR and Gram fp32 (bf16 products), r x r eigenproblem fp64, factors bf16",
            "streams": 1 if args.one_stream else len(bufs),
        },
        "roofline": {
            "bound": "hbm", "kernel": "tcl_factor_balanced (tsqr_leaf, gram_kernel, "
                                      "factor_core, factor_out; timed together)",
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": stored_traffic(PRODUCER_WORKLOAD, "tcl_factor_balanced"),
        },
    }
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = producer_cpu_baseline(classes, r)
    print(json.dumps(out), flush=True)


SCHED_METRIC = "LAG batch choice + BAM slot assignment, decisions/s (host)"


def sched_stream(seed, steps, A=128, per_step=32, burst=256):
    """Synthetic request stream standing in for the pages' ShareGPT traces: a
    burst of `burst` requests, then per_step arrivals per step (as many as a
    batch holds, so a backlog of about `burst` stays waiting), each a
    composite of 2-5 distinct adapters drawn Zipf(1.2) over A adapters."""
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, A + 1) ** 1.2
    p /= p.sum()

    def req():
        return list(int(a) for a in rng.choice(A, int(rng.integers(2, 6)), replace=False, p=p))
    return [[req() for _ in range(per_step + (burst if t == 0 else 0))] for t in range(steps)]


def sched_replay(stream, select, make_pool, theta, B, S):
    """Runs the stream: each step adds its arrivals, picks a batch, makes its
    adapters resident.  Returns (loads per batch, seconds in select+acquire)."""
    pool = make_pool(S)
    arr, ads, loads, t_used = [], [], 0, 0.0
    for step, new in enumerate(stream):
        for a in new:
            arr.append(float(step))
            ads.append(a)
        t0 = time.perf_counter()
        res = pool.resident()
        ch = select(float(step), theta, arr, ads, res, B, S)
        loads += pool.acquire([a for i in ch for a in ads[i]])
        t_used += time.perf_counter() - t0
        chs = set(ch)
        keep = [i for i in range(len(arr)) if i not in chs]
        arr, ads = [arr[i] for i in keep], [ads[i] for i in keep]
    return loads / len(stream), t_used


def sched_main(args):
    from tenant_composite_lora_amd import tclora

    class LibPool:
        def __init__(self, S):
            self.b = tclora.Bam(S)

        def resident(self):
            return [a for a in self.b.slots().tolist() if a >= 0]

        def acquire(self, batch):
            return len(self.b.acquire(batch)[1])

    steps = args.steps
    stream = sched_stream(11, steps + args.warmup)
    B, S, theta = 32, 64, 16.0
    lag_loads, t = sched_replay(stream, tclora.lag_select, LibPool, theta, B, S)
    fifo_loads, _ = sched_replay(stream, tclora.lag_select, LibPool, float("-inf"), B, S)
    n_dec = len(stream)
    # bytes one load moves host to device (tcl_bam_load copies A and B rows):
    # a rank-16 bf16 adapter on the seven projections of each of the 32
    # layers of Llama-3-8B (d_in + d_out summed over q, k, v, o, gate, up, down)
    per_layer = (4096 + 4096) + 2 * (4096 + 1024) + (4096 + 4096) + 3 * (4096 + 14336)
    adapter_bytes = per_layer * 16 * 2 * 32
    out = {
        "metric": SCHED_METRIC, "value": n_dec / t, "unit": "decisions/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": t / n_dec * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": "zipf1.2_a128_slots64_batch32_backlog256_theta16",
                   "adapters": 128, "slots": S, "max_batch": B, "theta_steps": theta,
                   "arrivals_per_step": 32, "initial_burst": 256,
                   "composite": "2-5 adapters, Zipf(1.2)",
                   "loads_per_batch_lag": lag_loads, "loads_per_batch_fifo": fifo_loads,
                   "adapter_bytes": adapter_bytes,
                   "h2d_bytes_per_batch_lag": lag_loads * adapter_bytes,
                   "h2d_bytes_per_batch_fifo": fifo_loads * adapter_bytes,
                   "timed": "lag_select + bam acquire per step, binding included"},
        "roofline": None,
    }
    if not args.no_cpu_baseline:
        import oracle as O

        class OraclePool:
            def __init__(self, S):
                self.S, self.batches = S, []

            def resident(self):
                return [a for a in O.bam_run(self.S, self.batches)[1] if a >= 0]

            def acquire(self, batch):
                self.batches.append(batch)
                return len(O.bam_run(self.S, self.batches)[0][-1][2])

        sample = stream[:64]
        o_loads, o_t = sched_replay(sample, O.lag_select, OraclePool, theta, B, S)
        out["cpu_baseline"] = {"value": len(sample) / o_t, "unit": "decisions/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the first {len(sample)} steps of the same stream "
                                         f"(the oracle's pool replays its history each step), "
                                         f"{o_t:.1f} s"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 10 with --producer)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps (default 5; 2 with --producer)")
    ap.add_argument("--config", type=int, default=5,
                    help="the workload of the headline line (default: 5, the largest)")
    ap.add_argument("--full-rank", action="store_true",
                    help="every adapter at r_max (retained ranks ignored; the zero rows "
                         "beyond them are then read and multiplied): the padded-pool "
                         "comparison for the retained-rank batch")
    ap.add_argument("--no-nested", action="store_true",
                    help="measure only --config (no nested decode/prefill configurations)")
    ap.add_argument("--eager", action="store_true", help="no HIP graph capture")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the counter summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--producer", action="store_true",
                    help="time the retained-rank producer on the Llama fleet instead")
    ap.add_argument("--one-stream", action="store_true",
                    help="with --producer: the four shape batches in sequence on one stream")
    ap.add_argument("--scheduler", action="store_true",
                    help="time the host-side LAG/BAM decisions on a synthetic request stream")
    ap.add_argument("--pmc-into", metavar="JSON",
                    help="with --pmc-summary: merge into this existing summary")
    args = ap.parse_args()
    if args.pmc_summary:
        names = {1: "tiny_f32_256", 2: "distinct_decode_q4096_n64_r8_t32",
                 3: "skewed_decode_llama3_8b_7proj_n128_r8_t64",
                 4: "sparse_prefill_gated_8x256_n128_r16",
                 5: "retained_rank_mixed_n256_r32_t4224"}
        wname = PRODUCER_WORKLOAD if args.producer else names[args.config]
        print(json.dumps(pmc_summary(*args.pmc_summary, wname, args.pmc_into), indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(one GPU holds one data-parallel shard of the batch)",
              file=sys.stderr)
        sys.exit(2)
    if args.scheduler:
        args.steps = 2000 if args.steps is None else args.steps
        args.warmup = 0 if args.warmup is None else args.warmup
        sched_main(args)
        return
    if args.producer:
        args.steps = 10 if args.steps is None else args.steps
        args.warmup = 2 if args.warmup is None else args.warmup
        producer_main(args)
        return
    args.steps = 20 if args.steps is None else args.steps
    args.warmup = 5 if args.warmup is None else args.warmup
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    from tenant_composite_lora_amd import workloads as W

    print(f"[bench] generating config {args.config}", file=sys.stderr, flush=True)
    wl = W.make(args.config)
    if args.full_rank:
        for m in wl.modules:
            m.k = None
        wl.name += "_full_rank"
    cpu = None
    if not args.no_cpu_baseline:
        # before anything touches the GPU: the oracle's workers are forked
        print(f"[bench] timing the oracle on {host_cores()} host cores", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(wl)
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    # (not in counter runs: their copy calibration takes the run's largest
    # device copy, which must be the 256 MiB one below)
    fl = None if args.calibrate_copy else floors(dev, stream)
    head = measure(wl, dev, stream, args.steps, args.warmup, args.eager, args.replicas,
                   latency=True, copy_gbs=fl["copy_gbs"] if fl else None)
    nested = {}
    if not args.no_nested:
        for ci in NESTED_CONFIGS:
            if ci == args.config:
                continue
            print(f"[bench] generating config {ci} (nested)", file=sys.stderr, flush=True)
            wn = W.make(ci)
            r = measure(wn, dev, stream, None, None, args.eager, 0, latency=True,
                        copy_gbs=fl["copy_gbs"] if fl else None)
            nested[wn.name] = r
            del wn
            torch.cuda.empty_cache()
    K, Wu = args.steps, args.warmup
    t_steps = head["_t_steps"]
    out = {
        "metric": METRIC,
        "value": head["tokens"] * K / t_steps,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "ms_per_step": 1e3 * t_steps / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == W.BF16 else "f32",
        "data": "synthetic",
        "config": {k: v for k, v in head.items() if not k.startswith("_") and k != "roofline"},
        "roofline": head["roofline"],
    }
    if fl:
        out["config"]["floors"] = fl
    if nested:
        out["config"]["nested"] = {k: {kk: vv for kk, vv in v.items() if not kk.startswith("_")}
                                   for k, v in nested.items()}
    if args.calibrate_copy:
        # a plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE
        # counters of the same profiling run
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


# Configurations measured inside the same run and reported under
# config.nested (the decode configurations the bandwidth target names, and
# the sparse prefill).
NESTED_CONFIGS = (2, 3, 4)


def measure(wl, dev, stream, steps, warmup, eager, replicas, latency=False,
            copy_gbs=None) -> dict:
    """Times one workload on the GPU.  A step is tcl_remap_apply (mapping
    stage, shrink and expand of every module) on the next of R replicas of
    {pools, x, y}; R x working set >= 4 x the 256 MiB Infinity Cache, so the
    adapter bytes come from HBM.  With ``steps`` given, exactly that many
    steps are timed in one HIP graph after ``warmup`` untimed ones (a graph
    of their own); otherwise (nested configurations) whole passes over the
    replicas, at least 256 steps, replayed twice, the second replay timed.
    t_apply times tcl_fused_apply on the mapped plan the same way, and each
    kernel (mapping, shrink, expand) is timed alone in graphs of the same
    length.  Events are recorded on the stream every launch is queued on."""
    import ctypes

    import torch

    from tenant_composite_lora_amd import tclora
    from tenant_composite_lora_amd import workloads as W

    c = wl.composites
    T = c.n_tokens
    B_alg = algorithmic_bytes(wl)
    F_alg = algorithmic_flops(wl)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    ws_bytes = sum(m.A_t.nbytes + m.B_t.nbytes for m in wl.modules) + \
        sum(x.nbytes for x in wl.x) + sum(y.nbytes for y in wl.y_base)
    R = replicas or max(1, min(256, -(-4 * MALL_BYTES // ws_bytes)))
    base_mods = [tclora.Module(up(m.A_t), up(m.B_t), m.k) for m in wl.modules]
    base_x = [up(x) for x in wl.x]
    base_y = [up(y) for y in wl.y_base]
    reps = []
    for r in range(R):
        if r == 0:
            mods, xs, ys = base_mods, base_x, base_y
        else:
            mods = [tclora.Module(m.A_t.clone(), m.B_t.clone(), wl.modules[i].k)
                    for i, m in enumerate(base_mods)]
            xs = [x.clone() for x in base_x]
            ys = [y.clone() for y in base_y]
        reps.append((mods, xs, ys))
    gtp, gpp, pa, pw = (up(c.group_tok_ptr.astype(np.int32)), up(c.group_pair_ptr.astype(np.int32)),
                        up(c.pair_adapter.astype(np.int32)), up(c.pair_alpha.astype(np.float32)))
    P = c.n_tuples()
    plan = tclora.Plan(gtp, gpp, pa, pw, wl.n_adapters, n_tokens=T, max_tuples=P)
    rc, P_dev, U_dev = plan.status()
    tclora.check(rc)
    ws = torch.empty(tclora.workspace_bytes(plan, base_mods), dtype=torch.uint8, device=dev)
    calls = [tclora.FusedCall(plan, mods, xs, ys, ws) for (mods, xs, ys) in reps]
    comp_c = tclora.Composites(T, c.n_groups, c.n_pairs, wl.n_adapters, P, gtp.data_ptr(),
                               gpp.data_ptr(), pa.data_ptr(), pw.data_ptr())
    L = tclora.lib()

    def step(i, spp):
        # one step = tcl_remap_apply: mapping stage, shrink, expand
        cl = calls[i % R]
        tclora.check(L.tcl_remap_apply(plan.handle, ctypes.byref(comp_c), cl.descs, cl.n, cl.xp,
                                       cl.ldx, cl.xd, cl.yp, cl.ldy, cl.yd, cl.ws.data_ptr(),
                                       cl.ws.numel(), spp))

    # decode tables (the one-workgroup mapping mode) of bf16 pools run the
    # mapping stage inside the shrink launch; the shrink timing below then
    # times that launch (tcl_remap_shrink), as the step runs it
    fused = (wl.dtype == W.BF16 and c.n_pairs <= 512
             and os.environ.get("TCL_FUSED_MAPPING") != "0"
             and os.environ.get("TCL_SHRINK") != "valu")

    def shrink_only(i, spp):
        cl = calls[i % R]
        if fused:
            tclora.check(L.tcl_remap_shrink(plan.handle, ctypes.byref(comp_c), cl.descs, cl.n,
                                            cl.xp, cl.ldx, cl.xd, cl.ws.data_ptr(),
                                            cl.ws.numel(), spp))
        else:
            cl.shrink(spp)

    def plan_only(i, spp):
        tclora.check(L.tcl_plan_remap(plan.handle, ctypes.byref(comp_c), spp))

    phases = {
        "step": step,
        "apply": lambda i, spp: calls[i % R](spp),
        "plan": plan_only,
        "shrink": shrink_only,
        "expand": lambda i, spp: calls[i % R].expand(spp),
    }
    sp = int(stream.cuda_stream)
    print(f"[bench] {wl.name}: T={T} P={P_dev} U={U_dev} replicas={R} "
          f"alg bytes={B_alg} flops={F_alg}", file=sys.stderr, flush=True)
    with torch.cuda.stream(stream):
        for i in range(2):              # warm up before any capture
            step(i, sp)
    torch.cuda.synchronize()

    def runner(fn, n):
        """A callable that queues n launches of fn (replicas 0, 1, ...): one
        graph of n launches, or n eager calls."""
        if eager:
            return lambda: [fn(i, sp) for i in range(n)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            cs = int(torch.cuda.current_stream().cuda_stream)
            for i in range(n):
                fn(i, cs)
        return g.replay

    def timed(run):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            ev0.record(stream)
            run()
            ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3

    if steps is not None:
        K = steps
        if warmup:
            print(f"[bench] warmup {warmup} steps", file=sys.stderr, flush=True)
            timed(runner(step, warmup))
        run_k = runner(step, K)
        print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
        t_steps = timed(run_k)
    else:
        K = R * max(1, -(-256 // R))
        run_k = runner(step, K)
        timed(run_k)
        print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
        t_steps = timed(run_k)
    per = {}
    for name in ("apply", "plan", "shrink", "expand"):
        print(f"[bench] timing {K} launches of {name} alone", file=sys.stderr, flush=True)
        r = runner(phases[name], K)
        if steps is None:
            timed(r)
        per[name] = timed(r) / K
    lat = None
    if latency:
        # one step alone, replayed with the stream idle in between: the
        # single-call latency (median of 21)
        r1 = runner(step, 1)
        r1()
        samples = sorted(timed(r1) for _ in range(21))
        lat = samples[10] * 1e6
    gate = None
    if "gate_logits" in wl.meta:
        # the token-level gate that produces this workload's table from its
        # logits (tcl_gate_topk), timed alone in graphs of 64 launches
        lg = torch.from_numpy(np.ascontiguousarray(wl.meta["gate_logits"], np.float32)).to(dev)
        cd = torch.from_numpy(np.ascontiguousarray(wl.meta["gate_candidates"], np.int32)).to(dev)
        gk, C = int(wl.meta["gate_k"]), lg.shape[1]
        g_out = [torch.empty(T + 1, dtype=torch.int32, device=dev),
                 torch.empty(T + 1, dtype=torch.int32, device=dev),
                 torch.empty(T * gk, dtype=torch.int32, device=dev),
                 torch.empty(T * gk, dtype=torch.float32, device=dev)]

        def gate_call(i, spp):
            tclora.check(L.tcl_gate_topk(lg.data_ptr(), C, cd.data_ptr(), C, T, C, gk,
                                         *[o.data_ptr() for o in g_out], spp))

        GS = 64
        rg = runner(gate_call, GS)
        timed(rg)
        g_us = timed(rg) / GS * 1e6
        g_bytes = T * C * 8 + (T + 1) * 8 + T * gk * 8
        gate = {"kernel": "gate_count_kernel+gate_scan_kernel+gate_topk_kernel", "us": g_us,
                "alg_bytes": g_bytes,
                "gbs": g_bytes / g_us / 1e3, "k": gk, "candidates": C}
    kb = kernel_bytes(wl)
    dom = max(("shrink", "expand"), key=lambda n: per[n])
    names = kernel_names(wl, fused)
    achieved = kb[dom] / per[dom] / 1e9
    t_step = t_steps / K
    apply_bytes = kb["shrink"] + kb["expand"]
    res = {
        "workload": wl.name, "tokens": T, "tuples": int(P_dev), "adapters_touched": int(U_dev),
        "modules": [f"{m.name}:{m.d_in}->{m.d_out}" for m in wl.modules],
        "n_adapters": wl.n_adapters, "r_max": wl.modules[0].r_max,
        "accumulate": "f32", "replicas": R, "graph": not eager, "steps": K,
        "alg_bytes_per_step": B_alg, "alg_flops_per_step": F_alg,
        "step_us": t_step * 1e6,
        "tokens_per_s": T / t_step,
        "hbm_gbs_per_step": B_alg / t_step / 1e9,
        "hbm_frac_per_step": B_alg / t_step / 1e9 / HBM_PEAK_GBS,
        "t_apply_us": per["apply"] * 1e6,
        "apply_tokens_per_s": T / per["apply"],
        "apply_gbs": apply_bytes / per["apply"] / 1e9,
        "apply_frac": apply_bytes / per["apply"] / 1e9 / HBM_PEAK_GBS,
        **({"apply_frac_of_copy": apply_bytes / per["apply"] / 1e9 / copy_gbs}
           if copy_gbs else {}),
        **({"latency_us": lat} if lat is not None else {}),
        "kernel_us": {n: per[n] * 1e6 for n in ("plan", "shrink", "expand")},
        "kernel_alg_bytes": kb,
        "kernel_gbs": {n: kb[n] / per[n] / 1e9 for n in ("plan", "shrink", "expand")},
        "kernels": names,
        **({"gate": gate} if gate else {}),
        "roofline": {
            "bound": "hbm", "kernel": names[dom],
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": stored_traffic(wl.name, names[dom]),
        },
        "_t_steps": t_steps,
    }
    del calls, reps, ws, plan
    return res


def floors(dev, stream) -> dict:
    """Two floors measured in the same run, outside the timed steps: a
    kernel launch that does nothing useful (a one-element fill, 256 launches
    in one HIP graph, per launch), and the streaming bandwidth of a plain
    1 GiB device copy (bytes read plus bytes written per second), the
    practical HBM ceiling the apply is also reported against."""
    import torch
    one = torch.zeros(1, dtype=torch.float32, device=dev)
    src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for _ in range(3):
            one.fill_(1.0)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(256):
                one.fill_(1.0)
        g.replay()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        launch_us = e0.elapsed_time(e1) * 1e3 / 256
        for _ in range(2):
            dst.copy_(src)
        best = None
        for _ in range(5):
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
    copy_gbs = 2 * src.numel() * 4 / (best * 1e-3) / 1e9
    del g, src, dst, one
    torch.cuda.empty_cache()
    return {"empty_kernel_us_in_graph": launch_us, "copy_gbs": copy_gbs,
            "copy_bytes": 2 << 30}


def kernel_names(wl, fused: bool) -> dict:
    """The kernels each timed phase launches, by the library's dispatch rules:
    the decode step's shrink carries the mapping stage (plan_shrink); a
    prefill-sized shrink pairs its work items when that still leaves at least
    1024 jobs (two rounds of two workgroups on each of the 256 compute
    units); prefill-sized bf16 batches expand over token tiles on the matrix
    cores (tile_prep writes each tile's coefficients, expand_tile does the
    work), other batches on the per-token kernel."""
    from tenant_composite_lora_amd import workloads as W
    c = wl.composites
    bf = wl.dtype == W.BF16
    if not bf or os.environ.get("TCL_SHRINK") == "valu":
        shrink = "shrink_valu"
    elif fused:
        shrink = "plan_shrink"
    else:
        P = c.n_tuples()
        items_cap = min(P, wl.n_adapters) + P // 16 + 1
        units = sum(-(-m.r_max // 16) for m in wl.modules)
        shrink = "shrink_mfma_pair" if -(-items_cap // 2) * units >= 4 * 256 else "shrink_mfma"
    if not bf or c.n_tokens < 256 or os.environ.get("TCL_DISPATCH") == "valu":
        expand = "expand_kernel"
    else:
        expand = "tile_prep+expand_tile"
    return {"plan": "plan_kernel", "shrink": shrink, "expand": expand}


if __name__ == "__main__":
    main()
