"""bench.py's host-side logic without a GPU: the one-GPU rule, the
algorithmic byte counts and the counter summary."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from tenant_composite_lora_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_tiny(bench):
    """The tiny fp32 workload: 4 adapters of rank 8 on 256 -> 256, 16 tokens:
    adapters 4 * 8 * (256 + 256) * 4 B, x 16 * 256 * 4 B, y read and written
    2 * 16 * 256 * 4 B, plus 16 B per tuple."""
    wl = W.make(1)
    P = wl.composites.n_tuples()
    assert bench.algorithmic_bytes(wl) == 65536 + 16384 + 32768 + 16 * P
    kb = bench.kernel_bytes(wl)
    assert kb["shrink"] + kb["expand"] + kb["plan"] == bench.algorithmic_bytes(wl)


def test_algorithmic_bytes_retained_rank(bench):
    """Only the retained rows of touched adapters count."""
    wl = W.random_case(3, T=20, N=6, d_in=64, d_out=32, r_max=8, max_pairs=2, with_k=True)
    c, m = wl.composites, wl.modules[0]
    used = np.unique(c.pair_adapter)
    want = int(m.k[used].sum()) * (64 + 32) * 2 + 20 * 64 * 2 + 2 * 20 * 32 * 4 + 16 * c.n_tuples()
    assert bench.algorithmic_bytes(wl) == want


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_pmc_summary_scales_by_the_copy(bench, tmp_path):
    """Counters are KiB per dispatch, scaled so that the 256 MiB calibration
    copy reads 256 MiB."""
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    copy_kib = (256 << 20) / 1024
    _csv(fetch, [["__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_kib / 2],
                 ["void tcl::plan_shrink<8>(tcl::PlanArgs, tcl::ShrinkArgs)", "FETCH_SIZE", 100.0],
                 ["void tcl::plan_shrink<8>(tcl::PlanArgs, tcl::ShrinkArgs)", "FETCH_SIZE", 300.0],
                 ["void tcl::expand_kernel<8, 2, true>(tcl::ExpandArgs)", "FETCH_SIZE", 50.0]])
    _csv(write, [["__amd_rocclr_copyBuffer", "WRITE_SIZE", copy_kib],
                 ["void tcl::expand_kernel<8, 2, true>(tcl::ExpandArgs)", "WRITE_SIZE", 10.0]])
    out = bench.pmc_summary(str(fetch), str(write), "wl")
    e = out["entries"]["wl:plan_shrink"]
    assert e["fetch_factor"] == 2.0 and e["launches"] == 2
    assert e["fetch_bytes_per_launch"] == 200.0 * 1024 * 2
    x = out["entries"]["wl:expand_kernel"]
    assert x["write_bytes_per_launch"] == 10.0 * 1024 and x["hbm_bytes_per_launch"] == (50 * 2 + 10) * 1024
    assert x["source_hash"] == bench.kernel_source_hash("expand_kernel")


def test_pmc_summary_keeps_kernels_apart(bench, tmp_path):
    """Kernel names are matched as whole identifiers: the paired shrink is
    not counted as the plain one, and the two kernels of the token-tile
    expand keep their own entries, which the traffic lookup sums."""
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    copy_kib = (256 << 20) / 1024
    _csv(fetch, [["__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_kib],
                 ["void tcl::shrink_mfma<8>(tcl::ShrinkArgs)", "FETCH_SIZE", 1.0],
                 ["void tcl::shrink_mfma_pair<8>(tcl::ShrinkArgs)", "FETCH_SIZE", 4.0],
                 ["tcl::tile_prep(tcl::TileArgs)", "FETCH_SIZE", 2.0],
                 ["void tcl::expand_tile<tcl::bf16_t>(tcl::TileArgs)", "FETCH_SIZE", 8.0]])
    _csv(write, [["__amd_rocclr_copyBuffer", "WRITE_SIZE", copy_kib]])
    e = bench.pmc_summary(str(fetch), str(write), "wl")["entries"]
    assert e["wl:shrink_mfma"]["fetch_bytes_per_launch"] == 1024.0
    assert e["wl:shrink_mfma_pair"]["fetch_bytes_per_launch"] == 4096.0
    assert e["wl:tile_prep"]["source_hash"] == bench.kernel_source_hash("tile_prep")
    assert e["wl:expand_tile"]["fetch_bytes_per_launch"] == 8192.0


def test_stored_traffic_unknown_workload(bench):
    assert bench.stored_traffic("no_such_workload", "plan_shrink") is None


def test_producer_algorithmic_bytes():
    """Every factor read once and every output written once, bf16, plus
    sigma: for the Llama fleet at rank 16, 2 * 2.94 GB."""
    import bench
    classes = [(2240, 4096, 4096), (2240, 1024, 4096), (2240, 14336, 4096), (1120, 4096, 14336)]
    b, f = bench.producer_alg(classes, 16)
    per_adapter_layer = sum(d_in + d_out for _, d_in, d_out in
                            [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024),
                             ("o", 4096, 4096), ("g", 4096, 14336), ("u", 4096, 14336),
                             ("d", 14336, 4096)])
    n = 35 * 32
    assert b == n * per_adapter_layer * 16 * 2 * 2 + 7840 * 16 * 4
    assert f == sum(M * 4 * 16 * 16 * (d_out + d_in) for M, d_out, d_in in classes)


def test_scheduler_replay_library_matches_oracle():
    """The scheduler leg's replay gives the same loads through the library
    and through the oracle on a short stream."""
    import bench
    import oracle as O
    from tenant_composite_lora_amd import tclora

    class LibPool:
        def __init__(self, S):
            self.b = tclora.Bam(S)

        def resident(self):
            return [a for a in self.b.slots().tolist() if a >= 0]

        def acquire(self, batch):
            return len(self.b.acquire(batch)[1])

    class OraclePool:
        def __init__(self, S):
            self.S, self.batches = S, []

        def resident(self):
            return [a for a in O.bam_run(self.S, self.batches)[1] if a >= 0]

        def acquire(self, batch):
            self.batches.append(batch)
            return len(O.bam_run(self.S, self.batches)[0][-1][2])

    stream = bench.sched_stream(3, 12, A=40, per_step=8, burst=30)
    for theta in (4.0, float("-inf")):
        lib_loads, _ = bench.sched_replay(stream, tclora.lag_select, LibPool, theta, 8, 16)
        ora_loads, _ = bench.sched_replay(stream, O.lag_select, OraclePool, theta, 8, 16)
        assert lib_loads == ora_loads


def test_cpu_baseline_uses_the_cores_it_names():
    """The oracle baseline splits the batch over worker processes and
    reports their count; every token is covered once per repetition."""
    import bench
    wl = W.random_case(5, T=40, N=6, d_in=64, d_out=32, r_max=8, max_pairs=3)
    out = bench.cpu_baseline(wl, budget_s=0.2, cores=3)
    assert out["cores"] == 3 and out["kind"] == "oracle" and out["value"] > 0
    assert "3 contiguous token ranges" in out["sample"]


def test_kernel_names_follow_dispatch(bench):
    """The bench names the kernels the library's dispatch picks: the paired
    prefill shrink from 1024 pair jobs on, the token-tile expand for
    prefill-sized bf16 batches."""
    k4 = bench.kernel_names(W.make(4), False)
    assert k4["shrink"] == "shrink_mfma" and k4["expand"] == "tile_prep+expand_tile"
    small = W.random_case(1, T=40, N=8, d_in=32, d_out=32, r_max=8, max_pairs=2)
    k = bench.kernel_names(small, True)
    assert k["shrink"] == "plan_shrink" and k["expand"] == "expand_kernel"
