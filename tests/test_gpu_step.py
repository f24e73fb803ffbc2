"""tcl_remap_apply and tcl_remap_shrink (one step: mapping stage + fused
apply) against the fp64 oracle.  Decode-sized bf16 batches run the mapping
stage inside the shrink launch (workgroup 0 maps the table in LDS and
writes the plan, the others map it up to their work items); the others run
the plain remap + fused apply.  The step must match the oracle to the stated tolerance, match the
separate calls bit for bit, leave y untouched for a table the mapping stage
rejects, and handle consecutive steps with different tables on one plan."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import composites_to_dev, make_module, rel_err, to_dev
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W
from test_gpu_parity import CASES, TOL, _bad_tables, _pad_groups, banner, oracle_apply

pytestmark = pytest.mark.gpu

STEP_CASES = ["config1", "config2", "config3", "ragged_tiles", "static_groups", "empty_tokens",
              "ranks_with_zero", "rank_40", "rank_5", "single_token", "all_adapters",
              "64_pairs_per_token", "rank_64_f32", "mfma_ragged", "direct_400_groups",
              "direct_1500_groups"]


def _step(wl, y_dtype=torch.float32, plan_wl=None):
    """Build a plan (on plan_wl's table if given), then one tcl_remap_apply
    with wl's table; returns y of every module as float64."""
    pw = plan_wl or wl
    c0 = pw.composites
    g0 = composites_to_dev(c0)
    cap = max(c0.n_tuples(), wl.composites.n_tuples(), 1)
    plan = tclora.Plan(*g0, c0.n_adapters, n_tokens=c0.n_tokens, max_tuples=cap)
    mods = [make_module(m) for m in wl.modules]
    xs = [to_dev(x) for x in wl.x]
    ys = [to_dev(y).to(y_dtype) for y in wl.y_base]
    call = tclora.FusedCall(plan, mods, xs, ys)
    c = wl.composites
    g = composites_to_dev(c)
    call.remap_apply(*g, c.n_tokens)
    torch.cuda.synchronize()
    return [y.to(torch.float64).cpu().numpy() for y in ys], plan


def _check(wl, ys):
    for mi in range(len(wl.modules)):
        _, d_ora = oracle_apply(wl, mi)
        err = rel_err(ys[mi] - wl.y_base[mi].astype(np.float64), d_ora)
        print(f"  module {mi}: rel {err:.3e}", flush=True)
        assert err <= TOL[wl.dtype], (mi, err)


@pytest.mark.parametrize("name", STEP_CASES)
def test_step_vs_oracle(name, monkeypatch):
    monkeypatch.delenv("TCL_FUSED_MAPPING", raising=False)
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    wl = CASES[name]()
    banner(f"remap_apply {name}: T={wl.n_tokens} P={wl.composites.n_tuples()}")
    ys, _ = _step(wl)
    _check(wl, ys)
    # tokens with an empty composite keep y bit for bit
    c = wl.composites
    owner = np.repeat(np.arange(c.n_groups), np.diff(c.group_tok_ptr))
    empty = np.diff(c.group_pair_ptr)[owner] == 0 if c.n_tokens else np.zeros(0, bool)
    for mi in range(len(wl.modules)):
        assert np.array_equal(ys[mi][empty], wl.y_base[mi][empty].astype(np.float64))


@pytest.mark.parametrize("name", ["config2", "config3", "static_groups", "64_pairs_per_token",
                                  "empty_tokens", "ranks_with_zero", "all_adapters",
                                  "direct_400_groups", "direct_1500_groups"])
def test_step_paths_agree(name, monkeypatch):
    """The mapping stage inside the shrink launch and the separate mapping
    kernel give the same plan and the same y, bit for bit."""
    wl = CASES[name]()
    banner(f"fused vs separate mapping stage {name}")
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    monkeypatch.delenv("TCL_FUSED_MAPPING", raising=False)
    a, pa = _step(wl)
    monkeypatch.setenv("TCL_FUSED_MAPPING", "0")
    b, pb = _step(wl)
    for mi in range(len(wl.modules)):
        assert np.array_equal(a[mi], b[mi]), mi
    ca, cb = pa.copy_out(), pb.copy_out()
    for k in ca:
        assert np.array_equal(np.asarray(ca[k]).view(np.uint32) if k == "tup_alpha" else ca[k],
                              np.asarray(cb[k]).view(np.uint32) if k == "tup_alpha" else cb[k]), k


@pytest.mark.parametrize("name,kchunk", [("config3", 512), ("config2", 512), ("config2", 1536)])
def test_step_split_k(name, kchunk, monkeypatch):
    """Partial z rows of the shrink: config 3's two-slot expand batches read
    them through scalar loads, config 2's four-slot batches through vector
    loads (8 chunks: four issued before the B rows, four after; 3 chunks:
    a ragged group)."""
    wl = CASES[name]()
    banner(f"remap_apply with split-K partials: {name}, {kchunk}-element chunks")
    monkeypatch.setenv("TCL_KCHUNK", str(kchunk))
    ys, _ = _step(wl)
    _check(wl, ys)


def test_step_bf16_y(monkeypatch):
    monkeypatch.delenv("TCL_FUSED_MAPPING", raising=False)
    wl = CASES["config2"]()
    banner("remap_apply with bf16 y")
    yb16 = W.f32_to_bf16_bits(wl.y_base[0])
    wl2 = W.Workload(wl.name, wl.dtype, wl.n_adapters, wl.composites, wl.modules, wl.x,
                     [W.bf16_bits_to_f32(yb16)])
    ys, _ = _step(wl2, y_dtype=torch.bfloat16)
    _, d_ora = oracle_apply(wl2, 0)
    y_ora = W.bf16_bits_to_f32(yb16).astype(np.float64) + d_ora
    bound = np.abs(y_ora) * 2.0 ** -8 + 1e-2 * np.max(np.abs(d_ora))
    assert np.all(np.abs(ys[0] - y_ora) <= bound)


def test_consecutive_steps_on_one_plan(monkeypatch):
    """Three steps with different tables (and token counts) on one plan and
    one workspace, both sized for the largest batch."""
    monkeypatch.delenv("TCL_FUSED_MAPPING", raising=False)
    N = 48
    wls = [W.random_case(160 + i, T=T, N=N, d_in=256, d_out=264, r_max=8, max_pairs=5)
           for i, T in enumerate((40, 17, 64))]
    for wl in wls:  # one adapter pool for every step
        wl.modules[0] = wls[0].modules[0]
    big = wls[2].composites
    cap = max(w.composites.n_tuples() for w in wls)
    plan = tclora.Plan(*composites_to_dev(big), N, n_tokens=big.n_tokens, max_tuples=cap)
    mod = make_module(wls[0].modules[0])
    ws = torch.empty(tclora.workspace_bytes(plan, [mod]), dtype=torch.uint8, device="cuda:0")
    for i, wl in enumerate(wls):
        banner(f"step {i}: T={wl.n_tokens}")
        x = to_dev(wl.x[0])
        y = to_dev(wl.y_base[0])
        call = tclora.FusedCall(plan, [mod], [x], [y], ws)
        c = wl.composites
        call.remap_apply(*composites_to_dev(c), c.n_tokens)
        torch.cuda.synchronize()
        _check(wl, [y.double().cpu().numpy()])


@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("name", sorted(_bad_tables()))
def test_step_rejected_table_is_noop(name, padded, monkeypatch):
    monkeypatch.delenv("TCL_FUSED_MAPPING", raising=False)
    tp, pp, ad, al, T, cap = _bad_tables()[name]
    if padded:
        tp, pp = _pad_groups(tp, pp, 1100)
    N = 80 if name.startswith("too_many_pairs") else 4
    want = O.validate(np.array(tp), np.array(pp), np.array(ad, np.int32),
                      np.array(al, np.float32), T, N, max_tuples=cap)
    banner(f"remap_apply on table {name}: expect {want}")
    bad = (torch.tensor(tp, dtype=torch.int32, device="cuda:0"),
           torch.tensor(pp, dtype=torch.int32, device="cuda:0"),
           torch.tensor(ad, dtype=torch.int32, device="cuda:0"),
           torch.tensor(al, dtype=torch.float32, device="cuda:0"))
    cap_ = cap if cap is not None else 80
    plan = tclora.Plan(*bad, N, n_tokens=T, max_tuples=cap_)
    m = W.random_case(1, T=T, N=N, d_in=64, d_out=64, r_max=4, max_pairs=1).modules[0]
    mod = make_module(m)
    x = torch.randn(T, 64, device="cuda:0").to(torch.bfloat16)
    y = torch.randn(T, 64, device="cuda:0")
    y0 = y.clone()
    call = tclora.FusedCall(plan, [mod], [x], [y])
    call.remap_apply(*bad, T)
    torch.cuda.synchronize()
    rc, _, _ = plan.status()
    assert rc == want
    if rc != 0:
        assert torch.equal(y, y0)


def test_step_halves(monkeypatch):
    """tcl_remap_shrink then tcl_fused_expand equals tcl_remap_apply."""
    monkeypatch.delenv("TCL_FUSED_MAPPING", raising=False)
    wl = CASES["config3"]()
    banner("remap_shrink + fused_expand")
    a, _ = _step(wl)
    c = wl.composites
    g = composites_to_dev(c)
    plan = tclora.Plan(*g, c.n_adapters, n_tokens=c.n_tokens, max_tuples=c.n_tuples())
    mods = [make_module(m) for m in wl.modules]
    call = tclora.FusedCall(plan, mods, [to_dev(x) for x in wl.x], [to_dev(y) for y in wl.y_base])
    call.remap_shrink(*g, c.n_tokens)
    call.expand()
    torch.cuda.synchronize()
    for mi, y in enumerate(call.ys):
        assert np.array_equal(y.double().cpu().numpy(), a[mi]), mi
