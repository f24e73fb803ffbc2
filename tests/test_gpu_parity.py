"""GPU path (through the C ABI) against the fp64 oracle.

Mapping: bit-exact.  Apply: rel = max|D_gpu - D_oracle| / max|D_oracle| on
D = y - y_base, <= 1e-2 in bf16 mode and <= 1e-5 in fp32 mode; z from the
shrink alone against the oracle's z with the same bounds.  Every case prints
its name before it touches the GPU.
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (composites_to_dev, make_module, make_plan, rel_err, run_fused, run_split,
                      to_dev)
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.BF16: 1e-2, W.F32: 1e-5}


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


@functools.lru_cache(maxsize=None)
def cfg(i):
    return W.make(i)


def oracle_plan(c):
    return O.plan(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha)


def oracle_apply(wl, mi, k="module"):
    c, m = wl.composites, wl.modules[mi]
    kk = m.k if isinstance(k, str) else k
    return O.apply(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                   m.A_t, m.B_t, kk, wl.x[mi], wl.y_base[mi])


def assert_plan_equal(got, want):
    for key in want:
        g, w = np.asarray(got[key]), np.asarray(want[key])
        if key == "tup_alpha":
            g, w = g.view(np.uint32), w.astype(np.float32).view(np.uint32)
        assert g.shape == w.shape, (key, g.shape, w.shape)
        assert np.array_equal(g, w), (key, np.nonzero(g != w)[0][:10])


EDGE_CASES = {
    "ragged_tiles": dict(seed=101, T=37, N=11, d_in=1000, d_out=520, r_max=8, max_pairs=4),
    "static_groups": dict(seed=102, T=45, N=9, d_in=256, d_out=264, r_max=16, max_pairs=5,
                          tokens_per_group=7),
    "empty_tokens": dict(seed=103, T=29, N=6, d_in=128, d_out=136, r_max=8, max_pairs=3,
                         empty_frac=0.4),
    "ranks_with_zero": dict(seed=104, T=33, N=10, d_in=512, d_out=512, r_max=12, max_pairs=4,
                            with_k=True),
    "rank_40": dict(seed=105, T=21, N=5, d_in=264, d_out=200, r_max=40, max_pairs=3,
                    with_k=True),
    "rank_64_f32": dict(seed=106, T=19, N=4, d_in=96, d_out=104, r_max=64, max_pairs=4,
                        dtype=W.F32),
    "single_token": dict(seed=107, T=1, N=3, d_in=64, d_out=64, r_max=8, max_pairs=3),
    "rank_5": dict(seed=108, T=50, N=7, d_in=72, d_out=80, r_max=5, max_pairs=7),
    # prefill-sized batches take the matrix-core expand (>= 256 tokens)
    "mfma_ragged": dict(seed=130, T=300, N=20, d_in=520, d_out=520, r_max=8, max_pairs=4,
                        empty_frac=0.1),
    "mfma_ranks24": dict(seed=131, T=333, N=40, d_in=256, d_out=776, r_max=24, max_pairs=5,
                         with_k=True),
    "mfma_static": dict(seed=132, T=512, N=12, d_in=128, d_out=256, r_max=16, max_pairs=6,
                        tokens_per_group=37),
    "mfma_many_adapters": dict(seed=133, T=256, N=600, d_in=64, d_out=264, r_max=8,
                               max_pairs=8),
    # mapping-stage modes: more pairs than the one-workgroup direct path holds
    # (multi-workgroup), more adapters or more groups than the multi path
    # takes (one-workgroup counting sort)
    "multi_ragged": dict(seed=134, T=700, N=90, d_in=64, d_out=72, r_max=8, max_pairs=5,
                         empty_frac=0.05),
    "count_5000_adapters": dict(seed=135, T=600, N=5000, d_in=64, d_out=64, r_max=4,
                                max_pairs=3),
    "count_9000_groups": dict(seed=136, T=9000, N=64, d_in=32, d_out=32, r_max=4, max_pairs=2),
    # direct-mode tables with more groups than the mapping workgroup has
    # threads (mostly empty tokens): the general direct path, not the
    # one-thread-per-group one
    "direct_400_groups": dict(seed=137, T=400, N=20, d_in=64, d_out=72, r_max=4, max_pairs=2,
                              empty_frac=0.75),
    "direct_1500_groups": dict(seed=138, T=1500, N=30, d_in=64, d_out=72, r_max=4,
                               max_pairs=2, empty_frac=0.8),
}


def edge(name):
    return W.random_case(**EDGE_CASES[name])


def one_adapter_case():
    wl = W.random_case(109, T=300, N=4, d_in=256, d_out=256, r_max=8, max_pairs=1)
    c = W.csr_from_token_lists([[2]] * 300, [[0.5]] * 300, 4)
    wl.composites = c
    return wl


def all_adapters_case():
    N = 40
    rng = np.random.default_rng(110)
    wl = W.random_case(110, T=40, N=N, d_in=128, d_out=128, r_max=8, max_pairs=1)
    ads = [[int(a)] for a in rng.permutation(N)]
    wl.composites = W.csr_from_token_lists(ads, [[1.0]] * N, N)
    return wl


def max_pairs_case():
    N = 64
    wl = W.random_case(111, T=6, N=N, d_in=64, d_out=64, r_max=4, max_pairs=1)
    rng = np.random.default_rng(111)
    ads = [rng.permutation(N).tolist() for _ in range(6)]
    als = [rng.random(N).astype(np.float32).tolist() for _ in range(6)]
    wl.composites = W.csr_from_token_lists(ads, als, N)
    return wl


def all_cases():
    cases = {f"config{i}": (lambda i=i: cfg(i)) for i in (1, 2, 3, 4)}
    cases.update({n: (lambda n=n: edge(n)) for n in EDGE_CASES})
    cases["one_adapter_300_tokens"] = one_adapter_case
    cases["all_adapters"] = all_adapters_case
    cases["64_pairs_per_token"] = max_pairs_case
    return cases


CASES = all_cases()


# ---------------------------------------------------------------------------
# mapping stage
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", sorted(CASES))
def test_plan_bit_exact(name):
    wl = CASES[name]()
    banner(f"plan {name}: T={wl.n_tokens} pairs={wl.composites.n_pairs} "
           f"P={wl.composites.n_tuples()}")
    plan = make_plan(wl.composites)
    assert_plan_equal(plan.copy_out(), oracle_plan(wl.composites))


def _with_tail(c, extra=7, seed=0):
    """The same table with pair arrays longer than its pairs: entries past
    group_pair_ptr[G] hold ids out of range, repeats and NaN weights, which
    are unused capacity and must not be read."""
    rng = np.random.default_rng(seed)
    bad = rng.choice([-5, c.n_adapters, 10 ** 6, 0], extra).astype(np.int32)
    return W.Composites(c.n_tokens, c.n_adapters, c.group_tok_ptr, c.group_pair_ptr,
                        np.concatenate([c.pair_adapter.astype(np.int32), bad]),
                        np.concatenate([c.pair_alpha.astype(np.float32),
                                        np.full(extra, np.nan, np.float32)]))


TAIL_CASES = ["config2", "config3", "config4", "direct_400_groups", "direct_1500_groups",
              "count_5000_adapters", "count_9000_groups", "empty_tokens", "64_pairs_per_token"]


@pytest.mark.parametrize("name", TAIL_CASES)
def test_plan_ignores_unused_pair_capacity(name):
    """Every mapping mode reads the table's pairs only (those below
    group_pair_ptr[G]): with a tail of invalid entries the plan is the
    oracle's plan of the table, bit for bit."""
    wl = CASES[name]()
    ct = _with_tail(wl.composites)
    banner(f"plan with unused pair capacity {name}: pairs {wl.composites.n_pairs} "
           f"of {ct.n_pairs}")
    plan = make_plan(ct)
    assert plan.status()[0] == 0
    assert_plan_equal(plan.copy_out(), oracle_plan(wl.composites))


@pytest.mark.parametrize("name", ["config2", "config3", "config4"])
def test_step_ignores_unused_pair_capacity(name):
    """The whole step (tcl_remap_apply: the decode configs map inside the
    shrink launch) over a table with unused pair capacity, against the
    oracle apply of the table."""
    wl = CASES[name]()
    ct = _with_tail(wl.composites, seed=1)
    banner(f"step with unused pair capacity {name}")
    plan = make_plan(ct)
    mods = [make_module(m) for m in wl.modules]
    xs = [to_dev(x) for x in wl.x]
    ys = [to_dev(y) for y in wl.y_base]
    call = tclora.FusedCall(plan, mods, xs, ys)
    gtp, gpp, pa, pw = composites_to_dev(ct)
    call.remap_apply(gtp, gpp, pa, pw, ct.n_tokens)
    torch.cuda.synchronize()
    assert plan.status()[0] == 0
    for mi in range(len(wl.modules)):
        _, d_ora = oracle_apply(wl, mi)
        err = rel_err(ys[mi].double().cpu().numpy() - wl.y_base[mi].astype(np.float64), d_ora)
        print(f"  module {mi}: rel {err:.3e}", flush=True)
        assert err <= TOL[wl.dtype]


def test_plan_config5_bit_exact():
    c = cfg(5).composites
    banner(f"plan config5: T={c.n_tokens} P={c.n_tuples()}")
    assert_plan_equal(make_plan(c).copy_out(), oracle_plan(c))


def test_plan_capacity_slack():
    """A capacity larger than the tuple count changes nothing."""
    c = cfg(3).composites
    banner("plan config3 with capacity 4x")
    plan = make_plan(c, max_tuples=4 * c.n_tuples())
    assert_plan_equal(plan.copy_out(), oracle_plan(c))


def test_plan_empty_batch():
    banner("plan empty batch")
    c = W.csr_from_token_lists([], [], 5)
    plan = make_plan(c)
    rc, P, U = plan.status()
    assert (rc, P, U) == (0, 0, 0)
    c = W.csr_from_token_lists([[]] * 7, [[]] * 7, 5)
    plan = make_plan(c)
    out = plan.copy_out()
    assert out["tok_ptr"].tolist() == [0] * 8 and out["tup_token"].size == 0


def _bad_tables():
    good = ([0, 1, 3], [0, 2, 3], [0, 1, 3], [0.5, 0.5, 1.0])
    return {
        "tokens_mismatch": ([0, 1, 2], [0, 2, 3], [0, 1, 3], [.5, .5, 1.], 3, None),
        "decreasing": ([0, 2, 1, 3], [0, 1, 2, 3], [0, 1, 3], [.5, .5, 1.], 3, None),
        "adapter_oob": ([0, 1, 3], [0, 2, 3], [0, 4, 3], [.5, .5, 1.], 3, None),
        "adapter_neg": ([0, 1, 3], [0, 2, 3], [0, -1, 3], [.5, .5, 1.], 3, None),
        "duplicate": ([0, 1, 3], [0, 2, 3], [1, 1, 3], [.5, .5, 1.], 3, None),
        "nan_alpha": ([0, 1, 3], [0, 2, 3], [0, 1, 3], [.5, np.nan, 1.], 3, None),
        "inf_alpha": ([0, 1, 3], [0, 2, 3], [0, 1, 3], [.5, np.inf, 1.], 3, None),
        "over_capacity": good + (3, 3),
        "fits_capacity": good + (3, 4),
        "too_many_pairs": ([0, 1], [0, 65], list(range(65)), [1.0] * 65, 1, None),
        "too_many_pairs_with_dup": ([0, 1], [0, 65], list(range(64)) + [5], [1.0] * 65, 1,
                                    None),
        "too_many_pairs_and_bad_id": ([0, 1, 2], [0, 65, 66], list(range(65)) + [90],
                                      [1.0] * 66, 2, None),
    }


def _bad_large_tables():
    """Tables of a few hundred groups (the multi-workgroup mapping path) with
    one defect each; (group_tok_ptr, group_pair_ptr, adapters, alphas, T, N,
    max_tuples)."""
    base = W.random_case(150, T=400, N=50, d_in=16, d_out=16, r_max=4, max_pairs=4).composites
    gt, gp = base.group_tok_ptr.astype(np.int64), base.group_pair_ptr.astype(np.int64)
    ad, al = base.pair_adapter.astype(np.int64), base.pair_alpha.astype(np.float32)
    T, N, NP = base.n_tokens, base.n_adapters, base.n_pairs
    mid = NP // 2
    out = {}
    out["ok"] = (gt, gp, ad, al, T, N, None)
    a2 = ad.copy(); a2[mid] = N
    out["bad_id"] = (gt, gp, a2, al, T, N, None)
    w2 = al.copy(); w2[NP - 1] = np.nan
    out["nan_alpha"] = (gt, gp, ad, w2, T, N, None)
    g = int(np.searchsorted(gp, mid, side="right")) - 1
    while gp[g + 1] - gp[g] < 2:
        g += 1
    a3 = ad.copy(); a3[gp[g] + 1] = a3[gp[g]]
    out["duplicate"] = (gt, gp, a3, al, T, N, None)
    # one group of 70 pairs (beyond the limit) right before a group with a
    # repeated adapter: EINVAL outranks EUNSUPPORTED
    big = list(range(70))
    gp4 = np.concatenate([[0, 70], 70 + gp[1:]]).astype(np.int64)
    gt4 = np.concatenate([[0, 1], 1 + gt[1:]]).astype(np.int64)
    a4 = np.concatenate([big, a3]).astype(np.int64)
    w4 = np.concatenate([np.ones(70, np.float32), al]).astype(np.float32)
    out["oversized_then_dup"] = (gt4, gp4, a4, w4, T + 1, 80, None)
    out["oversized_only"] = (gt4, gp4, np.concatenate([big, ad]).astype(np.int64), w4, T + 1,
                             80, None)
    # the repeated adapter in the group right after the oversized one (the
    # same workgroup of the multi path)
    g1 = 0
    while gp[g1 + 1] - gp[g1] < 2:
        g1 += 1
    a6 = ad.copy(); a6[gp[g1] + 1] = a6[gp[g1]]
    out["oversized_dup_same_block"] = (gt4, gp4, np.concatenate([big, a6]).astype(np.int64), w4,
                                       T + 1, 80, None)
    out["over_capacity"] = (gt, gp, ad, al, T, N, base.n_tuples() - 1)
    gt5 = gt.copy(); gt5[200], gt5[201] = gt5[201], gt5[200]
    out["decreasing_tokens"] = (gt5, gp, ad, al, T, N, None)
    return out


@pytest.mark.parametrize("name", sorted(_bad_large_tables()))
def test_plan_multi_validation(name):
    tp, pp, ad, al, T, N, cap = _bad_large_tables()[name]
    want = O.validate(tp, pp, ad.astype(np.int32), al, T, N, max_tuples=cap)
    banner(f"multi-workgroup validation {name}: pairs={len(ad)} expect {want}")
    c = W.Composites(T, N, tp.astype(np.int32), pp.astype(np.int32), ad.astype(np.int32),
                     al.astype(np.float32))
    n_tup = int(np.sum(np.diff(tp).clip(0) * np.diff(pp).clip(0)))
    plan = make_plan(c, max_tuples=cap if cap is not None else max(n_tup, 1))
    rc, _, _ = plan.status()
    assert rc == want
    if rc == 0:
        assert_plan_equal(plan.copy_out(), oracle_plan(c))
    else:
        # a rejected plan turns the apply into a no-op
        m = W.random_case(2, T=T, N=N, d_in=16, d_out=16, r_max=4, max_pairs=1).modules[0]
        mod = make_module(m)
        x = torch.randn(T, 16, device="cuda:0").to(torch.bfloat16)
        y = torch.randn(T, 16, device="cuda:0")
        y0 = y.clone()
        tclora.fused_apply(plan, [mod], [x], [y])
        torch.cuda.synchronize()
        assert torch.equal(y, y0)


def _pad_groups(tp, pp, n):
    """The same table with n empty groups (no tokens, no pairs) appended:
    more groups than the direct mapping workgroup has threads."""
    return list(tp) + [tp[-1]] * n, list(pp) + [pp[-1]] * n


@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("name", sorted(_bad_tables()))
def test_plan_device_validation(name, padded):
    tp, pp, ad, al, T, cap = _bad_tables()[name]
    if padded:
        tp, pp = _pad_groups(tp, pp, 1100)
    N = 80 if name.startswith("too_many_pairs") else 4
    want = O.validate(np.array(tp), np.array(pp), np.array(ad, np.int32),
                      np.array(al, np.float32), T, N, max_tuples=cap)
    banner(f"validation {name}: expect {want}")
    c = W.Composites(T, N, np.array(tp, np.int32), np.array(pp, np.int32),
                     np.array(ad, np.int32), np.array(al, np.float32))
    plan = make_plan(c, max_tuples=cap if cap is not None else 16)
    rc, _, _ = plan.status()
    assert rc == want
    if rc != 0:
        # a rejected plan turns the apply into a no-op
        m = W.random_case(1, T=T, N=N, d_in=16, d_out=16, r_max=4, max_pairs=1).modules[0]
        mod = make_module(m)
        x = torch.randn(T, 16, device="cuda:0").to(torch.bfloat16)
        y = torch.randn(T, 16, device="cuda:0")
        y0 = y.clone()
        tclora.fused_apply(plan, [mod], [x], [y])
        torch.cuda.synchronize()
        assert torch.equal(y, y0)


# ---------------------------------------------------------------------------
# the apply
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_apply_parity(name):
    wl = CASES[name]()
    banner(f"fused_apply {name}: modules={len(wl.modules)} T={wl.n_tokens}")
    ys, _, _ = run_fused(wl)
    for mi in range(len(wl.modules)):
        _, d_ora = oracle_apply(wl, mi)
        d_gpu = ys[mi] - wl.y_base[mi].astype(np.float64)
        err = rel_err(d_gpu, d_ora)
        print(f"  module {wl.modules[mi].name}: rel {err:.3e}", flush=True)
        assert err <= TOL[wl.dtype], (wl.modules[mi].name, err)
        # tokens with an empty composite are left untouched
        c = wl.composites
        owner = np.repeat(np.arange(c.n_groups), np.diff(c.group_tok_ptr))
        empty = np.diff(c.group_pair_ptr)[owner] == 0 if c.n_tokens else np.zeros(0, bool)
        assert np.array_equal(ys[mi][empty], wl.y_base[mi][empty].astype(np.float64))


@pytest.mark.parametrize("name", ["config2", "config3", "config4", "ranks_with_zero",
                                  "static_groups"])
def test_valu_shrink_on_bf16_pools(name, monkeypatch):
    """TCL_SHRINK=valu: the fp32 VALU shrink on bf16 pools (whole-d_in z rows,
    the mapping kernel apart from the shrink), against the oracle."""
    monkeypatch.setenv("TCL_SHRINK", "valu")
    wl = CASES[name]()
    banner(f"valu shrink {name}: modules={len(wl.modules)} T={wl.n_tokens}")
    ys, _, _ = run_fused(wl)
    for mi in range(len(wl.modules)):
        _, d_ora = oracle_apply(wl, mi)
        err = rel_err(ys[mi] - wl.y_base[mi].astype(np.float64), d_ora)
        print(f"  module {wl.modules[mi].name}: rel {err:.3e}", flush=True)
        assert err <= TOL[wl.dtype], (wl.modules[mi].name, err)


@pytest.mark.parametrize("name", ["config1", "config2", "ragged_tiles", "ranks_with_zero",
                                  "rank_64_f32", "static_groups"])
def test_shrink_expand_parity(name):
    wl = CASES[name]()
    banner(f"shrink+expand {name}")
    y, z, plan = run_split(wl)
    pl = oracle_plan(wl.composites)
    m = wl.modules[0]
    z_ora = O.shrink(pl, m.A_t, m.k, wl.x[0])
    P = z_ora.shape[0]
    zerr = rel_err(z[:P], z_ora)
    print(f"  z rel {zerr:.3e}", flush=True)
    assert zerr <= TOL[wl.dtype]
    if m.k is not None:  # rows beyond the effective rank are exactly zero
        for p in range(P):
            assert np.all(z[p, m.k[pl["tup_adapter"][p]]:] == 0)
    _, d_ora = oracle_apply(wl, 0)
    err = rel_err(y - wl.y_base[0].astype(np.float64), d_ora)
    print(f"  y rel {err:.3e}", flush=True)
    assert err <= TOL[wl.dtype]


def test_expand_alone_from_oracle_z():
    """tcl_expand fed the oracle's z (rounded to fp32) against the oracle's expand."""
    wl = cfg(2)
    banner("expand alone, config2")
    m = wl.modules[0]
    pl = oracle_plan(wl.composites)
    z = O.shrink(pl, m.A_t, m.k, wl.x[0]).astype(np.float32)
    plan = make_plan(wl.composites)
    mod = make_module(m)
    y = to_dev(wl.y_base[0])
    tclora.expand(plan, mod, to_dev(z), y)
    torch.cuda.synchronize()
    want = O.expand(pl, m.B_t, m.k, z, wl.y_base[0]) - wl.y_base[0]
    got = y.double().cpu().numpy() - wl.y_base[0]
    assert rel_err(got, want) <= 1e-5


def test_bf16_output():
    wl = cfg(2)
    banner("fused_apply config2 with bf16 y")
    yb16 = W.f32_to_bf16_bits(wl.y_base[0])
    ys, _, _ = run_fused(W.Workload(wl.name, wl.dtype, wl.n_adapters, wl.composites, wl.modules,
                                    wl.x, [W.bf16_bits_to_f32(yb16)]), y_dtype=torch.bfloat16)
    _, d_ora = oracle_apply(wl, 0)
    y_ora = W.bf16_bits_to_f32(yb16).astype(np.float64) + d_ora
    # one final rounding to bf16 (half an ulp) on top of the stated tolerance
    half_ulp = np.abs(y_ora) * 2.0 ** -8
    bound = half_ulp + 1e-2 * np.max(np.abs(d_ora))
    assert np.all(np.abs(ys[0] - y_ora) <= bound)


@pytest.mark.parametrize("name", ["config4", "mfma_ragged", "mfma_ranks24", "mfma_static"])
def test_prefill_paths_agree(name, monkeypatch):
    """The token-tile expand on the matrix cores and the per-token VALU expand
    on the same batch: both within tolerance of the oracle."""
    wl = CASES[name]()
    banner(f"valu vs tile expand {name}")
    monkeypatch.setenv("TCL_DISPATCH", "valu")
    a, _, _ = run_fused(wl)
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    b, _, _ = run_fused(wl)
    for mi in range(len(wl.modules)):
        _, d_ora = oracle_apply(wl, mi)
        base = wl.y_base[mi].astype(np.float64)
        ea, eb = rel_err(a[mi] - base, d_ora), rel_err(b[mi] - base, d_ora)
        print(f"  module {mi}: valu rel {ea:.3e}, tile rel {eb:.3e}", flush=True)
        assert ea <= TOL[wl.dtype] and eb <= TOL[wl.dtype]


def test_tile_bf16_output(monkeypatch):
    wl = edge("mfma_ragged")
    banner("tile expand with bf16 y")
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    yb16 = W.f32_to_bf16_bits(wl.y_base[0])
    wl2 = W.Workload(wl.name, wl.dtype, wl.n_adapters, wl.composites, wl.modules, wl.x,
                     [W.bf16_bits_to_f32(yb16)])
    ys, _, _ = run_fused(wl2, y_dtype=torch.bfloat16)
    _, d_ora = oracle_apply(wl2, 0)
    y_ora = W.bf16_bits_to_f32(yb16).astype(np.float64) + d_ora
    bound = np.abs(y_ora) * 2.0 ** -8 + 1e-2 * np.max(np.abs(d_ora))
    assert np.all(np.abs(ys[0] - y_ora) <= bound)


def test_config5_sampled():
    """Full-size retained-rank batch in the benchmark's launch configuration;
    the oracle computes 48 sampled tokens (all columns) one by one."""
    wl = cfg(5)
    banner("fused_apply config5 full size, sampled rows")
    ys, plan, _ = run_fused(wl)
    c = wl.composites
    rng = np.random.default_rng(5)
    rows = sorted(set(rng.choice(c.n_tokens, 40, replace=False).tolist()
                      + [0, 1, c.n_tokens - 1, 4095, 4096, 4097]))
    for mi, m in enumerate(wl.modules):
        want = O.apply_rows(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                            m.A_t, m.B_t, m.k, wl.x[mi], wl.y_base[mi], rows)
        base = wl.y_base[mi][rows].astype(np.float64)
        err = rel_err(ys[mi][rows] - base, want - base)
        print(f"  module {m.name}: rel {err:.3e} over {len(rows)} rows", flush=True)
        assert err <= TOL[wl.dtype]


# ---------------------------------------------------------------------------
# invariants (bitwise)
# ---------------------------------------------------------------------------

def test_deterministic():
    wl = cfg(3)
    banner("determinism config3")
    a, _, _ = run_fused(wl)
    b, _, _ = run_fused(wl)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_pair_permutation_invariance():
    wl = cfg(2)
    banner("pair permutation config2")
    c = wl.composites
    rng = np.random.default_rng(3)
    ad, al = c.pair_adapter.copy(), c.pair_alpha.copy()
    for g in range(c.n_groups):
        lo, hi = c.group_pair_ptr[g], c.group_pair_ptr[g + 1]
        perm = rng.permutation(hi - lo) + lo
        ad[lo:hi], al[lo:hi] = c.pair_adapter[perm], c.pair_alpha[perm]
    wl2 = W.Workload(wl.name, wl.dtype, wl.n_adapters,
                     W.Composites(c.n_tokens, c.n_adapters, c.group_tok_ptr, c.group_pair_ptr,
                                  ad, al), wl.modules, wl.x, wl.y_base)
    a, _, _ = run_fused(wl)
    b, _, _ = run_fused(wl2)
    assert np.array_equal(a[0], b[0])


def test_token_permutation():
    wl = cfg(1)
    banner("token permutation config1")
    c = wl.composites
    perm = np.random.default_rng(4).permutation(c.n_tokens)
    rows_a = [c.pair_adapter[c.group_pair_ptr[t]:c.group_pair_ptr[t + 1]].tolist() for t in perm]
    rows_w = [c.pair_alpha[c.group_pair_ptr[t]:c.group_pair_ptr[t + 1]].tolist() for t in perm]
    wl2 = W.Workload(wl.name, wl.dtype, wl.n_adapters,
                     W.csr_from_token_lists(rows_a, rows_w, c.n_adapters), wl.modules,
                     [wl.x[0][perm]], [wl.y_base[0][perm]])
    a, _, _ = run_fused(wl)
    b, _, _ = run_fused(wl2)
    assert np.array_equal(a[0][perm], b[0])


def test_alpha_zero_and_rank_zero_are_noops():
    wl = cfg(2)
    banner("alpha = 0 and k = 0 no-ops")
    c = wl.composites
    wl0 = W.Workload(wl.name, wl.dtype, wl.n_adapters,
                     W.Composites(c.n_tokens, c.n_adapters, c.group_tok_ptr, c.group_pair_ptr,
                                  c.pair_adapter, np.zeros_like(c.pair_alpha)),
                     wl.modules, wl.x, wl.y_base)
    ys, _, _ = run_fused(wl0)
    assert np.array_equal(ys[0], wl.y_base[0].astype(np.float64))
    ys, _, _ = run_fused(wl, k=np.zeros(wl.n_adapters, np.int32))
    assert np.array_equal(ys[0], wl.y_base[0].astype(np.float64))


def test_fused_halves_equal_fused_apply():
    """tcl_fused_shrink then tcl_fused_expand computes exactly tcl_fused_apply."""
    wl = cfg(3)
    banner("fused halves vs fused apply, config3")
    a, plan, mods = run_fused(wl)
    xs = [to_dev(x) for x in wl.x]
    ys = [to_dev(y) for y in wl.y_base]
    call = tclora.FusedCall(plan, mods, xs, ys)
    call.shrink()
    call.expand()
    torch.cuda.synchronize()
    for u, v in zip(a, ys):
        assert np.array_equal(u, v.double().cpu().numpy())


def test_retained_rank_equals_padded():
    """k_m on a zero-padded pool equals k = r_max on the same pool, bitwise."""
    wl = W.random_case(120, T=64, N=16, d_in=1024, d_out=768, r_max=32, max_pairs=4,
                       with_k=True)
    banner("retained rank vs padded, r_max 32")
    a, _, _ = run_fused(wl)
    b, _, _ = run_fused(wl, k=None)
    assert np.array_equal(a[0], b[0])
