"""A whole step (mapping stage + fused apply) captured in a HIP graph and
replayed: every replay gives the eager result bit for bit.

The prefill cases run the split expand, whose two halves run on the
caller's stream and on the library's second stream joined by events; the
graph must hold both.  Between replays the outputs are overwritten with NaN
and an unrelated eager apply runs, so a replay that skipped or reused work
would show.
"""
import numpy as np
import pytest
import torch

from gpu_util import composites_to_dev, make_module, to_dev
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W
from test_gpu_tile import MFMA_CASES
from test_gpu_parity import CASES, banner

pytestmark = pytest.mark.gpu


def _case(name):
    return MFMA_CASES[name]() if name in MFMA_CASES else CASES[name]()


@pytest.mark.parametrize("name", ["config2", "config3", "config4", "mx_mixed",
                                  "mfma_many_adapters"])
@pytest.mark.parametrize("one_call", [False, True])
def test_graph_replays_match_eager(name, one_call, monkeypatch):
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    monkeypatch.delenv("TCL_KCHUNK", raising=False)
    monkeypatch.delenv("TCL_FUSED_MAPPING", raising=False)
    wl = _case(name)
    c = wl.composites
    banner(f"graph replay {name} ({'tcl_remap_apply' if one_call else 'remap + apply'}): "
           f"T={wl.n_tokens} P={c.n_tuples()}")
    gtp, gpp, pa, pw = composites_to_dev(c)
    plan = tclora.Plan(gtp, gpp, pa, pw, c.n_adapters, n_tokens=c.n_tokens,
                       max_tuples=c.n_tuples())
    mods = [make_module(m) for m in wl.modules]
    xs = [to_dev(x) for x in wl.x]
    ybs = [to_dev(y) for y in wl.y_base]
    ys = [y.clone() for y in ybs]
    call = tclora.FusedCall(plan, mods, xs, ys)
    # an unrelated batch run eagerly between replays
    other = W.random_case(7, T=24, N=c.n_adapters, d_in=wl.modules[0].d_in,
                          d_out=wl.modules[0].d_out, r_max=wl.modules[0].r_max, max_pairs=3)
    o_gtp, o_gpp, o_pa, o_pw = composites_to_dev(other.composites)
    o_plan = tclora.Plan(o_gtp, o_gpp, o_pa, o_pw, c.n_adapters, n_tokens=24,
                         max_tuples=other.composites.n_tuples())
    o_y = torch.zeros(24, wl.modules[0].d_out, device="cuda:0")
    o_x = to_dev(other.x[0])

    def step(st):
        if one_call:
            call.remap_apply(gtp, gpp, pa, pw, c.n_tokens, stream=st)
        else:
            plan.remap(gtp, gpp, pa, pw, c.n_tokens, stream=st)
            call(st)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for y, yb in zip(ys, ybs):
            y.copy_(yb)
        step(s)
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        cs = torch.cuda.current_stream()
        for y, yb in zip(ys, ybs):
            y.copy_(yb)
        step(cs)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        tclora.fused_apply(o_plan, [mods[0]], [o_x], [o_y])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for mi, (y, r) in enumerate(zip(ys, ref)):
            bad = torch.nonzero(y != r)
            assert bad.numel() == 0, (rep, mi, bad[:5].tolist())
    assert np.all(np.isfinite(o_y.cpu().numpy()))


def _permuted_table(c, seed):
    """The same group structure with every adapter id sent through one
    permutation of the pool: a table of the same sizes whose segments (and so
    its per-tile tuple ranges) differ."""
    perm = np.random.default_rng(seed).permutation(c.n_adapters).astype(np.int32)
    return W.Composites(c.n_tokens, c.n_adapters, c.group_tok_ptr.copy(),
                        c.group_pair_ptr.copy(), perm[c.pair_adapter], c.pair_alpha.copy())


def _oracle_check(wl, c, ys, label):
    import oracle as O
    from gpu_util import rel_err
    for mi, m in enumerate(wl.modules):
        _, delta = O.apply(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                           m.A_t, m.B_t, m.k, wl.x[mi], wl.y_base[mi])
        got = ys[mi].double().cpu().numpy() - wl.y_base[mi]
        rel = rel_err(got, delta)
        assert rel <= 1e-2, (label, mi, rel)


@pytest.mark.parametrize("name", ["mx_mixed", "mfma_many_adapters"])
def test_apply_graph_sees_later_remap(name, monkeypatch):
    """An apply-only graph captured after an eager apply, replayed after an
    eager remap to a different table of the same sizes, applies the new table:
    the per-tile tuple ranges the matrix-core expand reads are written by
    every mapping launch, not once per plan."""
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    monkeypatch.delenv("TCL_FUSED_MAPPING", raising=False)
    wl = _case(name)
    c0 = wl.composites
    c1 = _permuted_table(c0, 5)
    banner(f"apply-only graph after a remap {name}: T={wl.n_tokens} P={c0.n_tuples()}")
    t0 = composites_to_dev(c0)
    t1 = composites_to_dev(c1)
    plan = tclora.Plan(*t0, c0.n_adapters, n_tokens=c0.n_tokens, max_tuples=c0.n_tuples())
    mods = [make_module(m) for m in wl.modules]
    xs = [to_dev(x) for x in wl.x]
    ybs = [to_dev(y) for y in wl.y_base]
    ys = [y.clone() for y in ybs]
    call = tclora.FusedCall(plan, mods, xs, ys)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(s)                      # eager apply of table 0
    torch.cuda.synchronize()
    _oracle_check(wl, c0, ys, "eager table 0")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        cs = torch.cuda.current_stream()
        for y, yb in zip(ys, ybs):
            y.copy_(yb)
        call(cs)
    torch.cuda.synchronize()
    for rep, (tab, c) in enumerate([(t1, c1), (t0, c0), (t1, c1)]):
        with torch.cuda.stream(s):
            plan.remap(*tab, c.n_tokens, stream=s)   # eager remap, then replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _oracle_check(wl, c, ys, f"replay {rep}")


def test_eager_apply_before_first_replay(monkeypatch):
    """A graph captured on a fresh plan, then an eager apply before any
    replay: the eager apply reads tile ranges the mapping launch wrote."""
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    wl = _case("mx_mixed")
    c = wl.composites
    banner(f"eager apply before the first replay: T={wl.n_tokens}")
    tab = composites_to_dev(c)
    plan = tclora.Plan(*tab, c.n_adapters, n_tokens=c.n_tokens, max_tuples=c.n_tuples())
    mods = [make_module(m) for m in wl.modules]
    xs = [to_dev(x) for x in wl.x]
    ybs = [to_dev(y) for y in wl.y_base]
    ys = [y.clone() for y in ybs]
    call = tclora.FusedCall(plan, mods, xs, ys)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        cs = torch.cuda.current_stream()
        for y, yb in zip(ys, ybs):
            y.copy_(yb)
        call(cs)
    torch.cuda.synchronize()
    for y, yb in zip(ys, ybs):
        y.copy_(yb)
    with torch.cuda.stream(s):
        call(s)
    torch.cuda.synchronize()
    _oracle_check(wl, c, ys, "eager")
    g.replay()
    torch.cuda.synchronize()
    _oracle_check(wl, c, ys, "replay")
