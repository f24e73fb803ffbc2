"""tcl_gate_topk (the token-level gate on the GPU) against the fp64 oracle's
gate, then the gated table through the whole step against the oracle apply.

The kept adapters, their order and the table's pointer arrays are integers:
they must match bit for bit (the selection compares the fp32 logits both
sides are given, so no rounding decides it).  The weights are an fp32
softmax against the oracle's fp64 one: relative error at most 2e-6 (the
exponentials are within about 2 ulp, and the pairwise sum of at most 64 of
them adds at most 6 roundings, about 4e-7 relative).
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import make_module, rel_err, to_dev
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W
from test_gpu_parity import TOL, banner

pytestmark = pytest.mark.gpu


def _inputs(seed, T, C, n_adapters=100, pad_frac=0.0, tie_frac=0.0, short_frac=0.0,
            bad_frac=0.0):
    """fp32 logits and int32 candidates [T, C]: random candidate lists,
    padding (-1) at random places, some tokens with tied logits, some with
    fewer valid candidates than 2, some with a NaN or infinite logit."""
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, C)).astype(np.float32)
    cd = np.stack([rng.permutation(n_adapters)[:C] for _ in range(T)]).astype(np.int32)
    cd[rng.random((T, C)) < pad_frac] = -1
    for t in np.nonzero(rng.random(T) < tie_frac)[0]:
        lg[t, rng.integers(0, C, 3)] = lg[t].max()
    for t in np.nonzero(rng.random(T) < short_frac)[0]:
        cd[t, 1:] = -1
    for t in np.nonzero(rng.random(T) < bad_frac)[0]:
        lg[t, rng.integers(0, C)] = [np.nan, np.inf, -np.inf][int(rng.integers(0, 3))]
    return lg, cd


def _gate(lg, cd, k):
    out = tclora.gate_topk(to_dev(lg), to_dev(cd), k)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def _check(lg, cd, k):
    gtp, gpp, pa, pw = _gate(lg, cd, k)
    ogtp, ogpp, opa, opw = O.gate_topk(lg.astype(np.float64), cd, k)
    assert np.array_equal(gtp, ogtp) and np.array_equal(gpp, ogpp)
    assert np.array_equal(pa, opa), np.nonzero(pa != opa)[0][:8]
    kept = opa >= 0
    assert np.all(pw[~kept] == 0)
    err = np.abs(pw[kept].astype(np.float64) - opw[kept]) / np.maximum(opw[kept], 1e-30)
    assert np.all(err <= 2e-6), float(err.max())
    return pa, pw


CASES = {
    "sparse_prefill_like": dict(seed=1, T=2048, C=8, k=2),
    "padding": dict(seed=2, T=500, C=8, k=2, pad_frac=0.3),
    "ties": dict(seed=3, T=300, C=8, k=3, tie_frac=0.5),
    "short_and_bad": dict(seed=4, T=400, C=6, k=2, short_frac=0.1, bad_frac=0.1),
    "short_only": dict(seed=9, T=300, C=6, k=3, short_frac=0.3, pad_frac=0.2),
    "full_wave": dict(seed=5, T=130, C=64, k=64),
    "one_candidate": dict(seed=6, T=77, C=1, k=1),
    "k_equals_C_with_padding": dict(seed=7, T=200, C=5, k=5, pad_frac=0.2),
    "single_token": dict(seed=8, T=1, C=8, k=2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gate_vs_oracle(name):
    a = dict(CASES[name])
    k = a.pop("k")
    banner(f"gate {name}: {a} k={k}")
    seed, T, C = a.pop("seed"), a.pop("T"), a.pop("C")
    lg, cd = _inputs(seed, T, C, **a)
    _check(lg, cd, k)


def test_gate_no_tokens():
    banner("gate with no tokens")
    lg = np.zeros((0, 4), np.float32)
    cd = np.zeros((0, 4), np.int32)
    gtp, gpp, pa, pw = _gate(lg, cd, 2)
    assert gtp.tolist() == [0] and gpp.tolist() == [0] and pa.size == 0 and pw.size == 0


def test_gate_reproduces_sparse_prefill_table():
    """The 8 x 256 sparse-prefill workload's gate inputs give its composite
    table: the same adapters, weights within an fp32 softmax of the
    workload's (fp64, then rounded) ones."""
    wl = W.make(4)
    m = wl.meta
    lg = m["gate_logits"].astype(np.float32)
    banner("gate on the sparse-prefill workload's logits")
    pa, pw = _check(lg, m["gate_candidates"], m["gate_k"])
    c = wl.composites
    # rounding the fp64 logits to fp32 may swap two nearly equal logits;
    # the draws here have none
    assert np.array_equal(pa, c.pair_adapter)
    assert np.max(np.abs(pw - c.pair_alpha) / c.pair_alpha) <= 2e-6


@pytest.mark.parametrize("T", [40, 300])
def test_gated_step_vs_oracle(T):
    """Gate -> mapping stage -> shrink -> expand in device memory, against the
    oracle apply of the oracle gate's table.  Some tokens have one valid
    candidate (a one-pair list) and some none (an empty composite, left
    unchanged): the table ends before its arrays do.  40 tokens run the
    decode step (mapping inside the shrink launch), 300 the prefill path."""
    rng = np.random.default_rng(11)
    N, C, k = 64, 8, 2
    wl = W.random_case(12, T=T, N=N, d_in=256, d_out=264, r_max=16, max_pairs=2)
    refs = [rng.choice(N, int(rng.integers(5, 9)), replace=False) for _ in range(3)]
    cd = np.full((T, C), -1, np.int32)
    for t in range(T):
        r = refs[t * 3 // T]
        cd[t, :len(r)] = r
    short = rng.choice(T, T // 8, replace=False)
    cd[short[: len(short) // 2], 1:] = -1          # one valid candidate
    cd[short[len(short) // 2:], :] = -1            # none
    lg = rng.standard_normal((T, C)).astype(np.float32)
    banner(f"gated step: T={T} N={N}, {len(short)} short or empty tokens")
    gtp, gpp, pa, pw = tclora.gate_topk(to_dev(lg), to_dev(cd), k)
    plan = tclora.Plan(gtp, gpp, pa, pw, N, n_tokens=T, max_tuples=T * k)
    mod = make_module(wl.modules[0])
    x = to_dev(wl.x[0])
    y = to_dev(wl.y_base[0])
    call = tclora.FusedCall(plan, [mod], [x], [y])
    call.remap_apply(gtp, gpp, pa, pw, T)
    torch.cuda.synchronize()
    ogtp, ogpp, opa, opw = O.gate_topk(lg.astype(np.float64), cd, k)
    assert int(ogpp[-1]) < T * k
    rc, P, U = plan.status()
    assert rc == 0 and P == int(ogpp[-1])
    m = wl.modules[0]
    y_ora, d_ora = O.apply(ogtp, ogpp, opa, opw.astype(np.float32), m.A_t, m.B_t, m.k, wl.x[0],
                           wl.y_base[0])
    got = y.double().cpu().numpy()
    err = rel_err(got - wl.y_base[0].astype(np.float64), d_ora)
    print(f"  rel {err:.3e}", flush=True)
    assert err <= TOL[wl.dtype]
    empty = short[len(short) // 2:]
    assert np.array_equal(got[empty], wl.y_base[0][empty].astype(np.float64))


def test_gated_table_with_a_nonfinite_logit_is_rejected():
    """A token with a NaN logit lists adapter -1, which the mapping stage
    rejects; the step leaves y untouched."""
    T, C, k, N = 40, 4, 2, 16
    lg = np.random.default_rng(13).standard_normal((T, C)).astype(np.float32)
    cd = np.tile(np.arange(C, dtype=np.int32), (T, 1))
    lg[17, 2] = np.nan
    banner("gated table with a NaN logit")
    gtp, gpp, pa, pw = tclora.gate_topk(to_dev(lg), to_dev(cd), k)
    plan = tclora.Plan(gtp, gpp, pa, pw, N, n_tokens=T, max_tuples=T * k)
    assert plan.status()[0] == tclora.EINVAL
    m = W.random_case(1, T=T, N=N, d_in=64, d_out=64, r_max=4, max_pairs=1).modules[0]
    mod = make_module(m)
    x = torch.randn(T, 64, device="cuda:0").to(torch.bfloat16)
    y = torch.randn(T, 64, device="cuda:0")
    y0 = y.clone()
    call = tclora.FusedCall(plan, [mod], [x], [y])
    call.remap_apply(gtp, gpp, pa, pw, T)
    torch.cuda.synchronize()
    assert plan.status()[0] == tclora.EINVAL
    assert torch.equal(y, y0)


def test_gated_step_in_a_graph():
    """Gate, mapping stage and apply captured in one HIP graph: every replay
    gives the eager result bit for bit (outputs poisoned between replays)."""
    rng = np.random.default_rng(17)
    N, T, C, k = 48, 96, 6, 2
    wl = W.random_case(18, T=T, N=N, d_in=256, d_out=264, r_max=8, max_pairs=2)
    cd = np.stack([rng.permutation(N)[:C] for _ in range(T)]).astype(np.int32)
    lg_d = to_dev(rng.standard_normal((T, C)).astype(np.float32))
    cd_d = to_dev(cd)
    banner(f"gated step in a graph: T={T} N={N}")
    gtp, gpp, pa, pw = tclora.gate_topk(lg_d, cd_d, k)
    plan = tclora.Plan(gtp, gpp, pa, pw, N, n_tokens=T, max_tuples=T * k)
    mod = make_module(wl.modules[0])
    x = to_dev(wl.x[0])
    yb = to_dev(wl.y_base[0])
    y = yb.clone()
    call = tclora.FusedCall(plan, [mod], [x], [y])
    L = tclora.lib()

    def step(st):
        sp = int(st.cuda_stream)
        tclora.check(L.tcl_gate_topk(lg_d.data_ptr(), C, cd_d.data_ptr(), C, T, C, k,
                                     gtp.data_ptr(), gpp.data_ptr(), pa.data_ptr(),
                                     pw.data_ptr(), sp))
        call.remap_apply(gtp, gpp, pa, pw, T, stream=st)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y.copy_(yb)
        step(s)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        y.copy_(yb)
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        pa.fill_(-7)
        pw.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), rep
