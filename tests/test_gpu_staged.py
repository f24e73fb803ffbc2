"""The staged expand (a token tile's B rows staged once in LDS) against the
per-token expand and the fp64 oracle.

Both expands do the same fp32 operations in the same order for every output
(alpha * z, one fma per rank in rank order, slots in slot order, y added
once), so their results must agree bit for bit; both must also be within the
bf16 tolerance of the oracle.  The stress cases force every control path of
the staged kernel: several passes over a tile (more tuples than the
coefficient buffer holds), several staging chunks (rank-64 adapters),
several segment windows (more than 256 touched adapters), zero-rank
segments, ragged tiles and column slices, split-K partial z and bf16 y.
"""
import numpy as np
import pytest
import torch

from gpu_util import make_module, make_plan, rel_err, run_fused, to_dev
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W
from test_gpu_parity import CASES, TOL, banner, oracle_apply

pytestmark = pytest.mark.gpu


def _all_pairs_case(seed, T, N, r_max, d_in, d_out):
    """Every token carries every adapter (N <= 64 pairs per token)."""
    wl = W.random_case(seed, T=T, N=N, d_in=d_in, d_out=d_out, r_max=r_max, max_pairs=1,
                       with_k=True)
    rng = np.random.default_rng(seed)
    ads = [rng.permutation(N).tolist() for _ in range(T)]
    als = [rng.random(N).astype(np.float32).tolist() for _ in range(T)]
    wl.composites = W.csr_from_token_lists(ads, als, N)
    return wl


STRESS = {
    # R = 32 holds 128 tuples per pass: 2 tokens of 64 slots each per pass
    "st_passes": lambda: _all_pairs_case(140, T=64, N=64, r_max=32, d_in=64, d_out=264),
    # rank-64 rows, zero-rank adapters, two tiles (the second ragged)
    "st_chunks": lambda: W.random_case(141, T=96, N=48, d_in=128, d_out=512, r_max=64,
                                       max_pairs=12, with_k=True),
    # several hundred touched adapters: more than one window of segments
    "st_windows": lambda: W.random_case(142, T=200, N=900, d_in=64, d_out=128, r_max=8,
                                        max_pairs=8),
    # requests of 64 tokens sharing one composite
    "st_requests": lambda: W.random_case(143, T=192, N=30, d_in=256, d_out=392, r_max=16,
                                         max_pairs=6, tokens_per_group=64, with_k=True),
}

BITWISE_CASES = ["config2", "config3", "config4", "ragged_tiles", "static_groups",
                 "empty_tokens", "ranks_with_zero", "rank_40", "rank_5", "mfma_ranks24",
                 "mfma_many_adapters", "64_pairs_per_token", "one_adapter_300_tokens",
                 "all_adapters"] + sorted(STRESS)


def _case(name):
    return STRESS[name]() if name in STRESS else CASES[name]()


def _run(wl, monkeypatch, dispatch, scpl=None, y_dtype=torch.float32, kchunk=None):
    monkeypatch.setenv("TCL_DISPATCH", dispatch)
    if scpl is not None:
        monkeypatch.setenv("TCL_SCPL", str(scpl))
    else:
        monkeypatch.delenv("TCL_SCPL", raising=False)
    if kchunk is not None:
        monkeypatch.setenv("TCL_KCHUNK", str(kchunk))
    else:
        monkeypatch.delenv("TCL_KCHUNK", raising=False)
    ys, _, _ = run_fused(wl, y_dtype=y_dtype)
    return ys


@pytest.mark.parametrize("name", BITWISE_CASES)
@pytest.mark.parametrize("scpl", [1, 2])
def test_staged_bitwise_equals_per_token(name, scpl, monkeypatch):
    wl = _case(name)
    if wl.dtype != W.BF16:
        pytest.skip("the staged expand serves bf16 pools")
    banner(f"staged (cpl {scpl}) vs per-token expand {name}: T={wl.n_tokens} "
           f"N={wl.n_adapters} P={wl.composites.n_tuples()}")
    ref = _run(wl, monkeypatch, "valu")
    got = _run(wl, monkeypatch, "staged", scpl=scpl)
    for mi in range(len(wl.modules)):
        _, d_ora = oracle_apply(wl, mi)
        base = wl.y_base[mi].astype(np.float64)
        err = rel_err(got[mi] - base, d_ora)
        print(f"  module {mi}: rel {err:.3e}", flush=True)
        assert err <= TOL[wl.dtype]
        bad = np.nonzero(got[mi] != ref[mi])
        assert bad[0].size == 0, (mi, bad[0][:5], bad[1][:5])


@pytest.mark.parametrize("name", ["config3", "st_chunks", "st_requests"])
def test_staged_split_k(name, monkeypatch):
    """Split-K partial z rows (the shrink cut into 64-element chunks of d_in)
    summed by the staged expand exactly as by the per-token expand."""
    wl = _case(name)
    banner(f"staged vs per-token with split-K partials {name}")
    ref = _run(wl, monkeypatch, "valu", kchunk=64 if wl.modules[0].d_in <= 1024 else 512)
    got = _run(wl, monkeypatch, "staged", kchunk=64 if wl.modules[0].d_in <= 1024 else 512)
    for mi in range(len(wl.modules)):
        _, d_ora = oracle_apply(wl, mi)
        base = wl.y_base[mi].astype(np.float64)
        assert rel_err(got[mi] - base, d_ora) <= TOL[wl.dtype]
        assert np.array_equal(got[mi], ref[mi]), mi


def test_staged_bf16_output(monkeypatch):
    wl = _case("st_requests")
    banner("staged expand with bf16 y")
    yb16 = W.f32_to_bf16_bits(wl.y_base[0])
    wl2 = W.Workload(wl.name, wl.dtype, wl.n_adapters, wl.composites, wl.modules, wl.x,
                     [W.bf16_bits_to_f32(yb16)])
    for scpl in (1, 2):
        ref = _run(wl2, monkeypatch, "valu", y_dtype=torch.bfloat16)
        got = _run(wl2, monkeypatch, "staged", scpl=scpl, y_dtype=torch.bfloat16)
        assert np.array_equal(got[0], ref[0]), scpl
    _, d_ora = oracle_apply(wl2, 0)
    y_ora = W.bf16_bits_to_f32(yb16).astype(np.float64) + d_ora
    bound = np.abs(y_ora) * 2.0 ** -8 + 1e-2 * np.max(np.abs(d_ora))
    assert np.all(np.abs(got[0] - y_ora) <= bound)


def test_staged_public_expand(monkeypatch):
    """tcl_expand (single module, caller's z) takes the staged kernel too."""
    wl = _case("st_chunks")
    banner("tcl_shrink + tcl_expand, staged vs per-token")
    plan = make_plan(wl.composites)
    mod = make_module(wl.modules[0])
    x = to_dev(wl.x[0])
    z = tclora.shrink(plan, mod, x)
    out = {}
    for disp in ("valu", "staged"):
        monkeypatch.setenv("TCL_DISPATCH", disp)
        y = to_dev(wl.y_base[0])
        tclora.expand(plan, mod, z, y)
        torch.cuda.synchronize()
        out[disp] = y.double().cpu().numpy()
    assert np.array_equal(out["valu"], out["staged"])


def test_staged_rejected_plan_is_noop(monkeypatch):
    """A composite table the device validation rejects leaves y untouched."""
    T, N = 64, 4
    tp = np.arange(T + 1, dtype=np.int32)
    pp = np.arange(T + 1, dtype=np.int32)
    ad = np.zeros(T, np.int32)
    ad[7] = N  # adapter id out of range
    c = W.Composites(T, N, tp, pp, ad, np.ones(T, np.float32))
    banner("staged expand after a rejected plan")
    plan = make_plan(c, max_tuples=T)
    assert plan.status()[0] != 0
    m = W.random_case(1, T=T, N=N, d_in=64, d_out=128, r_max=8, max_pairs=1).modules[0]
    mod = make_module(m)
    monkeypatch.setenv("TCL_DISPATCH", "staged")
    x = torch.randn(T, 64, device="cuda:0").to(torch.bfloat16)
    y = torch.randn(T, 128, device="cuda:0")
    y0 = y.clone()
    tclora.fused_apply(plan, [mod], [x], [y])
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
