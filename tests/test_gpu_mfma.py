"""The matrix-core prefill expand (tile union along K, alpha * z in bf16)
against the fp64 oracle, forced with TCL_DISPATCH=mfma.

The cases drive every control path of the kernel: several union windows (more
than 128 touched segments in a tile), several coefficient chunks (unions
beyond 128 rank rows), rank-64 adapters and zero-rank adapters, ragged token
tiles and column tiles, tokens without pairs, split-K partial z rows, a z
row stride that is not a multiple of 4 (the public expand), bf16 y, several
modules in one launch, and a rejected plan.  Padding rows at or beyond an
adapter's retained rank are filled with NaN in one case, so a read of any of
them would show in the result.
"""
import numpy as np
import pytest
import torch

from gpu_util import make_module, make_plan, rel_err, run_fused, to_dev
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W
from test_gpu_parity import CASES, TOL, banner, oracle_apply

pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC0)

MFMA_CASES = {
    # more than 128 segments touched by one 64-token tile: two union windows
    "mx_windows": lambda: W.random_case(150, T=320, N=700, d_in=64, d_out=264, r_max=8,
                                        max_pairs=12),
    # rank-64 adapters with retained ranks in [0, 64]: up to 8 octets each,
    # unions of several chunks
    "mx_rank64": lambda: W.random_case(151, T=260, N=24, d_in=128, d_out=520, r_max=64,
                                       max_pairs=6, with_k=True),
    # half the tokens without pairs, ragged last tile and column tile
    "mx_empty": lambda: W.random_case(152, T=290, N=16, d_in=96, d_out=136, r_max=16,
                                      max_pairs=3, empty_frac=0.5),
    # requests of 64 tokens sharing one composite (dense unions)
    "mx_requests": lambda: W.random_case(153, T=384, N=30, d_in=256, d_out=1032, r_max=16,
                                         max_pairs=6, tokens_per_group=64, with_k=True),
}


def _mixed_case():
    """Four dense tiles (requests of 64 tokens sharing 3 adapters) then four
    sparse ones (1-4 random adapters of 400 per token), over two modules of
    different ranks: the auto dispatch splits the batch between the two
    expands, per module."""
    N, T = 400, 512
    wl = W.random_case(155, T=T, N=N, d_in=128, d_out=520, r_max=16, max_pairs=4, with_k=True)
    w2 = W.random_case(156, T=T, N=N, d_in=64, d_out=264, r_max=32, max_pairs=4, with_k=True)
    rng = np.random.default_rng(155)
    ads = []
    for t in range(T):
        if t < 256:
            ads.append([(t // 64) * 7 + j for j in range(3)])
        else:
            ads.append(rng.choice(N, int(rng.integers(1, 5)), replace=False).tolist())
    als = [rng.random(len(a)).astype(np.float32).tolist() for a in ads]
    wl.composites = W.csr_from_token_lists(ads, als, N)
    wl.modules.append(w2.modules[0])
    wl.x.append(w2.x[0])
    wl.y_base.append(w2.y_base[0])
    return wl


MFMA_CASES["mx_mixed"] = _mixed_case


def _case(name):
    return MFMA_CASES[name]() if name in MFMA_CASES else CASES[name]()


def _pairs_per_token(c):
    tl = np.diff(c.group_tok_ptr.astype(np.int64))
    pl = np.diff(c.group_pair_ptr.astype(np.int64))
    return np.repeat(pl, tl)


def _check(wl, ys, label):
    for mi in range(len(wl.modules)):
        _, d_ora = oracle_apply(wl, mi)
        base = wl.y_base[mi].astype(np.float64)
        err = rel_err(ys[mi] - base, d_ora)
        print(f"  {label} module {mi}: rel {err:.3e}", flush=True)
        assert np.all(np.isfinite(ys[mi]))
        assert err <= TOL[wl.dtype], (mi, err)
        # tokens without pairs keep y bit for bit
        idle = np.nonzero(_pairs_per_token(wl.composites) == 0)[0]
        assert np.array_equal(ys[mi][idle], wl.y_base[mi][idle].astype(np.float64))


def _mfma(monkeypatch, kchunk=None):
    monkeypatch.setenv("TCL_DISPATCH", "mfma")
    if kchunk is None:
        monkeypatch.delenv("TCL_KCHUNK", raising=False)
    else:
        monkeypatch.setenv("TCL_KCHUNK", str(kchunk))


@pytest.mark.parametrize("name", ["config4", "mfma_ragged", "mfma_ranks24", "mfma_static",
                                  "mfma_many_adapters", "one_adapter_300_tokens"]
                         + sorted(MFMA_CASES))
def test_mfma_expand_vs_oracle(name, monkeypatch):
    wl = _case(name)
    banner(f"mfma expand {name}: T={wl.n_tokens} N={wl.n_adapters} "
           f"P={wl.composites.n_tuples()}")
    _mfma(monkeypatch)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, "mfma")


@pytest.mark.parametrize("name", ["mfma_ranks24", "mx_rank64", "mx_requests"])
def test_mfma_expand_split_k(name, monkeypatch):
    """Partial z rows of a shrink split into 64-element chunks of d_in."""
    wl = _case(name)
    banner(f"mfma expand with split-K partials {name}")
    _mfma(monkeypatch, kchunk=64)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, "mfma split-K")


@pytest.mark.parametrize("name", ["mx_mixed", "config4", "mfma_many_adapters", "mx_requests"])
@pytest.mark.parametrize("min_tok", [None, "1", "64"])
def test_auto_dispatch(name, min_tok, monkeypatch):
    """Default dispatch: the matrix-core expand takes the dense tiles, the
    per-token expand the others (threshold forced both ways too)."""
    wl = _case(name)
    banner(f"auto dispatch {name}, min_tok {min_tok}")
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    monkeypatch.delenv("TCL_KCHUNK", raising=False)
    if min_tok is None:
        monkeypatch.delenv("TCL_MFMA_MIN_TOK", raising=False)
    else:
        monkeypatch.setenv("TCL_MFMA_MIN_TOK", min_tok)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, "auto")


def test_mfma_expand_bf16_y(monkeypatch):
    wl = _case("mfma_ragged")
    banner("mfma expand with bf16 y")
    yb16 = W.f32_to_bf16_bits(wl.y_base[0])
    wl2 = W.Workload(wl.name, wl.dtype, wl.n_adapters, wl.composites, wl.modules, wl.x,
                     [W.bf16_bits_to_f32(yb16)])
    _mfma(monkeypatch)
    ys, _, _ = run_fused(wl2, y_dtype=torch.bfloat16)
    _, d_ora = oracle_apply(wl2, 0)
    y_ora = W.bf16_bits_to_f32(yb16).astype(np.float64) + d_ora
    bound = np.abs(y_ora) * 2.0 ** -8 + 1e-2 * np.max(np.abs(d_ora))
    assert np.all(np.abs(ys[0] - y_ora) <= bound)


@pytest.mark.parametrize("dispatch", ["valu", "mfma"])
def test_padding_rows_never_read(dispatch, monkeypatch):
    """Rank rows at or beyond k hold NaN in both pools; neither the shrink nor
    either expand may read them."""
    wl = _case("mx_rank64")
    m = wl.modules[0]
    pad = (np.arange(m.r_max)[None, :] >= m.k[:, None])[:, :, None]
    m.A_t = np.where(pad, BF16_NAN, m.A_t).astype(np.uint16)
    m.B_t = np.where(pad, BF16_NAN, m.B_t).astype(np.uint16)
    banner(f"NaN in padding rows, {dispatch} expand")
    monkeypatch.setenv("TCL_DISPATCH", dispatch)
    monkeypatch.delenv("TCL_KCHUNK", raising=False)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, dispatch)


def test_mfma_public_expand_odd_rank(monkeypatch):
    """tcl_shrink + tcl_expand: z rows of r_max = 6 floats (not a multiple of 4)."""
    wl = W.random_case(154, T=270, N=12, d_in=128, d_out=392, r_max=6, max_pairs=4,
                       with_k=True)
    banner("mfma public expand, r_max 6")
    plan = make_plan(wl.composites)
    mod = make_module(wl.modules[0])
    z = tclora.shrink(plan, mod, to_dev(wl.x[0]))
    _mfma(monkeypatch)
    y = to_dev(wl.y_base[0])
    tclora.expand(plan, mod, z, y)
    torch.cuda.synchronize()
    _check(wl, [y.double().cpu().numpy()], "public")


def test_mfma_rejected_plan_is_noop(monkeypatch):
    """A composite table the device validation rejects leaves y untouched."""
    T, N = 300, 4
    tp = np.arange(T + 1, dtype=np.int32)
    ad = np.zeros(T, np.int32)
    ad[123] = N  # adapter id out of range
    c = W.Composites(T, N, tp, tp.copy(), ad, np.ones(T, np.float32))
    banner("mfma expand after a rejected plan")
    plan = make_plan(c, max_tuples=T)
    assert plan.status()[0] != 0
    m = W.random_case(1, T=T, N=N, d_in=64, d_out=128, r_max=8, max_pairs=1).modules[0]
    mod = make_module(m)
    _mfma(monkeypatch)
    x = torch.randn(T, 64, device="cuda:0").to(torch.bfloat16)
    y = torch.randn(T, 128, device="cuda:0")
    y0 = y.clone()
    tclora.fused_apply(plan, [mod], [x], [y])
    torch.cuda.synchronize()
    assert torch.equal(y, y0)


@pytest.mark.parametrize("name", ["config4", "mx_windows", "mx_mixed", "mx_empty",
                                  "mfma_many_adapters", "mx_requests"])
@pytest.mark.parametrize("dispatch", [None, "mfma"])
def test_tile_ranges_from_token_index(name, dispatch, monkeypatch):
    """Per-tile tuple ranges and totals from the token index (the default for
    pools of up to 4096 adapters) against the binary searches over each
    segment (TCL_RANGES_TOK=0): y bit for bit, under the automatic dispatch
    (which splits tiles by the totals) and with every tile on the matrix
    cores."""
    wl = _case(name)
    banner(f"tile ranges from the token index {name}, dispatch {dispatch}")
    monkeypatch.delenv("TCL_KCHUNK", raising=False)
    if dispatch is None:
        monkeypatch.delenv("TCL_DISPATCH", raising=False)
    else:
        monkeypatch.setenv("TCL_DISPATCH", dispatch)
    monkeypatch.setenv("TCL_RANGES_TOK", "0")
    ys0, _, _ = run_fused(wl)
    monkeypatch.delenv("TCL_RANGES_TOK", raising=False)
    ys1, _, _ = run_fused(wl)
    for a, b in zip(ys0, ys1):
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
    _check(wl, ys1, "ranges")
