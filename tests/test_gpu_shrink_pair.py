"""The item-pair shrink (TCL_SHRINK_PAIR=1): one workgroup job takes two
consecutive work items and shares the A-row loads when both belong to one
adapter.  Its z must be bit for bit that of the one-item shrink (same K steps
per accumulator, same wave order in the sum), through the public shrink (final
z rows, zero tail) and through the fused apply (split-K partial rows too), and
the applied y must meet the oracle's tolerance.

Cases: segments of many items (requests sharing adapters), segments of one
item next to each other (many adapters), rank-64 adapters with retained ranks
in [0, 64] (rank tiles past the retained rank), a ragged last item, tokens
without pairs, an odd item count, and NaN in every padding row.
"""
import numpy as np
import pytest
import torch

from gpu_util import make_module, make_plan, run_fused, run_split
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W
from test_gpu_tile import BF16_NAN, MFMA_CASES, _check
from test_gpu_parity import CASES, banner

pytestmark = pytest.mark.gpu

NAMES = ["config4", "mfma_ranks24", "mfma_many_adapters", "one_adapter_300_tokens",
         "mx_rank64", "mx_empty", "mx_requests", "mx_mixed"]


def _case(name):
    return MFMA_CASES[name]() if name in MFMA_CASES else CASES[name]()


def _mode(monkeypatch, pair, steps=None, kchunk=None):
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    if pair:
        monkeypatch.setenv("TCL_SHRINK_PAIR", "1")
    else:
        monkeypatch.setenv("TCL_SHRINK_PAIR", "0")
    if steps is None:
        monkeypatch.delenv("TCL_PSTEPS", raising=False)
    else:
        monkeypatch.setenv("TCL_PSTEPS", str(steps))
    if kchunk is None:
        monkeypatch.delenv("TCL_KCHUNK", raising=False)
    else:
        monkeypatch.setenv("TCL_KCHUNK", str(kchunk))


@pytest.mark.parametrize("steps", [4, 8])
@pytest.mark.parametrize("name", NAMES)
def test_pair_public_shrink_bitwise(name, steps, monkeypatch):
    wl = _case(name)
    banner(f"item-pair public shrink {name}, {steps} steps: T={wl.n_tokens} "
           f"N={wl.n_adapters} P={wl.composites.n_tuples()}")
    for mi in range(len(wl.modules)):
        _mode(monkeypatch, False)
        y0, z0, _ = run_split(wl, mi)
        _mode(monkeypatch, True, steps)
        y1, z1, _ = run_split(wl, mi)
        assert np.array_equal(z0.view(np.uint64), z1.view(np.uint64)), mi
        assert np.array_equal(y0.view(np.uint64), y1.view(np.uint64)), mi


@pytest.mark.parametrize("kchunk", [None, 64])
@pytest.mark.parametrize("name", NAMES)
def test_pair_fused_vs_oracle(name, kchunk, monkeypatch):
    wl = _case(name)
    banner(f"item-pair fused apply {name}, kchunk {kchunk}")
    _mode(monkeypatch, False, kchunk=kchunk)
    ys0, _, _ = run_fused(wl)
    _mode(monkeypatch, True, kchunk=kchunk)
    ys1, _, _ = run_fused(wl)
    for a, b in zip(ys0, ys1):
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
    _check(wl, ys1, "pair")


def test_pair_padding_rows_never_read(monkeypatch):
    """Rank rows at or beyond k hold NaN in A; the pair shrink may not read them."""
    wl = _case("mx_rank64")
    m = wl.modules[0]
    pad = (np.arange(m.r_max)[None, :] >= m.k[:, None])[:, :, None]
    m.A_t = np.where(pad, BF16_NAN, m.A_t).astype(np.uint16)
    m.B_t = np.where(pad, BF16_NAN, m.B_t).astype(np.uint16)
    banner("item-pair shrink, NaN in padding rows")
    _mode(monkeypatch, True)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, "pair")


def test_pair_rejected_plan_is_noop(monkeypatch):
    """A table the mapping stage rejects has no work items: y stays as it was."""
    T, N = 300, 4
    tp = np.arange(T + 1, dtype=np.int32)
    ad = np.zeros(T, np.int32)
    ad[77] = N  # adapter id out of range
    c = W.Composites(T, N, tp, tp.copy(), ad, np.ones(T, np.float32))
    banner("item-pair shrink after a rejected plan")
    plan = make_plan(c, max_tuples=T)
    assert plan.status()[0] != 0
    m = W.random_case(2, T=T, N=N, d_in=64, d_out=128, r_max=8, max_pairs=1).modules[0]
    mod = make_module(m)
    _mode(monkeypatch, True)
    x = torch.randn(T, 64, device="cuda:0").to(torch.bfloat16)
    y = torch.randn(T, 128, device="cuda:0")
    y0 = y.clone()
    tclora.fused_apply(plan, [mod], [x], [y])
    torch.cuda.synchronize()
    assert torch.equal(y, y0)


def test_pair_retained_rank_full_size_bitwise(monkeypatch):
    """The full retained-rank batch, where the default dispatch takes item
    pairs: the step's y equals that of the one-item shrink bit for bit."""
    from test_gpu_parity import cfg
    wl = cfg(5)
    banner("item-pair shrink, retained-rank batch at full size, auto vs one-item")
    _mode(monkeypatch, False)
    ys0, _, _ = run_fused(wl)
    monkeypatch.delenv("TCL_SHRINK_PAIR", raising=False)
    ys1, _, _ = run_fused(wl)
    for a, b in zip(ys0, ys1):
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


@pytest.mark.parametrize("pair", [False, True])
@pytest.mark.parametrize("name", ["mfma_ranks24", "mx_rank64", "mx_mixed"])
def test_rank_tile_pairs_bitwise(name, pair, monkeypatch):
    """Both 16-rank tiles of an item in one job (the default when a module
    keeps more than 16 ranks: one x load feeds two accumulators) against one
    tile a job: z and y bit for bit through the public shrink (zero tail) and
    the fused apply (split-K partial rows too)."""
    wl = _case(name)
    assert max(m.r_max for m in wl.modules) > 16
    banner(f"rank-tile pairs {name}, item pairs {pair}: ranks {[m.r_max for m in wl.modules]}")
    for mi in range(len(wl.modules)):
        _mode(monkeypatch, pair)
        monkeypatch.setenv("TCL_SHRINK_RT", "1")
        y0, z0, _ = run_split(wl, mi)
        monkeypatch.delenv("TCL_SHRINK_RT")
        y1, z1, _ = run_split(wl, mi)
        assert np.array_equal(z0.view(np.uint64), z1.view(np.uint64)), mi
        assert np.array_equal(y0.view(np.uint64), y1.view(np.uint64)), mi
    for kchunk in (None, 64):
        _mode(monkeypatch, pair, kchunk=kchunk)
        monkeypatch.setenv("TCL_SHRINK_RT", "1")
        ys0, _, _ = run_fused(wl)
        monkeypatch.delenv("TCL_SHRINK_RT")
        ys1, _, _ = run_fused(wl)
        for a, b in zip(ys0, ys1):
            assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
    _check(wl, ys1, "rank-tile pairs")
