"""The library's rank-allocation policies (host code, LoRAForge approach
(2)) against the oracle's: the kept ranks are integers decided by fp64
comparisons both sides make the same way, so they must match exactly."""
import numpy as np
import pytest

import oracle as O
from tenant_composite_lora_amd import tclora


def _instance(rng, M, r_max, tie=False):
    ranks = rng.integers(0, r_max + 1, M).astype(np.int32)
    costs = rng.integers(1, 50, M).astype(np.int64)
    floors = rng.integers(0, 3, M).astype(np.int32)
    sig = np.zeros((M, r_max))
    for m in range(M):
        s = np.sort(rng.random(ranks[m]))[::-1]
        if tie and ranks[m] > 1:
            s[1] = s[0]
        sig[m, :ranks[m]] = s
    return sig, ranks, costs, floors


@pytest.mark.parametrize("seed", range(12))
def test_spectral_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    M, r_max = int(rng.integers(1, 60)), int(rng.integers(1, 33))
    sig, ranks, costs, floors = _instance(rng, M, r_max, tie=seed % 3 == 0)
    if seed % 4 == 1:  # equal costs: many equal eta
        costs[:] = 7
    total = int(sum(int(ranks[m]) * int(costs[m]) for m in range(M)))
    for budget in (0, total // 7, total // 2, total, total + 5):
        k = tclora.rank_spectral(sig, ranks, costs, floors, budget)
        ko = O.spectral_ranks([sig[m, :ranks[m]] for m in range(M)], costs, budget, floors)
        assert k.tolist() == ko.tolist(), (seed, budget)


def test_spectral_fleet_sized():
    """7840 modules of rank 16 (the Llama fleet), budget from LoRAForge-U at
    d = 12, floor 1."""
    rng = np.random.default_rng(5)
    M, r = 7840, 16
    sig = np.sort(rng.random((M, r)) ** 3, axis=1)[:, ::-1].copy()
    costs = np.array([8192, 5120, 5120, 8192, 18432, 18432, 18432] * (M // 7), dtype=np.int64)
    ranks = np.full(M, r, np.int32)
    u, budget = tclora.rank_uniform(ranks, costs, 12)
    uo = O.uniform_ranks(ranks, 12)
    assert u.tolist() == uo.tolist() and budget == O.uniform_budget(ranks, costs, 12)
    k = tclora.rank_spectral(sig, ranks, costs, np.ones(M, np.int32), budget)
    ko = O.spectral_ranks(list(sig), costs, budget, [1] * M)
    assert k.tolist() == ko.tolist()
    assert int((k * costs).sum()) <= budget


def test_uniform_matches_oracle():
    ranks = np.array([16, 8, 12, 4, 24, 0, 64], np.int32)
    costs = np.array([10, 3, 7, 9, 2, 5, 100], np.int64)
    for d in (1, 3, 8, 12, 100):
        u, b = tclora.rank_uniform(ranks, costs, d)
        assert u.tolist() == O.uniform_ranks(ranks, d).tolist()
        assert b == O.uniform_budget(ranks, costs, d)


def test_rank_host_errors():
    sig = np.ones((2, 3))
    ok = dict(ranks=[3, 3], costs=[1, 1], floors=[0, 0], budget=5)
    tclora.rank_spectral(sig, **ok)
    for bad in (dict(ranks=[4, 3]), dict(ranks=[-1, 3]), dict(costs=[0, 1]),
                dict(floors=[-1, 0])):
        a = dict(ok, **bad)
        with pytest.raises(RuntimeError):
            tclora.rank_spectral(sig, **a)
    s2 = sig.copy()
    s2[1, 2] = np.nan
    with pytest.raises(RuntimeError):
        tclora.rank_spectral(s2, **ok)
    s2[1, 2] = -1.0
    with pytest.raises(RuntimeError):
        tclora.rank_spectral(s2, **ok)

    with pytest.raises(RuntimeError):
        tclora.rank_uniform([4], [1], 0)
    with pytest.raises(RuntimeError):
        tclora.rank_uniform([4], [0], 2)


def test_factor_host_errors():
    L = tclora.lib()
    import ctypes
    nb = ctypes.c_size_t()
    assert L.tcl_factor_workspace_bytes(10, 4096, 4096, 16, ctypes.byref(nb)) == tclora.OK
    assert nb.value > 0
    assert L.tcl_factor_workspace_bytes(10, 4096, 4096, 33, ctypes.byref(nb)) == tclora.EUNSUPPORTED
    assert L.tcl_factor_workspace_bytes(10, 4096, 4095, 16, ctypes.byref(nb)) == tclora.EALIGN
    assert L.tcl_factor_workspace_bytes(10, 4095, 4096, 16, ctypes.byref(nb)) == tclora.EALIGN
    assert L.tcl_factor_workspace_bytes(-1, 4096, 4096, 16, ctypes.byref(nb)) == tclora.EINVAL
    assert L.tcl_factor_workspace_bytes(70000, 64, 64, 16, ctypes.byref(nb)) == tclora.EINVAL
    assert L.tcl_factor_workspace_bytes(1, 64, 64, 16, None) == tclora.EINVAL
    # no modules: nothing to launch, NULL data allowed
    assert L.tcl_factor_balanced(None, None, 0, 64, 64, 8, None, None, None, None, 0, None) == tclora.OK
    # NULL pointers and a short workspace are caught on the host
    assert L.tcl_factor_balanced(None, None, 2, 64, 64, 8, None, None, None, None, 0, None) == tclora.EINVAL
    buf = (ctypes.c_char * 4096)()
    p = ctypes.addressof(buf)
    p16 = (p + 15) & ~15
    assert L.tcl_factor_balanced(p16, p16, 2, 64, 64, 8, p16, p16, p16, p16, 16, None) == tclora.ENOSPC
    assert L.tcl_factor_balanced(p16, p16 + 2, 2, 64, 64, 8, p16, p16, p16, p16, 1 << 20, None) == tclora.EALIGN
