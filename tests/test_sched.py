"""The library's BAM slot pool and LAG batch choice (host code,
DyMerge-LoRA section 4) against the oracle's: every decision is integer
bookkeeping, so slots, loads, evictions and chosen requests must match
exactly."""
import numpy as np
import pytest

import oracle as O
from tenant_composite_lora_amd import tclora


@pytest.mark.parametrize("seed", range(10))
def test_bam_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    S, A = int(rng.integers(1, 9)), int(rng.integers(2, 30))
    batches = [list(int(a) for a in rng.integers(0, A, int(rng.integers(0, 7)))) for _ in range(80)]
    recs, final = O.bam_run(S, batches)
    bam = tclora.Bam(S)
    for t, (b, (st, where, loads)) in enumerate(zip(batches, recs)):
        if st != O.OK:
            with pytest.raises(tclora.TclError) as e:
                bam.acquire(b)
            assert e.value.code == tclora.ENOSPC
            continue
        slot_of, got = bam.acquire(b)
        assert got == loads, (seed, t)
        assert slot_of.tolist() == [where[a] for a in b], (seed, t)
    assert bam.slots().tolist() == final


@pytest.mark.parametrize("seed", range(12))
def test_lag_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    n, A = int(rng.integers(0, 60)), int(rng.integers(1, 40))
    arr = list(np.round(rng.random(n) * 20, 1))  # ties in arrival are common
    ads = [list(int(a) for a in rng.integers(0, A, int(rng.integers(0, 5)))) for _ in range(n)]
    res = list(set(int(a) for a in rng.integers(0, A, int(rng.integers(0, 10)))))
    for now, theta, B, S in ((20.0, 5.0, 8, 12), (20.0, 1e9, 16, 6), (20.0, -1.0, 4, 40),
                             (10.0, 3.0, 32, 2), (0.0, 0.0, 0, 5)):
        got = tclora.lag_select(now, theta, arr, ads, res, B, S)
        want = O.lag_select(now, theta, arr, ads, res, B, S)
        assert got == want, (seed, now, theta, B, S)


def test_bam_and_lag_stream():
    """A Zipf request stream: LAG picks, BAM loads, the pool stays within its
    slots, and every chosen request's adapters are resident afterwards."""
    rng = np.random.default_rng(7)
    A, S, B = 64, 24, 8
    p = 1.0 / np.arange(1, A + 1) ** 1.2
    p /= p.sum()
    bam = tclora.Bam(S)
    obam = []
    arr, ads, now = [], [], 0.0
    for step in range(60):
        for _ in range(6):
            arr.append(now)
            ads.append(list(int(a) for a in rng.choice(A, int(rng.integers(1, 4)), replace=False, p=p)))
        res = [a for a in bam.slots().tolist() if a >= 0]
        ch = tclora.lag_select(now, 4.0, arr, ads, res, B, S)
        assert ch == O.lag_select(now, 4.0, arr, ads, res, B, S)
        batch = [a for i in ch for a in ads[i]]
        obam.append(batch)
        bam.acquire(batch)
        assert set(batch) <= set(bam.slots().tolist())
        keep = [i for i in range(len(arr)) if i not in set(ch)]
        arr, ads = [arr[i] for i in keep], [ads[i] for i in keep]
        now += 1.0
    recs, final = O.bam_run(S, obam)
    assert bam.slots().tolist() == final


def test_sched_host_errors():
    with pytest.raises(tclora.TclError):
        tclora.Bam(0)
    bam = tclora.Bam(2)
    with pytest.raises(tclora.TclError):
        bam.acquire([1, -2])
    with pytest.raises(tclora.TclError):
        bam.acquire([1, 2, 3])
    assert bam.slots().tolist() == [-1, -1]
    with pytest.raises(tclora.TclError):
        tclora.lag_select(float("nan"), 1.0, [0.0], [[1]], [], 1, 1)
    with pytest.raises(tclora.TclError):
        tclora.lag_select(0.0, 1.0, [float("nan")], [[1]], [], 1, 1)
    with pytest.raises(tclora.TclError):
        tclora.lag_select(0.0, 1.0, [0.0], [[-1]], [], 1, 1)
    assert tclora.lag_select(0.0, 1.0, [], [], [], 4, 4) == []
