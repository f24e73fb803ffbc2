"""BAM on the GPU (DyMerge-LoRA section 4: the slot pool keeps the raw
factors of resident adapters on the GPU; a batch pins its adapters, misses
evict the least recently used unpinned slot).  A Zipf stream of decode and
prefill batches over 40 logical adapters runs through a pool of 10 slots
for two modules: each batch's adapters are made resident (tcl_bam_acquire,
then tcl_bam_load copies the missing adapters' retained rows from pinned
host pools into their slots and re-packs those slots), its composite table
is re-written in slot ids, and the apply over the pool is compared with the
oracle's apply over the logical pools.  The loads must be the oracle's
(bam_run) batch by batch, and fewer than the adapters the batches use."""
import numpy as np
import pytest
import torch

from gpu_util import make_plan, rel_err, to_dev
from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W
from test_gpu_parity import TOL, banner
import oracle as O

pytestmark = pytest.mark.gpu

N_LOGICAL, N_SLOTS = 40, 10


def _cpu_tensor(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def _stream(seed, n_batches):
    """Batches of token composites (1-3 distinct adapters a token, Zipf(1.2)
    over the logical ids), at most N_SLOTS distinct adapters a batch;
    decode-sized and prefill-sized batches alternate."""
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, N_LOGICAL + 1) ** 1.2
    w /= w.sum()
    perm = rng.permutation(N_LOGICAL)     # hot adapters at random ids
    out = []
    for b in range(n_batches):
        T = 24 if b % 2 == 0 else 300
        ads, seen = [], set()
        while len(ads) < T:
            n = int(rng.integers(1, 4))
            tok = [int(perm[i]) for i in rng.choice(N_LOGICAL, n, replace=False, p=w)]
            if len(seen | set(tok)) > N_SLOTS:
                continue
            seen |= set(tok)
            ads.append(tok)
        als = [rng.random(len(a)).astype(np.float32).tolist() for a in ads]
        out.append((ads, als))
    return out


def test_bam_zipf_stream_applies_over_slots(monkeypatch):
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    rng = np.random.default_rng(181)
    shapes = [(256, 264, 16), (128, 520, 8)]          # (d_in, d_out, r_max)
    pools = []
    for d_in, d_out, r in shapes:
        A = W._normal(rng, (N_LOGICAL, r, d_in), 0.02, W.BF16)
        B = W._normal(rng, (N_LOGICAL, r, d_out), 0.02, W.BF16)
        k = rng.integers(0, r + 1, N_LOGICAL).astype(np.int32)
        pools.append((A, B, k))
    sp = tclora.SlotPool(N_SLOTS, [(_cpu_tensor(A), _cpu_tensor(B), k) for A, B, k in pools],
                         "cuda:0")
    batches = _stream(182, 14)
    hist, total_uses, total_loads = [], 0, 0
    for bi, (ads, als) in enumerate(batches):
        order = []
        for tok in ads:
            for a in tok:
                if a not in order:
                    order.append(a)
        slot_of, loads = sp.load(order)
        hist.append(order)
        want = O.bam_run(N_SLOTS, hist)[0][-1]
        assert want[0] == O.OK
        assert [tuple(x) for x in loads] == [tuple(x) for x in want[2]], bi
        total_uses += len(order)
        total_loads += len(loads)
        slot = {a: int(s) for a, s in zip(order, slot_of)}
        assert slot == {int(a): int(s) for a, s in want[1].items()}, bi
        c_log = W.csr_from_token_lists(ads, als, N_LOGICAL)
        c_slot = W.csr_from_token_lists([[slot[a] for a in tok] for tok in ads], als, N_SLOTS)
        T = c_log.n_tokens
        xs = [W._normal(rng, (T, d_in), 1.0, W.BF16) for d_in, _, _ in shapes]
        ys = [rng.standard_normal(size=(T, d_out), dtype=np.float32) for _, d_out, _ in shapes]
        plan = make_plan(c_slot)
        y_dev = [to_dev(y) for y in ys]
        tclora.fused_apply(plan, sp.modules, [to_dev(x) for x in xs], y_dev)
        torch.cuda.synchronize()
        errs = []
        for mi, (A, B, k) in enumerate(pools):
            _, d_ora = O.apply(c_log.group_tok_ptr, c_log.group_pair_ptr, c_log.pair_adapter,
                               c_log.pair_alpha, A, B, k, xs[mi], ys[mi])
            got = y_dev[mi].double().cpu().numpy() - ys[mi].astype(np.float64)
            errs.append(rel_err(got, d_ora))
            assert errs[-1] <= TOL[W.BF16], (bi, mi, errs[-1])
        banner(f"bam batch {bi}: T={T} adapters={len(order)} loads={len(loads)} "
               f"rel {max(errs):.2e}")
    print(f"  {total_loads} loads for {total_uses} adapter uses, "
          f"{sp.h2d_bytes} bytes host to device", flush=True)
    assert total_loads < total_uses
    resident = [a for a in sp.bam.slots().tolist() if a >= 0]
    assert sorted(resident) == sorted(a for a in O.bam_run(N_SLOTS, hist)[1] if a >= 0)
