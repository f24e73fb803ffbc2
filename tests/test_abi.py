"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

from tenant_composite_lora_amd import tclora

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tcl.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tcl_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return tclora.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(tclora.EXPORTS) == names


def test_version(L):
    assert b"gfx950" in L.tcl_version()


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"(TCL_E[A-Z]+|TCL_OK)\s*=\s*(-?\d+)", text))
    assert int(consts["TCL_OK"]) == tclora.OK
    assert int(consts["TCL_EINVAL"]) == tclora.EINVAL
    assert int(consts["TCL_EALIGN"]) == tclora.EALIGN
    assert int(consts["TCL_ENOSPC"]) == tclora.ENOSPC
    assert int(consts["TCL_EUNSUPPORTED"]) == tclora.EUNSUPPORTED
    assert int(consts["TCL_EHIP"]) == tclora.EHIP
    assert f"TCL_MAX_RANK {tclora.MAX_RANK}" in text
    assert f"TCL_MAX_PAIRS_PER_GROUP {tclora.MAX_PAIRS_PER_GROUP}" in text
    m = re.search(r"#define TCL_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == tclora.SCRATCH_BYTES


def test_status_codes_match_oracle():
    import oracle as O
    assert (O.OK, O.EINVAL, O.ENOSPC, O.EUNSUPPORTED) == (
        tclora.OK, tclora.EINVAL, tclora.ENOSPC, tclora.EUNSUPPORTED)


def test_plan_bytes(L):
    out = ctypes.c_size_t(0)
    assert L.tcl_plan_bytes(32, 32, 96, 64, 96, ctypes.byref(out)) == 0
    small = out.value
    assert small > 0 and small % 256 == 0
    assert L.tcl_plan_bytes(4224, 4224, 10600, 256, 10600, ctypes.byref(out)) == 0
    assert out.value > small
    assert L.tcl_plan_bytes(0, 0, 0, 1, 0, ctypes.byref(out)) == 0
    for args in [(-1, 1, 1, 1, 1), (1, -1, 1, 1, 1), (1, 1, -1, 1, 1), (1, 1, 1, 0, 1),
                 (1, 1, 1, 1, -1), (1 << 25, 1, 1, 1, 1)]:
        assert L.tcl_plan_bytes(*args, ctypes.byref(out)) == tclora.EINVAL, args
        assert len(L.tcl_last_error()) > 0
    assert L.tcl_plan_bytes(1, 1, 1, 1, 1, None) == tclora.EINVAL


def _comp(T=3, G=2, NP=3, N=4, cap=4, ptr=0x1000):
    return tclora.Composites(T, G, NP, N, cap, ptr, ptr, ptr, ptr)


def test_plan_map_host_errors(L):
    h = ctypes.c_void_p(0)
    need = tclora.plan_bytes(3, 2, 3, 4, 4)
    # null composites / out
    assert L.tcl_plan_map(None, 0x10000, need, None, ctypes.byref(h)) == tclora.EINVAL
    c = _comp()
    assert L.tcl_plan_map(ctypes.byref(c), 0x10000, need, None, None) == tclora.EINVAL
    # null arrays
    c0 = tclora.Composites(3, 2, 3, 4, 4, None, 0x1000, 0x1000, 0x1000)
    assert L.tcl_plan_map(ctypes.byref(c0), 0x10000, need, None, ctypes.byref(h)) == tclora.EINVAL
    c1 = tclora.Composites(3, 2, 3, 4, 4, 0x1000, 0x1000, None, 0x1000)
    assert L.tcl_plan_map(ctypes.byref(c1), 0x10000, need, None, ctypes.byref(h)) == tclora.EINVAL
    # sizes
    cbad = _comp(N=0)
    assert L.tcl_plan_map(ctypes.byref(cbad), 0x10000, need, None, ctypes.byref(h)) == tclora.EINVAL
    # buffer
    assert L.tcl_plan_map(ctypes.byref(c), None, need, None, ctypes.byref(h)) == tclora.EINVAL
    assert L.tcl_plan_map(ctypes.byref(c), 0x10010, need, None, ctypes.byref(h)) == tclora.EALIGN
    assert L.tcl_plan_map(ctypes.byref(c), 0x10000, need - 1, None, ctypes.byref(h)) == tclora.ENOSPC
    assert b"needs" in L.tcl_last_error()
    assert h.value is None


def test_null_plan_rejected(L):
    m = tclora.ModuleDesc(4, 16, 16, 4, tclora.BF16, 0x1000, 0x2000, None)
    out = ctypes.c_size_t(0)
    assert L.tcl_workspace_bytes(None, ctypes.byref(m), 1, ctypes.byref(out)) == tclora.EINVAL
    assert L.tcl_shrink(None, ctypes.byref(m), 0x1000, 16, 0, 0x1000, None) == tclora.EINVAL
    assert L.tcl_expand(None, ctypes.byref(m), 0x1000, 0x1000, 16, 1, None) == tclora.EINVAL
    assert L.tcl_plan_status(None, None, None, None) == tclora.EINVAL
    c = tclora.Composites(4, 4, 4, 4, 4, 0x1000, 0x2000, 0x3000, 0x4000)
    ptrs = (ctypes.c_void_p * 1)(0x1000)
    lds = (ctypes.c_int64 * 1)(16)
    assert L.tcl_remap_apply(None, ctypes.byref(c), ctypes.byref(m), 1, ptrs, lds, 0, ptrs,
                             lds, 1, 0x1000, 1 << 20, None) == tclora.EINVAL
    assert L.tcl_remap_shrink(None, ctypes.byref(c), ctypes.byref(m), 1, ptrs, lds, 0, 0x1000,
                              1 << 20, None) == tclora.EINVAL
    assert L.tcl_plan_copy_out(None, *([None] * 9)) == tclora.EINVAL
    L.tcl_plan_free(None)


def test_load_ranks_host_errors(L):
    m = tclora.ModuleDesc(4, 16, 16, 8, tclora.BF16, 0x1000, 0x2000, None)
    k = np.array([0, 8, 9, 1], np.int32)          # 9 > r_max
    rc = L.tcl_module_load_ranks(ctypes.byref(m), k.ctypes.data_as(ctypes.c_void_p), 0x3000,
                                 None)
    assert rc == tclora.EINVAL and b"k[2]" in L.tcl_last_error()
    k = np.array([0, -1, 2, 1], np.int32)
    rc = L.tcl_module_load_ranks(ctypes.byref(m), k.ctypes.data_as(ctypes.c_void_p), 0x3000,
                                 None)
    assert rc == tclora.EINVAL
    assert L.tcl_module_load_ranks(ctypes.byref(m), None, 0x3000, None) == tclora.EINVAL


def test_gate_host_errors(L):
    """tcl_gate_topk rejects bad sizes and pointers on the host (no GPU)."""
    P = 0x1000

    def call(T=4, C=8, k=2, ldl=8, ldc=8, lg=P, cd=P, out=P):
        return L.tcl_gate_topk(lg, ldl, cd, ldc, T, C, k, out, out, out, out, None)

    assert call(T=-1) == tclora.EINVAL
    assert call(C=0) == tclora.EINVAL
    assert call(C=65, ldl=65, ldc=65) == tclora.EINVAL
    assert call(k=0) == tclora.EINVAL
    assert call(k=9) == tclora.EINVAL              # k > n_candidates
    assert call(ldl=7) == tclora.EINVAL
    assert call(ldc=7) == tclora.EINVAL
    assert call(lg=None) == tclora.EINVAL
    assert call(cd=None) == tclora.EINVAL
    assert call(out=None) == tclora.EINVAL
    assert call(T=1 << 30, k=4, C=8) == tclora.EINVAL  # T * k beyond 32-bit indexing
    assert call(lg=P + 2) == tclora.EALIGN
    assert b"gate" in L.tcl_last_error()


# ---------------------------------------------------------------------------
# host-resident composite tables: validated on the host, before any HIP call
# ---------------------------------------------------------------------------

def _mutations(seed, n):
    """Random tables with random defects (or none): every error class of the
    validation, alone and together, over a few hundred groups."""
    from tenant_composite_lora_amd import workloads as W
    rng = np.random.default_rng(seed)
    for i in range(n):
        T = int(rng.integers(0, 60))
        base = W.random_case(int(rng.integers(1 << 30)), T=max(T, 1), N=12, d_in=8, d_out=8,
                             r_max=2, max_pairs=6, empty_frac=0.2,
                             tokens_per_group=int(rng.integers(1, 4))).composites
        gt = base.group_tok_ptr.astype(np.int64).copy()
        gp = base.group_pair_ptr.astype(np.int64).copy()
        ad = base.pair_adapter.astype(np.int64).copy()
        al = base.pair_alpha.astype(np.float32).copy()
        N, Tn = base.n_adapters, base.n_tokens
        cap = None
        kinds = rng.choice(9, size=int(rng.integers(0, 3)), replace=False)
        for k in kinds:
            G, NP = len(gt) - 1, len(ad)
            if k == 0 and NP:
                ad[rng.integers(NP)] = rng.choice([-1, N, N + 7])
            elif k == 1 and NP:
                al[rng.integers(NP)] = rng.choice([np.nan, np.inf, -np.inf])
            elif k == 2 and G > 1:
                g = int(rng.integers(1, G))
                gt[g] = gt[g - 1] - 1 if gt[g - 1] > 0 else gt[g + 1] + 1
            elif k == 3 and G > 1:
                g = int(rng.integers(1, G))
                gp[g] = gp[g + 1] + 1
            elif k == 4:
                Tn += 1
            elif k == 5:
                for g in range(G):
                    if gp[g + 1] - gp[g] >= 2:
                        ad[gp[g] + 1] = ad[gp[g]]
                        break
            elif k == 6:
                # a group of 70 pairs appended (beyond the limit)
                ad = np.concatenate([ad, np.arange(70) % N + 0]).astype(np.int64)
                ad[-70:] = np.arange(70)
                N = max(N, 70)
                al = np.concatenate([al, np.ones(70, np.float32)])
                gp = np.concatenate([gp, [gp[-1] + 70]])
                gt = np.concatenate([gt, [gt[-1] + 1]])
                Tn += 1
            elif k == 7:
                P = int(np.sum(np.diff(gt).clip(0) * np.diff(gp).clip(0)))
                cap = max(P - 1, 0)
            elif k == 8:
                gp[-1] += 1
        yield i, gt, gp, ad, al, Tn, N, cap


def _validate_both(gt, gp, ad, al, T, N, cap):
    import oracle as O
    want = O.validate(gt, gp, ad.astype(np.int32), al, T, N, max_tuples=cap)
    rc, P, U = tclora.validate_composites(gt, gp, ad, al, N, n_tokens=T, max_tuples=cap)
    return want, rc, P, U


def test_host_validation_matches_oracle_on_hand_tables():
    """Every hand-made defect (and the defect-free tables) gets the oracle's
    code, including the precedence of EINVAL over EUNSUPPORTED over
    ENOSPC."""
    from test_gpu_parity import _bad_large_tables, _bad_tables, _pad_groups
    for name, (tp, pp, ad, al, T, cap) in _bad_tables().items():
        N = 80 if name.startswith("too_many_pairs") else 4
        for padded in (False, True):
            tq, pq = _pad_groups(tp, pp, 1100) if padded else (tp, pp)
            want, rc, _, _ = _validate_both(np.array(tq), np.array(pq), np.array(ad),
                                            np.array(al, np.float32), T, N, cap)
            assert rc == want, (name, padded, rc, want)
    for name, (tp, pp, ad, al, T, N, cap) in _bad_large_tables().items():
        want, rc, _, _ = _validate_both(tp, pp, ad, al, T, N, cap)
        assert rc == want, (name, rc, want)


def test_host_validation_matches_oracle_on_random_defects():
    import oracle as O
    seen = set()
    for i, gt, gp, ad, al, T, N, cap in _mutations(5, 400):
        want, rc, P, U = _validate_both(gt, gp, ad, al, T, N, cap)
        assert rc == want, (i, rc, want)
        seen.add(want)
        if rc == 0:
            pl = O.plan(gt, gp, ad.astype(np.int32), al)
            assert P == len(pl["tup_token"]) and U == len(pl["seg_adapter"])
    assert seen == {O.OK, O.EINVAL, O.EUNSUPPORTED, O.ENOSPC}


def test_host_plan_map_rejects_before_any_hip_call(L):
    """A bad host table is refused with its code before the library touches
    the GPU (this container has none: a HIP call would fail with EHIP)."""
    from test_gpu_parity import _bad_tables
    h = ctypes.c_void_p(0)
    for name, (tp, pp, ad, al, T, cap) in _bad_tables().items():
        if name == "fits_capacity":
            continue
        N = 80 if name.startswith("too_many_pairs") else 4
        arrs = tclora._host_table(tp, pp, ad, al)
        c = tclora._host_composites(arrs, T, N, cap if cap is not None else 16)
        import oracle as O
        want = O.validate(np.array(tp), np.array(pp), np.array(ad, np.int32),
                          np.array(al, np.float32), T, N, max_tuples=cap)
        assert want != 0
        rc = L.tcl_plan_map_host(ctypes.byref(c), 0x10000, 1 << 30, None, ctypes.byref(h))
        assert rc == want, (name, rc, want)
        assert h.value is None
        assert len(L.tcl_last_error()) > 0


def test_plan_info_and_status_async_host_errors(L):
    P, U = ctypes.c_int32(0), ctypes.c_int32(0)
    assert L.tcl_plan_info(None, ctypes.byref(P), ctypes.byref(U)) == tclora.EINVAL
    assert L.tcl_plan_status_async(None, 0x1000, None) == tclora.EINVAL
    assert L.tcl_plan_remap_host(None, None, None) == tclora.EINVAL


def test_module_init_host_errors(L):
    ok = dict(n=4, d_in=16, d_out=16, r=8, dt=tclora.BF16, A=0x1000, B=0x2000)

    def m(**kw):
        a = {**ok, **kw}
        return tclora.ModuleDesc(a["n"], a["d_in"], a["d_out"], a["r"], a["dt"], a["A"], a["B"],
                                 None)

    k = np.array([0, 8, 3, 1], np.int32)
    kp = k.ctypes.data_as(ctypes.c_void_p)
    assert L.tcl_module_init(None, kp, 0x3000, None) == tclora.EINVAL
    assert L.tcl_module_init(ctypes.byref(m(A=0)), kp, 0x3000, None) == tclora.EINVAL
    assert L.tcl_module_init(ctypes.byref(m(n=0)), kp, 0x3000, None) == tclora.EINVAL
    assert L.tcl_module_init(ctypes.byref(m(r=65)), kp, 0x3000, None) == tclora.EUNSUPPORTED
    assert L.tcl_module_init(ctypes.byref(m(r=0)), kp, 0x3000, None) == tclora.EUNSUPPORTED
    assert L.tcl_module_init(ctypes.byref(m(d_in=12)), kp, 0x3000, None) == tclora.EALIGN
    assert L.tcl_module_init(ctypes.byref(m(A=0x1008)), kp, 0x3000, None) == tclora.EALIGN
    assert L.tcl_module_init(ctypes.byref(m(dt=7)), kp, 0x3000, None) == tclora.EINVAL
    bad = np.array([0, 9, 3, 1], np.int32)
    assert L.tcl_module_init(ctypes.byref(m()), bad.ctypes.data_as(ctypes.c_void_p), 0x3000,
                             None) == tclora.EINVAL
    assert L.tcl_module_init(ctypes.byref(m()), kp, None, None) == tclora.EINVAL
    # no ranks: every adapter at r_max, no GPU call
    d = m()
    d.k_dev = 0x5000
    assert L.tcl_module_init(ctypes.byref(d), None, None, None) == tclora.OK
    assert d.k_dev is None


def test_bam_load_host_errors(L):
    """tcl_bam_load and tcl_bam_pool_init check everything on the host before
    any HIP call (the pointers here are never dereferenced)."""
    pool = tclora.ModuleDesc(4, 16, 16, 8, tclora.BF16, 0x1000, 0x2000, 0x3000, None)
    plain = tclora.ModuleDesc(4, 16, 16, 8, tclora.BF16, 0x1000, 0x2000, None, None)
    k = np.array([8, 3, 9, 0, 2], np.int32)       # adapter 2 has rank 9 > r_max
    kp = k.ctypes.data_as(ctypes.c_void_p)

    def load(desc, slots, ads, n_logical=5, kk=kp):
        s = np.ascontiguousarray(slots, np.int32)
        a = np.ascontiguousarray(ads, np.int32)
        return L.tcl_bam_load(ctypes.byref(desc), 0x4000, 0x5000, kk, n_logical, len(s),
                              s.ctypes.data, a.ctypes.data, None)

    assert load(plain, [0], [0]) == tclora.EINVAL               # not a slot pool
    assert b"slot pool" in L.tcl_last_error()
    assert load(pool, [4], [0]) == tclora.EINVAL                # slot out of range
    assert load(pool, [-1], [0]) == tclora.EINVAL
    assert load(pool, [0], [5]) == tclora.EINVAL                # adapter out of range
    assert load(pool, [1, 1], [0, 1]) == tclora.EINVAL          # slot twice
    assert load(pool, [0], [2]) == tclora.EINVAL                # rank beyond r_max
    assert b"rank 9" in L.tcl_last_error()
    assert load(pool, [0], [0], n_logical=0) == tclora.EINVAL
    assert load(pool, [], []) == tclora.OK                      # nothing to do
    assert L.tcl_bam_load(None, 0x4000, 0x5000, kp, 5, 0, None, None, None) == tclora.EINVAL
    assert L.tcl_bam_pool_init(ctypes.byref(plain), None, None, 0, None) == tclora.EINVAL
    assert L.tcl_bam_pool_init(ctypes.byref(plain), 0x3002, None, 0, None) == tclora.EALIGN
    assert L.tcl_bam_pool_init(ctypes.byref(plain), 0x3000, 0x6010, 1 << 20, None) == tclora.EALIGN
    assert L.tcl_bam_pool_init(ctypes.byref(plain), 0x3000, 0x6000, 16, None) == tclora.ENOSPC
    f32 = tclora.ModuleDesc(4, 16, 16, 8, tclora.F32, 0x1000, 0x2000, None, None)
    assert L.tcl_bam_pool_init(ctypes.byref(f32), 0x3000, 0x6000, 1 << 20, None) == \
        tclora.EUNSUPPORTED


def test_host_validation_ignores_the_unused_tail():
    """Pair entries at or beyond group_pair_ptr[G] are unused capacity: a
    tail of invalid ids, repeats and NaN weights changes neither the verdict
    nor the counts, on the host as in the oracle; a table whose pairs end
    beyond the arrays is EINVAL."""
    import oracle as O
    from tenant_composite_lora_amd import workloads as W
    rng = np.random.default_rng(31)
    for trial in range(40):
        T, N = int(rng.integers(1, 30)), int(rng.integers(2, 12))
        wl = W.random_case(300 + trial, T=T, N=N, d_in=8, d_out=8, r_max=4,
                           max_pairs=min(4, N), empty_frac=0.2)
        c = wl.composites
        gt, gp = c.group_tok_ptr.astype(np.int32), c.group_pair_ptr.astype(np.int32)
        ad, al = c.pair_adapter.astype(np.int32), c.pair_alpha.astype(np.float32)
        extra = int(rng.integers(1, 9))
        ad_t = np.concatenate([ad, rng.choice([-5, N, 10 ** 6, 0], extra).astype(np.int32)])
        al_t = np.concatenate([al, np.full(extra, np.nan, np.float32)])
        want_cut = O.validate(gt, gp, ad, al, T, N)
        want_tail = O.validate(gt, gp, ad_t, al_t, T, N)
        assert want_cut == want_tail == tclora.OK
        rc, P, U = tclora.validate_composites(gt, gp, ad_t, al_t, N, n_tokens=T)
        rc0, P0, U0 = tclora.validate_composites(gt, gp, ad, al, N, n_tokens=T)
        assert (rc, P, U) == (rc0, P0, U0) == (tclora.OK, P0, U0)
        # pairs that end beyond the arrays
        gp_bad = gp.copy()
        gp_bad[-1] = len(ad_t) + 1
        assert O.validate(gt, gp_bad, ad_t, al_t, T, N) == O.EINVAL
        assert tclora.validate_composites(gt, gp_bad, ad_t, al_t, N, n_tokens=T)[0] == \
            tclora.EINVAL
