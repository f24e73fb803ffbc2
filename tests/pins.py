"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes the oracle module ``O`` and raises
AssertionError if the oracle disagrees with the fact.  The same functions run
against the real oracle (tests/test_oracle_pins.py) and against deliberately
broken copies of it (tests/test_oracle_mutants.py), which shows that a
plausible mistake anywhere in the oracle is caught by at least one pin.
"""
import json
import os

import numpy as np
import torch

from tenant_composite_lora_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


_MODULE_K = object()


def _apply(O, c, m, x, yb, k=_MODULE_K):
    kk = m.k if k is _MODULE_K else k
    return O.apply(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                   m.A_t, m.B_t, kk, x, yb)


def _plan(O, c):
    return O.plan(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha)


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _rel(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den) if a.size else 0.0


# ---------------------------------------------------------------------------
# X1: ELORA worked example (single LoRA, d = 2, r = 1), exact small integers
# ---------------------------------------------------------------------------

def pin_x1_elora_example(O):
    g = json.load(open(os.path.join(GOLDEN, "elora_worked_example.json")))
    WK = np.array(g["W_K"], dtype=np.float64)
    h = np.array(g["h"], dtype=np.float64)
    yb = (WK @ h)[None, :]
    assert np.array_equal(yb[0], np.array(g["K_base"], dtype=np.float64))
    pool_A, pool_B = [], []
    for ad in g["adapters"]:
        A_page = np.array(ad["A_page"], dtype=np.float64)    # d x r
        B_page = np.array(ad["B_page"], dtype=np.float64)    # r x d
        pool_A.append(B_page)          # A_t[a] = A_a^T = B_page   (r x d_in)
        pool_B.append(A_page.T)        # B_t[a] = B_a^T = A_page^T (r x d_out)
    A_t = np.stack(pool_A).astype(np.float32)
    B_t = np.stack(pool_B).astype(np.float32)
    x = h[None, :].astype(np.float32)
    for i, ad in enumerate(g["adapters"]):
        c = W.csr_from_token_lists([[i]], [[1.0]], len(pool_A))
        y, _ = O.apply(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                       A_t, B_t, None, x, yb.astype(np.float32))
        assert np.array_equal(y[0], np.array(ad["K"], dtype=np.float64)), (ad["name"], y[0])
    names = [a["name"] for a in g["adapters"]]
    dc = g["derived_composite"]
    ids = [names.index(n) for n, _ in dc["pairs"]]
    als = [w for _, w in dc["pairs"]]
    c = W.csr_from_token_lists([ids], [als], len(pool_A))
    y, _ = O.apply(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                   A_t, B_t, None, x, yb.astype(np.float32))
    assert np.array_equal(y[0], np.array(dc["K"], dtype=np.float64)), y[0]


# ---------------------------------------------------------------------------
# X2: composite = dense pre-merged Delta W (DyMerge-LoRA section 3.1, M1)
# ---------------------------------------------------------------------------

def _dense_delta_w(c, m, t):
    """Delta W of token t built the pre-merge way: sum_i alpha_i B_i A_i^T as
    dense d_out x d_in matrices, then applied to x in one product."""
    g = int(np.searchsorted(c.group_tok_ptr, t, side="right") - 1)
    A = _f64(m.A_t)
    B = _f64(m.B_t)
    dW = np.zeros((m.d_out, m.d_in))
    for q in range(int(c.group_pair_ptr[g]), int(c.group_pair_ptr[g + 1])):
        a = int(c.pair_adapter[q])
        k = m.r_max if m.k is None else int(m.k[a])
        Bi = B[a, :k, :].T            # d_out x k
        Ai = A[a, :k, :].T            # d_in  x k
        dW += float(np.float32(c.pair_alpha[q])) * (Bi @ Ai.T)
    return dW


def pin_x2_dense_premerge(O):
    cases = [W.config1(0),
             W.random_case(3, T=9, N=5, d_in=24, d_out=40, r_max=4, max_pairs=4),
             W.random_case(4, T=7, N=6, d_in=32, d_out=16, r_max=8, max_pairs=5,
                           with_k=True, tokens_per_group=3, empty_frac=0.2)]
    for wl in cases:
        c, m = wl.composites, wl.modules[0]
        y, delta = _apply(O, c, m, wl.x[0], wl.y_base[0])
        X = _f64(wl.x[0])
        ref = np.stack([_dense_delta_w(c, m, t) @ X[t] for t in range(c.n_tokens)])
        assert _rel(delta, ref) < 1e-12, (wl.name, _rel(delta, ref))
        assert _rel(y, _f64(wl.y_base[0]) + ref) < 1e-12


# ---------------------------------------------------------------------------
# X3: one adapter, alpha = 1, is textbook LoRA (ELORA Eq. 1)
# ---------------------------------------------------------------------------

def pin_x3_textbook_lora(O):
    wl = W.random_case(5, T=6, N=3, d_in=48, d_out=20, r_max=8, max_pairs=1, dtype=W.F32)
    m = wl.modules[0]
    T = wl.n_tokens
    a = 1
    c = W.csr_from_token_lists([[a]] * T, [[1.0]] * T, 3)
    y, _ = _apply(O, c, m, wl.x[0], wl.y_base[0])
    x = torch.from_numpy(_f64(wl.x[0]))
    A_i_T = torch.from_numpy(_f64(m.A_t)[a])       # r x d_in, the down projection weight
    B_i = torch.from_numpy(_f64(m.B_t)[a].T.copy())   # d_out x r, the up projection weight
    ref = torch.from_numpy(_f64(wl.y_base[0])) + torch.nn.functional.linear(
        torch.nn.functional.linear(x, A_i_T), B_i)
    assert _rel(y, ref.numpy()) < 1e-12


# ---------------------------------------------------------------------------
# X4: linearity in alpha; X5: alpha = 0 and k = 0 are no-ops
# ---------------------------------------------------------------------------

def pin_x4_linearity(O):
    wl = W.random_case(6, T=10, N=6, d_in=32, d_out=24, r_max=8, max_pairs=4, with_k=True)
    c, m = wl.composites, wl.modules[0]
    rng = np.random.default_rng(11)
    # multiples of 1/64 below 1: sums and scalings stay exact in float32
    al = (rng.integers(0, 64, c.n_pairs) / 64).astype(np.float32)
    be = (rng.integers(0, 64, c.n_pairs) / 64).astype(np.float32)

    def delta(alpha):
        cc = W.Composites(c.n_tokens, c.n_adapters, c.group_tok_ptr, c.group_pair_ptr,
                          c.pair_adapter, alpha.astype(np.float32))
        return _apply(O, cc, m, wl.x[0], wl.y_base[0])[1]

    d_a, d_b, d_ab = delta(al), delta(be), delta(al + be)
    assert _rel(d_ab, d_a + d_b) < 1e-12
    assert _rel(delta(3 * al), 3 * d_a) < 1e-12
    assert np.max(np.abs(d_a)) > 0


def pin_x5_noop(O):
    wl = W.random_case(7, T=8, N=4, d_in=16, d_out=16, r_max=4, max_pairs=3)
    c, m = wl.composites, wl.modules[0]
    zero = W.Composites(c.n_tokens, c.n_adapters, c.group_tok_ptr, c.group_pair_ptr,
                        c.pair_adapter, np.zeros_like(c.pair_alpha))
    y, d = _apply(O, zero, m, wl.x[0], wl.y_base[0])
    assert np.all(d == 0) and np.array_equal(y, _f64(wl.y_base[0]))
    y, d = _apply(O, c, m, wl.x[0], wl.y_base[0], k=np.zeros(4, dtype=np.int32))
    assert np.all(d == 0) and np.array_equal(y, _f64(wl.y_base[0]))
    y, d = _apply(O, c, m, wl.x[0], wl.y_base[0])
    assert np.max(np.abs(d)) > 0
    empty = W.csr_from_token_lists([[]] * c.n_tokens, [[]] * c.n_tokens, 4)
    y, d = _apply(O, empty, m, wl.x[0], wl.y_base[0])
    assert np.all(d == 0)


# ---------------------------------------------------------------------------
# X6: truncating to k_m equals zero-padding and equals a dense rank-k copy
#     (LoRAForge retained-rank contract, approach (1))
# ---------------------------------------------------------------------------

def pin_x6_truncation(O):
    wl = W.random_case(8, T=12, N=6, d_in=40, d_out=24, r_max=8, max_pairs=4)
    c, m = wl.composites, wl.modules[0]
    rng = np.random.default_rng(12)
    k = rng.integers(0, 9, size=6).astype(np.int32)
    y_k, d_k = _apply(O, c, m, wl.x[0], wl.y_base[0], k=k)
    keep = (np.arange(8)[None, :] < k[:, None])[:, :, None]
    A0 = np.where(keep, _f64(m.A_t), 0.0)
    B0 = np.where(keep, _f64(m.B_t), 0.0)
    y_pad, d_pad = O.apply(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                           A0, B0, None, wl.x[0], wl.y_base[0])
    assert _rel(d_k, d_pad) < 1e-12
    # dense rank-k copy: explicit rank-k factors per adapter, no padding at all
    X = _f64(wl.x[0])
    ref = np.zeros_like(d_k)
    owner = np.repeat(np.arange(c.n_groups), np.diff(c.group_tok_ptr))
    for t in range(c.n_tokens):
        g = owner[t]
        for q in range(int(c.group_pair_ptr[g]), int(c.group_pair_ptr[g + 1])):
            a = int(c.pair_adapter[q])
            Ai = _f64(m.A_t)[a, :k[a], :].T     # d_in x k
            Bi = _f64(m.B_t)[a, :k[a], :].T     # d_out x k
            ref[t] += float(c.pair_alpha[q]) * (Bi @ (Ai.T @ X[t]))
    assert _rel(d_k, ref) < 1e-12
    # and k = r_max is the untruncated apply
    y_full, _ = _apply(O, c, m, wl.x[0], wl.y_base[0], k=np.full(6, 8, np.int32))
    y_none, _ = _apply(O, c, m, wl.x[0], wl.y_base[0], k=None)
    assert np.array_equal(y_full, y_none)


# ---------------------------------------------------------------------------
# X7: the merged update of a composite has rank <= sum of its ranks
#     (DyMerge-LoRA section 3.1: merging k rank-r adapters gives rank up to k*r)
# ---------------------------------------------------------------------------

def pin_x7_rank_bound(O):
    rng = np.random.default_rng(13)
    d = 40
    wl = W.random_case(9, T=1, N=6, d_in=d, d_out=d, r_max=3, max_pairs=1, dtype=W.F32)
    m = wl.modules[0]
    for ids in ([0], [1, 4], [0, 2, 5], [0, 1, 2, 3, 4, 5]):
        al = rng.random(len(ids)).astype(np.float32) + 0.1
        # one group covering d tokens with x = identity: token j receives column j
        c = W.Composites(d, 6, np.array([0, d], np.int32), np.array([0, len(ids)], np.int32),
                         np.array(ids, np.int32), al)
        eye = np.eye(d, dtype=np.float32)
        _, delta = O.apply(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                           m.A_t, m.B_t, None, eye, np.zeros((d, d), np.float32))
        dW = delta.T                     # column j = Delta W e_j
        rank = np.linalg.matrix_rank(dW, tol=1e-9)
        assert rank <= 3 * len(ids)
        assert rank == min(3 * len(ids), d)   # random factors: the bound is attained
        ref = np.zeros((d, d))
        for a, w in zip(ids, al):
            ref += float(w) * (_f64(m.B_t)[a].T @ _f64(m.A_t)[a])
        assert _rel(dW, ref) < 1e-12


# ---------------------------------------------------------------------------
# X8: mapping stage — hand-worked example and brute force on random inputs
# ---------------------------------------------------------------------------

def pin_x8_mapping(O):
    g = json.load(open(os.path.join(GOLDEN, "mapping_hand_example.json")))
    ads = [[a for a, _ in row] for row in g["token_pairs"]]
    als = [[w for _, w in row] for row in g["token_pairs"]]
    c = W.csr_from_token_lists(ads, als, g["n_adapters"])
    pl = _plan(O, c)
    for key, val in g["expected"].items():
        got = pl[key]
        want = np.array(val, dtype=got.dtype)
        assert np.array_equal(got, want), (key, got, want)
    for seed in range(4):
        wl = W.random_case(20 + seed, T=13, N=7, d_in=8, d_out=8, r_max=2, max_pairs=5,
                           tokens_per_group=1 + seed % 3, empty_frac=0.15)
        _check_plan_brute(_plan(O, wl.composites), wl.composites)


def _check_plan_brute(pl, c):
    """Position of each tuple = number of tuples with a smaller
    (adapter, token, slot) key, computed by direct counting."""
    T = c.n_tokens
    owner = np.repeat(np.arange(c.n_groups), np.diff(c.group_tok_ptr))
    tuples = []
    for t in range(T):
        g = owner[t]
        ids = c.pair_adapter[c.group_pair_ptr[g]:c.group_pair_ptr[g + 1]]
        w = c.pair_alpha[c.group_pair_ptr[g]:c.group_pair_ptr[g + 1]]
        for q in range(len(ids)):
            slot = int(np.sum(ids < ids[q]))          # rank among the composite's ids
            tuples.append((int(ids[q]), t, slot, np.float32(w[q])))
    P = len(tuples)
    assert pl["tup_token"].shape[0] == P
    for (a, t, s, w) in tuples:
        pos = sum(1 for (a2, t2, s2, _) in tuples if (a2, t2, s2) < (a, t, s))
        assert pl["tup_adapter"][pos] == a and pl["tup_token"][pos] == t
        assert pl["tup_slot"][pos] == s
        assert pl["tup_alpha"][pos].view(np.uint32) == w.view(np.uint32)
    counts = {}
    for (a, _, _, _) in tuples:
        counts[a] = counts.get(a, 0) + 1
    assert pl["seg_adapter"].tolist() == sorted(counts)
    assert np.diff(pl["seg_begin"]).tolist() == [counts[a] for a in sorted(counts)]
    assert pl["seg_begin"][0] == 0 and pl["seg_begin"][-1] == P
    n_t = np.array([np.sum(np.array([tt for (_, tt, _, _) in tuples]) == t) for t in range(T)])
    assert pl["tok_ptr"].tolist() == [0] + np.cumsum(n_t).tolist()
    for t in range(T):
        for s in range(n_t[t]):
            p = pl["tok_tuple"][pl["tok_ptr"][t] + s]
            assert pl["tup_token"][p] == t and pl["tup_slot"][p] == s


# ---------------------------------------------------------------------------
# X9: adapter size next to the base weight (ELORA section III-A size example)
# ---------------------------------------------------------------------------

def pin_x9_adapter_fraction(O):
    d, r = 4096, 32
    assert d * d == 16_777_216                      # "about 16.8 million values"
    assert 2 * d * r == 262_144                     # "about 260 thousand values"
    f = O.adapter_fraction(d, d, r)
    assert f == 0.015625
    assert abs(round(100 * f, 1) - 1.6) < 1e-9      # "about 1.6 %"


# ---------------------------------------------------------------------------
# X10: permutation invariance
# ---------------------------------------------------------------------------

def pin_x10_permutation(O):
    wl = W.random_case(10, T=11, N=8, d_in=24, d_out=24, r_max=4, max_pairs=5)
    c, m = wl.composites, wl.modules[0]
    y, _ = _apply(O, c, m, wl.x[0], wl.y_base[0])
    pl = _plan(O, c)
    rng = np.random.default_rng(14)
    # shuffle the pairs inside every composite: nothing changes, bit for bit
    ad, al = c.pair_adapter.copy(), c.pair_alpha.copy()
    for g in range(c.n_groups):
        lo, hi = c.group_pair_ptr[g], c.group_pair_ptr[g + 1]
        perm = rng.permutation(hi - lo) + lo
        ad[lo:hi], al[lo:hi] = c.pair_adapter[perm], c.pair_alpha[perm]
    c2 = W.Composites(c.n_tokens, c.n_adapters, c.group_tok_ptr, c.group_pair_ptr, ad, al)
    y2, _ = _apply(O, c2, m, wl.x[0], wl.y_base[0])
    assert np.array_equal(y, y2)
    pl2 = _plan(O, c2)
    for key in pl:
        assert np.array_equal(pl[key], pl2[key]), key
    # permute tokens: rows permute
    tperm = rng.permutation(c.n_tokens)
    rows_a = [c.pair_adapter[c.group_pair_ptr[t]:c.group_pair_ptr[t + 1]].tolist() for t in tperm]
    rows_w = [c.pair_alpha[c.group_pair_ptr[t]:c.group_pair_ptr[t + 1]].tolist() for t in tperm]
    c3 = W.csr_from_token_lists(rows_a, rows_w, c.n_adapters)
    y3, _ = O.apply(c3.group_tok_ptr, c3.group_pair_ptr, c3.pair_adapter, c3.pair_alpha,
                    m.A_t, m.B_t, m.k, wl.x[0][tperm], wl.y_base[0][tperm])
    assert np.array_equal(y3, y[tperm])


# ---------------------------------------------------------------------------
# shrink / expand split agrees with the one-pass apply; sampled rows agree
# ---------------------------------------------------------------------------

def pin_split_and_rows(O):
    for wl in (W.config1(0),
               W.random_case(15, T=9, N=5, d_in=32, d_out=48, r_max=8, max_pairs=4,
                             with_k=True, tokens_per_group=2, empty_frac=0.2)):
        c, m = wl.composites, wl.modules[0]
        y, _ = _apply(O, c, m, wl.x[0], wl.y_base[0])
        pl = _plan(O, c)
        z = O.shrink(pl, m.A_t, m.k, wl.x[0])
        # z is A^T x, checked against a direct product per tuple
        A = _f64(m.A_t)
        X = _f64(wl.x[0])
        for p in range(z.shape[0]):
            a, t = pl["tup_adapter"][p], pl["tup_token"][p]
            kk = m.r_max if m.k is None else m.k[a]
            want = np.zeros(m.r_max)
            want[:kk] = A[a, :kk] @ X[t]
            assert _rel(z[p], want) < 1e-12 or np.all(want == 0) and np.all(z[p] == 0)
        y2 = O.expand(pl, m.B_t, m.k, z, wl.y_base[0])
        assert _rel(y2 - _f64(wl.y_base[0]), y - _f64(wl.y_base[0])) < 1e-12
        rows = [0, c.n_tokens - 1, c.n_tokens // 2]
        cols = [0, 3, m.d_out - 1]
        ys = O.apply_rows(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                          m.A_t, m.B_t, m.k, wl.x[0], wl.y_base[0], rows, cols)
        assert _rel(ys, y[np.ix_(rows, cols)]) < 1e-12


# ---------------------------------------------------------------------------
# validation codes
# ---------------------------------------------------------------------------

def pin_validation(O):
    def v(tp, pp, ad, al, T=3, N=4, **kw):
        return O.validate(np.array(tp), np.array(pp), np.array(ad, np.int32),
                          np.array(al, np.float32), T, N, **kw)
    good = ([0, 1, 3], [0, 2, 3], [0, 1, 3], [0.5, 0.5, 1.0])
    assert v(*good) == O.OK
    assert v([0, 1, 2], [0, 2, 3], [0, 1, 3], [.5, .5, 1.]) == O.EINVAL        # tokens != T
    assert v([0, 2, 1], [0, 2, 3], [0, 1, 3], [.5, .5, 1.]) == O.EINVAL        # decreasing
    assert v([0, 1, 3], [0, 2, 4], [0, 1, 3], [.5, .5, 1.]) == O.EINVAL        # past the arrays
    # entries at or beyond group_pair_ptr[G] are unused capacity, never read:
    # bad ids, repeats and NaN there change nothing
    assert v([0, 1, 3], [0, 2, 2], [0, 1, 3], [.5, .5, 1.]) == O.OK
    assert v([0, 1, 3], [0, 1, 2], [0, 1, -1, 9, 1], [.5, .5, np.nan, 1., 2.]) == O.OK
    assert v([0, 1, 3], [0, 1, 2], [0, -1, 2], [.5, .5, 1.]) == O.EINVAL       # inside: still checked
    assert v([0, 1, 3], [0, 2, 3], [0, 4, 3], [.5, .5, 1.]) == O.EINVAL        # id >= N
    assert v([0, 1, 3], [0, 2, 3], [0, -1, 3], [.5, .5, 1.]) == O.EINVAL       # id < 0
    assert v([0, 1, 3], [0, 2, 3], [1, 1, 3], [.5, .5, 1.]) == O.EINVAL        # duplicate
    assert v([0, 1, 3], [0, 2, 3], [0, 1, 3], [.5, np.nan, 1.]) == O.EINVAL    # nan
    assert v([0, 1, 3], [0, 2, 3], [0, 1, 3], [.5, np.inf, 1.]) == O.EINVAL    # inf
    assert v(*good, max_pairs_per_group=1) == O.EUNSUPPORTED
    assert v(*good, max_tuples=3) == O.ENOSPC                                  # P = 2 + 2
    assert v(*good, max_tuples=4) == O.OK
    assert v([0, 1, 3], [0, 2, 3], [1, 1, 3], [.5, .5, 1.], max_tuples=0) == O.EINVAL
    assert v([0], [0], [], [], T=0) == O.OK                                    # empty batch
    # a group beyond the pair limit is EUNSUPPORTED even when it repeats an
    # adapter; an EINVAL elsewhere in the table still outranks it
    assert v([0, 1, 3], [0, 2, 3], [1, 1, 3], [.5, .5, 1.], max_pairs_per_group=1) \
        == O.EUNSUPPORTED
    assert v([0, 1, 3], [0, 2, 3], [1, 1, 3], [.5, np.nan, 1.], max_pairs_per_group=1) \
        == O.EINVAL
    assert v([0, 1, 3], [0, 2, 3], [1, 2, 3], [.5, .5, 1.], max_pairs_per_group=1) \
        == O.EUNSUPPORTED


def pin_gate(O):
    """The token-level gate (DyMerge-LoRA, section 3.1 dynamic composition,
    section 5.1 Sparse workload): top-k of the softmax of the gate logits over
    a token's valid candidates, not renormalised, ties to the earlier
    candidate."""
    rng = np.random.default_rng(71)
    T, C, k = 40, 8, 2
    lg = rng.standard_normal((T, C))
    cand = np.stack([rng.permutation(100)[:C] for _ in range(T)]).astype(np.int64)
    gtp, gpp, pa, pw = O.gate_topk(lg, cand, k)
    assert np.array_equal(gtp, np.arange(T + 1)) and np.array_equal(gpp, np.arange(T + 1) * k)
    # library routines: torch.topk picks the indices, torch.softmax the weights
    lt = torch.tensor(lg, dtype=torch.float64)
    idx = torch.topk(lt, k, dim=1).indices.numpy()
    sm = torch.softmax(lt, dim=1).numpy()
    for t in range(T):
        assert pa[t * k:(t + 1) * k].tolist() == cand[t, idx[t]].tolist(), t
        assert np.allclose(pw[t * k:(t + 1) * k], sm[t, idx[t]], rtol=1e-13, atol=0), t
    # keeping every candidate: the weights are the whole softmax, in
    # descending order, summing to 1
    _, _, pa2, pw2 = O.gate_topk(lg, cand, C)
    w2 = pw2.reshape(T, C)
    assert np.allclose(w2.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w2, axis=1) <= 0)
    # a common shift of the logits changes nothing
    _, _, pa3, pw3 = O.gate_topk(lg + 3.75, cand, k)
    assert np.array_equal(pa3, pa) and np.allclose(pw3, pw, rtol=1e-13, atol=0)
    # ties go to the earlier candidate; equal logits give equal weights
    _, _, pa4, pw4 = O.gate_topk([[1.0, 1.0, 1.0, 0.0]], [[10, 11, 12, 13]], 2)
    e = np.e
    assert pa4.tolist() == [10, 11]
    assert np.allclose(pw4, [e / (3 * e + 1)] * 2, rtol=1e-15, atol=0)
    # padding (-1) is not a candidate: the same as the compacted list
    _, _, pa5, pw5 = O.gate_topk([[0.3, 9.0, -0.2, 0.7]], [[4, -1, 6, 8]], 2)
    _, _, pa6, pw6 = O.gate_topk([[0.3, -0.2, 0.7]], [[4, 6, 8]], 2)
    assert np.array_equal(pa5, pa6) and np.allclose(pw5, pw6, rtol=1e-15, atol=0)
    # fewer valid candidates than k: a shorter pair list (one valid
    # candidate keeps weight 1); none: an empty composite; the arrays keep
    # T * k entries, the unused tail adapter -1 and weight 0
    g7, gp7, pa7, pw7 = O.gate_topk([[0.5, 0.0, 0.0]], [[5, -1, -1]], 2)
    assert gp7.tolist() == [0, 1] and pa7.tolist() == [5, -1] and pw7.tolist() == [1.0, 0.0]
    assert O.validate(g7, gp7, pa7, pw7, 1, 6) == O.OK
    g9, gp9, pa9, pw9 = O.gate_topk([[0.1, 0.2], [0.3, 0.4], [1.0, 2.0]],
                                    [[-1, -1], [7, -1], [3, 4]], 2)
    assert gp9.tolist() == [0, 0, 1, 3] and pa9.tolist() == [7, 4, 3, -1, -1, -1]
    e1 = 1.0 / (1.0 + np.exp(-1.0))
    assert np.allclose(pw9[:3], [1.0, e1, 1.0 - e1], rtol=1e-15, atol=0)
    assert O.validate(g9, gp9, pa9, pw9, 3, 8) == O.OK
    # the unused tail is not part of the table: the plan equals that of the
    # trimmed arrays, and the empty token is left as it was
    trim = (g9, gp9, pa9[:3], pw9[:3])
    full, cut = O.plan(g9, gp9, pa9, pw9), O.plan(*trim)
    assert all(np.array_equal(full[key], cut[key]) for key in cut)
    Ag = np.ones((8, 1, 2))
    Bg = np.ones((8, 1, 2))
    xg = np.ones((3, 2))
    y0 = np.zeros((3, 2))
    yg, _ = O.apply(g9, gp9, pa9, pw9, Ag, Bg, None, xg, y0)
    assert np.array_equal(yg[0], [0.0, 0.0])
    assert np.allclose(yg[1], [2.0, 2.0]) and np.allclose(yg[2], [2.0, 2.0])
    # a non-finite logit: k pairs of adapter -1, a table the mapping rejects
    g8, gp8, pa8, pw8 = O.gate_topk([[float("nan"), 0.0]], [[5, 6]], 2)
    assert gp8.tolist() == [0, 2] and pa8.tolist() == [-1, -1] and pw8.tolist() == [0.0, 0.0]
    assert O.validate(g8, gp8, pa8, pw8, 1, 7) == O.EINVAL
    # brute force on small cases: the kept set has the largest total weight
    # of all k-subsets
    from itertools import combinations
    for trial in range(20):
        n = int(rng.integers(3, 7))
        kk = int(rng.integers(1, n + 1))
        l1 = rng.standard_normal((1, n))
        c1 = np.arange(n)[None, :]
        _, _, a1, w1 = O.gate_topk(l1, c1, kk)
        p1 = np.exp(l1[0] - l1[0].max()) / np.exp(l1[0] - l1[0].max()).sum()
        best = max(combinations(range(n), kk), key=lambda S: sum(p1[i] for i in S))
        assert sorted(a1.tolist()) == sorted(best), trial


def pin_factor(O):
    """Balanced factor construction (LoRAForge, approach (3)) against the
    library SVD of the explicit product: same singular values, the first k
    directions give the Eckart-Young truncation for every k, F T = X Y, and
    F^T F = T T^T = diag(sigma)."""
    rng = np.random.default_rng(81)
    for trial, (r, d_out, d_in) in enumerate([(4, 40, 24), (8, 96, 64), (16, 130, 70), (1, 9, 5)]):
        scale = 0.8 ** np.arange(r)
        Bt = rng.standard_normal((r, d_out)) * scale[:, None]
        At = rng.standard_normal((r, d_in))
        F_t, T, sigma = O.factor_balanced(Bt, At)
        D = Bt.T @ At
        U, S, Vt = np.linalg.svd(D)
        assert np.allclose(sigma, S[:r], rtol=1e-10, atol=0), trial
        assert np.all(np.diff(sigma) <= 0)
        assert np.allclose(F_t.T @ T, D, rtol=0, atol=1e-12 * S[0]), trial
        assert np.allclose(F_t @ F_t.T, np.diag(sigma), rtol=0, atol=1e-12 * S[0]), trial
        assert np.allclose(T @ T.T, np.diag(sigma), rtol=0, atol=1e-12 * S[0]), trial
        for k in range(1, r + 1):
            trunc = (U[:, :k] * S[:k]) @ Vt[:k]
            assert np.allclose(F_t[:k].T @ T[:k], trunc, rtol=0, atol=1e-11 * S[0]), (trial, k)
    # closed form: B with orthogonal columns of norms 3, 2 and A with
    # orthonormal columns give sigma = (3, 2) and balanced factors
    # sqrt(3) e_0 (x) a_0 and sqrt(2) e_1 (x) a_1, up to the sign of each
    Bt = np.zeros((2, 5))
    Bt[0, 0], Bt[1, 1] = 2.0, 3.0
    At = np.zeros((2, 4))
    At[0, 2], At[1, 3] = 1.0, 1.0
    F_t, T, sigma = O.factor_balanced(Bt, At)
    assert np.allclose(sigma, [3.0, 2.0], rtol=1e-15, atol=0)
    s0 = np.sign(F_t[0, 1])
    assert np.allclose(F_t[0] * s0, [0, np.sqrt(3), 0, 0, 0], atol=1e-15)
    assert np.allclose(T[0] * s0, [0, 0, 0, np.sqrt(3)], atol=1e-15)
    s1 = np.sign(F_t[1, 0])
    assert np.allclose(F_t[1] * s1, [np.sqrt(2), 0, 0, 0, 0], atol=1e-15)
    assert np.allclose(T[1] * s1, [0, 0, np.sqrt(2), 0], atol=1e-15)
    # rank-deficient B (a repeated column): the dead direction is exactly
    # zero and the live ones still reproduce the product
    Bt = rng.standard_normal((4, 30))
    Bt[3] = Bt[1]
    At = rng.standard_normal((4, 20))
    F_t, T, sigma = O.factor_balanced(Bt, At)
    S = np.linalg.svd(Bt.T @ At, compute_uv=False)
    assert sigma[3] == 0.0 and not F_t[3].any() and not T[3].any()
    assert np.allclose(sigma[:3], S[:3], rtol=1e-10, atol=0)
    assert np.allclose(F_t.T @ T, Bt.T @ At, rtol=0, atol=1e-12 * S[0])
    # fewer output rows than the rank: the spectrum is the product's, padded
    # with zeros, and the factors still reproduce it
    Bt = rng.standard_normal((6, 3))
    At = rng.standard_normal((6, 10))
    F_t, T, sigma = O.factor_balanced(Bt, At)
    S = np.linalg.svd(Bt.T @ At, compute_uv=False)
    assert F_t.shape == (6, 3) and T.shape == (6, 10)
    assert np.allclose(sigma[:3], S[:3], rtol=1e-10, atol=0) and not sigma[3:].any()
    assert np.allclose(F_t.T @ T, Bt.T @ At, rtol=0, atol=1e-12 * S[0])
    # bf16 bit patterns are widened exactly first
    bits = (np.arange(12, dtype=np.uint32).reshape(2, 6) * 613 + 0x3f00).astype(np.uint16)
    a_bits = (np.arange(8, dtype=np.uint32).reshape(2, 4) * 977 + 0x3e80).astype(np.uint16)
    f1 = O.factor_balanced(bits, a_bits)
    f2 = O.factor_balanced(O.widen(bits), O.widen(a_bits))
    assert all(np.array_equal(u, v) for u, v in zip(f1, f2))


def pin_rank_allocation(O):
    """LoRAForge-U and LoRAForge-S (LoRAForge, approach (2)).  U: a worked
    example.  S: with equal costs the kept directions are the budget's worth
    of largest sigma^2, which brute force over every prefix choice confirms
    is the least discarded energy; with unequal costs, a hand-worked
    example."""
    assert O.uniform_ranks([16, 8, 12, 4, 24], 12).tolist() == [1, 1, 1, 1, 2]
    assert O.uniform_ranks([64, 32], 8).tolist() == [8, 4]
    assert O.uniform_budget([16, 24], [10, 7], 12) == 1 * 10 + 2 * 7
    from itertools import product
    rng = np.random.default_rng(83)
    for trial in range(30):
        M = int(rng.integers(2, 4))
        r = [int(rng.integers(1, 5)) for _ in range(M)]
        sig = [np.sort(rng.random(rm))[::-1] for rm in r]
        c = 3
        floors = [int(rng.integers(0, 2)) for _ in range(M)]
        budget = c * int(rng.integers(sum(floors), sum(r) + 2))
        k = O.spectral_ranks(sig, [c] * M, budget, floors)
        best, best_k = None, None
        for ks in product(*[range(rm + 1) for rm in r]):
            if any(ks[m] < floors[m] for m in range(M)) or c * sum(ks) > budget:
                continue
            lost = sum(float(np.sum(sig[m][ks[m]:] ** 2)) for m in range(M))
            if best is None or lost < best - 1e-15:
                best, best_k = lost, ks
        assert tuple(k.tolist()) == best_k, (trial, k, best_k)
    # unequal costs by hand: module 0 costs 10 with sigma (4, 3, 1), eta
    # 1.6, 0.9, 0.1; module 1 costs 4 with sigma (3, 2, 2), eta 2.25, 1.0,
    # 1.0.  Floors (1, 0), so 10 of the budget is spent first; then the
    # visiting order is (1,0) (1,1) (1,2) (0,1) (0,2).
    sg, cs = [[4.0, 3.0, 1.0], [3.0, 2.0, 2.0]], [10, 4]
    # budget 30: 20 left -> 16, 12, 8; (0,1) needs 10: skipped; (0,2) would
    # leave a gap
    assert O.spectral_ranks(sg, cs, 30, [1, 0]).tolist() == [1, 3]
    # budget 32: 22 left -> 18, 14, 10, (0,1) fits exactly -> 0
    assert O.spectral_ranks(sg, cs, 32, [1, 0]).tolist() == [2, 3]
    # budget 41: 31 -> 27, 23, 19, 9; (0,2) needs 10.  Budget 42: all kept
    assert O.spectral_ranks(sg, cs, 41, [1, 0]).tolist() == [2, 3]
    assert O.spectral_ranks(sg, cs, 42, [1, 0]).tolist() == [3, 3]
    # budget 21: 11 -> 7, 3; (1,2) needs 4: skipped
    assert O.spectral_ranks(sg, cs, 21, [1, 0]).tolist() == [1, 2]
    # a skipped expensive direction does not stop cheaper ones: with sigma
    # (4, 3.5) module 0's second direction (eta 1.225) comes before module
    # 1's (1.0).  Budget 23: 13 left -> (1,0) 9; (0,1) needs 10: skipped;
    # (1,1) 5; (1,2) 1.  Budget 24: 14 -> 10; (0,1) fits -> 0.
    sg2 = [[4.0, 3.5], [3.0, 2.0, 2.0]]
    assert O.spectral_ranks(sg2, cs, 23, [1, 0]).tolist() == [1, 3]
    assert O.spectral_ranks(sg2, cs, 24, [1, 0]).tolist() == [2, 1]
    # floors above the budget are kept, and nothing else is
    k = O.spectral_ranks([[4.0, 3.0], [3.0, 2.0]], [10, 4], 5, [1, 1])
    assert k.tolist() == [1, 1]
    # a floor beyond a module's rank keeps all of it
    k = O.spectral_ranks([[4.0], [3.0, 2.0]], [10, 4], 100, [3, 0])
    assert k.tolist() == [1, 2]


def pin_bam(O):
    """BAM (DyMerge-LoRA, section 4): a hand-worked replay; residency
    invariants on a random stream; single-adapter batches reduce to a
    textbook LRU cache (collections.OrderedDict); enough slots means no
    evictions."""
    from collections import OrderedDict
    # two slots.  t0 [1, 2]: empty slots 0, 1.  t1 [3]: both last used at 0,
    # the lower slot goes (adapter 1 out).  t2 [1, 4]: 1 takes slot 1 (used
    # at 0, older than slot 0's 1), then 4 takes slot 0 (3 out).  t3 [5, 6,
    # 7]: three adapters, two slots: rejected, nothing changes.  t4 [2]:
    # slots used at 2 and 2: slot 0 (adapter 4) goes.
    recs, final = O.bam_run(2, [[1, 2], [3], [1, 4], [5, 6, 7], [2]])
    assert [r[0] for r in recs] == [O.OK, O.OK, O.OK, O.ENOSPC, O.OK]
    assert recs[0][2] == [(0, 1, -1), (1, 2, -1)]
    assert recs[1][2] == [(0, 3, 1)]
    assert recs[2][1] == {1: 1, 4: 0} and recs[2][2] == [(1, 1, 2), (0, 4, 3)]
    assert recs[3][1] == {} and recs[4][2] == [(0, 2, 4)] and final == [2, 1]
    # a hit is pinned before any load: [1, 9] with 1 resident never evicts 1
    recs, _ = O.bam_run(2, [[1], [2], [9, 1]])
    assert recs[2][1] == {1: 0, 9: 1} and recs[2][2] == [(1, 9, 2)]
    rng = np.random.default_rng(91)
    for trial in range(20):
        S, A = int(rng.integers(1, 6)), int(rng.integers(2, 12))
        batches = [list(rng.integers(0, A, int(rng.integers(1, 5)))) for _ in range(40)]
        recs, final = O.bam_run(S, batches)
        # replay the records to rebuild the pool and check every step
        pool = [-1] * S
        for b, (st, where, loads) in zip(batches, recs):
            distinct = set(int(a) for a in b)
            before = set(a for a in pool if a >= 0)
            if st != O.OK:
                assert len(distinct) > S and where == {} and loads == []
                continue
            assert set(where) == distinct
            assert [ld[1] for ld in loads] == [a for a in dict.fromkeys(int(x) for x in b)
                                               if a not in before]
            empty_before = pool.count(-1)
            for sl, a, ev in loads:
                assert pool[sl] == ev and ev not in distinct
                pool[sl] = a
            assert sum(1 for ld in loads if ld[2] >= 0) == max(0, len(loads) - empty_before)
            assert all(pool[where[a]] == a for a in distinct)
            assert len(set(a for a in pool if a >= 0)) == S - pool.count(-1)
        assert pool == final
        # single-adapter batches: the textbook LRU cache of S entries
        seq = [int(x) for x in rng.integers(0, A, 60)]
        recs, final = O.bam_run(S, [[a] for a in seq])
        lru = OrderedDict()
        for a, (st, where, loads) in zip(seq, recs):
            hit = a in lru
            evicted = -1
            if hit:
                lru.move_to_end(a)
            else:
                if len(lru) == S:
                    evicted = lru.popitem(last=False)[0]
                lru[a] = True
            assert st == O.OK
            assert loads == [] if hit else [ld[1:] for ld in loads] == [(a, evicted)]
        assert set(a for a in final if a >= 0) == set(lru)
        # slots for every adapter: nothing is ever evicted
        recs, _ = O.bam_run(A, batches[:10])
        assert all(ev == -1 for st, _, loads in recs for _, _, ev in loads)


def pin_lag(O):
    """LAG (DyMerge-LoRA, section 4): hand-worked batches; with every
    request waiting too long it is FIFO under the slot limit; with every
    adapter resident it is arrival order; without starvation the first pick
    has the fewest new loads of all requests (brute force)."""
    # now 10, theta 5: request 0 (arrived at 0) has waited too long and goes
    # first; then request 3 needs nothing new (5 is resident), request 2
    # needs 4, request 1 needs 2 and 3
    assert O.lag_select(10.0, 5.0, [0, 8, 9, 9.5], [[1], [2, 3], [1, 4], [5]], [1, 5], 2, 4) == [0, 3]
    assert O.lag_select(10.0, 5.0, [0, 8, 9, 9.5], [[1], [2, 3], [1, 4], [5]], [1, 5], 3, 4) == [0, 3, 2]
    # an adapter brought in by the batch is free for later picks: after
    # request 1 loads 2 and 3, request 4 (adapter 3) needs nothing
    got = O.lag_select(0.0, 9.0, [0, 1, 2, 3, 4], [[7, 8], [2, 3], [6], [5, 4], [3]], [], 3, 8)
    # fewest new loads: 2 (one), 4 (one; arrival 4 > 2) -> 2 first; then 4
    # (one: adapter 3), then 1 (one: adapter 2, since 3 is now in the batch)
    assert got == [2, 4, 1], got
    # slots limit: a request whose adapters would overflow is skipped
    assert O.lag_select(0.0, 9.0, [0, 1, 2], [[1, 2, 3], [4], [5]], [], 3, 2) == [1, 2]
    rng = np.random.default_rng(93)
    for trial in range(30):
        n, A = int(rng.integers(1, 9)), int(rng.integers(2, 10))
        arr = list(np.round(rng.random(n) * 10, 1))
        ads = [list(set(int(a) for a in rng.integers(0, A, int(rng.integers(1, 4))))) for _ in range(n)]
        B, S = int(rng.integers(1, 5)), int(rng.integers(1, 6))
        res = list(set(int(a) for a in rng.integers(0, A, 3)))
        # every request waiting too long: FIFO, each taken if it fits
        got = O.lag_select(100.0, -1.0, arr, ads, res, B, S)
        fifo, inb = [], set()
        for i in sorted(range(n), key=lambda i: (arr[i], i)):
            if len(fifo) < B and len(inb | set(ads[i])) <= S:
                fifo.append(i)
                inb |= set(ads[i])
        assert got == fifo, (trial, got, fifo)
        # every adapter resident and slots for all: arrival order
        got = O.lag_select(0.0, 1e9, arr, ads, list(range(A)), B, A)
        assert got == sorted(range(n), key=lambda i: (arr[i], i))[:B]
        # no starvation: the first pick has the fewest new loads (brute force)
        got = O.lag_select(0.0, 1e9, arr, ads, res, B, S)
        feas = [i for i in range(n) if len(ads[i]) <= S]
        if feas:
            best = min(len(set(ads[i]) - set(res)) for i in feas)
            assert len(set(ads[got[0]]) - set(res)) == best
        assert len(got) <= B and len(set(got)) == len(got)
        assert len(set(a for i in got for a in ads[i])) <= S


ALL_PINS = [pin_x1_elora_example, pin_x2_dense_premerge, pin_x3_textbook_lora,
            pin_x4_linearity, pin_x5_noop, pin_x6_truncation, pin_x7_rank_bound,
            pin_x8_mapping, pin_x9_adapter_fraction, pin_x10_permutation,
            pin_split_and_rows, pin_validation, pin_gate,
            pin_factor, pin_rank_allocation, pin_bam, pin_lag]
