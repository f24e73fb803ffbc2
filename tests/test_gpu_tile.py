"""The prefill expand over token tiles (tile_prep + expand_tile: the default
for bf16 batches of at least 256 tokens) against the fp64 oracle.

The cases reach every path of the two kernels: tiles with many union entries
(several hundred adapters), rank-64 adapters (eight octets each) and
zero-rank adapters, ragged token tiles and column blocks, every K-loop
step count from 1 to 14, tokens without pairs, static groups, split-K partial z rows, bf16 y, several modules in one
launch, and tiles beyond the record's limits (more than 1024 tuples, more
than 128 union entries, more than 1024 coefficient octets), whose jobs
run the per-token fp32 loop; those are also compared bit for bit with the
per-token expand kernel, which does the same arithmetic.  Rank rows at or
beyond an adapter's retained rank hold NaN in one case, so a read of any of
them would show.
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
    # about a hundred distinct adapters per tile (within the record's 128)
    "mx_wide_union": lambda: W.random_case(157, T=256, N=150, d_in=64, d_out=264, r_max=8,
                                           max_pairs=4),
    # rank-64 adapters with retained ranks in [0, 64]: up to 8 octets each,
    # unions of several chunks
    "mx_rank64": lambda: W.random_case(151, T=260, N=24, d_in=128, d_out=520, r_max=64,
                                       max_pairs=6, with_k=True),
    # half the tokens without pairs, ragged last tile and column tile
    "mx_empty": lambda: W.random_case(152, T=290, N=16, d_in=96, d_out=136, r_max=16,
                                      max_pairs=3, empty_frac=0.5),
    # rank-64 adapters at full rank, about 45 a tile: 330-400 K octets a tile
    # (more than 256), within the record
    "mx_octets": lambda: W.random_case(158, T=260, N=60, d_in=64, d_out=264, r_max=64,
                                       max_pairs=2),
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

# limits of a tile record (the kernel's constants)
MAX_Q, MAX_U, MAX_OCT, MAX_COEF = 1024, 128, 512, 1024

FALLBACK_CASES = {
    # more than 1024 tuples in a tile (up to 40 pairs a token)
    "fb_tuples": lambda: W.random_case(160, T=300, N=64, d_in=64, d_out=264, r_max=8,
                                       max_pairs=40),
    # more than 128 distinct adapters in a tile
    "fb_union": lambda: W.random_case(161, T=256, N=3000, d_in=64, d_out=136, r_max=4,
                                      max_pairs=16),
    # more than 1024 coefficient octets (rank 64, up to 16 pairs a token)
    "fb_coef": lambda: W.random_case(162, T=256, N=200, d_in=64, d_out=136, r_max=64,
                                     max_pairs=16, with_k=True),
}


def _case(name):
    if name in FALLBACK_CASES:
        return FALLBACK_CASES[name]()
    return MFMA_CASES[name]() if name in MFMA_CASES else CASES[name]()


def tile_order(c):
    """The plan's token order for the tiles: tokens with pairs, grouped by
    their rarest adapter (largest id of the composite), adapters ascending,
    in token order within an adapter."""
    owner = np.repeat(np.arange(c.n_groups), np.diff(c.group_tok_ptr))
    comps = [sorted(int(a) for a in c.pair_adapter[c.group_pair_ptr[g]:c.group_pair_ptr[g + 1]])
             for g in owner]
    busy = [t for t in range(c.n_tokens) if comps[t]]
    return sorted(busy, key=lambda t: (comps[t][-1], t)), comps


def tile_limits_hit(wl, mi=0):
    """Per 64-token tile of module mi (in the plan's tile order): (token
    rows of the tile, whether the record's limits send it to the per-token
    loop)."""
    c, m = wl.composites, wl.modules[mi]
    k = np.full(c.n_adapters, m.r_max) if m.k is None else m.k
    order, comps = tile_order(c)
    out = []
    for t0 in range(0, len(order), 64):
        rows = order[t0:t0 + 64]
        slots = [comps[t] for t in rows]
        Q = sum(len(s) for s in slots)
        union = sorted(set(a for s in slots for a in s))
        octs = lambda a: (int(k[a]) + 7) // 8
        H = sum(octs(a) for a in union)
        C = sum(octs(a) for s in slots for a in s)
        out.append((rows, Q > MAX_Q or len(union) > MAX_U or H > MAX_OCT or C > MAX_COEF))
    return out


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
        idle = np.nonzero(_pairs_per_token(wl.composites) == 0)[0]
        assert np.array_equal(ys[mi][idle], wl.y_base[mi][idle].astype(np.float64))


def _auto(monkeypatch, kchunk=None):
    monkeypatch.delenv("TCL_DISPATCH", raising=False)
    if kchunk is None:
        monkeypatch.delenv("TCL_KCHUNK", raising=False)
    else:
        monkeypatch.setenv("TCL_KCHUNK", str(kchunk))


TILE_NAMES = (["config4", "mfma_ragged", "mfma_ranks24", "mfma_static", "mfma_many_adapters",
               "one_adapter_300_tokens", "multi_ragged", "direct_400_groups"]
              + sorted(MFMA_CASES) + sorted(FALLBACK_CASES))


@pytest.mark.parametrize("name", TILE_NAMES)
def test_tile_expand_vs_oracle(name, monkeypatch):
    wl = _case(name)
    hit = [h for _, h in tile_limits_hit(wl)]
    banner(f"tile expand {name}: T={wl.n_tokens} N={wl.n_adapters} "
           f"P={wl.composites.n_tuples()} fallback tiles {sum(hit)}/{len(hit)}")
    if name in FALLBACK_CASES:
        assert any(hit)
    _auto(monkeypatch)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, "tile")


@pytest.mark.parametrize("name", ["mfma_ranks24", "mx_rank64", "mx_requests", "fb_tuples"])
def test_tile_expand_split_k(name, monkeypatch):
    """Partial z rows of a shrink split into 64-element chunks of d_in."""
    wl = _case(name)
    banner(f"tile expand with split-K partials {name}")
    _auto(monkeypatch, kchunk=64)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, "tile split-K")


@pytest.mark.parametrize("name", sorted(FALLBACK_CASES))
@pytest.mark.parametrize("kchunk", [None, 64])
def test_fallback_tiles_equal_per_token_kernel(name, kchunk, monkeypatch):
    """Tiles beyond the record's limits take the per-token fp32 loop, whose
    arithmetic is that of the per-token expand kernel: y bit for bit."""
    wl = _case(name)
    tiles = tile_limits_hit(wl)
    rows = np.array(sorted(t for r, h in tiles if h for t in r), np.int64)
    banner(f"fallback tiles vs per-token kernel {name} kchunk {kchunk}: "
           f"{sum(h for _, h in tiles)}/{len(tiles)} tiles, {len(rows)} tokens")
    assert len(rows) > 0
    _auto(monkeypatch, kchunk)
    ys, _, _ = run_fused(wl)
    monkeypatch.setenv("TCL_DISPATCH", "valu")
    yv, _, _ = run_fused(wl)
    assert np.array_equal(ys[0][rows], yv[0][rows])


def test_tile_expand_bf16_y(monkeypatch):
    """bf16 y: the base is bf16-exact, so the result is within half an ulp
    of the final rounding plus the bf16-mode tolerance of the oracle's."""
    wl = _case("mx_mixed")
    banner("tile expand with bf16 y")
    yb16 = [W.f32_to_bf16_bits(y) for y in wl.y_base]
    wl.y_base = [W.bf16_bits_to_f32(b) for b in yb16]
    _auto(monkeypatch)
    ys, _, _ = run_fused(wl, y_dtype=torch.bfloat16)
    for mi in range(len(wl.modules)):
        _, d_ora = oracle_apply(wl, mi)
        y_ora = wl.y_base[mi].astype(np.float64) + d_ora
        bound = np.abs(y_ora) * 2.0 ** -8 + TOL[W.BF16] * np.max(np.abs(d_ora))
        assert np.all(np.abs(ys[mi] - y_ora) <= bound), mi


@pytest.mark.parametrize("name", ["mx_rank64", "fb_coef"])
def test_tile_padding_rows_never_read(name, monkeypatch):
    """Rank rows at or beyond k hold NaN in both pools."""
    wl = _case(name)
    banner(f"tile expand, NaN padding rows {name}")
    m = wl.modules[0]
    pad = np.arange(m.r_max)[None, :, None] >= m.k[:, None, None]
    m.A_t = np.where(pad, BF16_NAN, m.A_t).astype(np.uint16)
    m.B_t = np.where(pad, BF16_NAN, m.B_t).astype(np.uint16)
    _auto(monkeypatch)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, "tile nan-padded")


def test_tile_config5_rows(monkeypatch):
    """The retained-rank batch at full size through the default dispatch:
    44 sampled tokens (prefill and decode) of both modules against the
    oracle, all columns."""
    import oracle as O
    from test_gpu_parity import cfg
    wl = cfg(5)
    c = wl.composites
    banner(f"tile expand on the full retained-rank batch: T={wl.n_tokens}")
    _auto(monkeypatch)
    ys, _, _ = run_fused(wl)
    rows = np.unique(np.concatenate([np.arange(0, 4224, 97), [4095, 4096, 4200, 4223]]))
    for mi, m in enumerate(wl.modules):
        want = O.apply_rows(c.group_tok_ptr, c.group_pair_ptr, c.pair_adapter, c.pair_alpha,
                            m.A_t, m.B_t, m.k, wl.x[mi], wl.y_base[mi], rows)
        base = wl.y_base[mi][rows].astype(np.float64)
        err = rel_err(ys[mi][rows] - base, want - base)
        print(f"  module {mi}: rel {err:.3e}", flush=True)
        assert err <= TOL[W.BF16]


def _two_modules(wl, seed):
    w2 = W.random_case(seed, T=wl.n_tokens, N=wl.n_adapters, d_in=136, d_out=264, r_max=8,
                       max_pairs=3, with_k=True)
    wl.modules.append(w2.modules[0])
    wl.x.append(w2.x[0])
    wl.y_base.append(w2.y_base[0])
    return wl


def _dense_and_sparse():
    """Four requests of 64 tokens over three adapters each, then 192 tokens
    over the whole pool of 64 adapters: tiles with small and large unions."""
    wl = W.random_case(166, T=448, N=64, d_in=384, d_out=200, r_max=16, max_pairs=4,
                       with_k=True)
    rng = np.random.default_rng(167)
    ads = []
    for _ in range(4):
        cand = rng.choice(64, 3, replace=False)
        for _ in range(64):
            ads.append(rng.choice(cand, int(rng.integers(1, 3)), replace=False).tolist())
    for _ in range(192):
        ads.append(rng.choice(64, int(rng.integers(2, 5)), replace=False).tolist())
    als = [rng.random(len(a)).astype(np.float32).tolist() for a in ads]
    wl.composites = W.csr_from_token_lists(ads, als, 64)
    return wl


REQUEST_CASES = {
    # requests of 64 tokens sharing one composite of up to 6 adapters
    "rq_requests": lambda: W.random_case(163, T=384, N=30, d_in=512, d_out=264, r_max=16,
                                         max_pairs=6, tokens_per_group=64, with_k=True),
    # two modules, d_in not a multiple of 32 and a ragged last tile
    "rq_two_modules": lambda: _two_modules(W.random_case(164, T=300, N=12, d_in=264, d_out=136,
                                                         r_max=16, max_pairs=3,
                                                         tokens_per_group=50, with_k=True), 165),
    # small-union and large-union tiles in one batch
    "rq_mixed": _dense_and_sparse,
}


@pytest.mark.parametrize("name", sorted(REQUEST_CASES))
def test_tile_expand_request_batches(name, monkeypatch):
    """Request-shaped prefill batches through the token-tile expand."""
    wl = REQUEST_CASES[name]()
    banner(f"tile expand {name}: T={wl.n_tokens} modules={len(wl.modules)}")
    assert wl.n_tokens >= 256
    _auto(monkeypatch)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, "tile")


def test_tile_expand_many_partial_planes(monkeypatch):
    """Ten K-chunk partial planes a tuple (rank 8, d_in 600 in chunks of 64):
    the expand sums a full group of eight planes and a ragged group of two."""
    wl = W.random_case(168, T=320, N=24, d_in=600, d_out=264, r_max=8, max_pairs=4, with_k=True)
    banner("tile expand, 10 partial planes")
    _auto(monkeypatch, kchunk=64)
    ys, _, _ = run_fused(wl)
    _check(wl, ys, "tile 10 planes")


def _step_count_case():
    """Fourteen 64-token tiles whose unions hold 4 g + 4 - (g mod 3) rank
    octets (g = 0..13): the K loop runs 1..14 steps of four octets, so whole
    groups of six steps run 0, 1 and 2 times and every tail length 0..5
    follows them, some with a last step of fewer than four octets.  Each
    tile is one request of its own adapters (each token holds two of them,
    or the one), ranks 8 o - 3 for o octets, rows at or beyond k NaN."""
    T, r_max = 14 * 64, 64
    octs, ads = [], []
    for g in range(14):
        H = 4 * (g + 1) - g % 3
        own = [8] * (H // 8) + ([H % 8] if H % 8 else [])
        base = len(octs)
        octs += own
        n = len(own)
        for i in range(64):
            ads.append([base + i % n] if n == 1 else [base + i % n, base + (i + 1) % n])
    N = len(octs)
    wl = W.random_case(169, T=T, N=N, d_in=64, d_out=264, r_max=r_max, max_pairs=2)
    rng = np.random.default_rng(169)
    als = [rng.random(len(a)).astype(np.float32).tolist() for a in ads]
    wl.composites = W.csr_from_token_lists(ads, als, N)
    m = wl.modules[0]
    m.k = np.array([8 * o - 3 for o in octs], np.int32)
    pad = np.arange(r_max)[None, :, None] >= m.k[:, None, None]
    m.A_t = np.where(pad, BF16_NAN, m.A_t).astype(np.uint16)
    m.B_t = np.where(pad, BF16_NAN, m.B_t).astype(np.uint16)
    return wl


@pytest.mark.parametrize("y16", [False, True])
def test_tile_expand_every_step_count(y16, monkeypatch):
    """The tile expand's K loop (whole groups of six steps, then the last
    steps after the loop) at 1..14 steps a tile, fp32 and bf16 y (the two
    instances of the kernel)."""
    wl = _step_count_case()
    c, m = wl.composites, wl.modules[0]
    order, comps = tile_order(c)
    steps = []
    for t0 in range(0, len(order), 64):
        union = sorted(set(a for t in order[t0:t0 + 64] for a in comps[t]))
        steps.append((sum((int(m.k[a]) + 7) // 8 for a in union) + 3) // 4)
    assert steps == list(range(1, 15)), steps
    assert not any(h for _, h in tile_limits_hit(wl))
    banner(f"tile expand, 1..14 K steps a tile (bf16 y {y16}): T={wl.n_tokens} N={wl.n_adapters}")
    _auto(monkeypatch)
    if not y16:
        ys, _, _ = run_fused(wl)
        _check(wl, ys, "tile steps 1..14")
        return
    wl.y_base = [W.bf16_bits_to_f32(W.f32_to_bf16_bits(y)) for y in wl.y_base]
    ys, _, _ = run_fused(wl, y_dtype=torch.bfloat16)
    _, d_ora = oracle_apply(wl, 0)
    y_ora = wl.y_base[0].astype(np.float64) + d_ora
    bound = np.abs(y_ora) * 2.0 ** -8 + TOL[W.BF16] * np.max(np.abs(d_ora))
    assert np.all(np.abs(ys[0] - y_ora) <= bound)
