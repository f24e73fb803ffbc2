"""Seeded synthetic workloads for the composite multi-LoRA apply.

This module only draws inputs: adapter pools, effective ranks, per-token
composites (adapter id, weight alpha), activations x and base outputs y_base.
It performs none of the apply's arithmetic and is shared by the tests, the
benchmark and the oracle harness alike; both the GPU path and the CPU oracle
consume exactly the arrays produced here.

The five configurations follow the workload descriptions of the DyMerge-LoRA
page (section 5.1: Single / Distinct / Skewed / Sparse adapter assignment,
Llama-3 projection shapes, rank 8, bf16) and the LoRAForge page (retained-rank
exports with a per-module effective rank k_m).  The public traces and adapter
fleets those pages evaluate on are not available; these draws stand in for
them.

Conventions
-----------
* bf16 tensors are carried as ``uint16`` bit patterns (numpy has no bfloat16);
  values are produced in float32 and rounded to bf16 with round-to-nearest-even.
* Pools are stored rank-major: ``A_t[a, j, :]`` is row j of A_a^T (length
  d_in) and ``B_t[a, j, :]`` is row j of B_a^T (length d_out), so the first k
  rows of an adapter are its retained prefix.
* Composites are a CSR over *groups*: group g covers tokens
  ``group_tok_ptr[g] .. group_tok_ptr[g+1]-1`` and owns pairs
  ``group_pair_ptr[g] .. group_pair_ptr[g+1]-1``.  Every configuration below
  uses one group per token (token-level composition); request-level groups
  (static composition) are produced by :func:`regroup_by_request`.
* One ``numpy.random.default_rng(seed)`` (PCG64) per configuration, consumed in
  the fixed order: pools (module order, A_t then B_t) -> effective ranks ->
  composites -> alpha -> x -> y_base.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even) and return the bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Module:
    """One projection's adapter pool (d_in -> d_out)."""
    name: str
    d_in: int
    d_out: int
    r_max: int
    A_t: np.ndarray            # [N, r_max, d_in]  uint16 (bf16 bits) or float32
    B_t: np.ndarray            # [N, r_max, d_out] uint16 (bf16 bits) or float32
    k: Optional[np.ndarray]    # [N] int32 effective ranks, or None (= r_max)

    def A_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.A_t) if self.A_t.dtype == np.uint16 else self.A_t

    def B_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.B_t) if self.B_t.dtype == np.uint16 else self.B_t


@dataclass
class Composites:
    """Group CSR of (adapter, alpha) pairs; see the module docstring."""
    n_tokens: int
    n_adapters: int
    group_tok_ptr: np.ndarray   # [G+1] int32
    group_pair_ptr: np.ndarray  # [G+1] int32
    pair_adapter: np.ndarray    # [n_pairs] int32
    pair_alpha: np.ndarray      # [n_pairs] float32

    @property
    def n_groups(self) -> int:
        return int(self.group_tok_ptr.shape[0] - 1)

    @property
    def n_pairs(self) -> int:
        return int(self.pair_adapter.shape[0])

    def n_tuples(self) -> int:
        """Number of (token, pair) tuples the composites expand to."""
        tl = np.diff(self.group_tok_ptr.astype(np.int64))
        pl = np.diff(self.group_pair_ptr.astype(np.int64))
        return int((tl * pl).sum())

    def max_pairs_per_group(self) -> int:
        pl = np.diff(self.group_pair_ptr.astype(np.int64))
        return int(pl.max()) if pl.size else 0


@dataclass
class Workload:
    name: str
    dtype: str                       # "bf16" (bf16 x/A/B, fp32 y) or "f32"
    n_adapters: int
    composites: Composites
    modules: List[Module]
    x: List[np.ndarray]              # per module [T, d_in] uint16 bits or float32
    y_base: List[np.ndarray]         # per module [T, d_out] float32
    n_prefill: int = 0               # tokens [0, n_prefill) are prefill (dispatch hint only)
    meta: dict = field(default_factory=dict)

    def x_f32(self, m: int) -> np.ndarray:
        xm = self.x[m]
        return bf16_bits_to_f32(xm) if xm.dtype == np.uint16 else xm

    @property
    def n_tokens(self) -> int:
        return self.composites.n_tokens


def csr_from_token_lists(adapters: List[List[int]], alphas: List[List[float]],
                         n_adapters: int) -> Composites:
    """One group per token, pairs in the order given."""
    T = len(adapters)
    tok_ptr = np.arange(T + 1, dtype=np.int32)
    counts = np.array([len(a) for a in adapters], dtype=np.int64)
    pair_ptr = np.zeros(T + 1, dtype=np.int32)
    pair_ptr[1:] = np.cumsum(counts)
    flat_a = np.array([a for row in adapters for a in row], dtype=np.int32)
    flat_w = np.array([w for row in alphas for w in row], dtype=np.float32)
    return Composites(T, n_adapters, tok_ptr, pair_ptr, flat_a, flat_w)


def regroup_by_request(c: Composites, tokens_per_group: int) -> Composites:
    """Static (request-level) composition: consecutive runs of
    ``tokens_per_group`` tokens share the composite of their first token."""
    T = c.n_tokens
    starts = list(range(0, T, tokens_per_group))
    tok_ptr = np.array(starts + [T], dtype=np.int32)
    pair_ptr = [0]
    ad, al = [], []
    for t0 in starts:
        g = int(np.searchsorted(c.group_tok_ptr, t0, side="right") - 1)
        lo, hi = int(c.group_pair_ptr[g]), int(c.group_pair_ptr[g + 1])
        ad.extend(c.pair_adapter[lo:hi].tolist())
        al.extend(c.pair_alpha[lo:hi].tolist())
        pair_ptr.append(len(ad))
    return Composites(T, c.n_adapters, tok_ptr, np.array(pair_ptr, dtype=np.int32),
                      np.array(ad, dtype=np.int32), np.array(al, dtype=np.float32))


def zipf_probs(n: int, s: float) -> np.ndarray:
    """p(rank k) proportional to k^-s over k = 1..n; adapter id = rank - 1."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def _normal(rng, shape, std, dtype_out):
    v = rng.standard_normal(size=shape, dtype=np.float32)
    v *= np.float32(std)
    return f32_to_bf16_bits(v) if dtype_out == BF16 else v


def _make_pool(rng, name, N, r, d_in, d_out, dtype, std=0.02) -> Module:
    A = _normal(rng, (N, r, d_in), std, dtype)
    B = _normal(rng, (N, r, d_out), std, dtype)
    return Module(name, d_in, d_out, r, A, B, None)


def _x(rng, T, d, dtype):
    return _normal(rng, (T, d), 1.0, dtype)


def _ybase(rng, T, d):
    return rng.standard_normal(size=(T, d), dtype=np.float32)


# --------------------------------------------------------------------------
# the five configurations
# --------------------------------------------------------------------------

def config1(seed: int = 0) -> Workload:
    """Tiny fp32 case: 256->256, N=4 adapters of rank 8, 16 tokens, each token
    1-3 distinct adapters drawn uniformly, alpha ~ U[0,1)."""
    rng = np.random.default_rng(seed)
    N, r, d, T = 4, 8, 256, 16
    mod = _make_pool(rng, "proj", N, r, d, d, F32)
    ads = []
    for _ in range(T):
        n = int(rng.integers(1, 4))
        ads.append(rng.choice(N, n, replace=False).tolist())
    als = [rng.random(len(a)).astype(np.float32).tolist() for a in ads]
    comp = csr_from_token_lists(ads, als, N)
    x = [_x(rng, T, d, F32)]
    yb = [_ybase(rng, T, d)]
    return Workload("tiny_f32_256", F32, N, comp, [mod], x, yb, n_prefill=0)


def config2(seed: int = 0) -> Workload:
    """Distinct decode: q_proj 4096->4096, 64 adapters rank 8 bf16, 32 tokens,
    3 non-overlapping adapters per token, alpha = softmax of N(0,1) logits.

    32 x 3 = 96 > 64 adapters, so global disjointness is impossible: tokens take
    consecutive triples from a random permutation of the pool, drawing a fresh
    permutation when fewer than 3 ids remain."""
    rng = np.random.default_rng(seed)
    N, r, d, T = 64, 8, 4096, 32
    mod = _make_pool(rng, "q_proj", N, r, d, d, BF16)
    ads = []
    perm = rng.permutation(N).tolist()
    pos = 0
    for _ in range(T):
        if N - pos < 3:
            perm = rng.permutation(N).tolist()
            pos = 0
        ads.append(perm[pos:pos + 3])
        pos += 3
    als = []
    for _ in range(T):
        lg = rng.standard_normal(3)
        e = np.exp(lg - lg.max())
        als.append((e / e.sum()).astype(np.float32).tolist())
    comp = csr_from_token_lists(ads, als, N)
    x = [_x(rng, T, d, BF16)]
    yb = [_ybase(rng, T, d)]
    return Workload("distinct_decode_q4096_n64_r8_t32", BF16, N, comp, [mod], x, yb)


LLAMA3_8B_PROJ = [
    ("q_proj", 4096, 4096), ("k_proj", 4096, 1024), ("v_proj", 4096, 1024),
    ("o_proj", 4096, 4096), ("gate_proj", 4096, 14336), ("up_proj", 4096, 14336),
    ("down_proj", 14336, 4096),
]


def config3(seed: int = 0) -> Workload:
    """Skewed decode: the seven Llama-3-8B projections, 128 adapters rank 8
    bf16 per projection, 64 tokens, 2-5 adapters per token drawn Zipf(s=1.5)
    without replacement, alpha ~ U[0,1); one composite table for all modules."""
    rng = np.random.default_rng(seed)
    N, r, T = 128, 8, 64
    mods = [_make_pool(rng, nm, N, r, di, do, BF16) for nm, di, do in LLAMA3_8B_PROJ]
    p = zipf_probs(N, 1.5)
    ads = []
    for _ in range(T):
        n = int(rng.integers(2, 6))
        ads.append(rng.choice(N, n, replace=False, p=p).tolist())
    als = [rng.random(len(a)).astype(np.float32).tolist() for a in ads]
    comp = csr_from_token_lists(ads, als, N)
    x = [_x(rng, T, m.d_in, BF16) for m in mods]
    yb = [_ybase(rng, T, m.d_out) for m in mods]
    return Workload("skewed_decode_llama3_8b_7proj_n128_r8_t64", BF16, N, comp, mods, x, yb)


def config4(seed: int = 0) -> Workload:
    """Sparse prefill with token-level gating: 8 requests x 256 tokens,
    4096->4096 and 4096->14336, N=128 adapters rank 16 bf16.  Each request
    references 5-8 adapters (uniform, without replacement); every token draws
    N(0,1) gate logits over its request's referenced adapters, takes the
    softmax and keeps the two largest probabilities (not renormalised; ties go
    to the earlier reference) as its composite."""
    rng = np.random.default_rng(seed)
    N, r, R, L = 128, 16, 8, 256
    T = R * L
    mods = [_make_pool(rng, "q_proj", N, r, 4096, 4096, BF16),
            _make_pool(rng, "up_proj", N, r, 4096, 14336, BF16)]
    refs = []
    for _ in range(R):
        n = int(rng.integers(5, 9))
        refs.append(rng.choice(N, n, replace=False).tolist())
    ads, als = [], []
    # the gate's inputs as a device gate takes them: per token, the request's
    # referenced adapters padded with -1 to 8 candidates, and the logits
    cand = np.full((T, 8), -1, dtype=np.int32)
    logits = np.zeros((T, 8), dtype=np.float64)
    for q in range(R):
        ref = refs[q]
        for i in range(L):
            lg = rng.standard_normal(len(ref))
            t = q * L + i
            cand[t, :len(ref)] = ref
            logits[t, :len(ref)] = lg
            e = np.exp(lg - lg.max())
            pr = e / e.sum()
            order = np.argsort(-pr, kind="stable")[:2]
            ads.append([ref[i] for i in order])
            als.append([float(np.float32(pr[i])) for i in order])
    comp = csr_from_token_lists(ads, als, N)
    x = [_x(rng, T, m.d_in, BF16) for m in mods]
    yb = [_ybase(rng, T, m.d_out) for m in mods]
    return Workload("sparse_prefill_gated_8x256_n128_r16", BF16, N, comp, mods, x, yb,
                    n_prefill=T, meta={"refs": refs, "gate_candidates": cand,
                                       "gate_logits": logits, "gate_k": 2})


def config5(seed: int = 0, scale_tokens: float = 1.0) -> Workload:
    """Retained-rank mixed batch: N=256 adapters stored at r_max=32 bf16 with a
    per-(adapter, module) effective rank k ~ U{1..32}; rows j < k are
    N(0,0.02) scaled by 0.8^(j/2) (so pair j carries energy ~ 0.8^j, the
    geometric spectral decay), rows >= k are zero (zero-padded export).
    4096 prefill + 128 decode tokens, modules 8192->8192 and 8192->28672,
    1-4 adapters per token drawn Zipf(s=1.2), alpha ~ U[0,1).

    ``scale_tokens`` < 1 shrinks the token count proportionally (tests only)."""
    rng = np.random.default_rng(seed)
    N, r = 256, 32
    n_pre = int(round(4096 * scale_tokens))
    n_dec = int(round(128 * scale_tokens))
    T = n_pre + n_dec
    shapes = [("q_proj", 8192, 8192), ("up_proj", 8192, 28672)]
    mods = []
    for nm, di, do in shapes:
        A = rng.standard_normal(size=(N, r, di), dtype=np.float32)
        B = rng.standard_normal(size=(N, r, do), dtype=np.float32)
        mods.append([nm, di, do, A, B])
    decay = (np.float32(0.02) * (np.float32(0.8) ** (np.arange(r, dtype=np.float32) / 2))
             ).astype(np.float32)
    out = []
    for nm, di, do, A, B in mods:
        k = rng.integers(1, r + 1, size=N).astype(np.int32)
        keep = (np.arange(r)[None, :] < k[:, None]).astype(np.float32)
        fac = (keep * decay[None, :])[:, :, None]
        A *= fac
        B *= fac
        out.append(Module(nm, di, do, r, f32_to_bf16_bits(A), f32_to_bf16_bits(B), k))
        del A, B
    p = zipf_probs(N, 1.2)
    ads = []
    for _ in range(T):
        n = int(rng.integers(1, 5))
        ads.append(rng.choice(N, n, replace=False, p=p).tolist())
    als = [rng.random(len(a)).astype(np.float32).tolist() for a in ads]
    comp = csr_from_token_lists(ads, als, N)
    x = [_x(rng, T, m.d_in, BF16) for m in out]
    yb = [_ybase(rng, T, m.d_out) for m in out]
    return Workload("retained_rank_mixed_n256_r32_t4224", BF16, N, comp, out, x, yb,
                    n_prefill=n_pre)


# --------------------------------------------------------------------------
# retained-rank producer inputs (LoRAForge, approach (3); the Llama fleet of
# its Figure 1: 35 adapters, 7840 LoRA matrices = 35 x 32 layers x 7
# projections)
# --------------------------------------------------------------------------

# (name, d_in, d_out) of the Llama-3.1-8B projections
LLAMA31_8B_PROJ = [("q_proj", 4096, 4096), ("k_proj", 4096, 1024), ("v_proj", 4096, 1024),
                   ("o_proj", 4096, 4096), ("gate_proj", 4096, 14336),
                   ("up_proj", 4096, 14336), ("down_proj", 14336, 4096)]
FLEET_ADAPTERS, FLEET_LAYERS, FLEET_RANK = 35, 32, 16


def factor_batch(seed: int, M: int, r: int, d_out: int, d_in: int, decay: float = 0.85,
                 repeated_rows=()):
    """Synthetic LoRA factors for the producer, bf16 bits: B_t [M, r, d_out]
    and A_t [M, r, d_in].  A_t rows are N(0, 1/d_in) (the usual
    initialisation scale of A); B_t row j is N(0, 0.02^2) * decay^j, so the
    update's spectrum falls off with the direction like a trained adapter's.
    repeated_rows: B_t rows j that copy row 0, leaving B without full rank."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, r, d_in), dtype=np.float32) * np.float32(1.0 / np.sqrt(d_in))
    B = rng.standard_normal((M, r, d_out), dtype=np.float32) * np.float32(0.02)
    B *= (np.float32(decay) ** np.arange(r, dtype=np.float32))[None, :, None]
    for j in repeated_rows:
        B[:, j] = B[:, 0]
    return f32_to_bf16_bits(B), f32_to_bf16_bits(A)



def factor_batch_torch(seed: int, M: int, r: int, d_out: int, d_in: int, device,
                       decay: float = 0.85):
    """The recipe of factor_batch drawn with torch's generator on `device`
    (fleet-sized batches, too large to draw and copy from the host): bf16
    tensors B_t [M, r, d_out] and A_t [M, r, d_in]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    A = torch.randn((M, r, d_in), generator=g, device=device) * (1.0 / float(np.sqrt(d_in)))
    B = torch.randn((M, r, d_out), generator=g, device=device) * 0.02
    B *= (decay ** torch.arange(r, device=device, dtype=torch.float32))[None, :, None]
    return B.to(torch.bfloat16), A.to(torch.bfloat16)

CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def make(cfg: int, seed: int = 0, **kw) -> Workload:
    return CONFIGS[cfg](seed, **kw)


# --------------------------------------------------------------------------
# small random cases for property and edge-case tests
# --------------------------------------------------------------------------

def random_case(seed: int, T: int, N: int, d_in: int, d_out: int, r_max: int,
                max_pairs: int, dtype: str = BF16, with_k: bool = False,
                tokens_per_group: int = 1, empty_frac: float = 0.0,
                std: float = 0.02) -> Workload:
    """A small random workload with arbitrary shapes (edge-case coverage).

    ``empty_frac`` of the tokens get an empty composite; with ``with_k`` each
    adapter gets an effective rank in [0, r_max] and rows >= k are zeroed."""
    rng = np.random.default_rng(seed)
    mod = _make_pool(rng, "proj", N, r_max, d_in, d_out, dtype, std)
    if with_k:
        k = rng.integers(0, r_max + 1, size=N).astype(np.int32)
        keep = (np.arange(r_max)[None, :] < k[:, None])[:, :, None]
        if dtype == BF16:
            mod.A_t = np.where(keep, mod.A_t, np.uint16(0)).astype(np.uint16)
            mod.B_t = np.where(keep, mod.B_t, np.uint16(0)).astype(np.uint16)
        else:
            mod.A_t = np.where(keep, mod.A_t, 0).astype(np.float32)
            mod.B_t = np.where(keep, mod.B_t, 0).astype(np.float32)
        mod.k = k
    ads = []
    for _ in range(T):
        if rng.random() < empty_frac:
            ads.append([])
            continue
        n = int(rng.integers(1, min(max_pairs, N) + 1))
        ads.append(rng.choice(N, n, replace=False).tolist())
    als = [rng.random(len(a)).astype(np.float32).tolist() for a in ads]
    comp = csr_from_token_lists(ads, als, N)
    if tokens_per_group > 1:
        comp = regroup_by_request(comp, tokens_per_group)
    x = [_x(rng, T, d_in, dtype)]
    yb = [_ybase(rng, T, d_out)]
    return Workload(f"random_s{seed}", dtype, N, comp, [mod], x, yb)
