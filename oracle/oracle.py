"""Plain fp64 CPU oracle for the batched composite multi-LoRA apply.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library
path never calls it, and it shares no code with the library: no kernels, no
headers, no helpers, no constants.  It is slow on purpose; every function is
the plainest statement of what the pages define.

What is computed (pages cited by title and section):

* DyMerge-LoRA, section 3.1 (M1): a composite update is the weighted sum of
  low-rank adapter updates, Delta W = sum_i alpha_i B_i A_i^T, with alpha fixed
  per request (static composition) or per token (dynamic composition).
  Evaluated after the merge point, token t receives
      y_t = y_base_t + sum_{(i, alpha) in C_t} alpha * B_i (A_i^T x_t).
* ELORA, section III-A, Eq. 1 / Eq. 2: the single-adapter case W' = W + A B.
  ELORA writes the update as A_t B_t with A_t of size d x r; in the
  orientation used here that is B_i (d_out x r) times A_i^T (r x d_in).
* LoRAForge, approach (1): the retained-rank contract.  Each adapter of a
  module keeps an ordered factor prefix and an effective rank k_m; only the
  first k_m rank directions take part and a padded store holds zeros beyond.
* DyMerge-LoRA, section 4.3: token-adapter pairs become mapping tuples and are
  reordered by adapter (LoRA) id so one adapter's tokens are contiguous.  The
  tuple's fields are not spelled out on the page; they are read here as
  (token, adapter, alpha, out-slot), with the out-slot being the pair's
  position inside its token's composite once that composite is ordered by
  adapter id, and ties in the reorder broken by (token, slot).

Storage conventions (shared by every consumer, stated not imported):
pools are rank-major, ``A_t[a, j, :]`` = row j of A_a^T (length d_in) and
``B_t[a, j, :]`` = row j of B_a^T (length d_out); bf16 arrays arrive as uint16
bit patterns and are widened exactly; composites are a group CSR
(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha).

Status codes returned by :func:`validate` use the same numbering as the
library's documented status codes so that the two can be compared.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

OK = 0
EINVAL = -1
ENOSPC = -3
EUNSUPPORTED = -4


# ---------------------------------------------------------------------------
# input handling
# ---------------------------------------------------------------------------

def widen(a: np.ndarray) -> np.ndarray:
    """float64 view of an input array.  uint16 arrays are bfloat16 bit
    patterns: the 16 bits are the top half of an IEEE float32, so the value is
    exact once placed there."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def validate(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
             n_tokens: int, n_adapters: int, max_pairs_per_group: int = 64,
             max_tuples: Optional[int] = None) -> int:
    """Status of a composite table.

    The pair arrays may be longer than the table: its pairs are those below
    group_pair_ptr[G], and entries at or beyond it are unused capacity,
    never read (a gate writing variable-length pair lists into fixed-size
    arrays; DyMerge-LoRA one-minute summary, padding and masking of the
    gate's vectorised form).

    EINVAL: CSR pointers that do not start at 0, end at the token count (and
    at most at the pair arrays' length), or decrease; an adapter id outside
    [0, n_adapters); a non-finite alpha; the same adapter twice in one
    composite (composites within the pair limit).  EUNSUPPORTED: a group
    with more than ``max_pairs_per_group`` pairs.  ENOSPC: more tuples than
    ``max_tuples``.  EINVAL outranks EUNSUPPORTED, which outranks ENOSPC."""
    gt = [int(v) for v in group_tok_ptr]
    gp = [int(v) for v in group_pair_ptr]
    ad = [int(v) for v in pair_adapter]
    al = [float(v) for v in np.asarray(pair_alpha, dtype=np.float32)]
    if n_tokens < 0 or n_adapters < 1 or len(gt) < 1 or len(gt) != len(gp):
        return EINVAL
    if gt[0] != 0 or gt[-1] != n_tokens or gp[0] != 0 or gp[-1] > len(ad):
        return EINVAL
    if len(al) != len(ad):
        return EINVAL
    for g in range(len(gt) - 1):
        if gt[g + 1] < gt[g] or gp[g + 1] < gp[g]:
            return EINVAL
    n_pairs = gp[-1]
    for a in ad[:n_pairs]:
        if a < 0 or a >= n_adapters:
            return EINVAL
    for w in al[:n_pairs]:
        if not math.isfinite(w):
            return EINVAL
    for g in range(len(gt) - 1):
        ids = ad[gp[g]:gp[g + 1]]
        # a group beyond the pair limit is unsupported whatever it holds, so
        # it is not searched for duplicates
        if len(ids) <= max_pairs_per_group and len(set(ids)) != len(ids):
            return EINVAL
    for g in range(len(gt) - 1):
        if gp[g + 1] - gp[g] > max_pairs_per_group:
            return EUNSUPPORTED
    if max_tuples is not None:
        P = sum((gt[g + 1] - gt[g]) * (gp[g + 1] - gp[g]) for g in range(len(gt) - 1))
        if P > max_tuples:
            return ENOSPC
    return OK


def canonical_composite(group_pair_ptr, pair_adapter, pair_alpha, g: int):
    """Pairs of group g ordered by adapter id; position in this list is the
    pair's out-slot.  Returns a list of (adapter, alpha) with alpha kept as
    its float32 value."""
    lo, hi = int(group_pair_ptr[g]), int(group_pair_ptr[g + 1])
    pairs = [(int(pair_adapter[q]), np.float32(pair_alpha[q])) for q in range(lo, hi)]
    return sorted(pairs, key=lambda p: p[0])


def group_of_token(group_tok_ptr) -> np.ndarray:
    T = int(group_tok_ptr[-1])
    owner = np.empty(T, dtype=np.int64)
    for g in range(len(group_tok_ptr) - 1):
        owner[int(group_tok_ptr[g]):int(group_tok_ptr[g + 1])] = g
    return owner


# ---------------------------------------------------------------------------
# token-level gate: the composite of each token from its gate logits
# (DyMerge-LoRA, section 3.1 dynamic composition; section 5.1 Sparse
# workload: a request references 5-8 adapters and two are active per token)
# ---------------------------------------------------------------------------

def gate_topk(logits, candidates, k: int):
    """Composite table of a token-level gate.

    Token t has candidate adapters ``candidates[t, c]`` (entries < 0 are
    padding) with gate logits ``logits[t, c]``.  Its weights are the softmax
    of the logits over the valid candidates; the k largest weights are kept,
    not renormalised, ties going to the earlier candidate (the softmax is
    increasing in the logit, so this is the order of the logits), listed in
    that order.  A token with fewer than k valid candidates keeps them all:
    its pair list is shorter (no valid candidate: an empty composite, which
    leaves the token unchanged).  A token with a non-finite valid logit lists
    k pairs of adapter -1 and weight 0, a table the mapping stage rejects.

    The pair lists follow one another; the pair arrays keep n_tokens * k
    entries, and those at or beyond group_pair_ptr[T] are unused capacity
    (adapter -1, weight 0).

    Returns (group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha) with one
    group per token; pair_alpha is float64 here."""
    lg = np.asarray(logits, dtype=np.float64)
    cd = np.asarray(candidates, dtype=np.int64)
    T = lg.shape[0]
    gtp = np.arange(T + 1, dtype=np.int64)
    gpp = np.zeros(T + 1, dtype=np.int64)
    pa = np.full(T * k, -1, dtype=np.int64)
    pw = np.zeros(T * k, dtype=np.float64)
    for t in range(T):
        valid = [c for c in range(cd.shape[1]) if cd[t, c] >= 0]
        if not all(math.isfinite(lg[t, c]) for c in valid):
            gpp[t + 1] = gpp[t] + k          # k pairs of adapter -1: rejected
            continue
        kept = []
        if valid:
            top = max(lg[t, c] for c in valid)
            e = {c: math.exp(lg[t, c] - top) for c in valid}
            total = sum(e[c] for c in valid)
            # largest logit first; equal logits keep the candidate order
            order = sorted(valid, key=lambda c: (-lg[t, c], c))
            kept = [(int(cd[t, c]), e[c] / total) for c in order[:k]]
        base = int(gpp[t])
        for i, (a, w) in enumerate(kept):
            pa[base + i] = a
            pw[base + i] = w
        gpp[t + 1] = base + len(kept)
    return gtp, gpp, pa, pw


# ---------------------------------------------------------------------------
# mapping stage: tuples reordered by adapter id (DyMerge-LoRA, section 4.3)
# ---------------------------------------------------------------------------

def plan(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha) -> Dict[str, np.ndarray]:
    """Expand composites into (token, adapter, alpha, slot) tuples and reorder
    them by adapter id.

    Tuples are first listed token-major (token ascending, slot ascending) and
    then stably sorted by adapter id, which makes the order the total order on
    (adapter, token, slot).  Also returns the segment table (one entry per
    adapter that owns tuples, ascending) and the per-token index
    (``tok_tuple[tok_ptr[t] + s]`` is the sorted position of token t's slot s).
    """
    T = int(group_tok_ptr[-1])
    tokens, adapters, alphas, slots = [], [], [], []
    n_per_token = np.zeros(T, dtype=np.int64)
    owner = group_of_token(group_tok_ptr)
    for t in range(T):
        comp = canonical_composite(group_pair_ptr, pair_adapter, pair_alpha, int(owner[t]))
        n_per_token[t] = len(comp)
        for s, (a, w) in enumerate(comp):
            tokens.append(t)
            adapters.append(a)
            alphas.append(w)
            slots.append(s)
    tokens = np.array(tokens, dtype=np.int32)
    adapters = np.array(adapters, dtype=np.int32)
    alphas = np.array(alphas, dtype=np.float32)
    slots = np.array(slots, dtype=np.int32)
    order = np.argsort(adapters, kind="stable")
    tup_token = tokens[order]
    tup_adapter = adapters[order]
    tup_alpha = alphas[order]
    tup_slot = slots[order]
    P = len(order)

    seg_adapter, seg_begin = [], []
    for p in range(P):
        if p == 0 or tup_adapter[p] != tup_adapter[p - 1]:
            seg_adapter.append(int(tup_adapter[p]))
            seg_begin.append(p)
    seg_begin.append(P)

    tok_ptr = np.zeros(T + 1, dtype=np.int32)
    tok_ptr[1:] = np.cumsum(n_per_token)
    tok_tuple = np.full(P, -1, dtype=np.int32)
    for p in range(P):
        tok_tuple[tok_ptr[tup_token[p]] + tup_slot[p]] = p
    return {
        "tup_token": tup_token, "tup_adapter": tup_adapter,
        "tup_alpha": tup_alpha, "tup_slot": tup_slot,
        "seg_adapter": np.array(seg_adapter, dtype=np.int32),
        "seg_begin": np.array(seg_begin, dtype=np.int32),
        "tok_ptr": tok_ptr, "tok_tuple": tok_tuple,
    }


# ---------------------------------------------------------------------------
# the apply, straight from the definition
# ---------------------------------------------------------------------------

def effective_rank(k, a: int, r_max: int) -> int:
    """k_m of adapter a (LoRAForge retained-rank contract); r_max if absent."""
    return r_max if k is None else int(k[a])


def apply(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
          A_t, B_t, k, x, y_base):
    """y_t = y_base_t + sum over token t's composite, in slot order, of
    alpha * B_a[:, :k_a] (A_a[:, :k_a]^T x_t), all in float64.

    Returns (y, delta) as float64 arrays of shape [T, d_out]."""
    T = int(group_tok_ptr[-1])
    r_max = A_t.shape[1]
    d_out = B_t.shape[2]
    delta = np.zeros((T, d_out), dtype=np.float64)
    owner = group_of_token(group_tok_ptr)
    for t in range(T):
        xt = widen(x[t])
        for a, w in canonical_composite(group_pair_ptr, pair_adapter, pair_alpha, int(owner[t])):
            kk = effective_rank(k, a, r_max)
            if kk == 0:
                continue
            A_a_T = widen(A_t[a, :kk, :])      # A_a^T restricted to the retained prefix
            B_a_T = widen(B_t[a, :kk, :])      # B_a^T restricted likewise
            z = A_a_T @ xt                     # A_a^T x_t   (length k)
            delta[t] += float(w) * (B_a_T.T @ z)   # alpha * B_a z
    return widen(y_base) + delta, delta


def shrink(pl: Dict[str, np.ndarray], A_t, k, x) -> np.ndarray:
    """z_p = A_{a_p}[:, :k]^T x_{t_p} for every tuple p, in sorted-tuple order;
    float64 [P, r_max] with zeros beyond each adapter's effective rank.
    alpha is not applied."""
    P = pl["tup_token"].shape[0]
    r_max = A_t.shape[1]
    z = np.zeros((P, r_max), dtype=np.float64)
    for p in range(P):
        a, t = int(pl["tup_adapter"][p]), int(pl["tup_token"][p])
        kk = effective_rank(k, a, r_max)
        if kk:
            z[p, :kk] = widen(A_t[a, :kk, :]) @ widen(x[t])
    return z


def expand(pl: Dict[str, np.ndarray], B_t, k, z, y_base) -> np.ndarray:
    """y_t = y_base_t + sum over token t's slots s of alpha * B_a[:, :k] z_(t,s),
    where z is given per sorted tuple.  float64 [T, d_out]."""
    T = pl["tok_ptr"].shape[0] - 1
    r_max = B_t.shape[1]
    y = widen(y_base).copy()
    z = np.asarray(z, dtype=np.float64)
    for t in range(T):
        acc = np.zeros(y.shape[1], dtype=np.float64)
        for i in range(int(pl["tok_ptr"][t]), int(pl["tok_ptr"][t + 1])):
            p = int(pl["tok_tuple"][i])
            a = int(pl["tup_adapter"][p])
            kk = effective_rank(k, a, r_max)
            if kk:
                acc += float(pl["tup_alpha"][p]) * (widen(B_t[a, :kk, :]).T @ z[p, :kk])
        y[t] += acc
    return y


def apply_rows(group_tok_ptr, group_pair_ptr, pair_adapter, pair_alpha,
               A_t, B_t, k, x, y_base, rows, cols=None):
    """The apply for selected tokens (and optionally selected output columns)
    only: float64 [len(rows), len(cols) or d_out].  Same arithmetic as
    :func:`apply`, used to sample outputs of full-size problems."""
    r_max = A_t.shape[1]
    owner = group_of_token(group_tok_ptr)
    cols = slice(None) if cols is None else np.asarray(cols)
    out = []
    for t in rows:
        t = int(t)
        xt = widen(x[t])
        acc = None
        for a, w in canonical_composite(group_pair_ptr, pair_adapter, pair_alpha, int(owner[t])):
            kk = effective_rank(k, a, r_max)
            if kk == 0:
                continue
            z = widen(A_t[a, :kk, :]) @ xt
            term = float(w) * (widen(B_t[a, :kk, :][:, cols]).T @ z)
            acc = term if acc is None else acc + term
        base = widen(y_base[t][cols])
        out.append(base + (acc if acc is not None else 0.0))
    return np.array(out)


# ---------------------------------------------------------------------------
# sizes (ELORA, section III-A: adapter size next to the base weight)
# ---------------------------------------------------------------------------

def adapter_fraction(d_in: int, d_out: int, r: int) -> float:
    """Values of one rank-r adapter (A: d_in x r, B: d_out x r) as a fraction
    of the d_out x d_in base weight it modifies."""
    return (d_in + d_out) * r / (d_in * d_out)


# ---------------------------------------------------------------------------
# retained-rank producer (LoRAForge, approach (2) rank allocation and
# approach (3) factor construction)
# ---------------------------------------------------------------------------

def factor_balanced(B_t, A_t):
    """Balanced factors of one module's update, spectrum first.

    The update is Delta W = B A^T = X Y with X = B (d_out x r, the tall-skinny
    factor; ``B_t`` holds its columns as rows) and Y = A^T (r x d_in, the rows
    of ``A_t``).  Following LoRAForge approach (3): a thin QR of X gives R,
    then H = R Y, and the eigendecomposition of H H^T = U diag(lambda) U^T
    gives the spectrum, sigma_j = sqrt(lambda_j), largest first.  The balanced
    factors are F = Q U diag(sigma)^(1/2) and T = diag(sigma)^(-1/2) U^T H, so
    F T = X Y, F^T F = T T^T = diag(sigma), and the first k columns of F with
    the first k rows of T are the rank-k truncated SVD of Delta W.

    Directions whose eigenvalue is at most r * 2^-52 times the largest (the
    rounding level of the r x r eigenproblem) are taken as exactly zero:
    sigma 0, a zero column of F and a zero row of T.

    Returns (F_t, T, sigma): F_t = F^T (r x d_out, the new B_t rows), T (r x
    d_in, the new A_t rows), sigma (r,), all float64."""
    X = widen(B_t).T
    Y = widen(A_t)
    r = X.shape[1]
    # with fewer rows than r (d_out < r) the thin QR has min(d_out, r) rows
    # of R and the remaining directions are zero
    Q, R = np.linalg.qr(X, mode="reduced")
    H = R @ Y
    lam, U = np.linalg.eigh(H @ H.T)
    order = np.argsort(-lam, kind="stable")
    lam, U = lam[order], U[:, order]
    kq = len(lam)
    live = lam > r * 2.0 ** -52 * max(lam[0], 0.0)
    sigma = np.zeros(r)
    sigma[:kq] = np.where(live, np.sqrt(np.where(live, lam, 1.0)), 0.0)
    F = np.zeros((X.shape[0], r))
    T = np.zeros((r, Y.shape[1]))
    for j in range(kq):
        if live[j]:
            F[:, j] = (Q @ U[:, j]) * math.sqrt(sigma[j])
            T[j, :] = (U[:, j] @ H) / math.sqrt(sigma[j])
    return F.T.copy(), T, sigma


def uniform_ranks(ranks, denominator: int):
    """LoRAForge-U (LoRAForge, approach (2)): module m keeps
    u_m = max(1, floor(r_m / d)) of its r_m directions."""
    return np.array([max(1, int(r) // int(denominator)) for r in ranks], dtype=np.int64)


def uniform_budget(ranks, costs, denominator: int) -> int:
    """The parameter budget P_U of LoRAForge-U: sum over modules of
    u_m * (d_in + d_out), the values its retained prefixes hold."""
    u = uniform_ranks(ranks, denominator)
    return int(sum(int(a) * int(c) for a, c in zip(u, costs)))


def spectral_ranks(sigmas, costs, budget: int, floors):
    """LoRAForge-S (LoRAForge, approach (2)): spend the budget on the
    directions with the most spectral energy per parameter.

    Module m has singular values sigma_{m,0} >= sigma_{m,1} >= ... and each
    retained direction costs c_m = d_in + d_out values.  Every module first
    keeps its floor of l_m directions (capped at its rank).  The remaining
    directions are then visited by decreasing eta_{m,j} = sigma_{m,j}^2 / c_m
    (equal ratios: lower module index, then lower j), and a direction is kept
    when its cost still fits in what is left of the budget.  Since sigma is
    non-increasing within a module, the kept directions of each module are a
    prefix.  Returns k_m for every module (int64)."""
    M = len(sigmas)
    k = np.array([min(int(floors[m]), len(sigmas[m])) for m in range(M)], dtype=np.int64)
    left = int(budget) - sum(int(k[m]) * int(costs[m]) for m in range(M))
    items = []
    for m in range(M):
        s = np.asarray(sigmas[m], dtype=np.float64)
        for j in range(int(k[m]), len(s)):
            items.append((-(s[j] * s[j]) / float(costs[m]), m, j))
    items.sort()
    for _, m, j in items:
        if j == k[m] and int(costs[m]) <= left:
            k[m] += 1
            left -= int(costs[m])
    return k


# ---------------------------------------------------------------------------
# adapter residency and batch choice (DyMerge-LoRA, section 4: BAM and the
# LAG scheduler)
# ---------------------------------------------------------------------------

def bam_run(n_slots: int, batches):
    """Replay batches through BAM, the slot pool that keeps raw adapter
    factors on the GPU (DyMerge-LoRA, section 4: adapters the running batch
    uses are pinned, the others leave least recently used first).

    Each batch is a list of adapter ids.  Batch number t (time t):
      1. its adapters already in a slot are hits: pinned, last use = t;
      2. each missing adapter, in the batch's order (a repeat counts once),
         takes the lowest-numbered empty slot, else the slot whose adapter
         was used longest ago among the slots this batch has not pinned
         (equal times: the lower slot); it is loaded there, pinned, last
         use = t;
      3. if some adapter finds no slot the batch is rejected (status
         ENOSPC) and the pool is left as it was before the batch.
    Pins last for the batch only.

    Returns one record per batch: (status, {adapter: slot}, [(slot, loaded
    adapter, evicted adapter or -1), ...]) and the final slot contents."""
    slot_ad = [-1] * n_slots
    last = [-1] * n_slots
    out = []
    for t, batch in enumerate(batches):
        ad_list = []
        for a in batch:
            if a not in ad_list:
                ad_list.append(int(a))
        s_ad, s_last = list(slot_ad), list(last)
        pinned = set()
        where = {}
        for a in ad_list:
            if a in s_ad:
                s = s_ad.index(a)
                pinned.add(s)
                s_last[s] = t
                where[a] = s
        loads = []
        ok = True
        for a in ad_list:
            if a in where:
                continue
            empty = [s for s in range(n_slots) if s_ad[s] == -1]
            if empty:
                s = empty[0]
            else:
                cand = [s for s in range(n_slots) if s not in pinned]
                if not cand:
                    ok = False
                    break
                s = min(cand, key=lambda q: (s_last[q], q))
            loads.append((s, a, s_ad[s]))
            s_ad[s] = a
            s_last[s] = t
            pinned.add(s)
            where[a] = s
        if ok:
            slot_ad, last = s_ad, s_last
            out.append((OK, where, loads))
        else:
            out.append((ENOSPC, {}, []))
    return out, slot_ad


def lag_select(now: float, theta: float, arrival, adapters, resident, max_batch: int,
               n_slots: int):
    """The next batch, chosen the LAG way (DyMerge-LoRA, section 4: batch
    the requests that need the fewest adapters not already resident, and
    serve requests that have waited longer than theta first, in arrival
    order).

    Request i arrived at arrival[i] and uses the adapters adapters[i].  A
    batch holds at most max_batch requests, and the distinct adapters of its
    requests must fit in n_slots slots.  First the waiting-too-long requests
    (now - arrival > theta), by arrival (equal: lower index), each taken if
    it still fits.  Then, while the batch has room, the remaining request
    with the fewest new loads |L(r) minus (resident + adapters already in the
    batch)| among those that fit, ties by arrival then index.  Returns the
    chosen request indices in the order taken."""
    n = len(arrival)
    res = set(int(a) for a in resident)
    chosen = []
    in_batch = set()

    def fits(i):
        return len(in_batch | set(int(a) for a in adapters[i])) <= n_slots

    def take(i):
        chosen.append(i)
        in_batch.update(int(a) for a in adapters[i])

    old = sorted((i for i in range(n) if now - arrival[i] > theta),
                 key=lambda i: (arrival[i], i))
    for i in old:
        if len(chosen) < max_batch and fits(i):
            take(i)
    while len(chosen) < max_batch:
        best = None
        for i in range(n):
            if i in chosen or not fits(i):
                continue
            new = len(set(int(a) for a in adapters[i]) - res - in_batch)
            key = (new, arrival[i], i)
            if best is None or key < best[0]:
                best = (key, i)
        if best is None:
            break
        take(best[1])
    return chosen
