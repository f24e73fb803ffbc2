"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them."""
import os
import types

import pytest

import pins

SRC = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "oracle.py")).read()

MUTANTS = {
    "dropped_alpha": ("delta[t] += float(w) * (B_a_T.T @ z)", "delta[t] += (B_a_T.T @ z)"),
    "wrong_sign": ("delta[t] += float(w) * (B_a_T.T @ z)", "delta[t] -= float(w) * (B_a_T.T @ z)"),
    "swapped_factors": ("A_a_T = widen(A_t[a, :kk, :])", "A_a_T = widen(B_t[a, :kk, :])"),
    "ignored_rank": ("            kk = effective_rank(k, a, r_max)\n            if kk == 0:\n                continue\n            A_a_T",
                     "            kk = r_max\n            if kk == 0:\n                continue\n            A_a_T"),
    "uncanonical_slots": ("return sorted(pairs, key=lambda p: p[0])", "return pairs"),
    "sorted_by_token": ('order = np.argsort(adapters, kind="stable")',
                        'order = np.argsort(tokens, kind="stable")'),
    "dropped_pair": ("for s, (a, w) in enumerate(comp):", "for s, (a, w) in enumerate(comp[1:]):"),
    "shifted_tok_ptr": ("tok_ptr[1:] = np.cumsum(n_per_token)", "tok_ptr[:-1] = np.cumsum(n_per_token)"),
    "dropped_base": ("return widen(y_base) + delta, delta", "return delta, delta"),
    "bf16_truncated": ("return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)",
                       "return (a.astype(np.uint32) << 8).view(np.float32).astype(np.float64)"),
    "dup_allowed": ("if len(ids) <= max_pairs_per_group and len(set(ids)) != len(ids):",
                    "if False:"),
    "adapter_fraction_one_side": ("return (d_in + d_out) * r / (d_in * d_out)",
                                  "return d_in * r / (d_in * d_out)"),
    "gate_renormalised": ("e[c] / total) for c in order[:k]]",
                          "e[c] / sum(e[o] for o in order[:k])) for c in order[:k]]"),
    "gate_short_padded": ("gpp[t + 1] = base + len(kept)", "gpp[t + 1] = base + k"),
    "validate_full_arrays": ("gp[-1] > len(ad)", "gp[-1] != len(ad)"),
    "validate_reads_tail": ("for a in ad[:n_pairs]:", "for a in ad:"),
    "gate_ties_to_later": ("order = sorted(valid, key=lambda c: (-lg[t, c], c))",
                           "order = sorted(valid, key=lambda c: (-lg[t, c], -c))"),
    "gate_smallest": ("order = sorted(valid, key=lambda c: (-lg[t, c], c))",
                      "order = sorted(valid, key=lambda c: (lg[t, c], c))"),
    "gate_padding_kept": ("valid = [c for c in range(cd.shape[1]) if cd[t, c] >= 0]",
                          "valid = [c for c in range(cd.shape[1])]"),
    "factor_ascending": ('order = np.argsort(-lam, kind="stable")', 'order = np.argsort(lam, kind="stable")'),
    "factor_unbalanced": ("F[:, j] = (Q @ U[:, j]) * math.sqrt(sigma[j])", "F[:, j] = (Q @ U[:, j]) * sigma[j]"),
    "factor_h_transposed": ("H = R @ Y", "H = R.T @ Y"),
    "factor_no_sqrt": ("sigma[:kq] = np.where(live, np.sqrt(np.where(live, lam, 1.0)), 0.0)",
                       "sigma[:kq] = np.where(live, np.where(live, lam, 1.0), 0.0)"),
    "factor_tail_not_zero": ("    sigma = np.zeros(r)\n", "    sigma = np.ones(r)\n"),
    "uniform_ceil": ("max(1, int(r) // int(denominator))", "max(1, -(-int(r) // int(denominator)))"),
    "uniform_no_min": ("max(1, int(r) // int(denominator))", "max(0, int(r) // int(denominator))"),
    "spectral_sigma_not_squared": ("items.append((-(s[j] * s[j]) / float(costs[m]), m, j))",
                                   "items.append((-s[j] / float(costs[m]), m, j))"),
    "spectral_cost_ignored": ("items.append((-(s[j] * s[j]) / float(costs[m]), m, j))",
                              "items.append((-(s[j] * s[j]), m, j))"),
    "spectral_stop_at_first_misfit": ("        if j == k[m] and int(costs[m]) <= left:\n            k[m] += 1\n            left -= int(costs[m])",
                                      "        if j == k[m] and int(costs[m]) <= left:\n            k[m] += 1\n            left -= int(costs[m])\n        else:\n            break"),
    "spectral_no_floor": ("k = np.array([min(int(floors[m]), len(sigmas[m])) for m in range(M)], dtype=np.int64)",
                          "k = np.array([0 for m in range(M)], dtype=np.int64)"),
    "bam_most_recent": ("s = min(cand, key=lambda q: (s_last[q], q))", "s = max(cand, key=lambda q: (s_last[q], -q))"),
    "bam_ties_high_slot": ("s = min(cand, key=lambda q: (s_last[q], q))", "s = min(cand, key=lambda q: (s_last[q], -q))"),
    "bam_no_pins": ("cand = [s for s in range(n_slots) if s not in pinned]", "cand = [s for s in range(n_slots)]"),
    "bam_hits_not_touched": ("                pinned.add(s)\n                s_last[s] = t\n                where[a] = s",
                             "                pinned.add(s)\n                where[a] = s"),
    "bam_no_rollback": ("            out.append((ENOSPC, {}, []))", "            slot_ad, last = s_ad, s_last\n            out.append((ENOSPC, {}, []))"),
    "lag_ignores_residency": ("new = len(set(int(a) for a in adapters[i]) - res - in_batch)",
                              "new = len(set(int(a) for a in adapters[i]) - in_batch)"),
    "lag_ignores_batch": ("new = len(set(int(a) for a in adapters[i]) - res - in_batch)",
                          "new = len(set(int(a) for a in adapters[i]) - res)"),
    "lag_starving_by_index": ("key=lambda i: (arrival[i], i))\n    for i in old:", "key=lambda i: i)\n    for i in old:"),
    "lag_ties_latest": ("key = (new, arrival[i], i)", "key = (new, -arrival[i], i)"),
    "lag_no_slot_limit": ("        return len(in_batch | set(int(a) for a in adapters[i])) <= n_slots",
                          "        return True"),

}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, name
    mod = types.ModuleType("oracle_mutant_" + name)
    exec(compile(SRC.replace(old, new), "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    O = _mutant(name)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(O)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
