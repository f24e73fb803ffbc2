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
    "gate_renormalised": ("pw[t * k + i] = e[c] / total",
                          "pw[t * k + i] = e[c] / sum(e[o] for o in order[:k])"),
    "gate_ties_to_later": ("order = sorted(valid, key=lambda c: (-lg[t, c], c))",
                           "order = sorted(valid, key=lambda c: (-lg[t, c], -c))"),
    "gate_smallest": ("order = sorted(valid, key=lambda c: (-lg[t, c], c))",
                      "order = sorted(valid, key=lambda c: (lg[t, c], c))"),
    "gate_padding_kept": ("valid = [c for c in range(cd.shape[1]) if cd[t, c] >= 0]",
                          "valid = [c for c in range(cd.shape[1])]"),
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
