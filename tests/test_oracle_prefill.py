"""The Token-Sparse prefill oracle against its pins, and planted mistakes in a copy of it."""
import inspect
import types

import pytest

from oracle import sparse_prefill_ref
from tests import pins_prefill as pins


@pytest.mark.parametrize("pin", pins.PREFILL_PINS, ids=lambda f: f.__name__)
def test_prefill_pin(pin):
    pin(sparse_prefill_ref)


MUTATIONS = {
    "proxy_not_causal": ("vis = pos0 + i + 1", "vis = K.shape[0]"),
    "proxy_unnormalised": ("imp[:vis] = imp[:vis] + e / math.fsum(e.tolist())", "imp[:vis] = imp[:vis] + e"),
    "proxy_missing_last_row": ("for i in range(Qw.shape[0]):\n        vis", "for i in range(Qw.shape[0] - 1):\n        vis"),
    "budget_from_first_head": ("k, margin = coverage_budget(total, w.tau)", "k, margin = coverage_budget(imps[0], w.tau)"),
    "attention_not_causal": ("keys = S[:i + 1]", "keys = S"),
    "attention_wrong_kv_group": ("    g = h // G\n    o =", "    g = h % w.n_kv_heads\n    o ="),
    "query_at_compact_index": ("src.q_rows(b, h, S[i:i + 1])", "src.q_rows(b, h, [i])"),
    "scatter_not_zeroed": ("            O[b, h] = 0.0\n", "            O[b, h] = 1.0\n"),
    "full_heads_in_budget": ("        if not modes[h]:\n            total = total + imps[h]", "        total = total + imps[h]"),
    "full_head_uses_budget": ("        if modes[h]:\n            sets[h], gaps[h] = np.arange(L), math.inf\n            continue\n", ""),
    "modes_ignored": ("return [0] * w.n_q_heads if m is None else", "return [0] * w.n_q_heads if True else"),
}


def _mutant(old, new):
    src = inspect.getsource(sparse_prefill_ref)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace("from .sparse_decode_ref import", "from oracle.sparse_decode_ref import")
    mod = types.ModuleType("prefill_mutant")
    exec(compile(src.replace(old, new, 1), "prefill_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_prefill_mutation_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins.PREFILL_PINS:
        try:
            pin(mod)
        except Exception:  # a failed assertion or a crash both count
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
