"""The gist-masked prefill oracle against its pins, and planted mistakes in a copy of it."""
import inspect
import types

import pytest

from oracle import gist_prefill_ref
from tests import pins_gist as pins


@pytest.mark.parametrize("pin", pins.GIST_PINS, ids=lambda f: f.__name__)
def test_gist_pin(pin):
    pin(gist_prefill_ref)


MUTATIONS = {
    "raw_sees_own_gist": ("return np.arange(m), np.arange(m * C, i + 1)", "return np.arange(m + 1), np.arange(m * C, i + 1)"),
    "raw_not_causal": ("return np.arange(m), np.arange(m * C, i + 1)", "return np.arange(m), np.arange(m * C, (m + 1) * C)"),
    "raw_sees_earlier_chunks": ("return np.arange(m), np.arange(m * C, i + 1)", "return np.arange(m), np.arange(0, i + 1)"),
    "gist_not_self": ("return np.arange(i + 1), np.arange(i * C, (i + 1) * C)", "return np.arange(i), np.arange(i * C, (i + 1) * C)"),
    "gist_sees_next_chunk": ("return np.arange(i + 1), np.arange(i * C, (i + 1) * C)", "return np.arange(i + 1), np.arange((i + 1) * C, (i + 2) * C)"),
    "gist_without_raw": ("return np.arange(i + 1), np.arange(i * C, (i + 1) * C)", "return np.arange(i + 1), np.arange(0)"),
    "wrong_kv_group": ("g = h // (w.n_q_heads // w.n_kv_heads)\n    o =", "g = h % w.n_kv_heads\n    o ="),
    "gist_values_are_raw": ("Vc = np.concatenate([Vg, Vr], axis=0)", "Vc = np.concatenate([Kg, Vr], axis=0)"),
}


def _mutant(old, new):
    src = inspect.getsource(gist_prefill_ref)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace("from .sparse_decode_ref import", "from oracle.sparse_decode_ref import")
    mod = types.ModuleType("gist_mutant")
    exec(compile(src.replace(old, new, 1), "gist_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_gist_mutation_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in pins.GIST_PINS:
        try:
            pin(mod)
        except Exception:  # a failed assertion or a crash both count
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
