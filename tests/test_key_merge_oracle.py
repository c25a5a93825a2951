"""The key-merge oracle against its pins, and the pins against planted mistakes
in copies of the oracle.  CPU only."""
import importlib.util
import os

import pytest

from oracle import key_merge
from key_merge_pins import ALL_PINS

SRC = key_merge.__file__

MUTATIONS = {
    "numerator_drops_Sb": ("(Wa @ Sa + Wb @ Sb) @", "(Wa @ Sa + Wb) @"),
    "pinv_of_Sa_only": ("pinv_psd(Sa + Sb, rtol)", "pinv_psd(Sa, rtol)"),
    "pinv_transposed_basis": ("(V * inv) @ V.T", "(V.T * inv) @ V"),
    "pinv_no_cutoff": ("keep = lam > rtol * top", "keep = lam != 0"),
    "gram_keeps_last_head": ("S += Qj.T @ Qj", "S = Qj.T @ Qj"),
    "loss_one_group": ("for r in (a, b):\n        Kr", "for r in (a,):\n        Kr"),
    "loss_wrong_key": ("Kr = X @ W[r]", "Kr = X @ W[a]"),
    "group_modulo": ("return (j * h_kt) // h_q", "return j % h_kt"),
    "matching_partial": ("for k in range(1, len(heads)):", "for k in range(1, min(len(heads), 3)):"),
    "matching_drops_heads": ("rest = heads[1:k] + heads[k + 1:]", "rest = heads[k + 1:]"),
    "matching_maximises": ("if cost < best_cost:", "if -cost < -best_cost or best is None:"),
}


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(key_merge)


def _load_mutant(name, path):
    spec = importlib.util.spec_from_file_location(f"km_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / f"{name}.py"
    path.write_text(src.replace(old, new))
    mod = _load_mutant(name, str(path))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, TypeError, IndexError, ZeroDivisionError,
                FloatingPointError, KeyError, np_linalg_error()):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutation {name}"


def np_linalg_error():
    import numpy as np

    return np.linalg.LinAlgError
