"""The text-encoder oracle against its pins, and planted mistakes (CPU)."""
import inspect
import types

import pytest

import text_encoder_pins as P
from oracle import text_encoder


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_text_encoder_oracle_pin(pin):
    pin(text_encoder)


MUTANTS = [
    ("mask_excludes_self", "S = np.where(kj <= qi, S, -np.inf)", "S = np.where(kj < qi, S, -np.inf)"),
    ("mask_non_causal", "S = np.where(kj <= qi, S, -np.inf)", "S = np.where(kj >= 0, S, -np.inf)"),
    ("kv_head_modulo", "K = k[a:b, h // g, :]", "K = k[a:b, h % Hkv, :]"),
    ("rms_subtracts_mean", "ms = (x * x).mean(axis=-1, keepdims=True)",
     "ms = ((x - x.mean(axis=-1, keepdims=True)) ** 2).mean(axis=-1, keepdims=True)"),
    ("rope_clockwise", "out[..., 0::2] = x0 * c - x1 * s", "out[..., 0::2] = x0 * c + x1 * s"),
    ("positions_global", "pos[a:b] = np.arange(b - a)", "pos[a:b] = np.arange(a, b)"),
    ("lse_no_max", "lse[h, r0:r1] = (m + np.log(l))[:, 0]", "lse[h, r0:r1] = np.log(l)[:, 0]"),
]


def _mutant(name, old, new):
    src = inspect.getsource(text_encoder)
    assert src.count(old) == 1, (name, src.count(old))
    mod = types.ModuleType("oracle.text_encoder_mutant_" + name)
    mod.__file__ = text_encoder.__file__
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), text_encoder.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_text_encoder_mutant_is_caught(name, old, new):
    m = _mutant(name, old, new)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(m)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
