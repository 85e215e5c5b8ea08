"""The packed-CFG sampler oracle against its pins, and planted mistakes (CPU)."""
import inspect
import types

import pytest

import sampler_pins as P
from oracle import sampler


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_sampler_oracle_pin(pin):
    pin(sampler)


MUTANTS = [
    ("step_sign", "return np.asarray(z, dtype=np.float64) + (t - t_next) *",
     "return np.asarray(z, dtype=np.float64) + (t_next - t) *"),
    ("guidance_swapped", "return vu + w * (vc - vu)", "return vc + w * (vu - vc)"),
    ("first_frame", "bc = int(cu[c]) + tc + (fc - 1) * n", "bc = int(cu[c]) + tc"),
    ("no_text_offset", "bu = int(cu[u]) + tu + (fu - 1) * n", "bu = int(cu[u]) + (fu - 1) * n"),
    ("scatter_cond_only", "    x[rows[:, 1]] = z_next\n", ""),
]


def _mutant(name, old, new):
    src = inspect.getsource(sampler)
    assert src.count(old) == 1, (name, src.count(old))
    mod = types.ModuleType("oracle.sampler_mutant_" + name)
    mod.__file__ = sampler.__file__
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), sampler.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_sampler_mutant_is_caught(name, old, new):
    m = _mutant(name, old, new)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(m)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
