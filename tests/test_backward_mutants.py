"""Plant plausible mistakes in copies of the backward oracle (on the CPU) and
check that at least one pin rejects each copy."""
import inspect
import types

import pytest

import backward_pins as P
from oracle import backward

# (name, text in oracle/backward.py, planted replacement)
MUTANTS = [
    ("no_rowsum_term", "dS = P * (dP - Dr)", "dS = P * dP"),
    ("dq_uses_v", "dQ[r0:r1, h, :] = scale * (dS @ K)", "dQ[r0:r1, h, :] = scale * (dS @ V)"),
    ("dk_unscaled", "dK[a:b, h, :] += scale * (dS.T @ Q)", "dK[a:b, h, :] += (dS.T @ Q)"),
    ("dv_uses_dp", "dV[a:b, h, :] += P.T @ G", "dV[a:b, h, :] += dS.T @ G"),
    ("rope_back_same_turn", "out[:, :, e0] = g0 * c + g1 * s", "out[:, :, e0] = g0 * c - g1 * s"),
    ("ln_bwd_no_mean", "dx = (gx - gx.mean(axis=-1, keepdims=True) - xh *", "dx = (gx - xh *"),
    ("ln_bwd_no_proj", " - xh * (gx * xh).mean(axis=-1, keepdims=True)) / sig", ") / sig"),
    ("mod_no_one_plus", "gx = du2 * (1.0 + scale[mod_row])", "gx = du2 * scale[mod_row]"),
    ("dscale_no_xh", "np.add.at(dscale, mod_row, du2 * xh)", "np.add.at(dscale, mod_row, du2)"),
    ("dgate_uses_y", "np.add.at(dgate, mod_row, dyt * o)", "np.add.at(dgate, mod_row, dyt * y)"),
    ("residual_drops_ln", "dyt = dyt + dln", "dyt = dyt"),
    ("dshift2_uses_dy", "np.add.at(dshift2, mod_row, dz)", "np.add.at(dshift2, mod_row, dyt)"),
]


def _mutant(name, old, new):
    src = inspect.getsource(backward)
    assert src.count(old) == 1, (name, src.count(old))
    mod = types.ModuleType("oracle.backward_mutant_" + name)
    mod.__file__ = backward.__file__
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), backward.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_mutant_is_caught(name, old, new):
    m = _mutant(name, old, new)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(m)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
