"""Plant plausible mistakes in copies of the block-projection oracle (on the
CPU) and check that at least one pin rejects each copy."""
import inspect
import types

import pytest

import block_pins as P
from oracle import block

# (name, text in oracle/block.py, planted replacement)
MUTANTS = [
    ("w_not_transposed", "    qkv = u @ w.T\n", "    qkv = u @ w.reshape(C, 3 * C)\n"),
    ("k_takes_v_columns", "k = qkv[:, C:2 * C].reshape(T, H, d)", "k = qkv[:, 2 * C:].reshape(T, H, d)"),
    ("v_rotated", "return R.rope(q, pos, dims, base), R.rope(k, pos, dims, base), v",
     "return R.rope(q, pos, dims, base), R.rope(k, pos, dims, base), R.rope(v, pos, dims, base)"),
    ("no_modulation", "u = R.modulate(x, shift, scale, mod_row, eps) if shift is not None else x", "u = x"),
    ("k_not_rotated", "return R.rope(q, pos, dims, base), R.rope(k, pos, dims, base), v",
     "return R.rope(q, pos, dims, base), k, v"),
    ("out_w_not_transposed", "(o2 @ w.T)", "(o2 @ w)"),
    ("gate_on_residual", "return x + np.asarray(gate, dtype=np.float64)[mod_row] * (o2 @ w.T)",
     "return np.asarray(gate, dtype=np.float64)[mod_row] * x + (o2 @ w.T)"),
    ("rows_keep_all_mod_rows", "mr = None if mod_row is None else np.asarray(mod_row)[rows]",
     "mr = None if mod_row is None else np.asarray(mod_row)[:len(rows)]"),
]


def _mutant(name, old, new):
    src = inspect.getsource(block)
    assert src.count(old) == 1, (name, src.count(old))
    mod = types.ModuleType("oracle.block_mutant_" + name)
    mod.__file__ = block.__file__
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), block.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_block_mutant_is_caught(name, old, new):
    m = _mutant(name, old, new)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(m)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
