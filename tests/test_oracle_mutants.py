"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
at least one pin rejects each copy, so the pins would catch such a slip in the
real oracle."""
import inspect
import types

import numpy as np
import pytest

import oracle_pins as P
from oracle import reference


def _mutant(name, **overrides):
    """Fresh copy of the oracle module with some functions replaced.  The
    replacement functions are re-bound to the copy's globals so that callers
    inside the copy use them too."""
    src = inspect.getsource(reference)
    mod = types.ModuleType("oracle_mutant_" + name)
    mod.__file__ = reference.__file__
    exec(compile(src, reference.__file__, "exec"), mod.__dict__)
    for fname, fn in overrides.items():
        setattr(mod, fname, types.FunctionType(fn.__code__, mod.__dict__, fname,
                                               fn.__defaults__, fn.__closure__))
    return mod


# --- the planted mistakes ---------------------------------------------------

def rope_clockwise(u, pos, dims, base):
    out = u.copy(); o = 0
    for axis, Da in enumerate(dims):
        if Da == 0:
            continue
        th = rope_thetas(Da, base)                                         # noqa: F821
        phi = pos[:, axis].astype(np.float64)[:, None] * th[None, :]
        c = np.cos(phi)[:, None, :]; s = np.sin(phi)[:, None, :]
        e0 = o + 2 * np.arange(Da // 2); e1 = e0 + 1
        x0 = u[:, :, e0]; x1 = u[:, :, e1]
        out[:, :, e0] = x0 * c + x1 * s
        out[:, :, e1] = -x0 * s + x1 * c
        o += Da
    return out


def rope_half_split(u, pos, dims, base):
    out = u.copy(); o = 0
    for axis, Da in enumerate(dims):
        if Da == 0:
            continue
        th = rope_thetas(Da, base)                                         # noqa: F821
        phi = pos[:, axis].astype(np.float64)[:, None] * th[None, :]
        c = np.cos(phi)[:, None, :]; s = np.sin(phi)[:, None, :]
        e0 = o + np.arange(Da // 2); e1 = e0 + Da // 2
        x0 = u[:, :, e0]; x1 = u[:, :, e1]
        out[:, :, e0] = x0 * c - x1 * s
        out[:, :, e1] = x0 * s + x1 * c
        o += Da
    return out


def rope_thetas_wrong_ladder(D_axis, base):
    j = np.arange(D_axis // 2, dtype=np.float64)
    return base ** (-1.0 * j / D_axis)


def rope_axes_swapped(u, pos, dims, base):
    return _orig_rope(u, pos[:, [0, 2, 1]], dims, base)                   # noqa: F821


def layer_norm_unbiased(x, eps):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
    return (x - mu) / np.sqrt(var + eps)


def modulate_no_one_plus(x2d, shift, scale, mod_row, eps):
    return layer_norm(x2d, eps) * scale[mod_row] + shift[mod_row]         # noqa: F821


def attention_no_scale(q, k, v, cu, scale=None, chunk=1024):
    return _orig_attention(q, k, v, cu, 1.0, chunk)                       # noqa: F821


def attention_cross_sample(q, k, v, cu, scale=None, chunk=1024):
    return _orig_attention(q, k, v, np.array([0, q.shape[0]]), scale, chunk)  # noqa: F821


def attention_transposed_scores(q, k, v, cu, scale=None, chunk=1024):
    import math as _m
    T, H, d = q.shape
    scale = 1.0 / _m.sqrt(d) if scale is None else scale
    O = np.zeros((T, H, d)); LSE = np.zeros((H, T))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            S = scale * (k[a:b, h] @ q[a:b, h].T)          # K Q^T in place of Q K^T
            m = S.max(axis=1, keepdims=True); E = np.exp(S - m); l = E.sum(axis=1, keepdims=True)
            O[a:b, h] = (E @ v[a:b, h]) / l
            LSE[h, a:b] = (m + np.log(l))[:, 0]
    return O, LSE


def tables_column_major(descs):
    cu, pos, sid, mr = _orig_pack_tables(descs)                           # noqa: F821
    for s, (t, F, h, w, _, _) in enumerate(descs):
        a = int(cu[s]) + t
        for i in range(F * h * w):
            hw = h * w
            pos[a + i] = (i // hw, i % h, (i % hw) // h)
    return cu, pos, sid, mr


def gated_residual_seq_gate(x, o, gate, mod_row, shift2=None, scale2=None, eps=1e-6):
    y, z = _orig_gated_residual(x, o, gate, np.zeros_like(mod_row), shift2, scale2, eps)  # noqa
    return y, z


MUTANTS = {
    "rope_clockwise": dict(rope=rope_clockwise),
    "rope_half_split": dict(rope=rope_half_split),
    "rope_wrong_ladder": dict(rope_thetas=rope_thetas_wrong_ladder),
    "rope_axes_swapped": dict(rope=rope_axes_swapped),
    "ln_unbiased_variance": dict(layer_norm=layer_norm_unbiased),
    "modulate_missing_one_plus": dict(modulate=modulate_no_one_plus),
    "attention_no_scale": dict(attention=attention_no_scale),
    "attention_cross_sample": dict(attention=attention_cross_sample),
    "attention_transposed_scores": dict(attention=attention_transposed_scores),
    "tables_column_major": dict(pack_tables=tables_column_major),
    "gated_residual_wrong_row": dict(gated_residual=gated_residual_seq_gate),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    # keep the originals reachable for mutants that wrap them
    mod.__dict__["_orig_rope"] = mod.rope
    mod.__dict__["_orig_attention"] = mod.attention
    mod.__dict__["_orig_pack_tables"] = mod.pack_tables
    mod.__dict__["_orig_gated_residual"] = mod.gated_residual
    for fname, fn in MUTANTS[name].items():
        setattr(mod, fname, types.FunctionType(fn.__code__, mod.__dict__, fname,
                                               fn.__defaults__, fn.__closure__))
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin rejects mutant {name}"
