"""fp64 oracle of the block projections around the attention.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library: it imports numpy and the oracle's own reference steps.

The pages fuse the adaptive normalisation, the rotary embedding and the
gating / residual chains with the operators around them (picx.dev summary of
Mage-Flow, Methodology > Training Infrastructure; gist.science "Resumo
Tecnico: Mage-Flow", Metodologia > 3. Otimizacao de Nivel de Sistema >
Kernels Fundidos), inside NR-MMDiT blocks whose attention is joint over the
packed text and image tokens (picx.dev, Methodology > Native-Resolution
MMDiT).  In a block those operators are the projections into and out of the
attention.  Readings (the plainest the pages support; listed in the design
notes):

  * the residual stream x [T][C] is adaLN-modulated as in the reference step
    2 (LayerNorm over the C channels without affine, population variance,
    then * (1 + scale[m(t)]) + shift[m(t)]) and projected by one linear map
    W_qkv of shape [3C][C] (output x input, no bias): q, k and v are the
    output columns [0, C), [C, 2C) and [2C, 3C), each viewed as [H][d];
  * q and k are rotated as in the reference step 3; v is not;
  * the out projection maps the attention output o [T][C] by W_o [C][C]
    (output x input, no bias) and the gated residual adds it:
        y = x + gate[m(t)] * (o W_o^T).

Each function is that definition in float64 from the exact input values; the
products are plain matrix products.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import reference as R


def qkv_projection(x: np.ndarray, w_qkv: np.ndarray, pos: np.ndarray, dims: Tuple[int, int, int],
                   base: float, H: int, shift: Optional[np.ndarray] = None,
                   scale: Optional[np.ndarray] = None, mod_row: Optional[np.ndarray] = None,
                   eps: float = 1e-6):
    """(q', k', v), each [T][H][d] float64.

    u = modulate(x) (or x when shift/scale are None); qkv = u W_qkv^T;
    q' = RoPE(q), k' = RoPE(k).
    """
    x = np.asarray(x, dtype=np.float64)
    T, C = x.shape
    d = C // H
    w = np.asarray(w_qkv, dtype=np.float64)
    assert w.shape == (3 * C, C), w.shape
    u = R.modulate(x, shift, scale, mod_row, eps) if shift is not None else x
    qkv = u @ w.T
    q = qkv[:, :C].reshape(T, H, d)
    k = qkv[:, C:2 * C].reshape(T, H, d)
    v = qkv[:, 2 * C:].reshape(T, H, d)
    return R.rope(q, pos, dims, base), R.rope(k, pos, dims, base), v


def out_projection(o: np.ndarray, w_o: np.ndarray, x: np.ndarray, gate: np.ndarray,
                   mod_row: np.ndarray) -> np.ndarray:
    """y = x + gate[m(t)] * (o W_o^T), [T][C] float64; o is [T][H][d] or [T][C]."""
    x = np.asarray(x, dtype=np.float64)
    T, C = x.shape
    o2 = np.asarray(o, dtype=np.float64).reshape(T, C)
    w = np.asarray(w_o, dtype=np.float64)
    assert w.shape == (C, C), w.shape
    return x + np.asarray(gate, dtype=np.float64)[mod_row] * (o2 @ w.T)


def qkv_projection_rows(x, w_qkv, pos, dims, base, H, rows, shift=None, scale=None, mod_row=None,
                        eps: float = 1e-6):
    """qkv_projection restricted to the given token rows (each row depends
    only on its own x row, table entries and the weights)."""
    rows = np.asarray(rows)
    mr = None if mod_row is None else np.asarray(mod_row)[rows]
    return qkv_projection(np.asarray(x)[rows], w_qkv, np.asarray(pos)[rows], dims, base, H,
                          shift, scale, mr, eps)
