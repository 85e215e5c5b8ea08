"""Pins of the block-projection oracle against facts fixed outside it.

Each pin takes a module ``b`` (the real ``oracle.block`` or a deliberately
broken copy) and raises AssertionError when ``b`` disagrees.  The real module
passes every pin; each mutant in ``test_block_mutants.py`` fails at least one.

What pins what (no expected value comes from ``oracle.block`` itself):
  * pure-Python loops on a tiny case: LayerNorm, modulation, the projection
    sum and the pair rotation written out element by element;
  * torch in float64 on the CPU through its own library routines
    (``layer_norm``, ``linear``), with RoPE as a complex multiplication (a
    different formulation from the oracle's pair rotation);
  * structure: a permutation weight matrix moves channels (orientation of
    W and the q / k / v column split), the identity out projection reduces
    to the gated residual, rows evaluated alone equal the full evaluation.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import reference as R


def _case(seed, T=7, H=2, d=8, n_rows=2, dims=(0, 4, 4)):
    rng = np.random.default_rng(seed)
    C = H * d
    x = rng.standard_normal((T, C)) * 1.5 + 0.3
    w = rng.standard_normal((3 * C, C)) / math.sqrt(C)
    shift = rng.standard_normal((n_rows, C)) * 0.2
    scale = rng.standard_normal((n_rows, C)) * 0.2
    mod_row = rng.integers(0, n_rows, size=T)
    pos = np.stack([rng.integers(0, 3, T), rng.integers(0, 9, T), rng.integers(0, 11, T)], axis=1)
    return dict(x=x, w=w, shift=shift, scale=scale, mod_row=mod_row, pos=pos, H=H, d=d, dims=dims)


def _close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * max(1.0, float(np.max(np.abs(b))) if b.size else 1.0), err


def pin_brute_loops(b):
    """Every step written out with scalar loops on a tiny case."""
    c = _case(11, T=5, H=2, d=4, dims=(0, 2, 2))
    x, w, H, d = c["x"], c["w"], c["H"], c["d"]
    T, C = x.shape
    eps, base = 1e-6, 10000.0
    q = [[0.0] * C for _ in range(T)]
    k = [[0.0] * C for _ in range(T)]
    v = [[0.0] * C for _ in range(T)]
    for t in range(T):
        row = [float(x[t][i]) for i in range(C)]
        mu = sum(row) / C
        var = sum((r - mu) ** 2 for r in row) / C
        m = int(c["mod_row"][t])
        u = [(row[i] - mu) / math.sqrt(var + eps) * (1.0 + c["scale"][m][i]) + c["shift"][m][i]
             for i in range(C)]
        for n in range(3 * C):
            acc = 0.0
            for i in range(C):
                acc += u[i] * float(w[n][i])
            (q, k, v)[n // C][t][n % C] = acc
    # dims (0, 2, 2): per head, dims 0-1 turn with the row position, 2-3 with
    # the column position, one pair each, theta = base^0 = 1
    for t in range(T):
        for X in (q, k):
            for h in range(H):
                for e0, axis in ((0, 1), (2, 2)):
                    phi = float(c["pos"][t][axis]) * base ** 0.0
                    a0, a1 = X[t][h * d + e0], X[t][h * d + e0 + 1]
                    X[t][h * d + e0] = a0 * math.cos(phi) - a1 * math.sin(phi)
                    X[t][h * d + e0 + 1] = a0 * math.sin(phi) + a1 * math.cos(phi)
    got = b.qkv_projection(x, w, c["pos"], c["dims"], base, H, c["shift"], c["scale"], c["mod_row"], eps)
    for g, e in zip(got, (q, k, v)):
        _close(g.reshape(T, C), np.array(e))


def _torch_rope(X, pos, dims, base):
    """RoPE as a complex multiplication of each adjacent pair by exp(i phi)."""
    import torch
    T, H, d = X.shape
    z = torch.view_as_complex(X.reshape(T, H, d // 2, 2).contiguous())
    phis = []
    for axis, Da in enumerate(dims):
        if Da == 0:
            continue
        theta = base ** (-2.0 * torch.arange(Da // 2, dtype=torch.float64) / Da)
        phis.append(pos[:, axis].to(torch.float64)[:, None] * theta[None, :])
    phi = torch.cat(phis, dim=1)                                    # [T][d/2]
    rot = torch.polar(torch.ones_like(phi), phi)[:, None, :]
    return torch.view_as_real(z * rot).reshape(T, H, d)


def pin_torch(b):
    """torch float64: layer_norm, linear, complex-multiplication RoPE."""
    import torch
    import torch.nn.functional as F
    c = _case(12, T=9, H=2, d=8, dims=(0, 4, 4))
    x, w, H, d = (torch.tensor(c["x"]), torch.tensor(c["w"]), c["H"], c["d"])
    T, C = x.shape
    m = torch.tensor(c["mod_row"])
    u = F.layer_norm(x, (C,), eps=1e-6) * (1.0 + torch.tensor(c["scale"])[m]) + torch.tensor(c["shift"])[m]
    qkv = F.linear(u, w)
    pos = torch.tensor(c["pos"])
    q = _torch_rope(qkv[:, :C].reshape(T, H, d), pos, c["dims"], 10000.0)
    k = _torch_rope(qkv[:, C:2 * C].reshape(T, H, d), pos, c["dims"], 10000.0)
    v = qkv[:, 2 * C:].reshape(T, H, d)
    got = b.qkv_projection(c["x"], c["w"], c["pos"], c["dims"], 10000.0, H, c["shift"], c["scale"],
                           c["mod_row"], 1e-6)
    for g, e in zip(got, (q, k, v)):
        _close(g, e.numpy(), 1e-9)
    # the out projection: y = x + gate * linear(o, W_o)
    rng = np.random.default_rng(13)
    o = rng.standard_normal((T, C))
    wo = rng.standard_normal((C, C)) / math.sqrt(C)
    gate = rng.standard_normal((2, C)) * 0.3
    y = x + torch.tensor(gate)[m] * F.linear(torch.tensor(o), torch.tensor(wo))
    _close(b.out_projection(o.reshape(T, H, d), wo, c["x"], gate, c["mod_row"]), y.numpy(), 1e-9)


def pin_permutation(b):
    """A permutation W moves channels: with all positions 0 (no rotation) and
    no modulation, q[:, n] = x[:, perm[n]] for W[n][perm[n]] = 1, and the
    three column blocks of the output are q, k and v in that order."""
    c = _case(14, T=6, H=2, d=8)
    x, H, d = c["x"], c["H"], c["d"]
    T, C = x.shape
    rng = np.random.default_rng(15)
    perm = rng.permutation(C * 3) % C
    w = np.zeros((3 * C, C))
    w[np.arange(3 * C), perm] = 1.0
    got = b.qkv_projection(x, w, np.zeros((T, 3), dtype=np.int64), c["dims"], 10000.0, H)
    for blk, g in enumerate(got):
        _close(g.reshape(T, C), x[:, perm[blk * C:(blk + 1) * C]])
    wo = np.zeros((C, C))
    p2 = rng.permutation(C)
    wo[np.arange(C), p2] = 1.0
    o = rng.standard_normal((T, C))
    gate = rng.standard_normal((2, C))
    _close(b.out_projection(o, wo, x, gate, c["mod_row"]), x + gate[c["mod_row"]] * o[:, p2])


def pin_identity_reduces(b):
    """W_qkv = [I; I; I] turns the projection into the reference's
    modulate + RoPE step (v = the modulated row), and W_o = I turns the out
    projection into the reference's gated residual; both reference steps are
    pinned on their own."""
    c = _case(16, T=8, H=2, d=8)
    x, H, d = c["x"], c["H"], c["d"]
    T, C = x.shape
    w = np.concatenate([np.eye(C)] * 3, axis=0)
    q, k, v = b.qkv_projection(x, w, c["pos"], c["dims"], 10000.0, H, c["shift"], c["scale"], c["mod_row"])
    xr = x.reshape(T, H, d)
    qe, ke = R.modulate_rope(xr, xr, c["pos"], c["dims"], 10000.0, c["shift"], c["scale"], c["mod_row"])
    _close(q, qe)
    _close(k, ke)
    _close(v.reshape(T, C), R.modulate(x, c["shift"], c["scale"], c["mod_row"], 1e-6))
    o = np.random.default_rng(17).standard_normal((T, C))
    gate = np.random.default_rng(18).standard_normal((2, C))
    _close(b.out_projection(o, np.eye(C), x, gate, c["mod_row"]),
           R.gated_residual(x, o, gate, c["mod_row"])[0])


def pin_rows(b):
    """Rows evaluated alone equal the full evaluation."""
    c = _case(19, T=10, H=2, d=8)
    full = b.qkv_projection(c["x"], c["w"], c["pos"], c["dims"], 10000.0, c["H"], c["shift"], c["scale"],
                            c["mod_row"])
    rows = np.array([9, 0, 4, 4, 7])
    part = b.qkv_projection_rows(c["x"], c["w"], c["pos"], c["dims"], 10000.0, c["H"], rows, c["shift"],
                                 c["scale"], c["mod_row"])
    for f, p in zip(full, part):
        _close(p, f[rows])


ALL_PINS = [pin_brute_loops, pin_torch, pin_permutation, pin_identity_reduces, pin_rows]
