"""Pure-Python loop versions of each oracle step, for tiny packs.

TEST INFRASTRUCTURE ONLY (same rule as the numpy oracle).  Written
independently of the numpy oracle: no numpy, no vectorisation, every sum an
explicit loop, so that an indexing or broadcasting slip in one is not shared
by the other.  Same sources and readings as the numpy oracle.
"""
from __future__ import annotations

import math


def tables(descs):
    cu = [0]
    pos, seq_id, mod_row = [], [], []
    for s, d in enumerate(descs):
        t, F, h, w, rt, ri = d
        L = t + F * h * w
        for j in range(L):
            if j < t:
                pos.append([0, 0, 0])
                mod_row.append(rt)
            else:
                i = j - t
                hw = h * w
                pos.append([i // hw, (i % hw) // w, i % w])
                mod_row.append(ri)
            seq_id.append(s)
        cu.append(cu[-1] + L)
    return cu, pos, seq_id, mod_row


def layer_norm_row(row, eps):
    n = len(row)
    mu = 0.0
    for a in row:
        mu += a
    mu /= n
    var = 0.0
    for a in row:
        var += (a - mu) * (a - mu)
    var /= n
    inv = 1.0 / math.sqrt(var + eps)
    return [(a - mu) * inv for a in row]


def modulate_row(row, shift_row, scale_row, eps):
    xh = layer_norm_row(row, eps)
    return [xh[c] * (1.0 + scale_row[c]) + shift_row[c] for c in range(len(row))]


def rope_head(vec, p, dims, base):
    """vec: list of d floats for one head; p: (frame, row, col)."""
    out = list(vec)
    off = 0
    for axis in range(3):
        Da = dims[axis]
        for j in range(Da // 2):
            theta = base ** (-(2.0 * j) / Da)
            phi = p[axis] * theta
            e0 = off + 2 * j
            e1 = e0 + 1
            a, b = vec[e0], vec[e1]
            out[e0] = a * math.cos(phi) - b * math.sin(phi)
            out[e1] = a * math.sin(phi) + b * math.cos(phi)
        off += Da
    return out


def modulate_rope(X, pos, dims, base, shift=None, scale=None, mod_row=None, eps=1e-6):
    """X: nested lists [T][H][d]."""
    T = len(X)
    H = len(X[0])
    d = len(X[0][0])
    out = []
    for t in range(T):
        flat = [X[t][h][e] for h in range(H) for e in range(d)]
        if shift is not None:
            m = mod_row[t]
            flat = modulate_row(flat, shift[m], scale[m], eps)
        heads = []
        for h in range(H):
            heads.append(rope_head(flat[h * d:(h + 1) * d], pos[t], dims, base))
        out.append(heads)
    return out


def attention(q, k, v, cu, scale=None):
    """q, k, v nested lists [T][H][d]; returns (O [T][H][d], LSE [H][T])."""
    T = len(q)
    H = len(q[0])
    d = len(q[0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = [[[0.0] * d for _ in range(H)] for _ in range(T)]
    LSE = [[0.0] * T for _ in range(H)]
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        for h in range(H):
            for i in range(a, b):
                scores = []
                for j in range(a, b):
                    acc = 0.0
                    for e in range(d):
                        acc += q[i][h][e] * k[j][h][e]
                    scores.append(scale * acc)
                mx = max(scores)
                ex = [math.exp(sc - mx) for sc in scores]
                tot = 0.0
                for w in ex:
                    tot += w
                for e in range(d):
                    acc = 0.0
                    for jj, j in enumerate(range(a, b)):
                        acc += ex[jj] * v[j][h][e]
                    O[i][h][e] = acc / tot
                LSE[h][i] = mx + math.log(tot)
    return O, LSE


def gated_residual(x, o, gate, mod_row, shift2=None, scale2=None, eps=1e-6):
    """x: [T][C] lists; o: [T][C] lists."""
    T = len(x)
    C = len(x[0])
    y = []
    for t in range(T):
        g = gate[mod_row[t]]
        y.append([x[t][c] + g[c] * o[t][c] for c in range(C)])
    z = None
    if shift2 is not None:
        z = [modulate_row(y[t], shift2[mod_row[t]], scale2[mod_row[t]], eps) for t in range(T)]
    return y, z
