"""Pins of the text-encoder oracle against facts fixed outside it.

Each pin takes a module ``e`` (the real ``oracle.text_encoder`` or a broken
copy) and raises AssertionError when ``e`` disagrees.  What pins what:
  * torch in float64 on the CPU: ``scaled_dot_product_attention`` with
    ``is_causal=True`` on each prompt alone, key/value heads repeated for the
    grouped query heads; ``rms_norm``; RoPE as a complex multiplication;
  * closed forms: a prompt's first token attends only to itself (O = its v,
    LSE = its own scaled score); position 0 leaves a row unrotated; a
    constant weight w scales the normalised row by w;
  * scalar loops on a tiny case (mask, grouping and softmax written out);
  * structure: packed equals each prompt alone.
"""
from __future__ import annotations

import math

import numpy as np


def _case(seed, lens=(5, 1, 9, 3), Hq=4, Hkv=2, d=8):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    return cu, q, k, v


def _close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.max(np.abs(a - b)) <= tol * max(1.0, float(np.max(np.abs(b)))), float(np.max(np.abs(a - b)))


def pin_torch_sdpa(e):
    import torch
    import torch.nn.functional as F
    cu, q, k, v = _case(21)
    O, L = e.causal_attention(q, k, v, cu)
    g = q.shape[1] // k.shape[1]
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        Q = torch.tensor(q[a:b]).transpose(0, 1)[None]                     # [1][H][L][d]
        K = torch.tensor(k[a:b]).transpose(0, 1).repeat_interleave(g, dim=0)[None]
        V = torch.tensor(v[a:b]).transpose(0, 1).repeat_interleave(g, dim=0)[None]
        ref = F.scaled_dot_product_attention(Q, K, V, is_causal=True)[0].transpose(0, 1).numpy()
        _close(O[a:b], ref, 1e-9)


def pin_first_token(e):
    cu, q, k, v = _case(22)
    O, L = e.causal_attention(q, k, v, cu)
    g = q.shape[1] // k.shape[1]
    d = q.shape[2]
    for s in range(len(cu) - 1):
        a = int(cu[s])
        for h in range(q.shape[1]):
            _close(O[a, h], v[a, h // g])
            _close(L[h, a], q[a, h] @ k[a, h // g] / math.sqrt(d))


def pin_brute(e):
    cu, q, k, v = _case(23, lens=(3, 4), Hq=2, Hkv=1, d=4)
    O, L = e.causal_attention(q, k, v, cu)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in range(2):
            for i in range(a, b):
                sc = [sum(q[i, h, x] * k[j, 0, x] for x in range(4)) / 2.0 for j in range(a, i + 1)]
                mx = max(sc)
                ws = [math.exp(z - mx) for z in sc]
                tot = sum(ws)
                for x in range(4):
                    o = sum(wj * v[j, 0, x] for wj, j in zip(ws, range(a, i + 1))) / tot
                    assert abs(O[i, h, x] - o) < 1e-12
                assert abs(L[h, i] - (mx + math.log(tot))) < 1e-12


def pin_packed_alone(e):
    cu, q, k, v = _case(24)
    O, L = e.causal_attention(q, k, v, cu)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        O1, L1 = e.causal_attention(q[a:b], k[a:b], v[a:b], np.array([0, b - a]))
        _close(O[a:b], O1)
        _close(L[:, a:b], L1)


def pin_norm_rope_torch(e):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(25)
    cu = np.array([0, 6, 7, 15])
    T, Hq, Hkv, d = 15, 4, 2, 8
    q = rng.standard_normal((T, Hq, d)) * 3.0
    k = rng.standard_normal((T, Hkv, d))
    wq = 1.0 + 0.1 * rng.standard_normal(d)
    wk = 1.0 + 0.1 * rng.standard_normal(d)
    pos = e.positions(cu)
    assert pos.tolist() == [0, 1, 2, 3, 4, 5, 0, 0, 1, 2, 3, 4, 5, 6, 7]
    qo, ko = e.qk_norm_rope(q, k, wq, wk, pos, 10000.0, 1e-6)
    theta = 10000.0 ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(T, d // 2, dtype=torch.float64),
                      torch.tensor(pos, dtype=torch.float64)[:, None] * theta[None])[:, None, :]
    for X, w, got in ((q, wq, qo), (k, wk, ko)):
        n = F.rms_norm(torch.tensor(X), (d,), weight=torch.tensor(w), eps=1e-6)
        z = torch.view_as_complex(n.reshape(T, -1, d // 2, 2).contiguous()) * rot
        _close(got, torch.view_as_real(z).reshape(T, -1, d).numpy(), 1e-12)
    # position 0 is unrotated; a constant weight scales the normalised row
    q0, _ = e.qk_norm_rope(q, k, np.full(d, 2.0), wk, np.zeros(T, dtype=np.int64), 10000.0, 1e-6)
    rms = np.sqrt((q * q).mean(axis=-1, keepdims=True) + 1e-6)
    _close(q0, 2.0 * q / rms)


def pin_rows(e):
    """The row-at-a-time evaluation equals the full one (first, middle and
    last rows of every prompt)."""
    cu, q, k, v = _case(26, lens=(5, 1, 9, 3, 12))
    O, L = e.causal_attention(q, k, v, cu)
    rows = [0, 2, 4, 5, 6, 10, 14, 15, 17, 18, 25, 29]
    Or, Lr = e.causal_attention_rows(q, k, v, cu, rows)
    _close(Or, O[rows])
    _close(Lr, L[:, rows])


ALL_PINS = [pin_torch_sdpa, pin_first_token, pin_brute, pin_packed_alone, pin_norm_rope_torch, pin_rows]
