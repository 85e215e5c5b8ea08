"""Pins of the oracle against facts fixed outside it.

Each pin is a function taking an oracle-like module ``o`` (the real
``oracle.reference`` or a deliberately broken copy) and raising
AssertionError when ``o`` disagrees with the fact.  The real oracle must pass
every pin; each mutant in ``test_oracle_mutants.py`` must fail at least one.

What pins what (none of these values comes from the oracle itself):
  * golden hand-derived tables and trigonometric closed values
    (``tests/golden``);
  * invariants of the definitions (RoPE preserves norms, relative-position
    dependence, composition; LN statistics; softmax weights);
  * special cases that reduce to an independent library routine (torch's
    float64 ``layer_norm`` and ``scaled_dot_product_attention``);
  * brute force by the pure-Python loop version on tiny packs.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Tables
# ---------------------------------------------------------------------------

def pin_tables_golden(o):
    g = _golden("tiny_pack_tables.json")
    for pack in g["packs"]:
        descs = [tuple(d) for d in pack["descs"]]
        cu, pos, seq_id, mod_row = o.pack_tables(descs)
        assert list(cu) == pack["cu_seqlens"], (pack["name"], list(cu))
        for t, p in pack["positions"].items():
            assert list(pos[int(t)]) == p, (pack["name"], t, list(pos[int(t)]), p)
        for t, s in pack["seq_id"].items():
            assert int(seq_id[int(t)]) == s
        for t, m in pack["mod_row"].items():
            assert int(mod_row[int(t)]) == m


def pin_tables_invariants(o, n_lists=200, seed=7):
    from packed_attention_amd.workloads import random_descs
    rng = _rng(seed)
    for _ in range(n_lists):
        descs = random_descs(rng)
        cu, pos, seq_id, mod_row = o.pack_tables(descs)
        assert cu[0] == 0 and np.all(np.diff(cu) >= 0)
        assert len(pos) == cu[-1] == len(seq_id) == len(mod_row)
        for s, (t, F, h, w, rt, ri) in enumerate(descs):
            a, b = int(cu[s]), int(cu[s + 1])
            assert b - a == t + F * h * w
            assert np.all(seq_id[a:b] == s)
            assert np.all(pos[a:a + t] == 0) and np.all(mod_row[a:a + t] == rt)
            img = pos[a + t:b]
            assert np.all(mod_row[a + t:b] == ri)
            if len(img):
                assert img[:, 0].max() < F and img[:, 1].max() < h and img[:, 2].max() < w
                assert len({tuple(r) for r in img}) == len(img)   # unique (f, r, c)
        # brute force agreement
        bcu, bpos, bsid, bmr = brute.tables(descs)
        assert list(cu) == bcu
        assert pos.tolist() == bpos if len(bpos) else len(pos) == 0
        assert seq_id.tolist() == bsid and mod_row.tolist() == bmr


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def pin_rope_closed_values(o):
    g = _golden("rope_closed_values.json")
    for case in g["cases"]:
        d = case["d"]
        u = np.asarray(case["input"], dtype=np.float64).reshape(1, 1, d)
        pos = np.asarray([case["pos"]], dtype=np.int32)
        out = o.rope(u, pos, tuple(case["dims"]), 10000.0)
        np.testing.assert_allclose(out.reshape(d), case["output"], rtol=0, atol=1e-15,
                                   err_msg=case["why"])
    for D, val in g["ladder"]["values"].items():
        th = o.rope_thetas(int(D), 10000.0)
        assert len(th) == int(D) // 2 and th[0] == 1.0
        assert abs(th[-1] - val) <= 1e-15 * 10, (D, th[-1], val)


def _rand_rope_inputs(seed, T=7, H=3, dims=(4, 6, 6)):
    rng = _rng(seed)
    d = sum(dims)
    u = rng.standard_normal((T, H, d))
    pos = np.stack([rng.integers(0, 3, T), rng.integers(0, 130, T), rng.integers(0, 130, T)],
                   axis=1).astype(np.int32)
    return u, pos, dims


def pin_rope_invariants(o, seed=11):
    u, pos, dims = _rand_rope_inputs(seed)
    T, H, d = u.shape
    base = 10000.0
    # zero angle is the identity
    z = o.rope(u, np.zeros_like(pos), dims, base)
    np.testing.assert_array_equal(z, u)
    r = o.rope(u, pos, dims, base)
    # per-pair norms preserved (hence per-head norms)
    n0 = u[..., 0::2] ** 2 + u[..., 1::2] ** 2
    n1 = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12, atol=1e-12)
    # <R(p) q, R(p') k> depends only on p' - p, axis by axis
    rng = _rng(seed + 1)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    for shift in ([0, 5, 0], [0, 0, 9], [1, 0, 0], [1, 3, 7]):
        shift = np.asarray(shift, dtype=np.int32)
        for p in ([0, 0, 0], [1, 17, 4], [0, 120, 33]):
            p = np.asarray([p], dtype=np.int32)
            a = np.sum(o.rope(q, p, dims, base) * o.rope(k, p + shift, dims, base))
            b = np.sum(q * o.rope(k, shift[None, :], dims, base))
            assert abs(a - b) < 1e-10, (shift, p, a, b)
    # R(p) R(p') = R(p + p')
    p1 = pos
    p2 = np.roll(pos, 1, axis=0)
    np.testing.assert_allclose(o.rope(o.rope(u, p1, dims, base), p2, dims, base),
                               o.rope(u, p1 + p2, dims, base), rtol=0, atol=1e-11)
    # brute-force agreement (single head lists)
    for t in range(T):
        for h in range(H):
            bb = brute.rope_head(list(u[t, h]), list(pos[t]), dims, base)
            np.testing.assert_allclose(r[t, h], bb, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Modulation
# ---------------------------------------------------------------------------

def pin_modulate(o, seed=13):
    import torch
    rng = _rng(seed)
    T, C, n_rows = 9, 48, 3
    eps = 1e-6
    x = rng.standard_normal((T, C)) * 2.0 + 0.7
    shift = rng.standard_normal((n_rows, C)) * 0.1
    scale = rng.standard_normal((n_rows, C)) * 0.1
    mod_row = rng.integers(0, n_rows, T).astype(np.int32)
    # plain LN when shift = scale = 0, against torch's float64 layer_norm
    zeros = np.zeros((n_rows, C))
    ln = o.modulate(x, zeros, zeros, mod_row, eps)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (C,), eps=eps).numpy()
    np.testing.assert_allclose(ln, ref, rtol=0, atol=1e-12)
    # statistics of the normalised row
    var = x.var(axis=1)
    np.testing.assert_allclose(ln.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(ln.var(axis=1), var / (var + eps), rtol=1e-12)
    # scale = -1 gives shift exactly (to rounding); constant row gives shift
    m = o.modulate(x, shift, -np.ones((n_rows, C)), mod_row, eps)
    np.testing.assert_allclose(m, shift[mod_row], rtol=0, atol=1e-15)
    xc = np.full((T, C), 3.25)
    m = o.modulate(xc, shift, scale, mod_row, eps)
    np.testing.assert_allclose(m, shift[mod_row], rtol=0, atol=1e-15)
    # brute force with real rows
    m = o.modulate(x, shift, scale, mod_row, eps)
    for t in range(T):
        b = brute.modulate_row(list(x[t]), list(shift[mod_row[t]]), list(scale[mod_row[t]]), eps)
        np.testing.assert_allclose(m[t], b, rtol=0, atol=1e-12)


def pin_modulate_rope_chain(o, seed=17):
    """modulate_rope = modulate over the H*d row, then per-head RoPE (brute force)."""
    rng = _rng(seed)
    T, H, dims = 5, 2, (2, 4, 6)
    d = sum(dims)
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    pos = np.stack([rng.integers(0, 2, T), rng.integers(0, 9, T), rng.integers(0, 9, T)], 1)
    pos = pos.astype(np.int32)
    shift = rng.standard_normal((2, H * d)) * 0.1
    scale = rng.standard_normal((2, H * d)) * 0.1
    mod_row = np.array([0, 1, 1, 0, 1], dtype=np.int32)
    qr, kr = o.modulate_rope(q, k, pos, dims, 10000.0, shift, scale, mod_row, 1e-6)
    bq = brute.modulate_rope(q.tolist(), pos.tolist(), dims, 10000.0, shift.tolist(),
                             scale.tolist(), mod_row.tolist(), 1e-6)
    bk = brute.modulate_rope(k.tolist(), pos.tolist(), dims, 10000.0, shift.tolist(),
                             scale.tolist(), mod_row.tolist(), 1e-6)
    np.testing.assert_allclose(qr, np.asarray(bq), rtol=0, atol=1e-12)
    np.testing.assert_allclose(kr, np.asarray(bk), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _tiny_attn_inputs(seed, lens=(3, 1, 6, 4), H=2, d=8):
    rng = _rng(seed)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    return q, k, v, cu


def pin_attention_brute(o, seed=19):
    for lens, H, d in (((3, 1, 6, 4), 2, 8), ((5,), 1, 4), ((2, 7), 3, 16)):
        q, k, v, cu = _tiny_attn_inputs(seed, lens, H, d)
        O, L = o.attention(q, k, v, cu)
        bO, bL = brute.attention(q.tolist(), k.tolist(), v.tolist(), list(cu))
        np.testing.assert_allclose(O, np.asarray(bO), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, np.asarray(bL), rtol=0, atol=1e-12)


def pin_attention_sdpa(o, seed=23):
    """With zero-angle RoPE, each sample reduces to plain softmax attention:
    compare per sample and head with torch's float64 SDPA."""
    import torch
    q, k, v, cu = _tiny_attn_inputs(seed, (9, 4, 13), 3, 16)
    O, _ = o.attention(q, k, v, cu)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        Q = torch.from_numpy(q[a:b]).permute(1, 0, 2)
        K = torch.from_numpy(k[a:b]).permute(1, 0, 2)
        V = torch.from_numpy(v[a:b]).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(O[a:b], ref, rtol=0, atol=1e-12)


def pin_attention_packed_equals_alone(o, seed=29):
    q, k, v, cu = _tiny_attn_inputs(seed, (5, 8, 3), 2, 8)
    O, L = o.attention(q, k, v, cu)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        Oa, La = o.attention(q[a:b], k[a:b], v[a:b], np.array([0, b - a]))
        np.testing.assert_array_equal(O[a:b], Oa)
        np.testing.assert_array_equal(L[:, a:b], La)


def pin_attention_special_cases(o, seed=31):
    q, k, v, cu = _tiny_attn_inputs(seed, (4, 1, 6), 2, 8)
    T, H, d = q.shape
    # q = 0: uniform weights -> mean of V over the sample; LSE = log L
    O, L = o.attention(np.zeros_like(q), k, v, cu)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        np.testing.assert_allclose(O[a:b], np.broadcast_to(v[a:b].mean(axis=0), O[a:b].shape),
                                   rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[:, a:b], math.log(b - a), rtol=0, atol=1e-14)
    # L = 1: O = V
    O, _ = o.attention(q, k, v, cu)
    np.testing.assert_allclose(O[4], v[4], rtol=0, atol=1e-15)
    # constant V inside a sample gives that constant
    vc = v.copy()
    vc[5:11] = 2.5
    O, _ = o.attention(q, k, vc, cu)
    np.testing.assert_allclose(O[5:11], 2.5, rtol=0, atol=1e-14)
    # permuting tokens inside a sample permutes its output rows
    O, _ = o.attention(q, k, v, cu)
    perm = np.arange(T)
    perm[5:11] = 5 + np.array([3, 0, 5, 1, 4, 2])
    Op, Lp = o.attention(q[perm], k[perm], v[perm], cu)
    np.testing.assert_allclose(Op, O[perm], rtol=0, atol=1e-13)
    # LSE of a single-key softmax is the scaled score
    _, L = o.attention(q, k, v, cu)
    assert abs(L[0, 4] - np.dot(q[4, 0], k[4, 0]) / math.sqrt(d)) < 1e-13


def pin_attention_rows(o, seed=37):
    """Sampled-row evaluation equals the full evaluation."""
    q, k, v, cu = _tiny_attn_inputs(seed, (7, 2, 9), 2, 8)
    O, L = o.attention(q, k, v, cu)
    rows = [0, 6, 7, 8, 9, 17]
    heads = [0, 1, 1, 0, 1, 0]
    Os, Ls = o.attention_rows(q, k, v, cu, rows, heads)
    for n, (t, h) in enumerate(zip(rows, heads)):
        np.testing.assert_allclose(Os[n], O[t, h], rtol=0, atol=1e-13)
        assert abs(Ls[n] - L[h, t]) < 1e-13


# ---------------------------------------------------------------------------
# Gated residual
# ---------------------------------------------------------------------------

def pin_gated_residual(o, seed=41):
    rng = _rng(seed)
    T, H, d, n_rows = 6, 2, 4, 2
    C = H * d
    x = rng.standard_normal((T, C))
    oo = rng.standard_normal((T, H, d))
    gate = rng.standard_normal((n_rows, C)) * 0.1
    sh = rng.standard_normal((n_rows, C)) * 0.1
    sc = rng.standard_normal((n_rows, C)) * 0.1
    mod_row = np.array([0, 0, 1, 1, 0, 1], dtype=np.int32)
    # gate = 0: y is x exactly
    y, z = o.gated_residual(x, oo, np.zeros_like(gate), mod_row)
    np.testing.assert_array_equal(y, x)
    assert z is None
    # gate = 1, o = -x: y = 0
    y, _ = o.gated_residual(x, -x.reshape(T, H, d), np.ones_like(gate), mod_row)
    np.testing.assert_array_equal(y, 0.0)
    # brute force, with z
    y, z = o.gated_residual(x, oo, gate, mod_row, sh, sc, 1e-6)
    by, bz = brute.gated_residual(x.tolist(), oo.reshape(T, C).tolist(), gate.tolist(),
                                  mod_row.tolist(), sh.tolist(), sc.tolist(), 1e-6)
    np.testing.assert_allclose(y, np.asarray(by), rtol=0, atol=1e-14)
    np.testing.assert_allclose(z, np.asarray(bz), rtol=0, atol=1e-12)
    # z with scale2 = -1 is shift2
    _, z = o.gated_residual(x, oo, gate, mod_row, sh, -np.ones_like(sc), 1e-6)
    np.testing.assert_allclose(z, sh[mod_row], rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# Whole chain on the tiny pack, against brute force
# ---------------------------------------------------------------------------

def pin_chain_brute(o):
    from packed_attention_amd import workloads as W
    w = W.tiny_mod()
    f = W.bf16_bits_to_f64
    q, k, v, x = f(w.q), f(w.k), f(w.v), f(w.x)
    sh, sc, g, sh2, sc2 = (f(a) for a in (w.shift, w.scale, w.gate, w.shift2, w.scale2))
    r = o.forward(w.descs, q, k, v, w.rope_dims, w.rope_base, sh, sc, x, g, sh2, sc2, w.eps)
    cu, pos, sid, mr = brute.tables(w.descs)
    bq = brute.modulate_rope(q.tolist(), pos, w.rope_dims, w.rope_base, sh.tolist(),
                             sc.tolist(), mr, w.eps)
    bk = brute.modulate_rope(k.tolist(), pos, w.rope_dims, w.rope_base, sh.tolist(),
                             sc.tolist(), mr, w.eps)
    bO, bL = brute.attention(bq, bk, v.tolist(), cu)
    T = w.T
    bo_flat = [[bO[t][h][e] for h in range(w.H) for e in range(w.D)] for t in range(T)]
    by, bz = brute.gated_residual(x.tolist(), bo_flat, g.tolist(), mr, sh2.tolist(),
                                  sc2.tolist(), w.eps)
    np.testing.assert_allclose(r["q"], np.asarray(bq), rtol=0, atol=1e-11)
    np.testing.assert_allclose(r["O"], np.asarray(bO), rtol=0, atol=1e-11)
    np.testing.assert_allclose(r["LSE"], np.asarray(bL), rtol=0, atol=1e-11)
    np.testing.assert_allclose(r["y"], np.asarray(by), rtol=0, atol=1e-11)
    np.testing.assert_allclose(r["z"], np.asarray(bz), rtol=0, atol=1e-10)


ALL_PINS = [
    pin_tables_golden, pin_tables_invariants, pin_rope_closed_values, pin_rope_invariants,
    pin_modulate, pin_modulate_rope_chain, pin_attention_brute, pin_attention_sdpa,
    pin_attention_packed_equals_alone, pin_attention_special_cases, pin_attention_rows,
    pin_gated_residual, pin_chain_brute,
]
