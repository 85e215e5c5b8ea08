"""Pins of the backward oracle against facts fixed outside it.

Each pin takes a backward-oracle-like module ``b`` (the real
``oracle.backward`` or a deliberately broken copy) and raises AssertionError
when ``b`` disagrees.  The real module passes every pin; each mutant in
``test_backward_mutants.py`` fails at least one.

What pins what (no expected value comes from ``oracle.backward`` itself):
  * torch automatic differentiation in float64 on the CPU through torch's own
    library routines: ``scaled_dot_product_attention`` for attention and
    ``layer_norm`` for the adaLN steps, with RoPE written as a complex
    multiplication (a different formulation from the oracle's pair rotation);
  * central finite differences of the pinned forward oracle
    (``oracle.reference``) along random directions;
  * closed forms: uniform attention (q = 0) gives dK = 0 and dV = the
    sample's mean of dO; a one-token sample gives dQ = dK = 0 and dV = dO;
    RoPE's gradient undoes the rotation; gate = 0 blocks the attention
    branch's gradient; without the fused adaLN, dx = dy and dgate = sum dy*o;
  * structure: packed equals each sample alone; sampled rows and keys equal
    the full evaluation.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import reference as R
from packed_attention_amd import workloads as W


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny_pack(seed, H=2, d=64, modulate=True):
    """The tiny pack's descriptors with float64 tensors drawn here."""
    descs = W.descs_tiny()
    cu, pos, _, mr = R.pack_tables(descs)
    T = int(cu[-1])
    C = H * d
    rng = _rng(seed)
    t = dict(q=rng.standard_normal((T, H, d)), k=rng.standard_normal((T, H, d)),
             v=rng.standard_normal((T, H, d)), dO=rng.standard_normal((T, H, d)),
             x=rng.standard_normal((T, C)), dy=rng.standard_normal((T, C)),
             dz=rng.standard_normal((T, C)))
    n_rows = len(descs)
    for name in ("shift", "scale", "gate", "shift2", "scale2"):
        t[name] = 0.1 * rng.standard_normal((n_rows, C)) if modulate else None
    return descs, cu, pos, mr, t


def _rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


# ---------------------------------------------------------------------------
# torch float64 autograd references (library routines)
# ---------------------------------------------------------------------------

def _torch_attention_grads(q, k, v, dO, cu):
    import torch
    import torch.nn.functional as F
    T, H, d = q.shape
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        tq = torch.tensor(q[a:b].transpose(1, 0, 2).copy(), dtype=torch.float64, requires_grad=True)
        tk = torch.tensor(k[a:b].transpose(1, 0, 2).copy(), dtype=torch.float64, requires_grad=True)
        tv = torch.tensor(v[a:b].transpose(1, 0, 2).copy(), dtype=torch.float64, requires_grad=True)
        out = F.scaled_dot_product_attention(tq, tk, tv)
        g = torch.tensor(dO[a:b].transpose(1, 0, 2).copy(), dtype=torch.float64)
        (out * g).sum().backward()
        dq[a:b] = tq.grad.numpy().transpose(1, 0, 2)
        dk[a:b] = tk.grad.numpy().transpose(1, 0, 2)
        dv[a:b] = tv.grad.numpy().transpose(1, 0, 2)
    return dq, dk, dv


def _torch_rope(u, pos, dims, base):
    """RoPE as a complex multiplication of (u[2j] + i u[2j+1]) by exp(i phi)."""
    import torch
    T, H, d = u.shape
    parts = []
    o = 0
    for axis, Da in enumerate(dims):
        if Da == 0:
            continue
        j = torch.arange(Da // 2, dtype=torch.float64)
        theta = torch.pow(torch.tensor(base, dtype=torch.float64), -2.0 * j / Da)
        phi = torch.tensor(pos[:, axis], dtype=torch.float64)[:, None] * theta[None, :]
        rot = torch.polar(torch.ones_like(phi), phi)[:, None, :]          # [T][1][Da/2]
        seg = u[:, :, o:o + Da].reshape(T, H, Da // 2, 2)
        z = torch.view_as_complex(seg.contiguous()) * rot
        parts.append(torch.view_as_real(z).reshape(T, H, Da))
        o += Da
    return torch.cat(parts, dim=-1)


def _torch_modulate(x2d, shift, scale, mr, eps):
    import torch
    import torch.nn.functional as F
    C = x2d.shape[-1]
    xh = F.layer_norm(x2d, (C,), eps=eps)
    idx = torch.tensor(mr, dtype=torch.long)
    return xh * (1.0 + scale[idx]) + shift[idx]


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def pin_attn_bwd_autograd(b, seed=101):
    descs, cu, pos, mr, t = _tiny_pack(seed)
    got = b.attention_bwd(t["q"], t["k"], t["v"], t["dO"], cu)
    ref = _torch_attention_grads(t["q"], t["k"], t["v"], t["dO"], cu)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert _rel(g, r) <= 1e-10, (name, _rel(g, r))


def pin_attn_bwd_finite_diff(b, seed=103, h=1e-5):
    descs, cu, pos, mr, t = _tiny_pack(seed)
    q, k, v, dO = t["q"], t["k"], t["v"], t["dO"]
    dq, dk, dv = b.attention_bwd(q, k, v, dO, cu)
    rng = _rng(seed + 1)
    f = lambda qq, kk, vv: float((R.attention(qq, kk, vv, cu)[0] * dO).sum())  # noqa: E731
    for which, g in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(3):
            dlt = rng.standard_normal(q.shape)
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[which] = args_p[which] + h * dlt
            args_m[which] = args_m[which] - h * dlt
            fd = (f(args_p["q"], args_p["k"], args_p["v"]) - f(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            an = float((g * dlt).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def pin_attn_bwd_closed_forms(b, seed=107):
    descs, cu, pos, mr, t = _tiny_pack(seed)
    T, H, d = t["q"].shape
    # q = 0: every softmax row is uniform over its sample
    q0 = np.zeros_like(t["q"])
    dq, dk, dv = b.attention_bwd(q0, t["k"], t["v"], t["dO"], cu)
    assert np.abs(dk).max() <= 1e-12
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        mean_dO = t["dO"][a:e].mean(axis=0)
        assert np.abs(dv[a:e] - mean_dO[None]).max() <= 1e-12
    # one-token samples: softmax weight 1 and no dependence on q or k
    cu1 = np.arange(T + 1, dtype=np.int32)
    dq, dk, dv = b.attention_bwd(t["q"], t["k"], t["v"], t["dO"], cu1)
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    assert np.abs(dv - t["dO"]).max() <= 1e-12


def pin_attn_bwd_packed_equals_alone(b, seed=109):
    descs, cu, pos, mr, t = _tiny_pack(seed)
    full = b.attention_bwd(t["q"], t["k"], t["v"], t["dO"], cu)
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        alone = b.attention_bwd(t["q"][a:e], t["k"][a:e], t["v"][a:e], t["dO"][a:e],
                                np.array([0, e - a], dtype=np.int32))
        for g, r in zip(full, alone):
            assert np.abs(g[a:e] - r).max() <= 1e-13


def pin_attn_bwd_sampled(b, seed=113):
    descs, cu, pos, mr, t = _tiny_pack(seed)
    T, H, d = t["q"].shape
    dq, dk, dv = b.attention_bwd(t["q"], t["k"], t["v"], t["dO"], cu, chunk=7)
    rng = _rng(seed)
    toks = rng.integers(0, T, size=20)
    heads = rng.integers(0, H, size=20)
    sq = b.attention_bwd_rows(t["q"], t["k"], t["v"], t["dO"], cu, toks, heads)
    sk, sv = b.attention_bwd_keys(t["q"], t["k"], t["v"], t["dO"], cu, toks, heads, chunk=5)
    assert np.abs(sq - dq[toks, heads]).max() <= 1e-12
    assert np.abs(sk - dk[toks, heads]).max() <= 1e-12
    assert np.abs(sv - dv[toks, heads]).max() <= 1e-12


# ---------------------------------------------------------------------------
# modulate + RoPE
# ---------------------------------------------------------------------------

def pin_rope_bwd_undoes_rotation(b, seed=127):
    descs, cu, pos, mr, t = _tiny_pack(seed)
    dims = (0, 32, 32)
    u = t["q"]
    back = b.rope_bwd(R.rope(u, pos, dims, 10000.0), pos, dims, 10000.0)
    assert np.abs(back - u).max() <= 1e-12
    # 3D split with frames
    descs3 = [(3, 2, 2, 3, 0, 0)]
    cu3, pos3, _, _ = R.pack_tables(descs3)
    u3 = _rng(seed + 1).standard_normal((int(cu3[-1]), 2, 32))
    back3 = b.rope_bwd(R.rope(u3, pos3, (8, 12, 12), 100.0), pos3, (8, 12, 12), 100.0)
    assert np.abs(back3 - u3).max() <= 1e-12


def pin_modrope_bwd_autograd(b, seed=131, eps=1e-6):
    import torch
    descs, cu, pos, mr, t = _tiny_pack(seed)
    T, H, d = t["q"].shape
    C = H * d
    dims, base = (0, 32, 32), 10000.0
    dq_out = _rng(seed + 2).standard_normal((T, H, d))
    dk_out = _rng(seed + 3).standard_normal((T, H, d))
    tq = torch.tensor(t["q"].reshape(T, C), requires_grad=True)
    tk = torch.tensor(t["k"].reshape(T, C), requires_grad=True)
    sh = torch.tensor(t["shift"], requires_grad=True)
    sc = torch.tensor(t["scale"], requires_grad=True)
    loss = 0
    for X, G in ((tq, dq_out), (tk, dk_out)):
        u = _torch_modulate(X, sh, sc, mr, eps).reshape(T, H, d)
        loss = loss + (_torch_rope(u, pos, dims, base) * torch.tensor(G)).sum()
    loss.backward()
    dq, dk, dsh, dsc = b.modulate_rope_bwd(t["q"], t["k"], pos, dims, base, dq_out, dk_out,
                                           t["shift"], t["scale"], mr, len(descs), eps)
    for name, g, r in (("dq", dq, tq.grad.numpy().reshape(T, H, d)),
                       ("dk", dk, tk.grad.numpy().reshape(T, H, d)),
                       ("dshift", dsh, sh.grad.numpy()), ("dscale", dsc, sc.grad.numpy())):
        assert _rel(g, r) <= 1e-10, (name, _rel(g, r))
    # RoPE only (no modulation): the gradient is the back-rotation alone
    tq2 = torch.tensor(t["q"], requires_grad=True)
    (_torch_rope(tq2, pos, dims, base) * torch.tensor(dq_out)).sum().backward()
    dq2, _, dsh2, _ = b.modulate_rope_bwd(t["q"], t["k"], pos, dims, base, dq_out, dk_out)
    assert dsh2 is None and _rel(dq2, tq2.grad.numpy()) <= 1e-12


def pin_modrope_bwd_finite_diff(b, seed=137, h=1e-6, eps=1e-6):
    descs, cu, pos, mr, t = _tiny_pack(seed)
    dims, base = (0, 32, 32), 10000.0
    T, H, d = t["q"].shape
    gq = _rng(seed + 2).standard_normal((T, H, d))
    gk = _rng(seed + 3).standard_normal((T, H, d))
    args = dict(q=t["q"], k=t["k"], shift=t["shift"], scale=t["scale"])

    def f(a):
        qr, kr = R.modulate_rope(a["q"], a["k"], pos, dims, base, a["shift"], a["scale"], mr, eps)
        return float((qr * gq).sum() + (kr * gk).sum())

    grads = dict(zip(("q", "k", "shift", "scale"),
                     b.modulate_rope_bwd(t["q"], t["k"], pos, dims, base, gq, gk, t["shift"],
                                         t["scale"], mr, len(descs), eps)))
    rng = _rng(seed + 4)
    for name in ("q", "k", "shift", "scale"):
        dlt = rng.standard_normal(args[name].shape)
        ap = dict(args); am = dict(args)
        ap[name] = args[name] + h * dlt
        am[name] = args[name] - h * dlt
        fd = (f(ap) - f(am)) / (2 * h)
        an = float((grads[name] * dlt).sum())
        assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (name, fd, an)


# ---------------------------------------------------------------------------
# Gated residual
# ---------------------------------------------------------------------------

def pin_gres_bwd_autograd(b, seed=139, eps=1e-6):
    import torch
    descs, cu, pos, mr, t = _tiny_pack(seed)
    T, H, d = t["q"].shape
    C = H * d
    o = _rng(seed + 5).standard_normal((T, C))
    tx = torch.tensor(t["x"], requires_grad=True)
    to = torch.tensor(o, requires_grad=True)
    tg = torch.tensor(t["gate"], requires_grad=True)
    ts = torch.tensor(t["shift2"], requires_grad=True)
    tc = torch.tensor(t["scale2"], requires_grad=True)
    idx = torch.tensor(mr, dtype=torch.long)
    y = tx + tg[idx] * to
    z = _torch_modulate(y, ts, tc, mr, eps)
    ((y * torch.tensor(t["dy"])).sum() + (z * torch.tensor(t["dz"])).sum()).backward()
    dx, do, dg, ds2, dc2 = b.gated_residual_bwd(t["x"], o, t["gate"], mr, t["dy"], t["dz"],
                                                t["shift2"], t["scale2"], len(descs), eps)
    for name, g, r in (("dx", dx, tx.grad), ("do", do, to.grad), ("dgate", dg, tg.grad),
                       ("dshift2", ds2, ts.grad), ("dscale2", dc2, tc.grad)):
        assert _rel(g, r.numpy()) <= 1e-10, (name, _rel(g, r.numpy()))


def pin_gres_bwd_closed_forms(b, seed=149):
    descs, cu, pos, mr, t = _tiny_pack(seed)
    T, C = t["x"].shape
    o = _rng(seed + 5).standard_normal((T, C))
    # no fused adaLN: dx = dy, do = gate * dy, dgate = per-row sum of dy * o
    dx, do, dg, ds2, dc2 = b.gated_residual_bwd(t["x"], o, t["gate"], mr, t["dy"], None,
                                                n_rows=len(descs))
    assert ds2 is None and dc2 is None
    assert np.array_equal(dx, t["dy"])
    assert np.abs(do - t["gate"][mr] * t["dy"]).max() <= 1e-15
    for r in range(len(descs)):
        sel = mr == r
        assert np.abs(dg[r] - (t["dy"][sel] * o[sel]).sum(axis=0)).max() <= 1e-12
    # gate = 0: nothing flows into the attention branch
    _, do0, _, _, _ = b.gated_residual_bwd(t["x"], o, np.zeros_like(t["gate"]), mr, t["dy"],
                                           t["dz"], t["shift2"], t["scale2"], len(descs))
    assert np.abs(do0).max() == 0.0


# ---------------------------------------------------------------------------
# Whole chain
# ---------------------------------------------------------------------------

def pin_chain_bwd_finite_diff(b, seed=151, h=1e-6, eps=1e-6):
    descs, cu, pos, mr, t = _tiny_pack(seed)
    dims, base = (0, 32, 32), 10000.0
    names = ("q", "k", "v", "x", "shift", "scale", "gate", "shift2", "scale2")
    args = {n: t[n] for n in names}

    def f(a):
        fw = R.forward(descs, a["q"], a["k"], a["v"], dims, base, a["shift"], a["scale"], a["x"],
                       a["gate"], a["shift2"], a["scale2"], eps)
        return float((fw["y"] * t["dy"]).sum() + (fw["z"] * t["dz"]).sum())

    g = b.backward(descs, t["q"], t["k"], t["v"], dims, base, t["dy"], t["dz"], t["shift"],
                   t["scale"], t["x"], t["gate"], t["shift2"], t["scale2"], eps)
    key = dict(q="dq", k="dk", v="dv", x="dx", shift="dshift", scale="dscale", gate="dgate",
               shift2="dshift2", scale2="dscale2")
    rng = _rng(seed + 7)
    for name in names:
        dlt = rng.standard_normal(args[name].shape)
        ap = dict(args); am = dict(args)
        ap[name] = args[name] + h * dlt
        am[name] = args[name] - h * dlt
        fd = (f(ap) - f(am)) / (2 * h)
        an = float((g[key[name]] * dlt).sum())
        assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (name, fd, an)


ALL_PINS = [
    pin_attn_bwd_autograd, pin_attn_bwd_finite_diff, pin_attn_bwd_closed_forms,
    pin_attn_bwd_packed_equals_alone, pin_attn_bwd_sampled, pin_rope_bwd_undoes_rotation,
    pin_modrope_bwd_autograd, pin_modrope_bwd_finite_diff, pin_gres_bwd_autograd,
    pin_gres_bwd_closed_forms, pin_chain_bwd_finite_diff,
]
