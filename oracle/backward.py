"""fp64 CPU oracle for the backward pass of the packed attention hot path.

TEST INFRASTRUCTURE ONLY.  Same rule as ``oracle.reference``: only the
test-suite, the smoke check and the benchmark's CPU-baseline leg may import
it; it imports numpy and nothing from the HIP package.

What it computes.  The pages train the NR-MMDiT with the fused kernels of the
forward path (picx.dev summary of Mage-Flow, Methodology > Training
Infrastructure: fused adaptive-norm / RoPE / gating kernels and the MFU they
reach in training; gist.science "Resumo Tecnico: Mage-Flow", Metodologia >
3. Otimizacao de Nivel de Sistema).  They print no backward formulas, so the
backward is the exact gradient, by the chain rule, of the forward steps as
``oracle.reference`` defines them, for a scalar loss whose gradients with
respect to the forward outputs are given (dO for attention, dy and dz for the
gated residual, dq' and dk' for modulate + RoPE).  Every function is that
gradient written out in float64 from the exact input values; sums over
tokens that share an adaLN row are plain sums.

Formulas (per packed sequence and head for attention; tau = softmax scale):
  attention   S = tau Q K^T, P = softmax_rows(S), O = P V,
              D_i = sum_e dO[i,e] O[i,e],
              dV = P^T dO, dP = dO V^T, dS = P * (dP - D),
              dQ = tau dS K, dK = tau dS^T Q.
  RoPE        each pair turns by phi, so its gradient turns back by -phi:
              g[e0] = h[e0] cos phi + h[e1] sin phi,
              g[e1] = -h[e0] sin phi + h[e1] cos phi.
  modulate    u = xh (1 + scale[m]) + shift[m], xh = (x - mu) / sigma,
              sigma = sqrt(var + eps) (population variance over the row):
              gx = du (1 + scale[m]),
              dx = (gx - mean(gx) - xh mean(gx xh)) / sigma,
              dshift[r] = sum_{t: m(t)=r} du[t], dscale[r] = sum du[t] xh[t].
  residual    y = x + gate[m] o, z = LN(y) (1 + scale2[m]) + shift2[m]:
              dy_tot = dy + (LN backward of dz (1 + scale2[m])),
              dx = dy_tot, do = gate[m] dy_tot,
              dgate[r] = sum dy_tot o, dshift2[r] = sum dz,
              dscale2[r] = sum dz yh.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from . import reference as R


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def attention_bwd(q, k, v, dO, cu, scale: Optional[float] = None, chunk: int = 1024):
    """dQ, dK, dV [T][H][d] (float64) of block-diagonal softmax attention.

    Query rows are taken in chunks of at most `chunk` rows (memory only): the
    chunk's P rows are the full softmax rows, dV and dK are sums over all
    query rows and so add up over the chunks.
    """
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dQ = np.zeros((T, H, d), dtype=np.float64)
    dK = np.zeros((T, H, d), dtype=np.float64)
    dV = np.zeros((T, H, d), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in range(H):
            K = np.asarray(k[a:b, h, :], dtype=np.float64)
            V = np.asarray(v[a:b, h, :], dtype=np.float64)
            for r0 in range(a, b, chunk):
                r1 = min(b, r0 + chunk)
                Q = np.asarray(q[r0:r1, h, :], dtype=np.float64)
                G = np.asarray(dO[r0:r1, h, :], dtype=np.float64)
                S = scale * (Q @ K.T)
                E = np.exp(S - S.max(axis=1, keepdims=True))
                P = E / E.sum(axis=1, keepdims=True)
                O = P @ V
                Dr = (G * O).sum(axis=1, keepdims=True)
                dP = G @ V.T
                dS = P * (dP - Dr)
                dV[a:b, h, :] += P.T @ G
                dK[a:b, h, :] += scale * (dS.T @ Q)
                dQ[r0:r1, h, :] = scale * (dS @ K)
    return dQ, dK, dV


def attention_bwd_keys(q, k, v, dO, cu, keys: Sequence[int], heads: Sequence[int],
                       scale: Optional[float] = None, chunk: int = 1024):
    """dK and dV at the listed (key token, head) pairs only: the same
    formulas, with the softmax rows of every query of the key's sequence
    evaluated in chunks.  Returns dK_sel[n][d], dV_sel[n][d]."""
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu = np.asarray(cu)
    keys = np.asarray(keys)
    heads = np.asarray(heads)
    dK = np.zeros((len(keys), d), dtype=np.float64)
    dV = np.zeros((len(keys), d), dtype=np.float64)
    seqs = np.searchsorted(cu, keys, side="right") - 1
    for s in np.unique(seqs):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in np.unique(heads[seqs == s]):
            sel = np.nonzero((seqs == s) & (heads == h))[0]
            K = np.asarray(k[a:b, h, :], dtype=np.float64)
            V = np.asarray(v[a:b, h, :], dtype=np.float64)
            Ks = K[keys[sel] - a]
            Vs = V[keys[sel] - a]
            for r0 in range(a, b, chunk):
                r1 = min(b, r0 + chunk)
                Q = np.asarray(q[r0:r1, h, :], dtype=np.float64)
                G = np.asarray(dO[r0:r1, h, :], dtype=np.float64)
                S = scale * (Q @ K.T)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                l = E.sum(axis=1, keepdims=True)
                O = (E @ V) / l
                Dr = (G * O).sum(axis=1, keepdims=True)
                Ps = np.exp(scale * (Q @ Ks.T) - m) / l          # [rows][n_sel]
                dPs = G @ Vs.T
                dSs = Ps * (dPs - Dr)
                dV[sel] += Ps.T @ G
                dK[sel] += scale * (dSs.T @ Q)
    return dK, dV


def attention_bwd_rows(q, k, v, dO, cu, rows: Sequence[int], heads: Sequence[int],
                       scale: Optional[float] = None):
    """dQ at the listed (query token, head) pairs only.  Returns dQ_sel[n][d]."""
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu = np.asarray(cu)
    out = np.zeros((len(rows), d), dtype=np.float64)
    for n, (t, h) in enumerate(zip(rows, heads)):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        a, b = int(cu[s]), int(cu[s + 1])
        K = np.asarray(k[a:b, h, :], dtype=np.float64)
        V = np.asarray(v[a:b, h, :], dtype=np.float64)
        Qt = np.asarray(q[t, h, :], dtype=np.float64)
        G = np.asarray(dO[t, h, :], dtype=np.float64)
        S = scale * (K @ Qt)
        E = np.exp(S - S.max())
        P = E / E.sum()
        O = P @ V
        Dr = float(G @ O)
        dS = P * (V @ G - Dr)
        out[n] = scale * (dS @ K)
    return out


# ---------------------------------------------------------------------------
# modulate + RoPE
# ---------------------------------------------------------------------------

def rope_bwd(h: np.ndarray, pos: np.ndarray, dims: Tuple[int, int, int], base: float) -> np.ndarray:
    """Gradient through the RoPE rotation: every pair turned back by -phi."""
    h = np.asarray(h, dtype=np.float64)
    out = h.copy()
    o = 0
    for axis, Da in enumerate(dims):
        if Da == 0:
            continue
        theta = R.rope_thetas(Da, base)
        phi = pos[:, axis].astype(np.float64)[:, None] * theta[None, :]
        c = np.cos(phi)[:, None, :]
        s = np.sin(phi)[:, None, :]
        e0 = o + 2 * np.arange(Da // 2)
        e1 = e0 + 1
        g0 = h[:, :, e0]
        g1 = h[:, :, e1]
        out[:, :, e0] = g0 * c + g1 * s
        out[:, :, e1] = -g0 * s + g1 * c
        o += Da
    return out


def layer_norm_bwd(x2d: np.ndarray, gx: np.ndarray, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Gradient of LN (no affine) given the gradient gx with respect to its
    output; also returns the normalised rows xh."""
    x = np.asarray(x2d, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    sig = np.sqrt(var + eps)
    xh = (x - mu) / sig
    dx = (gx - gx.mean(axis=-1, keepdims=True) - xh * (gx * xh).mean(axis=-1, keepdims=True)) / sig
    return dx, xh


def modulate_rope_bwd(q, k, pos, dims, base, dq_out, dk_out, shift=None, scale=None,
                      mod_row=None, n_rows: int = 0, eps: float = 1e-6):
    """Gradients of modulate_rope for q and k.

    q, k: the forward's inputs [T][H][d]; dq_out, dk_out: gradients with
    respect to its outputs q', k'.  Returns (dq, dk, dshift, dscale); the adaLN
    rows are shared by q and k, so dshift/dscale [n_rows][C] sum over both.
    Without modulation only the RoPE gradient applies and dshift/dscale are
    None.
    """
    T, H, d = q.shape
    C = H * d
    du_q = rope_bwd(dq_out, pos, dims, base)
    du_k = rope_bwd(dk_out, pos, dims, base)
    if shift is None:
        return du_q, du_k, None, None
    dshift = np.zeros((n_rows, C), dtype=np.float64)
    dscale = np.zeros((n_rows, C), dtype=np.float64)
    outs = []
    for X, du in ((q, du_q), (k, du_k)):
        du2 = du.reshape(T, C)
        gx = du2 * (1.0 + scale[mod_row])
        dx, xh = layer_norm_bwd(np.asarray(X, dtype=np.float64).reshape(T, C), gx, eps)
        np.add.at(dshift, mod_row, du2)
        np.add.at(dscale, mod_row, du2 * xh)
        outs.append(dx.reshape(T, H, d))
    return outs[0], outs[1], dshift, dscale


# ---------------------------------------------------------------------------
# Gated residual (+ next adaLN)
# ---------------------------------------------------------------------------

def gated_residual_bwd(x, o, gate, mod_row, dy, dz=None, shift2=None, scale2=None,
                       n_rows: int = 0, eps: float = 1e-6):
    """Gradients of gated_residual.  Returns (dx, do, dgate, dshift2,
    dscale2) with do shaped [T][C] and the last two None without the fused
    next adaLN.  dy may be None (only z is used downstream)."""
    T = x.shape[0]
    x = np.asarray(x, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64).reshape(T, -1)
    C = o.shape[1]
    y = x + gate[mod_row] * o
    dyt = np.zeros((T, C), dtype=np.float64) if dy is None else np.asarray(dy, dtype=np.float64).copy()
    dshift2 = dscale2 = None
    if dz is not None:
        dz = np.asarray(dz, dtype=np.float64)
        gy = dz * (1.0 + scale2[mod_row])
        dln, yh = layer_norm_bwd(y, gy, eps)
        dyt = dyt + dln
        dshift2 = np.zeros((n_rows, C), dtype=np.float64)
        dscale2 = np.zeros((n_rows, C), dtype=np.float64)
        np.add.at(dshift2, mod_row, dz)
        np.add.at(dscale2, mod_row, dz * yh)
    dx = dyt
    do = gate[mod_row] * dyt
    dgate = np.zeros((n_rows, C), dtype=np.float64)
    np.add.at(dgate, mod_row, dyt * o)
    return dx, do, dgate, dshift2, dscale2


# ---------------------------------------------------------------------------
# The whole chain backwards
# ---------------------------------------------------------------------------

def backward(descs, q, k, v, dims, base, dy, dz=None, shift=None, scale=None, x=None,
             gate=None, shift2=None, scale2=None, eps: float = 1e-6, softmax_scale=None):
    """Forward (oracle.reference) then the gradients of every input, float64:
    dq, dk, dv [T][H][d]; dx [T][C]; dshift, dscale, dgate, dshift2, dscale2
    [n_rows][C] (None where the forward had no such input)."""
    fw = R.forward(descs, q, k, v, dims, base, shift, scale, x, gate, shift2, scale2, eps,
                   softmax_scale)
    cu, pos, mod_row = fw["cu"], fw["pos"], fw["mod_row"]
    T, H, d = q.shape
    n_rows = int(max(max(dd[4], dd[5]) for dd in descs)) + 1 if len(descs) else 0
    dx, do, dgate, dshift2, dscale2 = gated_residual_bwd(
        x, fw["O"], gate, mod_row, dy, dz, shift2, scale2, n_rows, eps)
    dqr, dkr, dv = attention_bwd(fw["q"], fw["k"], v, do.reshape(T, H, d), cu, softmax_scale)
    dq, dk, dshift, dscale = modulate_rope_bwd(q, k, pos, dims, base, dqr, dkr, shift, scale,
                                               mod_row, n_rows, eps)
    return dict(dq=dq, dk=dk, dv=dv, dx=dx, do=do, dqr=dqr, dkr=dkr, dshift=dshift,
                dscale=dscale, dgate=dgate, dshift2=dshift2, dscale2=dscale2, fw=fw)
