"""fp64 oracle of the text-encoder variant of the hot path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library.

Sources: the pages fuse the normalisation and rotary-embedding chains inside
the frozen Qwen3-VL text encoder's blocks as well as in the backbone
(picx.dev summary of Mage-Flow, Methodology > Training Infrastructure;
gist.science "Resumo Tecnico: Mage-Flow", Metodologia > 3 > Kernels
Fundidos), whose prompts condition the backbone (picx.dev, Methodology >
Native-Resolution MMDiT, conditioning item); prompts of different lengths are
packed like the backbone's samples (same section, packing item).

Readings (plainest; listed in the design notes):
  * the encoder is a decoder-style language model: attention is causal inside
    each packed prompt (token i attends to tokens 0..i of its prompt) and
    nothing crosses prompts;
  * grouped heads: H_q query heads share H_kv key/value heads, query head h
    using key/value head h // (H_q / H_kv);
  * per-head norm: RMS normalisation over the d dims of each head of q and of
    k, x / sqrt(mean(x^2) + eps) * weight, one weight vector of d entries
    for q and one for k (shared by the heads);
  * RoPE: one axis, the token's index inside its prompt, on adjacent pairs
    with theta_j = base^(-2j/d) (the backbone's pairing and direction with all
    dims on one axis).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def rms_norm_heads(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """x [T][H][d] -> x / sqrt(mean over d of x^2 + eps) * weight[d]."""
    x = np.asarray(x, dtype=np.float64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


def positions(cu: np.ndarray) -> np.ndarray:
    """Index of every packed token inside its prompt."""
    T = int(cu[-1])
    pos = np.zeros(T, dtype=np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        pos[a:b] = np.arange(b - a)
    return pos


def rope_1d(u: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate adjacent pairs (2j, 2j+1) of every head by pos * base^(-2j/d)."""
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    theta = base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    phi = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    x0, x1 = u[..., 0::2], u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def qk_norm_rope(q: np.ndarray, k: np.ndarray, wq: np.ndarray, wk: np.ndarray, pos: np.ndarray,
                 base: float, eps: float = 1e-6):
    """(q', k') = (RoPE(RMS(q) * wq), RoPE(RMS(k) * wk)), [T][H][d] float64 each."""
    return (rope_1d(rms_norm_heads(q, wq, eps), pos, base),
            rope_1d(rms_norm_heads(k, wk, eps), pos, base))


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu: np.ndarray,
                     scale: Optional[float] = None, chunk: int = 1024):
    """O [T][H_q][d] and LSE [H_q][T] (natural log) of causal attention inside
    each prompt, query head h reading key/value head h // (H_q / H_kv)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((T, Hq, d))
    lse = np.zeros((Hq, T))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in range(Hq):
            K = k[a:b, h // g, :]
            V = v[a:b, h // g, :]
            for r0 in range(a, b, chunk):
                r1 = min(b, r0 + chunk)
                S = scale * (q[r0:r1, h, :] @ K.T)                     # [rows][L]
                qi = np.arange(r0, r1)[:, None] - a
                kj = np.arange(b - a)[None, :]
                S = np.where(kj <= qi, S, -np.inf)
                m = S.max(axis=1, keepdims=True)
                P = np.exp(S - m)
                l = P.sum(axis=1, keepdims=True)
                out[r0:r1, h, :] = (P / l) @ V
                lse[h, r0:r1] = (m + np.log(l))[:, 0]
    return out, lse


def causal_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu: np.ndarray, rows,
                          scale: Optional[float] = None):
    """O [len(rows)][H_q][d] and LSE [H_q][len(rows)] of causal attention at the
    given packed rows only, one query row at a time: row i of a prompt
    starting at a attends to keys a..i (for spot checks of long prompts)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, d = q.shape
    g = Hq // k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    first = np.asarray(cu, dtype=np.int64)[np.searchsorted(cu, rows, side="right") - 1]
    out = np.zeros((len(rows), Hq, d))
    lse = np.zeros((Hq, len(rows)))
    for n, (i, a) in enumerate(zip(rows, first)):
        for h in range(Hq):
            s = scale * (k[a:i + 1, h // g, :] @ q[i, h, :])
            m = s.max()
            p = np.exp(s - m)
            out[n, h] = (p @ v[a:i + 1, h // g, :]) / p.sum()
            lse[h, n] = m + np.log(p.sum())
    return out, lse

