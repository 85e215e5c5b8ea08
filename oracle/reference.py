"""fp64 CPU oracle for the packed varlen RoPE joint-attention forward.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library: it imports numpy and nothing from the package.

Every function is the plain definition of one step, evaluated in float64 from
the exact input values, with no blocking, fusion or reordering beyond what
the definition states (the attention loop over query chunks only bounds
memory; each chunk is the same formula).  Sources, by page and section:

  [packing]   picx.dev summary of Mage-Flow, Methodology > Native-Resolution
              MMDiT: images are flattened to variable-length latent token
              sequences, packed with variable-length text under a fixed token
              budget, and attention is delimited per sample by cumulative
              offsets; the same section's conditioning item gives the frame
              coordinate that separates edit source from target latents.
  [rope2d]    gist.science "Resumo Tecnico: Mage-Flow", Metodologia > 2.
              NR-MMDiT, native-resolution packing item: variable-length
              attention kernels together with per-sample 2D rotary embeddings.
              The molayo1419.me post (key-features list, system-level speed
              item) states the same pairing.
  [joint]     picx.dev summary, Methodology > Native-Resolution MMDiT: the
              backbone uses joint self-attention over text and image tokens
              with modality-specific normalisation.
  [fusion]    picx.dev summary, Methodology > Training Infrastructure, and
              gist.science summary, Metodologia > 3. Otimizacao de Nivel de
              Sistema > Kernels Fundidos: adaptive normalisation, rotary
              embedding and gating (residual) chains are fused kernels.

Where the pages are silent the readings used are (all also listed in the
design notes): LayerNorm without affine, population variance, eps 1e-6,
statistics over the H*d channels of a q or k row; modulation
x_hat * (1 + scale) + shift; per-axis RoPE frequency ladders
theta_j = base^(-2j/D_axis) on adjacent pairs, counter-clockwise; axes laid out
frame, row, col in contiguous blocks of each head; 0-based raster positions,
text at (0, 0, 0); tokens of a sample ordered text, then frames in order, each
frame row-major; non-causal block-diagonal attention with scale 1/sqrt(d);
gate multiplies the attention branch before the residual add.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

Desc = Tuple[int, int, int, int, int, int]


# ---------------------------------------------------------------------------
# Step 1: integer pack tables                                    [packing]
# ---------------------------------------------------------------------------

def pack_tables(descs: Sequence[Desc]):
    """cu_seqlens[n+1], pos[T][3] = (frame, row, col), seq_id[T], mod_row[T].

    For sample s with text length t, F frames of an h x w grid:
      L_s = t + F*h*w, cu[s+1] = cu[s] + L_s;
      local token j < t is text at position (0, 0, 0);
      local token j >= t, i = j - t, is image at
      (i // (h*w), (i % (h*w)) // w, i % w).
    """
    cu = [0]
    pos: List[Tuple[int, int, int]] = []
    seq_id: List[int] = []
    mod_row: List[int] = []
    for s, (t, F, h, w, row_text, row_image) in enumerate(descs):
        for _ in range(t):
            pos.append((0, 0, 0))
            seq_id.append(s)
            mod_row.append(row_text)
        for f in range(F):
            for r in range(h):
                for c in range(w):
                    pos.append((f, r, c))
                    seq_id.append(s)
                    mod_row.append(row_image)
        cu.append(cu[-1] + t + F * h * w)
    T = cu[-1]
    return (np.asarray(cu, dtype=np.int32),
            np.asarray(pos, dtype=np.int32).reshape(T, 3),
            np.asarray(seq_id, dtype=np.int32),
            np.asarray(mod_row, dtype=np.int32))


# ---------------------------------------------------------------------------
# Step 2: adaLN modulation of a q or k row                          [fusion]
# ---------------------------------------------------------------------------

def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """Per-row (last axis) LayerNorm without affine, population variance."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(x2d: np.ndarray, shift: np.ndarray, scale: np.ndarray,
             mod_row: np.ndarray, eps: float) -> np.ndarray:
    """u[t] = LN(x[t]) * (1 + scale[m(t)]) + shift[m(t)], rows of C channels."""
    xh = layer_norm(x2d, eps)
    return xh * (1.0 + scale[mod_row]) + shift[mod_row]


# ---------------------------------------------------------------------------
# Step 3: per-sample multi-axis rotary embedding                    [rope2d]
# ---------------------------------------------------------------------------

def rope_thetas(D_axis: int, base: float) -> np.ndarray:
    """Frequency ladder of one axis: theta_j = base^(-2j/D_axis), j < D_axis/2."""
    j = np.arange(D_axis // 2, dtype=np.float64)
    return base ** (-2.0 * j / D_axis)


def rope(u: np.ndarray, pos: np.ndarray, dims: Tuple[int, int, int], base: float) -> np.ndarray:
    """Rotate adjacent pairs of every head.

    u: [T][H][d] float64; pos: [T][3] (frame, row, col); dims: (D_f, D_r, D_c)
    with D_f + D_r + D_c = d.  Axis a owns the contiguous dims
    [o_a, o_a + D_a) of each head.  Pair j of axis a (dims e0 = o_a + 2j,
    e1 = e0 + 1) turns by phi = pos_a * theta_j:
        u'[e0] = u[e0] cos phi - u[e1] sin phi
        u'[e1] = u[e0] sin phi + u[e1] cos phi
    """
    u = np.asarray(u, dtype=np.float64)
    assert sum(dims) == u.shape[-1]
    out = u.copy()
    o = 0
    for axis, Da in enumerate(dims):
        if Da == 0:
            continue
        theta = rope_thetas(Da, base)                              # [Da/2]
        phi = pos[:, axis].astype(np.float64)[:, None] * theta[None, :]  # [T][Da/2]
        c = np.cos(phi)[:, None, :]
        s = np.sin(phi)[:, None, :]
        e0 = o + 2 * np.arange(Da // 2)
        e1 = e0 + 1
        x0 = u[:, :, e0]
        x1 = u[:, :, e1]
        out[:, :, e0] = x0 * c - x1 * s
        out[:, :, e1] = x0 * s + x1 * c
        o += Da
    return out


def modulate_rope(q: np.ndarray, k: np.ndarray, pos: np.ndarray, dims, base: float,
                  shift=None, scale=None, mod_row=None, eps: float = 1e-6):
    """Step 2 (when shift/scale are given) then step 3, for q and for k.

    q, k: [T][H][d] float64.  Returns (q', k') float64.
    """
    T, H, d = q.shape
    outs = []
    for X in (q, k):
        u = np.asarray(X, dtype=np.float64)
        if shift is not None:
            u = modulate(u.reshape(T, H * d), shift, scale, mod_row, eps).reshape(T, H, d)
        outs.append(rope(u, pos, dims, base))
    return outs[0], outs[1]


# ---------------------------------------------------------------------------
# Step 4: block-diagonal joint softmax attention           [packing] [joint]
# ---------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu: np.ndarray,
              scale: Optional[float] = None, chunk: int = 1024):
    """O[T][H][d] and LSE[H][T] (natural log).

    For each packed sequence s (tokens cu[s] .. cu[s+1]-1) and head h:
      S = scale * Q K^T, P = exp(S - rowmax) / sum, O = P V,
      LSE = rowmax + log(sum exp(S - rowmax)).
    No mask inside a sequence; nothing crosses sequences.  Query rows are
    taken in chunks of at most `chunk` rows so that the score matrix of a
    long sequence is never held whole.
    """
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = np.zeros((T, H, d), dtype=np.float64)
    LSE = np.zeros((H, T), dtype=np.float64)
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
                S = scale * (Q @ K.T)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                l = E.sum(axis=1, keepdims=True)
                O[r0:r1, h, :] = (E @ V) / l
                LSE[h, r0:r1] = (m + np.log(l))[:, 0]
    return O, LSE


def attention_rows(q, k, v, cu, rows: Sequence[int], heads: Sequence[int],
                   scale: Optional[float] = None):
    """The same definition evaluated only at the listed (row, head) pairs.

    Returns O_sel[n][d] and LSE_sel[n] for n = len(rows) = len(heads).  Used to
    check full-size outputs at sampled positions.
    """
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu = np.asarray(cu)
    out = np.zeros((len(rows), d), dtype=np.float64)
    lse = np.zeros(len(rows), dtype=np.float64)
    for n, (t, h) in enumerate(zip(rows, heads)):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        a, b = int(cu[s]), int(cu[s + 1])
        K = np.asarray(k[a:b, h, :], dtype=np.float64)
        V = np.asarray(v[a:b, h, :], dtype=np.float64)
        S = scale * (K @ np.asarray(q[t, h, :], dtype=np.float64))
        m = S.max()
        E = np.exp(S - m)
        l = E.sum()
        out[n] = (E @ V) / l
        lse[n] = m + math.log(l)
    return out, lse


# ---------------------------------------------------------------------------
# Step 5: gated residual (+ optional next-sublayer adaLN)           [fusion]
# ---------------------------------------------------------------------------

def gated_residual(x: np.ndarray, o: np.ndarray, gate: np.ndarray, mod_row: np.ndarray,
                   shift2=None, scale2=None, eps: float = 1e-6):
    """y = x + gate[m(t)] * o;  z = LN(y) * (1 + scale2[m(t)]) + shift2[m(t)].

    x: [T][C]; o: [T][H][d] or [T][C] (channel c = h*d + e).  Returns (y, z)
    with z None unless shift2/scale2 are given.
    """
    T = x.shape[0]
    x = np.asarray(x, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64).reshape(T, -1)
    y = x + gate[mod_row] * o
    z = None
    if shift2 is not None:
        z = modulate(y, shift2, scale2, mod_row, eps)
    return y, z


# ---------------------------------------------------------------------------
# The whole chain
# ---------------------------------------------------------------------------

def forward(descs, q, k, v, dims, base, shift=None, scale=None, x=None, gate=None,
            shift2=None, scale2=None, eps: float = 1e-6, softmax_scale=None):
    """Tables -> modulate+RoPE -> attention -> gated residual, all float64."""
    cu, pos, seq_id, mod_row = pack_tables(descs)
    qr, kr = modulate_rope(q, k, pos, dims, base, shift, scale, mod_row, eps)
    O, LSE = attention(qr, kr, v, cu, softmax_scale)
    y = z = None
    if x is not None:
        y, z = gated_residual(x, O, gate, mod_row, shift2, scale2, eps)
    return dict(cu=cu, pos=pos, seq_id=seq_id, mod_row=mod_row, q=qr, k=kr, O=O, LSE=LSE,
                y=y, z=z)
