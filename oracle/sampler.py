"""fp64 oracle of the packed-CFG sampler step after the last block.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library.

Sources:
  [flow]   gist.science "Resumo Tecnico: Mage-Flow", Metodologia and the
           picx.dev summary, Introduction and Theoretical Foundation, item 1:
           the backbone predicts a velocity v_theta(z_t, t, tau) for the
           straight interpolation z_t = (1 - t) z + t eps between data z
           (t = 0) and noise eps (t = 1), trained against the target z - eps.
  [cfg]    picx.dev summary, Methodology > Native-Resolution MMDiT: the
           conditional and unconditional branches of classifier-free guidance
           are packed into one forward pass; the Turbo variants sample in 4
           steps (picx.dev, Results; gist.science, Principais Resultados).

Readings (plainest, listed in the design notes):
  * guidance: v = v_u + w (v_c - v_u) per latent channel (the usual
    classifier-free combination; w = 1 is the conditional branch alone);
  * the step is Euler along t from t to t_next < t: dz_t/dt = eps - z, whose
    model estimate is -v, so z_{t_next} = z_t + (t - t_next) v;
  * a prompt p owns one conditional and one unconditional packed sample with
    the same latent grid; the latents that evolve are the last frame's
    (generation: the only frame; editing: the target frame, the source frame
    being conditioning), h*w tokens in raster order after the sample's text
    tokens and earlier frames;
  * the next forward's input rows of both copies receive the new latents.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from . import reference as R


def cfg_pair_rows(descs: Sequence[Tuple[int, int, int, int, int, int]], cond: Sequence[int],
                  uncond: Sequence[int]) -> np.ndarray:
    """rows[N][2]: packed row of the conditional and of the unconditional copy
    of every evolving latent token, prompts in order, raster order inside."""
    cu, _, _, _ = R.pack_tables(descs)
    out = []
    for c, u in zip(cond, uncond):
        tc, fc, hc, wc = descs[c][:4]
        tu, fu, hu, wu = descs[u][:4]
        if (hc, wc) != (hu, wu):
            raise ValueError(f"prompt ({c}, {u}): latent grids differ")
        n = hc * wc
        bc = int(cu[c]) + tc + (fc - 1) * n
        bu = int(cu[u]) + tu + (fu - 1) * n
        for j in range(n):
            out.append((bc + j, bu + j))
    return np.array(out, dtype=np.int64).reshape(-1, 2)


def guided_velocity(v: np.ndarray, rows: np.ndarray, w: float) -> np.ndarray:
    """v_u + w (v_c - v_u) for every evolving token: [N][Cl] float64."""
    v = np.asarray(v, dtype=np.float64)
    vc = v[rows[:, 0]]
    vu = v[rows[:, 1]]
    return vu + w * (vc - vu)


def cfg_euler_step(v: np.ndarray, rows: np.ndarray, z: np.ndarray, w: float, t: float,
                   t_next: float) -> np.ndarray:
    """z_next = z + (t - t_next) * (v_u + w (v_c - v_u)), [N][Cl] float64."""
    return np.asarray(z, dtype=np.float64) + (t - t_next) * guided_velocity(v, rows, w)


def scatter_rows(x: np.ndarray, rows: np.ndarray, z_next: np.ndarray) -> np.ndarray:
    """The next forward's input rows: both copies of every evolving token
    receive z_next; other rows are left as they are."""
    x = np.array(x, dtype=np.float64, copy=True)
    x[rows[:, 0]] = z_next
    x[rows[:, 1]] = z_next
    return x
