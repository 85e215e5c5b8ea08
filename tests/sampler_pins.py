"""Pins of the packed-CFG sampler oracle against facts fixed outside it.

Each pin takes a module ``s`` (the real ``oracle.sampler`` or a broken copy)
and raises AssertionError when ``s`` disagrees.  What pins what:
  * the pages' straight interpolation z_t = (1 - t) z + t eps with the
    velocity target z - eps: an Euler step with the exact target lands on
    z_{t_next} exactly, for one step or four (the Turbo schedule), which
    fixes the direction and sign of the step;
  * classifier-free guidance limits: w = 1 is the conditional branch, w = 0
    the unconditional one, and the combination is affine in w;
  * the row table against an independent walk over the packed order
    (text tokens, then frames, each frame row-major), including an edit
    sample whose second frame is the one that evolves;
  * the scatter writes both copies and nothing else.
"""
from __future__ import annotations

import numpy as np


def _pack_walk(descs):
    """(sample, frame, index-in-frame) of every packed position, by walking
    the pack in order: each sample's text tokens, then its frames."""
    out = []
    for s, (t, f, h, w, _, _) in enumerate(descs):
        out += [(s, -1, j) for j in range(t)]
        for fr in range(f):
            out += [(s, fr, j) for j in range(h * w)]
    return out


DESCS = [(5, 1, 3, 4, 0, 0), (2, 1, 3, 4, 1, 1), (7, 2, 2, 3, 2, 2), (1, 2, 2, 3, 3, 3),
         (4, 1, 2, 2, 4, 4), (3, 1, 2, 2, 5, 5)]
COND, UNCOND = [0, 2, 4], [1, 3, 5]


def pin_rows_walk(s):
    rows = s.cfg_pair_rows(DESCS, COND, UNCOND)
    walk = _pack_walk(DESCS)
    exp = []
    for c, u in zip(COND, UNCOND):
        last = DESCS[c][1] - 1
        pc = [i for i, (ss, fr, _) in enumerate(walk) if ss == c and fr == last]
        pu = [i for i, (ss, fr, _) in enumerate(walk) if ss == u and fr == DESCS[u][1] - 1]
        assert [walk[i][2] for i in pc] == list(range(len(pc)))
        exp += list(zip(pc, pu))
    assert rows.tolist() == [list(e) for e in exp]


def pin_straight_path(s):
    rng = np.random.default_rng(3)
    rows = s.cfg_pair_rows(DESCS, COND, UNCOND)
    N, Cl = rows.shape[0], 8
    z0 = rng.standard_normal((N, Cl))
    eps = rng.standard_normal((N, Cl))
    T = sum(d[0] + d[1] * d[2] * d[3] for d in DESCS)
    for w in (1.0, 4.5):
        v = rng.standard_normal((T, Cl))
        v[rows[:, 0]] = z0 - eps
        v[rows[:, 1]] = z0 - eps
        for t, tn in ((0.75, 0.0), (1.0, 0.5), (0.3, 0.1)):
            zt = (1 - t) * z0 + t * eps
            got = s.cfg_euler_step(v, rows, zt, w, t, tn)
            assert np.allclose(got, (1 - tn) * z0 + tn * eps, atol=1e-12)
        z = eps.copy()                       # four steps from noise (t = 1) to data
        sched = [1.0, 0.75, 0.5, 0.25, 0.0]
        for a, b in zip(sched[:-1], sched[1:]):
            z = s.cfg_euler_step(v, rows, z, w, a, b)
        assert np.allclose(z, z0, atol=1e-12)


def pin_guidance(s):
    rng = np.random.default_rng(4)
    rows = s.cfg_pair_rows(DESCS, COND, UNCOND)
    T = sum(d[0] + d[1] * d[2] * d[3] for d in DESCS)
    v = rng.standard_normal((T, 8))
    vc, vu = v[rows[:, 0]], v[rows[:, 1]]
    assert np.allclose(s.guided_velocity(v, rows, 1.0), vc)
    assert np.allclose(s.guided_velocity(v, rows, 0.0), vu)
    assert np.allclose(s.guided_velocity(v, rows, 3.0), 3.0 * vc - 2.0 * vu)
    z = rng.standard_normal((rows.shape[0], 8))
    assert np.allclose(s.cfg_euler_step(v, rows, z, 2.0, 0.6, 0.6), z)    # zero step


def pin_scatter(s):
    rng = np.random.default_rng(5)
    rows = s.cfg_pair_rows(DESCS, COND, UNCOND)
    T = sum(d[0] + d[1] * d[2] * d[3] for d in DESCS)
    x = rng.standard_normal((T, 8))
    zn = rng.standard_normal((rows.shape[0], 8))
    got = s.scatter_rows(x, rows, zn)
    assert np.array_equal(got[rows[:, 0]], zn) and np.array_equal(got[rows[:, 1]], zn)
    other = np.setdiff1d(np.arange(T), rows.ravel())
    assert np.array_equal(got[other], x[other])


ALL_PINS = [pin_rows_walk, pin_straight_path, pin_guidance, pin_scatter]
