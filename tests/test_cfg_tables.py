"""Host CFG pair tables (mf_cfg_pair_rows) against the sampler oracle: exact
integers on the CFG and edit packs and on random small packs; bad prompts
are rejected (CPU only)."""
import numpy as np
import pytest

import sampler_pins as P
from oracle import sampler
from packed_attention_amd import native, workloads as W

SHAPE, NULL = -2, -1


def test_pins_pack():
    assert np.array_equal(native.cfg_pair_rows(P.DESCS, P.COND, P.UNCOND),
                          sampler.cfg_pair_rows(P.DESCS, P.COND, P.UNCOND))


def test_cfg_workload_pack():
    w = W.cfg_pack()
    cond, uncond = W.cfg_prompts(w)
    rows = native.cfg_pair_rows(w.descs, cond, uncond)
    assert rows.shape == (4 * 64 * 64, 2)
    assert np.array_equal(rows, sampler.cfg_pair_rows(w.descs, cond, uncond))


def test_edit_pack_evolves_target_frame():
    descs = [(30, 2, 5, 6, 0, 0), (16, 2, 5, 6, 1, 1)]
    rows = native.cfg_pair_rows(descs, [0], [1])
    assert np.array_equal(rows, sampler.cfg_pair_rows(descs, [0], [1]))
    assert rows[0, 0] == 30 + 30 and rows[0, 1] == 30 + 60 + 16 + 30


@pytest.mark.parametrize("seed", range(6))
def test_random_packs(seed):
    rng = np.random.default_rng(seed)
    descs = []
    P_ = int(rng.integers(1, 4))
    for p in range(P_):
        h, wd, f = int(rng.integers(1, 6)), int(rng.integers(1, 6)), int(rng.integers(1, 3))
        descs.append((int(rng.integers(0, 9)), f, h, wd, 2 * p, 2 * p))
        descs.append((int(rng.integers(0, 9)), int(rng.integers(1, 3)), h, wd, 2 * p + 1, 2 * p + 1))
    perm = rng.permutation(len(descs))
    descs = [descs[i] for i in perm]
    inv = np.argsort(perm)
    cond, uncond = [int(inv[2 * p]) for p in range(P_)], [int(inv[2 * p + 1]) for p in range(P_)]
    assert np.array_equal(native.cfg_pair_rows(descs, cond, uncond), sampler.cfg_pair_rows(descs, cond, uncond))


def test_bad_prompts_rejected():
    import ctypes
    lib = native.lib()
    descs = [(3, 1, 2, 2, 0, 0), (1, 1, 2, 3, 1, 1), (2, 0, 0, 0, 2, 2)]
    arr = native._desc_array(descs)
    n = ctypes.c_int64(0)
    def call(c, u):
        ca = np.array(c, dtype=np.int32)
        ua = np.array(u, dtype=np.int32)
        return lib.mf_cfg_pair_count(arr, 3, ca.ctypes.data, ua.ctypes.data, len(c), ctypes.byref(n))
    assert call([0], [1]) == SHAPE        # grids differ
    assert call([0], [0]) == SHAPE        # same sample
    assert call([0], [3]) == SHAPE        # out of range
    assert call([0], [2]) == SHAPE        # no frame
    assert lib.mf_cfg_pair_count(arr, 3, None, None, 1, ctypes.byref(n)) == NULL
    assert lib.mf_cfg_pair_count(arr, 3, None, None, 0, ctypes.byref(n)) == 0 and n.value == 0
