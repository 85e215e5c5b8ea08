"""Host C++ pack tables (mf_pack_tables) against the oracle: exact integers."""
import numpy as np
import pytest

from oracle import reference as R
from packed_attention_amd import native, workloads as W


def _same(descs):
    a = native.pack_tables(descs)
    b = R.pack_tables(descs)
    for x, y, name in zip(a, b, ("cu_seqlens", "pos", "seq_id", "mod_row")):
        assert x.dtype == np.int32 and x.shape == y.shape, name
        np.testing.assert_array_equal(x, y, err_msg=name)
    assert native.pack_count(descs) == int(b[0][-1])


@pytest.mark.parametrize("make", [W.tiny, W.single_1024, W.cfg_pack, W.edit_pack],
                         ids=lambda f: f.__name__)
def test_named_workloads(make):
    rng = np.random.default_rng(0)
    w = make()
    _same(w.descs)


@pytest.mark.parametrize("seed", range(2000, 2008))
def test_native_budget_packs(seed):
    descs = W.descs_native_budget(np.random.default_rng(seed))
    T = sum(W.sample_len(d) for d in descs)
    assert 0 < T <= 16384
    for t, f, h, w, _, _ in descs:                       # 512..2048 per side at 16x
        assert 32 <= h <= 128 and 32 <= w <= 128 and 32 <= t <= 512 and f == 1
        assert max(h, w) <= 4 * min(h, w)
    _same(descs)


def test_random_descriptor_lists():
    rng = np.random.default_rng(123)
    for _ in range(1000):
        _same(W.random_descs(rng))


def test_empty_and_degenerate():
    _same([])
    _same([(0, 1, 0, 0, 0, 0)])
    _same([(0, 0, 5, 5, 0, 0), (3, 1, 1, 1, 1, 2)])
    _same([(1, 1, 0, 0, 0, 0)])


def test_count_errors():
    with pytest.raises(native.MFError) as e:
        native.pack_count([(-1, 1, 2, 2, 0, 0)])
    assert e.value.code == -2
    with pytest.raises(native.MFError) as e:
        native.pack_count([(0, 1, 65536, 65536, 0, 0)])   # T > INT32_MAX
    assert e.value.code == -2
