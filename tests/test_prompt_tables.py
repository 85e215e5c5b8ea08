"""Host prompt tables (mf_prompt_tables) against the text-encoder oracle's
positions: exact integers; bad lengths are rejected (CPU only)."""
import numpy as np
import pytest

from oracle import text_encoder as TE
from packed_attention_amd import native, workloads as W


@pytest.mark.parametrize("lens", [[5, 1, 9, 3], [1], [0, 4, 0, 2], [], W.text_pack().lens])
def test_prompt_tables_match_oracle(lens):
    cu, pos = native.prompt_tables(lens)
    assert cu.tolist() == np.concatenate([[0], np.cumsum(lens)]).astype(int).tolist()
    assert np.array_equal(pos, TE.positions(cu))


def test_bad_lengths_rejected():
    with pytest.raises(native.MFError):
        native.prompt_tables([3, -1])
    with pytest.raises(native.MFError):
        native.prompt_tables([2 ** 30, 2 ** 30, 2 ** 30])
