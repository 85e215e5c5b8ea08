"""The allocation-free attention forward (mf_varlen_attn_fwd_noalloc) against
the regular entry point (mf_varlen_attn_fwd) through the C ABI.

Both run the same kernels with the same schedule and persistent grid, so the
allocation-free call must reproduce the regular call's O and LSE bit for bit.
Two calls in a row share the library's scratch array, the second with a
smaller input (fewer sequences, fewer heads, D = 64).  A call whose workspace
would exceed the 80 MiB array is rejected before anything is enqueued."""
import numpy as np
import pytest

import gpu_common as G
from packed_attention_amd import native

pytestmark = pytest.mark.gpu

MF_ERR_UNSUPPORTED = -4


def _inputs(lens, H, D, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    T = int(sum(lens))
    mk = lambda: torch.randn((T, H, D), generator=g, device="cuda").to(torch.bfloat16)  # noqa: E731
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    return mk(), mk(), mk(), cu


def _call(fn, q, k, v, cu, lens, **kw):
    import torch
    T, H, D = q.shape
    o = torch.full_like(q, 7.0)
    lse = torch.full((H, T), 7.0, dtype=torch.float32, device="cuda")
    fn(q, k, v, o, cu, max(lens), lse=lse, **kw)
    torch.cuda.synchronize()
    return o, lse


def test_noalloc_matches_workspace_entry_point():
    import torch
    native.lib()
    for lens, H, D, seed in (([4352], 24, 128, 11), ([300, 41, 77, 1], 4, 64, 12)):
        G.say("noalloc vs workspace entry point", lens, H, D)
        q, k, v, cu = _inputs(lens, H, D, seed)
        o_ref, lse_ref = _call(native.varlen_attn_fwd, q, k, v, cu, lens)
        o, lse = _call(native.varlen_attn_fwd_noalloc, q, k, v, cu, lens)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), (lens, H, D)
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), (lens, H, D)


def test_noalloc_rejects_oversized_workspace():
    """A persistent grid of 400 workgroups needs 2 x 400 partial slots of
    133 KB at D = 128, beyond the 80 MiB array: MF_ERR_UNSUPPORTED, and the
    output is left untouched."""
    import torch
    q, k, v, cu = _inputs([600], 2, 128, 13)
    native.set_attn_fwd_grid(400)
    try:
        assert native.attn_workspace_bytes(1, 600, 2, 128) > 80 * (1 << 20)
        o = torch.full_like(q, 7.0)
        with pytest.raises(native.MFError) as exc:
            native.varlen_attn_fwd_noalloc(q, k, v, o, cu, 600)
        assert exc.value.code == MF_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert torch.all(o == 7.0)
    finally:
        native.set_attn_fwd_grid(0)
