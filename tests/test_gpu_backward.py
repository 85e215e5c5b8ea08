"""Attention backward (mf_varlen_attn_bwd) vs the fp64 backward oracle.

Per kernel: the oracle is fed the HIP path's own bf16 q', k' (from the GPU
forward chain), v and the seeded dO; the kernel also receives the GPU
forward's bf16 O and fp32 LSE.  Small packs are compared element by
element; the 1024^2 sample at full size on sampled query rows (dQ) and key
rows (dK, dV), each against its whole sequence.

Bar (derived in the design notes): the outputs are sums of L products whose
bf16 operands P and dS carry a relative rounding of at most 2^-9, so the
relative RMS error stays near 2^-9; the bar is relative RMS <= 1e-2 and
max-abs <= 2e-2 * max|ref| per output tensor.
"""
import numpy as np
import pytest

import gpu_common as G
from oracle import backward as B
from packed_attention_amd import native, runner, workloads as W

pytestmark = pytest.mark.gpu

GRAD_REL_RMS = 1e-2
GRAD_MAX_REL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    native.lib()


def check_grad(got, ref, name):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert rel <= GRAD_REL_RMS, f"{name}: relative RMS {rel:.3e}"
    assert err.max() <= GRAD_MAX_REL * scale, f"{name}: max-abs {err.max():.3e} vs max|ref| {scale:.3e}"
    return rel


def forward_and_grads(w, dO_scale=1.0):
    """GPU forward chain, then the backward on seeded dO; returns (b, dO, dq, dk, dv)."""
    import torch
    b = runner.to_device(w)
    runner.run_chain(b)
    g = W.upstream_grads(w)
    dO = runner.bf16_tensor(g["dO"]) * dO_scale
    dq, dk, dv = (torch.empty_like(b.q) for _ in range(3))
    native.varlen_attn_bwd(b.qr, b.kr, b.v, b.o, dO, b.lse, dq, dk, dv, b.cu, b.max_seqlen)
    torch.cuda.synchronize()
    return b, dO, dq, dk, dv


def run_and_check(w, dO_scale=1.0):
    G.say(w.name, "bwd", "T", w.T, "H", w.H, "D", w.D, "descs", w.descs)
    b, dO, dq, dk, dv = forward_and_grads(w, dO_scale)
    ref = B.attention_bwd(G.f64(b.qr), G.f64(b.kr), G.f64(b.v), G.f64(dO), b.cu_host)
    for name, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        check_grad(G.f64(got), r, f"{w.name}.{name}")
    return b, dq, dk, dv


def test_tiny_pack_bwd():
    run_and_check(W.tiny())


def test_tiny_modulated_bwd():
    run_and_check(W.tiny_mod())


# lengths around the 64-query, 128-key and 256-query tile edges, an empty
# sequence and a single token
RAGGED = [(1, 1, 0, 0), (1, 1, 1, 1), (3, 1, 6, 10), (0, 1, 8, 8), (1, 1, 8, 8), (0, 1, 0, 0),
          (7, 1, 8, 15), (0, 1, 8, 16), (1, 1, 8, 16), (12, 1, 16, 18), (5, 2, 4, 6),
          (1, 1, 15, 17)]


@pytest.mark.parametrize("D", [64, 128])
def test_ragged_pack_bwd(D):
    descs = [(t, f, h, ww, s, s) for s, (t, f, h, ww) in enumerate(RAGGED)]
    assert [W.sample_len(d) for d in descs] == [1, 2, 63, 64, 65, 0, 127, 128, 129, 300, 53, 256]
    dims = (0, D // 2, D // 2) if D == 64 else (16, 56, 56)
    w = W.custom(descs, H=3, D=D, rope_dims=dims, modulate=True, residual=True, seed=78,
                 name=f"ragged_bwd_d{D}")
    run_and_check(w)


@pytest.mark.parametrize("sigma", [4.0])
def test_peaky_softmax_bwd(sigma):
    descs = [(40, 1, 12, 12, 0, 0), (9, 1, 7, 5, 1, 1)]
    w = W.custom(descs, H=2, D=128, rope_dims=(0, 64, 64), seed=int(sigma) + 100, qk_sigma=sigma,
                 name=f"peaky_bwd_x{sigma:g}")
    run_and_check(w)


def test_bwd_packed_equals_alone_and_determinism():
    """Sequences are independent: the gradients of a pack equal those of each
    sample run alone, bitwise (the tiles start at each sequence's first row);
    two runs are bitwise identical."""
    import torch
    descs = [(20, 1, 9, 11, 0, 0), (3, 1, 17, 16, 1, 1), (0, 1, 5, 5, 2, 2)]
    w = W.custom(descs, H=2, D=128, seed=9, name="bwd_alone")
    G.say(w.name, "packed vs alone")
    b, dO, dq, dk, dv = forward_and_grads(w)
    dq2, dk2, dv2 = (torch.empty_like(b.q) for _ in range(3))
    native.varlen_attn_bwd(b.qr, b.kr, b.v, b.o, dO, b.lse, dq2, dk2, dv2, b.cu, b.max_seqlen)
    torch.cuda.synchronize()
    for x, y in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(x, y)
    cu = b.cu_host
    for s in range(len(descs)):
        a, e = int(cu[s]), int(cu[s + 1])
        sl = slice(a, e)
        cu1 = torch.tensor([0, e - a], dtype=torch.int32, device="cuda")
        lse1 = b.lse[:, sl].contiguous()
        outs = [torch.empty_like(b.q[sl]) for _ in range(3)]
        native.varlen_attn_bwd(b.qr[sl], b.kr[sl], b.v[sl], b.o[sl], dO[sl], lse1, *outs, cu1, e - a)
        torch.cuda.synchronize()
        for x, y in zip((dq, dk, dv), outs):
            assert torch.equal(x[sl], y), s


def test_bwd_single_1024_sampled():
    """Full size (256 + 64x64 tokens, H=24, d=128), sampled rows and keys."""
    import torch
    w = W.single_1024()
    G.say(w.name, "bwd full size")
    b, dO, dq, dk, dv = forward_and_grads(w)
    rng = np.random.default_rng(w.seed + 7)
    T = w.T
    rows = np.unique(np.concatenate([rng.choice(T, 48, replace=False), [0, T - 1]]))
    heads = rng.integers(0, w.H, size=len(rows))
    qr, kr, v, g = (runner.bf16_to_f64(t).astype(np.float32) for t in (b.qr, b.kr, b.v, dO))
    ref_q = B.attention_bwd_rows(qr, kr, v, g, b.cu_host, rows, heads)
    keys = np.unique(np.concatenate([rng.choice(T, 48, replace=False), [0, T - 1]]))
    kheads = rng.integers(0, w.H, size=len(keys))
    ref_k, ref_v = B.attention_bwd_keys(qr, kr, v, g, b.cu_host, keys, kheads)
    ti = lambda a: torch.as_tensor(a)  # noqa: E731
    check_grad(G.f64(dq.cpu()[ti(rows), ti(heads)]), ref_q, "single_1024.dQ")
    check_grad(G.f64(dk.cpu()[ti(keys), ti(kheads)]), ref_k, "single_1024.dK")
    check_grad(G.f64(dv.cpu()[ti(keys), ti(kheads)]), ref_v, "single_1024.dV")
