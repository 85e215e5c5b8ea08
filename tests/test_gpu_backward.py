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
RAGGED_DESCS = [(t, f, h, ww, s, s) for s, (t, f, h, ww) in enumerate(RAGGED)]


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


def test_bwd_orders_with_caller_stream():
    """The dQ kernel runs on a second stream forked from and joined to the
    caller's: on a non-default caller stream, inputs written just before the
    call and copies of the outputs taken just after it, with no host
    synchronisation between, match a run on the default stream bitwise."""
    import torch
    descs = [(30, 1, 16, 16, 0, 0), (2, 1, 9, 7, 1, 1)]
    w = W.custom(descs, H=4, D=128, seed=21, name="bwd_stream_order")
    G.say(w.name, "side caller stream")
    b, dO, dq, dk, dv = forward_and_grads(w)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    copies = []
    with torch.cuda.stream(s):
        for _ in range(3):
            dO2 = dO * 2.0 * 0.5
            outs = [torch.full_like(b.q, float("nan")) for _ in range(3)]
            native.varlen_attn_bwd(b.qr, b.kr, b.v, b.o, dO2, b.lse, *outs, b.cu, b.max_seqlen)
            copies.append([o.clone() for o in outs])
    torch.cuda.synchronize()
    for rep in copies:
        for x, y in zip((dq, dk, dv), rep):
            assert torch.equal(x, y)


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


# ---------------------------------------------------------------------------
# Elementwise backward kernels and the whole backward chain
# ---------------------------------------------------------------------------

ROWSUM_REL_RMS = 1e-4    # fp32 sums of fp32 per-token terms from bf16 data
CHAIN_REL_RMS = 2e-2     # three bf16-rounded stages, each near 2^-9 relative


def check_rows(got, ref, name):
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert np.all(np.isfinite(got)) and rel <= ROWSUM_REL_RMS, f"{name}: relative RMS {rel:.3e}"


def _f32(t):
    return t.detach().cpu().numpy().astype(np.float64)


def _use_rows(b, rows):
    """Replace the pack's adaLN row table (device and host copies)."""
    import torch
    if rows is not None:
        b.mod_row = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.int32)).to("cuda")
        b.mod_row_host = np.ascontiguousarray(rows, dtype=np.int32)


def modrope_bwd_check(w, rows=None):
    import torch
    G.say(w.name, "modulate_rope_bwd", "T", w.T, "H", w.H, "D", w.D)
    b = runner.to_device(w)
    _use_rows(b, rows)
    g = W.upstream_grads(w)
    dq_out, dk_out = runner.bf16_tensor(g["dq"]), runner.bf16_tensor(g["dk"])
    dq, dk = torch.empty_like(b.q), torch.empty_like(b.k)
    n_rows = len(w.descs)
    C = w.H * w.D
    dsh = torch.empty((n_rows, C), dtype=torch.float32, device="cuda") if w.modulate else None
    dsc = torch.empty((n_rows, C), dtype=torch.float32, device="cuda") if w.modulate else None
    native.modulate_rope_bwd(b.q, b.k, dq_out, dk_out, dq, dk, b.pos, w.rope_dims, w.rope_base,
                             b.scale, b.mod_row if w.modulate else None, dsh, dsc, w.eps)
    torch.cuda.synchronize()
    a = G.wl_f64(w)
    ref = B.modulate_rope_bwd(a["q"], a["k"], b.pos_host, w.rope_dims, w.rope_base,
                              G.f64(dq_out), G.f64(dk_out), a["shift"], a["scale"], b.mod_row_host,
                              n_rows, w.eps)
    check_grad(G.f64(dq), ref[0], w.name + ".dq")
    check_grad(G.f64(dk), ref[1], w.name + ".dk")
    if w.modulate:
        check_rows(_f32(dsh), ref[2], w.name + ".dshift")
        check_rows(_f32(dsc), ref[3], w.name + ".dscale")


def gres_bwd_check(w, fused=True, with_dy=True, rows=None):
    import torch
    G.say(w.name, "gated_residual_bwd", "fused", fused, "dy", with_dy)
    b = runner.to_device(w)
    _use_rows(b, rows)
    runner.run_chain(b)
    g = W.upstream_grads(w)
    T, C = w.T, w.H * w.D
    n_rows = len(w.descs)
    dy = runner.bf16_tensor(g["dy"]) if with_dy else None
    dz = runner.bf16_tensor(g["dz"]) if fused else None
    dx = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    do = torch.empty_like(dx)
    rows = lambda: torch.empty((n_rows, C), dtype=torch.float32, device="cuda")  # noqa: E731
    dgate, dsh2, dsc2 = rows(), (rows() if fused else None), (rows() if fused else None)
    o2 = b.o.view(T, C)
    native.gated_residual_bwd(b.x, o2, b.gate, b.mod_row, dy, dx, do, dgate,
                              b.scale2 if fused else None, dz, dsh2, dsc2, w.eps)
    torch.cuda.synchronize()
    a = G.wl_f64(w)
    ref = B.gated_residual_bwd(a["x"], G.f64(o2), a["gate"], b.mod_row_host,
                               G.f64(dy) if with_dy else None, G.f64(dz) if fused else None,
                               a["shift2"], a["scale2"], n_rows, w.eps)
    check_grad(G.f64(dx), ref[0], w.name + ".dx")
    check_grad(G.f64(do), ref[1], w.name + ".do")
    check_rows(_f32(dgate), ref[2], w.name + ".dgate")
    if fused:
        check_rows(_f32(dsh2), ref[3], w.name + ".dshift2")
        check_rows(_f32(dsc2), ref[4], w.name + ".dscale2")


def test_modulate_rope_bwd_tiny():
    modrope_bwd_check(W.tiny())          # RoPE only
    modrope_bwd_check(W.tiny_mod())


@pytest.mark.parametrize("D", [64, 128])
def test_modulate_rope_bwd_ragged(D):
    descs = [(t, f, h, ww, s, s) for s, (t, f, h, ww) in enumerate(RAGGED)]
    dims = (0, D // 2, D // 2) if D == 64 else (16, 56, 56)
    modrope_bwd_check(W.custom(descs, H=3, D=D, rope_dims=dims, modulate=True, residual=True,
                               seed=79, name=f"ragged_erbwd_d{D}"))


def test_gated_residual_bwd_variants():
    w = W.tiny_mod()
    gres_bwd_check(w, fused=True, with_dy=True)
    gres_bwd_check(w, fused=True, with_dy=False)
    gres_bwd_check(w, fused=False, with_dy=True)


def test_elementwise_bwd_single_1024():
    """Full size: every token (these kernels are cheap for the oracle)."""
    w = W.single_1024()
    modrope_bwd_check(w)
    gres_bwd_check(w)


def test_backward_chain_end_to_end():
    """GPU forward, then gated residual -> attention -> modulate+RoPE
    backward, against the fp64 oracle chain from the same seeded inputs."""
    import torch
    w = W.tiny_mod()
    G.say(w.name, "backward chain end to end")
    b = runner.to_device(w)
    runner.run_chain(b)
    g = W.upstream_grads(w)
    T, H, D = w.T, w.H, w.D
    C = H * D
    n_rows = len(w.descs)
    dy, dz = runner.bf16_tensor(g["dy"]), runner.bf16_tensor(g["dz"])
    rows = lambda: torch.empty((n_rows, C), dtype=torch.float32, device="cuda")  # noqa: E731
    dx = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    do = torch.empty_like(dx)
    dgate, dsh2, dsc2, dsh, dsc = rows(), rows(), rows(), rows(), rows()
    native.gated_residual_bwd(b.x, b.o.view(T, C), b.gate, b.mod_row, dy, dx, do, dgate, b.scale2,
                              dz, dsh2, dsc2, w.eps)
    dqr, dkr, dv = (torch.empty_like(b.q) for _ in range(3))
    native.varlen_attn_bwd(b.qr, b.kr, b.v, b.o, do.view(T, H, D), b.lse, dqr, dkr, dv, b.cu,
                           b.max_seqlen)
    dq, dk = torch.empty_like(b.q), torch.empty_like(b.k)
    native.modulate_rope_bwd(b.q, b.k, dqr, dkr, dq, dk, b.pos, w.rope_dims, w.rope_base, b.scale,
                             b.mod_row, dsh, dsc, w.eps)
    torch.cuda.synchronize()
    a = G.wl_f64(w)
    ref = B.backward(w.descs, a["q"], a["k"], a["v"], w.rope_dims, w.rope_base, G.f64(dy), G.f64(dz),
                     a["shift"], a["scale"], a["x"], a["gate"], a["shift2"], a["scale2"], w.eps)
    for name, got in (("dq", G.f64(dq)), ("dk", G.f64(dk)), ("dv", G.f64(dv)), ("dx", G.f64(dx)),
                      ("dshift", _f32(dsh)), ("dscale", _f32(dsc)), ("dgate", _f32(dgate)),
                      ("dshift2", _f32(dsh2)), ("dscale2", _f32(dsc2))):
        r = ref[name]
        rel = float(np.linalg.norm(got - r) / max(np.linalg.norm(r), 1e-30))
        assert rel <= CHAIN_REL_RMS, f"chain {name}: relative RMS {rel:.3e}"


@pytest.mark.parametrize("H", [32, 64])
def test_elementwise_bwd_wide_rows(H):
    """Rows of 4096 and 8192 channels: the modulate+RoPE backward's form for
    rows of more than 3072 channels, and the gated residual backward's
    per-token kernel at its largest workgroups."""
    descs = [(13, 1, 9, 10, 0, 0), (7, 1, 5, 6, 1, 1)]
    w = W.custom(descs, H=H, D=128, rope_dims=(0, 64, 64), modulate=True, residual=True, seed=80 + H,
                 name=f"wide_bwd_h{H}")
    modrope_bwd_check(w)
    gres_bwd_check(w)


def test_elementwise_bwd_rows_outside_table():
    """An adaLN row outside [0, n_rows) reads zeros and adds nothing: the
    per-token gradients equal, bit for bit, those of the same call with an
    explicit all-zero row for those tokens, and the table's rows sum the
    same tokens as in that call (within fp32 ordering)."""
    import torch
    w = W.custom(RAGGED_DESCS[:6], H=3, D=64, rope_dims=(0, 32, 32), modulate=True, residual=True, seed=83,
                 name="bwd_rows_outside")
    b = runner.to_device(w)
    runner.run_chain(b)
    g = W.upstream_grads(w)
    T, C = w.T, w.H * w.D
    n = len(w.descs)
    bad = b.mod_row.clone()
    bad[3], bad[T // 2], bad[T - 1] = n, -1, 1 << 20
    sub = torch.where((bad < 0) | (bad >= n), torch.full_like(bad, n), bad)
    zero = torch.zeros((1, C), dtype=torch.bfloat16, device="cuda")
    same = lambda a, c, name: torch.equal(a.view(torch.int16), c.view(torch.int16)) or pytest.fail(name)  # noqa

    dq_out, dk_out = runner.bf16_tensor(g["dq"]), runner.bf16_tensor(g["dk"])
    outs = []
    for rows, scale in ((bad, b.scale), (sub, torch.cat([b.scale, zero]))):
        dq, dk = torch.empty_like(b.q), torch.empty_like(b.k)
        dsh = torch.empty((scale.shape[0], C), dtype=torch.float32, device="cuda")
        dsc = torch.empty_like(dsh)
        native.modulate_rope_bwd(b.q, b.k, dq_out, dk_out, dq, dk, b.pos, w.rope_dims, w.rope_base, scale,
                                 rows, dsh, dsc, w.eps)
        outs.append((dq, dk, dsh, dsc))
    torch.cuda.synchronize()
    same(outs[0][0], outs[1][0], "dq")
    same(outs[0][1], outs[1][1], "dk")
    for i, name in ((2, "dshift"), (3, "dscale")):
        np.testing.assert_allclose(_f32(outs[0][i]), _f32(outs[1][i][:n]), rtol=1e-5, atol=1e-5, err_msg=name)

    dy, dz = runner.bf16_tensor(g["dy"]), runner.bf16_tensor(g["dz"])
    o2 = b.o.view(T, C)
    outs = []
    for rows, gate, scale2 in ((bad, b.gate, b.scale2), (sub, torch.cat([b.gate, zero]), torch.cat([b.scale2, zero]))):
        dx, do = torch.empty((T, C), dtype=torch.bfloat16, device="cuda"), torch.empty((T, C), dtype=torch.bfloat16,
                                                                                        device="cuda")
        r = lambda: torch.empty((gate.shape[0], C), dtype=torch.float32, device="cuda")  # noqa: E731
        dg, ds2, dc2 = r(), r(), r()
        native.gated_residual_bwd(b.x, o2, gate, rows, dy, dx, do, dg, scale2, dz, ds2, dc2, w.eps)
        outs.append((dx, do, dg, ds2, dc2))
    torch.cuda.synchronize()
    same(outs[0][0], outs[1][0], "dx")
    same(outs[0][1], outs[1][1], "do")
    for i, name in ((2, "dgate"), (3, "dshift2"), (4, "dscale2")):
        np.testing.assert_allclose(_f32(outs[0][i]), _f32(outs[1][i][:n]), rtol=1e-5, atol=1e-5, err_msg=name)


def _interleaved_rows(T, n, seed):
    """An adaLN row table whose row changes every one or two tokens and comes
    back: the row sums' runs hold several segments, and a row's tokens are
    not contiguous."""
    rng = np.random.default_rng(seed)
    rows = []
    while len(rows) < T:
        rows += [int(rng.integers(0, n))] * int(rng.integers(1, 3))
    return np.array(rows[:T], dtype=np.int32)


@pytest.mark.parametrize("H,D,descs", [
    (2, 64, [(40, 1, 24, 24, 0, 1), (9, 1, 7, 5, 2, 3)]),                    # runs of 8, one reduction level
    (2, 64, [(64, 1, 64, 64, s, s) for s in range(5)]),                       # 20 800 tokens: three levels
    (32, 128, [(31, 1, 16, 20, 0, 1), (5, 1, 9, 9, 2, 3)]),                   # 4096 channels: runs of 4
])
def test_elementwise_bwd_interleaved_rows(H, D, descs):
    """Row sums when the adaLN row changes every one or two tokens and rows
    recur: against the oracle, for both elementwise backward calls."""
    w = W.custom(descs, H=H, D=D, rope_dims=(0, D // 2, D // 2), modulate=True, residual=True,
                 seed=90 + H + len(descs), name=f"interleaved_h{H}_n{len(descs)}")
    rows = _interleaved_rows(w.T, len(w.descs), seed=7 + H)
    modrope_bwd_check(w, rows)
    gres_bwd_check(w, rows=rows)
    gres_bwd_check(w, fused=False, rows=rows)


@pytest.mark.parametrize("name", ["single_1024", "wide", "interleaved"])
def test_elementwise_bwd_row_sums_bitwise(name):
    """The row sums (dshift, dscale; dgate, dshift2, dscale2) are bitwise
    equal from call to call: every row sum is added in one fixed order."""
    import torch
    if name == "single_1024":
        w = W.NAMED["single_1024"]()
        rows = None
    elif name == "wide":
        w = W.custom([(60, 1, 24, 26, 0, 1), (11, 1, 13, 9, 2, 2)], H=32, D=128, rope_dims=(0, 64, 64),
                     modulate=True, residual=True, seed=95, name="bitwise_wide")
        rows = None
    else:
        w = W.custom([(64, 1, 40, 40, s, s) for s in range(3)], H=24, D=128, rope_dims=(0, 64, 64),
                     modulate=True, residual=True, seed=96, name="bitwise_interleaved")
        rows = _interleaved_rows(w.T, len(w.descs), seed=11)
    G.say(w.name, "row sums bitwise", "T", w.T, "C", w.H * w.D)
    b = runner.to_device(w)
    _use_rows(b, rows)
    runner.run_chain(b)
    g = W.upstream_grads(w)
    T, C, n = w.T, w.H * w.D, len(w.descs)
    dq_out, dk_out = runner.bf16_tensor(g["dq"]), runner.bf16_tensor(g["dk"])
    dy, dz = runner.bf16_tensor(g["dy"]), runner.bf16_tensor(g["dz"])
    o2 = b.o.view(T, C)
    f32 = lambda: torch.empty((n, C), dtype=torch.float32, device="cuda")  # noqa: E731
    bf = lambda: torch.empty((T, C), dtype=torch.bfloat16, device="cuda")  # noqa: E731
    runs = []
    for _ in range(3):
        dq, dk = torch.empty_like(b.q), torch.empty_like(b.k)
        dsh, dsc = f32(), f32()
        native.modulate_rope_bwd(b.q, b.k, dq_out, dk_out, dq, dk, b.pos, w.rope_dims, w.rope_base, b.scale,
                                 b.mod_row, dsh, dsc, w.eps)
        dx, do, dg, ds2, dc2 = bf(), bf(), f32(), f32(), f32()
        native.gated_residual_bwd(b.x, o2, b.gate, b.mod_row, dy, dx, do, dg, b.scale2, dz, ds2, dc2, w.eps)
        dx1, do1, dg1 = bf(), bf(), f32()
        native.gated_residual_bwd(b.x, o2, b.gate, b.mod_row, dy, dx1, do1, dg1, None, None, None, None, w.eps)
        runs.append((dsh, dsc, dg, ds2, dc2, dg1))
    torch.cuda.synchronize()
    names = ("dshift", "dscale", "dgate", "dshift2", "dscale2", "dgate (unfused)")
    for r in runs[1:]:
        for a, c, nm in zip(runs[0], r, names):
            assert torch.equal(a.view(torch.int32), c.view(torch.int32)), f"{w.name}: {nm} differs between calls"
