"""Block projections (mf_block_qkv, mf_block_out) vs the fp64 block oracle.

The oracle takes the same bf16 inputs (residual stream, seeded random-init
weights, modulation rows, tables) widened exactly to fp64.  Small and ragged
cases are compared element by element; the 1024^2 pack at full size on
sampled token rows (every output feature of each sampled row).

Bar (derived in the design notes): the kernel rounds the modulated rows to
bf16 before the products (relative 2^-9 per element, so about
2^-9/sqrt(3) relative RMS on a sum of many independent terms) and rounds the
output to bf16 (2^-9); relative RMS <= 5e-3 and max-abs <= 1e-2 * max|ref|
per output tensor.
"""
import numpy as np
import pytest

import gpu_common as G
from oracle import block as BO
from oracle import reference as R
from packed_attention_amd import native, runner, workloads as W

pytestmark = pytest.mark.gpu

REL_RMS = 5e-3
MAX_REL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    native.lib()


def check(got, ref, name):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    scale = max(float(np.abs(ref).max()), 1e-30)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    err = float(np.abs(got - ref).max())
    assert rel <= REL_RMS, f"{name}: relative RMS {rel:.3e}"
    assert err <= MAX_REL * scale, f"{name}: max-abs {err:.3e} vs max|ref| {scale:.3e}"


def run_qkv(w, modulate=True, rows=None):
    """GPU qkv for workload w; returns (qkv [T][3C] fp64, oracle (q', k', v) at `rows` or all)."""
    import torch
    G.say(w.name, "block_qkv", "T", w.T, "H", w.H, "D", w.D, "modulate", modulate)
    b = runner.to_device(w)
    bi = W.block_inputs(w)
    T, C = w.T, w.H * w.D
    x = runner.bf16_tensor(bi["x"])
    wq = runner.bf16_tensor(bi["w_qkv"])
    qkv = torch.full((T, 3 * C), float("nan"), dtype=torch.bfloat16, device="cuda")
    sh, sc = (b.shift, b.scale) if modulate else (None, None)
    native.block_qkv(x, wq, qkv, b.pos, w.H, w.rope_dims, w.rope_base, sh, sc,
                     b.mod_row if modulate else None, w.eps)
    torch.cuda.synchronize()
    got = G.f64(qkv)
    xs = W.bf16_bits_to_f64(bi["x"])
    ws = W.bf16_bits_to_f64(bi["w_qkv"])
    shf = W.bf16_bits_to_f64(w.shift) if modulate else None
    scf = W.bf16_bits_to_f64(w.scale) if modulate else None
    if rows is None:
        ref = BO.qkv_projection(xs, ws, b.pos_host, w.rope_dims, w.rope_base, w.H, shf, scf,
                                b.mod_row_host if modulate else None, w.eps)
    else:
        ref = BO.qkv_projection_rows(xs, ws, b.pos_host, w.rope_dims, w.rope_base, w.H, rows, shf, scf,
                                     b.mod_row_host if modulate else None, w.eps)
        got = got[rows]
    return got, ref


def check_qkv(w, modulate=True, rows=None):
    got, ref = run_qkv(w, modulate, rows)
    n, C = got.shape[0], w.H * w.D
    for i, name in enumerate(("q'", "k'", "v")):
        check(got[:, i * C:(i + 1) * C], ref[i].reshape(n, C), f"{w.name}.{name}")


def run_out(w, rows=None):
    import torch
    G.say(w.name, "block_out", "T", w.T, "C", w.H * w.D)
    b = runner.to_device(w)
    bi = W.block_inputs(w)
    T, C = w.T, w.H * w.D
    rng = np.random.default_rng(w.seed + 7)
    o_bits = W.f32_to_bf16_bits(rng.standard_normal((T, C)).astype(np.float32))
    o = runner.bf16_tensor(o_bits)
    x = runner.bf16_tensor(bi["x"])
    wo = runner.bf16_tensor(bi["w_o"])
    gate_bits = w.gate if w.gate is not None else W.f32_to_bf16_bits(
        (rng.standard_normal((len(w.descs), C)) * 0.1).astype(np.float32))
    gate = runner.bf16_tensor(gate_bits)
    y = torch.full((T, C), float("nan"), dtype=torch.bfloat16, device="cuda")
    native.block_out(o, wo, x, gate, b.mod_row, y)
    torch.cuda.synchronize()
    got = G.f64(y)
    of, xf, wf, gf = (W.bf16_bits_to_f64(a) for a in (o_bits, bi["x"], bi["w_o"], gate_bits))
    if rows is None:
        ref = BO.out_projection(of, wf, xf, gf, b.mod_row_host)
    else:
        ref = BO.out_projection(of[rows], wf, xf[rows], gf, b.mod_row_host[rows])
        got = got[rows]
    check(got, ref, f"{w.name}.y")


def test_block_qkv_tiny():
    check_qkv(W.tiny_mod())


def test_block_qkv_no_modulation():
    check_qkv(W.tiny(), modulate=False)


# T not a multiple of the 256-token tile, 3C not a multiple of the 256-feature tile
@pytest.mark.parametrize("D", [64, 128])
def test_block_qkv_ragged(D):
    descs = [(37, 1, 9, 11, 0, 0), (5, 1, 13, 14, 1, 1), (0, 1, 3, 5, 2, 2)]
    dims = (0, D // 2, D // 2) if D == 64 else (16, 56, 56)
    w = W.custom(descs, H=3, D=D, rope_dims=dims, modulate=True, residual=True, seed=31,
                 name=f"block_ragged_d{D}")
    assert w.T % 256 != 0 and (3 * w.H * D) % 256 != 0
    check_qkv(w)


# Small grids on a 256-CU device: the last round's tiles are cut into token
# slices that run side by side, each with the whole K (C = 512: 18 tiles, T =
# 600, four slices of 64 tokens, the last tile's two upper slices past the
# last token; C = 1024: 24 tiles, four slices; C = 3072: 108 tiles, T = 700,
# two slices of 128 tokens).  The 1024^2 pack's 612 tiles (a last round of
# 100, two slices) are in test_block_qkv_single_1024_sampled.
@pytest.mark.parametrize("H,descs", [(4, [(88, 1, 16, 32, 0, 0)]), (8, [(27, 1, 13, 21, 0, 0), (0, 1, 1, 1, 1, 1)]),
                                     (24, [(60, 1, 20, 32, 0, 0)])],
                         ids=["C512", "C1024", "C3072"])
def test_block_qkv_split_tail(H, descs):
    w = W.custom(descs, H=H, D=128, rope_dims=(0, 64, 64), modulate=True, residual=True, seed=41,
                 name=f"block_split_c{H * 128}")
    check_qkv(w)


def test_block_qkv_edit_3d_rope():
    """Frame positions > 0 (edit source and target) with the 3D split."""
    descs = [(12, 2, 8, 9, 0, 0), (4, 1, 6, 7, 1, 1)]
    w = W.custom(descs, H=2, D=128, rope_dims=(16, 56, 56), modulate=True, residual=True, seed=33,
                 name="block_edit3d")
    check_qkv(w)


def test_block_qkv_single_1024_sampled():
    """Full size (256 + 64x64 tokens, C = 3072, W_qkv 9216 x 3072): sampled rows."""
    w = W.single_1024()
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(w.T, 40, replace=False),
                                     [0, 255, 256, 4351]]))
    check_qkv(w, rows=rows)


def test_block_out_tiny_and_ragged():
    run_out(W.tiny_mod())
    descs = [(37, 1, 9, 11, 0, 0), (5, 1, 13, 14, 1, 1)]
    run_out(W.custom(descs, H=3, D=128, rope_dims=(0, 64, 64), modulate=True, residual=True, seed=35,
                     name="block_out_ragged"))


def test_block_out_single_1024_sampled():
    w = W.single_1024()
    rows = np.unique(np.concatenate([np.random.default_rng(6).choice(w.T, 40, replace=False), [0, 4351]]))
    run_out(w, rows=rows)


def test_block_identity_weights_match_elementwise_kernels():
    """W_qkv = [I; I; I] makes q', k' the modulate+RoPE kernel's outputs on
    the same rows and v the modulated rows; W_o = I makes y the gated
    residual kernel's output (the kernels round differently, so the bar is
    the bf16 one, not bitwise)."""
    import torch
    w = W.tiny_mod()
    b = runner.to_device(w)
    T, C = w.T, w.H * w.D
    x = b.x
    eye = torch.eye(C, dtype=torch.bfloat16, device="cuda")
    qkv = torch.empty((T, 3 * C), dtype=torch.bfloat16, device="cuda")
    native.block_qkv(x, torch.cat([eye] * 3, 0).contiguous(), qkv, b.pos, w.H, w.rope_dims, w.rope_base,
                     b.shift, b.scale, b.mod_row, w.eps)
    xr = x.view(T, w.H, w.D)
    qr, kr = torch.empty_like(xr), torch.empty_like(xr)
    native.modulate_rope(xr, xr, qr, kr, b.pos, w.rope_dims, w.rope_base, b.shift, b.scale, b.mod_row, w.eps)
    torch.cuda.synchronize()
    ref_u = R.modulate(G.f64(x), G.f64(b.shift), G.f64(b.scale), b.mod_row_host, w.eps)
    check(G.f64(qkv[:, :C]), G.f64(qr).reshape(T, C), "identity.q'")
    check(G.f64(qkv[:, C:2 * C]), G.f64(kr).reshape(T, C), "identity.k'")
    check(G.f64(qkv[:, 2 * C:]), ref_u, "identity.v")
