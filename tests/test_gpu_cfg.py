"""Packed-CFG guidance + Euler step (mf_cfg_euler_step) vs the sampler oracle.

The oracle takes the same bf16 velocities and fp32 state widened exactly to
fp64.  The kernel computes in fp32 from those exact values, so the new state
matches to fp32 rounding (a few ulps): max-abs <= 1e-6 * (1 + max|ref|); the
bf16 input rows of the next forward are the new state rounded to bf16,
within one bf16 ulp of the oracle's state (a rounding decision can flip
where fp32 and fp64 straddle a midpoint); rows outside the table are not
touched (bitwise).
"""
import numpy as np
import pytest

import gpu_common as G
from oracle import sampler
from packed_attention_amd import native, runner, workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    native.lib()


def run_step(w, cond, uncond, guidance, t, t_next, Cl=W.LATENT_CHANNELS, in_place=False):
    import torch
    G.say(w.name, "cfg_euler", "T", w.T, "prompts", len(cond), "Cl", Cl, "w", guidance, "t", t, t_next)
    rows_h = native.cfg_pair_rows(w.descs, cond, uncond)
    N = rows_h.shape[0]
    si = W.sampler_inputs(w, N, Cl)
    v = runner.bf16_tensor(si["v"])
    rows = torch.from_numpy(rows_h).cuda()
    z = torch.from_numpy(si["z"]).cuda()
    z_out = z if in_place else torch.empty_like(z)
    sentinel = np.full((w.T, Cl), 0x7F7F, dtype=np.uint16)          # a finite bf16 pattern
    x = runner.bf16_tensor(sentinel)
    native.cfg_euler_step(v, rows, z, z_out, guidance, t, t_next, x_next=x)
    torch.cuda.synchronize()
    ref = sampler.cfg_euler_step(W.bf16_bits_to_f64(si["v"]), rows_h.astype(np.int64), si["z"].astype(np.float64),
                                 guidance, t, t_next)
    got = z_out.cpu().numpy().astype(np.float64)
    err = float(np.abs(got - ref).max())
    assert err <= 1e-6 * (1.0 + float(np.abs(ref).max())), err
    xg = G.f64(x)
    ulp = G.bf16_ulp(ref)
    for col in (0, 1):
        assert np.all(np.abs(xg[rows_h[:, col]] - ref) <= ulp), col
    other = np.setdiff1d(np.arange(w.T), rows_h.ravel())
    assert np.array_equal(x.view(torch.int16).cpu().numpy()[other], sentinel.view(np.int16)[other])


def test_cfg_pack_step():
    w = W.cfg_pack()
    cond, uncond = W.cfg_prompts(w)
    run_step(w, cond, uncond, 4.5, 0.75, 0.5)


def test_edit_pack_step_in_place():
    descs = [(30, 2, 9, 7, 0, 0), (16, 2, 9, 7, 1, 1), (5, 1, 3, 3, 2, 2), (2, 1, 3, 3, 3, 3)]
    w = W.custom(descs, H=2, D=64, seed=41, name="cfg_edit_small")
    run_step(w, [0, 2], [1, 3], 2.0, 0.25, 0.0, Cl=64, in_place=True)


def test_turbo_schedule_lands_on_data():
    """Four steps with the exact straight-path velocity z - eps (both copies)
    take the noise to the data up to fp32 rounding."""
    import torch
    descs = [(12, 1, 8, 8, 0, 0), (4, 1, 8, 8, 1, 1)]
    w = W.custom(descs, H=2, D=64, seed=43, name="cfg_turbo")
    rows_h = native.cfg_pair_rows(w.descs, [0], [1])
    rng = np.random.default_rng(44)
    z0 = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((64, 16)).astype(np.float32)))
    eps = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((64, 16)).astype(np.float32)))
    vt = np.zeros((w.T, 16), dtype=np.float32)
    vt[rows_h[:, 0]] = z0 - eps
    vt[rows_h[:, 1]] = z0 - eps
    vbits = W.f32_to_bf16_bits(vt)
    v = runner.bf16_tensor(vbits)
    rows = torch.from_numpy(rows_h).cuda()
    z = torch.from_numpy(eps.copy()).cuda()
    sched = [1.0, 0.75, 0.5, 0.25, 0.0]
    for a, b in zip(sched[:-1], sched[1:]):
        native.cfg_euler_step(v, rows, z, z, 3.0, a, b)
    torch.cuda.synchronize()
    vexact = W.bf16_bits_to_f64(vbits)[rows_h[:, 0]]
    # the bf16 velocity is z0 - eps rounded: the landing point is eps + 1.0 * v
    assert np.abs(z.cpu().numpy() - (eps + vexact)).max() <= 1e-5
