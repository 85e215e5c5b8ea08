"""HIP path vs the fp64 oracle on small packs (full oracle, every element).

Each case runs the three kernels through the C-ABI binding and checks
  * the integer tables the library built: exactly equal to the oracle's;
  * per kernel: the oracle fed that kernel's own bf16 inputs;
  * end to end: the oracle chain in fp64 from the same seeded bf16 inputs.
Bar: max-abs <= 2e-2 and mean-abs <= 2e-3 on every bf16 output, plus the
internal checks (one bf16 ulp for the elementwise kernels, relative RMS and
LSE for attention).
"""
import numpy as np
import pytest

import gpu_common as G
from oracle import reference as R
from packed_attention_amd import native, runner, workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    native.lib()


def run_and_check(w, e2e=True, qk_sigma=1.0):
    import torch
    G.say(w.name, "T", w.T, "H", w.H, "D", w.D, "descs", w.descs)
    b = runner.to_device(w)
    # tables: exact
    cu, pos, sid, mr = R.pack_tables(w.descs)
    np.testing.assert_array_equal(b.cu_host, cu)
    np.testing.assert_array_equal(b.pos_host, pos)
    np.testing.assert_array_equal(b.mod_row_host, mr)
    runner.run_chain(b)
    torch.cuda.synchronize()
    a = G.wl_f64(w)
    T, H, D = w.T, w.H, w.D
    # per kernel: modulate + rope
    qr_ref, kr_ref = R.modulate_rope(a["q"], a["k"], pos, w.rope_dims, w.rope_base, a["shift"],
                                     a["scale"], mr, w.eps)
    qr, kr = G.f64(b.qr), G.f64(b.kr)
    # the absolute bar is stated for unit-scale rows; stress rows of scale
    # sigma carry sigma times the bf16 rounding, so it scales with sigma there
    G.check_bar(qr, qr_ref, w.name + ".q'", G.MAX_ABS * qk_sigma, G.MEAN_ABS * qk_sigma)
    G.check_bar(kr, kr_ref, w.name + ".k'", G.MAX_ABS * qk_sigma, G.MEAN_ABS * qk_sigma)
    G.check_rounded(qr, qr_ref, w.name + ".q'")
    G.check_rounded(kr, kr_ref, w.name + ".k'")
    # per kernel: attention on the kernel's own bf16 inputs
    O_ref, L_ref = R.attention(qr, kr, a["v"], cu)
    O = G.f64(b.o)
    lse = b.lse.cpu().numpy().astype(np.float64)
    G.check_attention(O, O_ref, w.name, lse, L_ref)
    # per kernel: gated residual on the kernel's own O
    if w.x is not None:
        y_ref, z_ref = R.gated_residual(a["x"], O, a["gate"], mr, a["shift2"], a["scale2"], w.eps)
        y, z = G.f64(b.y), G.f64(b.z)
        G.check_bar(y, y_ref, w.name + ".y")
        G.check_rounded(y, y_ref, w.name + ".y")
        G.check_bar(z, z_ref, w.name + ".z")
        G.check_rounded(z, z_ref, w.name + ".z", slack=1e-5)
    # end to end, fp64 throughout
    if e2e:
        r = R.forward(w.descs, a["q"], a["k"], a["v"], w.rope_dims, w.rope_base, a["shift"],
                      a["scale"], a["x"], a["gate"], a["shift2"], a["scale2"], w.eps)
        G.check_attention(O, r["O"], w.name + ".e2e", lse, r["LSE"], G.LSE_ABS_E2E * qk_sigma ** 2)
        if w.x is not None:
            G.check_bar(G.f64(b.y), r["y"], w.name + ".e2e.y")
            G.check_bar(G.f64(b.z), r["z"], w.name + ".e2e.z")
    return b


def test_tiny_pack():
    run_and_check(W.tiny())


def test_tiny_pack_modulated():
    run_and_check(W.tiny_mod())


# Sequence lengths around the 64-key and 128-query tile edges, an empty
# sequence and a single token; text + latent grid mixes.
RAGGED = [(1, 1, 0, 0), (1, 1, 1, 1), (3, 1, 6, 10), (0, 1, 8, 8), (1, 1, 8, 8), (0, 1, 0, 0),
          (7, 1, 8, 15), (0, 1, 8, 16), (1, 1, 8, 16), (12, 1, 16, 18), (5, 2, 4, 6)]


@pytest.mark.parametrize("D", [64, 128])
def test_ragged_pack(D):
    descs = [(t, f, h, ww, s, s) for s, (t, f, h, ww) in enumerate(RAGGED)]
    assert [W.sample_len(d) for d in descs] == [1, 2, 63, 64, 65, 0, 127, 128, 129, 300, 53]
    dims = (0, D // 2, D // 2) if D == 64 else (16, 56, 56)
    w = W.custom(descs, H=3, D=D, rope_dims=dims, modulate=True, residual=True, seed=77,
                 name=f"ragged_d{D}")
    run_and_check(w)


@pytest.mark.parametrize("sigma", [4.0, 8.0])
def test_peaky_softmax(sigma):
    descs = [(40, 1, 12, 12, 0, 0), (9, 1, 7, 5, 1, 1)]
    w = W.custom(descs, H=2, D=128, rope_dims=(0, 64, 64), modulate=False, residual=False,
                 seed=int(sigma), qk_sigma=sigma, name=f"peaky_x{sigma:g}")
    # per kernel only: with scores of standard deviation ~sigma^2 the softmax is
    # near one-hot, and the bf16 rounding of q'/k' (part of the kernel chain,
    # absent from an fp64-throughout chain) can swap near-tied maxima
    run_and_check(w, e2e=False, qk_sigma=sigma)


def test_leak_probe():
    """V = +100 in one sequence and 0 elsewhere: no other sequence sees it."""
    import torch
    descs = [(10, 1, 9, 9, 0, 0), (3, 1, 5, 7, 1, 1), (0, 1, 11, 13, 2, 2)]
    w = W.custom(descs, H=2, D=128, seed=5, name="leak")
    b = runner.to_device(w)
    cu = b.cu_host
    for s in range(len(descs)):
        G.say("leak probe, hot sequence", s)
        b.v.zero_()
        b.v[cu[s]:cu[s + 1]] = 100.0
        runner.run_modulate_rope(b)
        runner.run_attention(b)
        torch.cuda.synchronize()
        O = G.f64(b.o)
        for s2 in range(len(descs)):
            blk = O[cu[s2]:cu[s2 + 1]]
            if s2 == s:
                # P is rounded to bf16 before PV while the normaliser sums the
                # fp32 probabilities: within a few bf16 ulps of 100.
                assert np.abs(blk - 100.0).max() <= 1.0
            else:
                np.testing.assert_array_equal(blk, 0.0)


def test_packed_equals_alone_and_determinism():
    """Run-to-run bitwise determinism; each sample alone matches its slice of
    the pack."""
    import torch
    descs = [(17, 1, 10, 14, 0, 0), (2, 1, 3, 3, 1, 1), (0, 1, 16, 20, 2, 2)]
    w = W.custom(descs, H=2, D=128, seed=9, name="alone")
    b = runner.to_device(w)
    G.say("packed vs alone")
    runner.run_modulate_rope(b)
    runner.run_attention(b)
    torch.cuda.synchronize()
    O1 = b.o.clone()
    L1 = b.lse.clone()
    runner.run_attention(b)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), b.o.view(torch.int16)), "not deterministic"
    assert torch.equal(L1, b.lse)
    for s in range(len(descs)):
        a0, a1 = int(b.cu_host[s]), int(b.cu_host[s + 1])
        L = a1 - a0
        o = torch.full((L, w.H, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.H, L), float("nan"), dtype=torch.float32, device="cuda")
        cu1 = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        native.varlen_attn_fwd(b.qr[a0:a1], b.kr[a0:a1], b.v[a0:a1], o, cu1, L, lse=lse)
        torch.cuda.synchronize()
        # Alone, the sequence's tiles are split over the CUs differently than
        # inside the pack (stream-K ranges): the fp32 accumulation order
        # differs, and each piece of a cut tile takes its reference max from
        # its own first key step, so its bf16 probabilities round differently.
        # On these inputs O stays within one bf16 ulp and LSE (merged from
        # fp32 maxima and sums) within fp32 rounding.
        got, ref = G.f64(o), G.f64(O1[a0:a1])
        assert np.all(np.abs(got - ref) <= G.bf16_ulp(ref) + 1e-6), s
        np.testing.assert_allclose(lse.cpu().numpy(), L1[:, a0:a1].cpu().numpy(), rtol=0, atol=1e-5)


def test_guard_bands_and_strides():
    """Outputs written exactly where they belong: canary bands around every
    output stay intact; q/k/v as slices of one fused [T][3][H][D] buffer;
    q'/k' written in place."""
    import torch
    descs = [(13, 1, 9, 10, 0, 0), (4, 1, 6, 6, 1, 1)]
    w = W.custom(descs, H=2, D=128, modulate=True, residual=True, seed=21, name="guards")
    b = runner.to_device(w)
    T, H, D = w.T, w.H, w.D
    g = 64
    CANARY = 0x4B1D   # a finite bf16 bit pattern

    def banded(shape):
        buf = torch.full((shape[0] + 2 * g,) + tuple(shape[1:]), CANARY, dtype=torch.int16,
                         device="cuda").view(torch.bfloat16)
        return buf, buf[g:g + shape[0]]

    qkv = torch.empty((T, 3, H, D), dtype=torch.bfloat16, device="cuda")
    qkv[:, 0] = b.q
    qkv[:, 1] = b.k
    qkv[:, 2] = b.v
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    G.say("in-place modulate_rope on fused qkv")
    native.modulate_rope(q, k, q, k, b.pos, w.rope_dims, w.rope_base, b.shift, b.scale, b.mod_row,
                         w.eps)
    runner.run_modulate_rope(b)          # reference: separate buffers
    torch.cuda.synchronize()
    assert torch.equal(q.contiguous().view(torch.int16), b.qr.view(torch.int16))
    assert torch.equal(k.contiguous().view(torch.int16), b.kr.view(torch.int16))
    ob, o = banded((T, H, D))
    lse_buf = torch.full((H * T + 2 * g,), 12345.0, dtype=torch.float32, device="cuda")
    lse = lse_buf[g:g + H * T].view(H, T)
    G.say("attention with fused-qkv strides and banded outputs")
    native.varlen_attn_fwd(q, k, v, o, b.cu, b.max_seqlen, lse=lse)
    runner.run_attention(b)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), b.o.view(torch.int16))
    assert torch.equal(lse, b.lse)
    assert torch.all(ob[:g].view(torch.int16) == CANARY) and torch.all(ob[-g:].view(torch.int16) == CANARY)
    assert torch.all(lse_buf[:g] == 12345.0) and torch.all(lse_buf[-g:] == 12345.0)
    yb, y = banded((T, H * D))
    zb, z = banded((T, H * D))
    G.say("gated residual with banded outputs")
    native.gated_residual(b.x, o.view(T, -1), y, b.gate, b.mod_row, b.shift2, b.scale2, z, w.eps)
    runner.run_gated_residual(b)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), b.y.view(torch.int16))
    assert torch.equal(z.view(torch.int16), b.z.view(torch.int16))
    for buf in (yb, zb):
        assert torch.all(buf[:g].view(torch.int16) == CANARY)
        assert torch.all(buf[-g:].view(torch.int16) == CANARY)
    # gated residual in place (y == x) and without the fused norm
    x2 = b.x.clone()
    native.gated_residual(x2, o.view(T, -1), x2, b.gate, b.mod_row)
    torch.cuda.synchronize()
    assert torch.equal(x2.view(torch.int16), b.y.view(torch.int16))


def test_zero_tokens_is_noop():
    import torch
    q = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.empty((0, 3), dtype=torch.int32, device="cuda")
    native.modulate_rope(q, q, q, q, pos, (0, 32, 32))
    native.varlen_attn_fwd(q, q, q, q, cu, 0)
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    native.gated_residual(x, x, x, x, cu)
    torch.cuda.synchronize()


def test_gate_zero_is_exact_residual():
    """gate = 0: y equals x bit for bit."""
    import torch
    w = W.custom([(5, 1, 6, 6, 0, 0)], H=2, D=64, modulate=True, residual=True, seed=3, name="g0")
    b = runner.to_device(w)
    b.gate.zero_()
    runner.run_chain(b)
    torch.cuda.synchronize()
    assert torch.equal(b.y.view(torch.int16), b.x.view(torch.int16))


def test_many_sequences_prologue_schedule():
    """More sequences than the in-kernel scheduler takes: the schedule comes
    from the prologue kernel through the workspace (lengths 0..150, shuffled)."""
    rng = np.random.default_rng(314)
    descs = []
    for s in range(100):
        t = int(rng.integers(0, 20))
        h = int(rng.integers(0, 12))
        ww = int(rng.integers(0, 12)) if h else 0
        if s % 10 == 7:
            t, h, ww = 0, 0, 0          # empty sequences in the middle of the pack
        descs.append((t, 1, h, ww, s, s))
    w = W.custom(descs, H=2, D=128, modulate=True, residual=True, seed=315, name="many_seqs")
    assert w.n_seq > 64 and min(w.seq_lens) == 0
    run_and_check(w)


@pytest.mark.parametrize("which", ["modulated_pack", "many_sequences"])
def test_graph_replay_matches_eager(which):
    """The whole chain captured in a HIP graph: every replay (with eager work
    and synchronisation between replays) reproduces the eager outputs bit for
    bit, for the in-kernel schedule and for the prologue-kernel schedule."""
    import torch
    if which == "modulated_pack":
        w = W.custom([(40, 1, 12, 20, 0, 0), (7, 1, 9, 5, 1, 1)], H=2, D=128, modulate=True,
                     residual=True, seed=77, name="graph_pack")
    else:
        descs = [(s % 9, 1, s % 5, (s % 7) if s % 5 else 0, s, s) for s in range(80)]
        w = W.custom(descs, H=2, D=64, modulate=True, residual=True, seed=78, name="graph_many")
        assert w.n_seq > 64
    G.say("graph replay", w.name, "T", w.T, "n_seq", w.n_seq)
    b = runner.to_device(w)
    other = runner.to_device(W.custom([(5, 1, 6, 6, 0, 0)], H=2, D=128, modulate=True,
                                      residual=True, seed=79, name="graph_other"))
    outs = lambda: (b.qr, b.kr, b.o, b.lse, b.y, b.z)  # noqa: E731
    runner.run_chain(b)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs()]
    g = runner.capture_chain(b)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs():
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, r in zip(("q'", "k'", "O", "LSE", "y", "z"), outs(), ref):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                               r.view(torch.int32) if r.dtype == torch.float32 else r.view(torch.int16)), \
                f"replay {rep}: {name} differs from the eager result"
        runner.run_chain(other)          # unrelated eager work between replays
        torch.cuda.synchronize()


def _attn_inputs(lens, H, D, seed, q_shift=0.0):
    """Seeded bf16 q, k, v ~ N(0,1) for a pack of the given lengths."""
    import torch
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    mk = lambda: torch.from_numpy(rng.standard_normal((T, H, D)).astype(np.float32)).to(torch.bfloat16)  # noqa: E731
    q, k, v = mk(), mk(), mk()
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, cu


def _run_attn(q, k, v, cu, grid=0):
    """One attention call on the GPU with the persistent grid set to `grid`
    (0 = one workgroup per CU); returns O (f64) and LSE (f64)."""
    import torch
    native.set_attn_fwd_grid(grid)
    try:
        T, H, D = q.shape
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        # NaN-filled outputs: a row the kernels fail to write cannot pass on
        # a previous call's values left at the same address
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
        cud = torch.from_numpy(cu).cuda()
        ws = torch.empty(native.attn_workspace_bytes(len(cu) - 1, T, H, D), dtype=torch.uint8, device="cuda")
        native.varlen_attn_fwd(qd, kd, vd, o, cud, int(np.diff(cu).max()), lse=lse, workspace=ws)
        torch.cuda.synchronize()
        return G.f64(o), lse.cpu().numpy().astype(np.float64), ws
    finally:
        native.set_attn_fwd_grid(0)


def test_grid_size_invariance():
    """The stream-K cut points move with the number of persistent
    workgroups (1: every tile whole; 37, 128, 300, one per CU: different
    cuts).  Every grid matches the oracle, and all agree with each other:
    LSE within fp32 rounding, O within a fraction of the bf16 rounding of the
    probabilities (each piece of a cut tile takes its reference max from its
    own first key step, so its probabilities round differently; the pieces'
    unnormalised O is merged in fp32, so O is rounded to bf16 once)."""
    lens = [1300, 41, 700, 2]
    q, k, v, cu = _attn_inputs(lens, H=3, D=128, seed=4242)
    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    O_ref, L_ref = R.attention(f(q), f(k), f(v), cu)
    results, err = {}, {}
    for grid in (0, 1, 37, 128, 300):
        G.say("grid size", grid, "lens", lens)
        O, lse, _ = _run_attn(q, k, v, cu, grid)
        G.check_attention(O, O_ref, f"grid{grid}", lse, L_ref)
        results[grid] = (O, lse)
        err[grid] = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
    # Each grid's O carries its own bf16 rounding of the probabilities
    # (relative RMS near 2^-9 / sqrt(3) per term) and of its cut pieces, so
    # two grids differ by about sqrt(2) times one grid's error to the oracle.
    O0, L0 = results[0]
    for grid, (O, lse) in results.items():
        d = np.abs(O - O0)
        rel = np.linalg.norm(O - O0) / np.linalg.norm(O0)
        assert rel <= 5e-3 and d.max() <= 1e-2, (grid, rel, d.max(), err)
        np.testing.assert_allclose(lse, L0, rtol=0, atol=2e-5)
    # Cut tiles are no less accurate than whole ones: relative RMS error to
    # the oracle with cut tiles against whole tiles (grid 1).
    G.say("relative RMS error to the oracle by grid", {g: float(f"{e:.3e}") for g, e in err.items()})
    for grid, e in err.items():
        assert e <= 1.08 * err[1], (grid, err)


@pytest.mark.parametrize("grid", [1, 0])
def test_score_spike_redo(grid):
    """One key per (sequence, head) scores about 260 (log2 units) above the
    rest, and it does not sit in the tile a segment starts with: the
    probabilities overflow against the reference max taken from the first
    key step, the row sums show it, and the workgroup redoes the segment with
    exact row maxima.  O (then close to that key's value row) and LSE match
    the oracle; grid 1 takes whole tiles, the default grid cut ones."""
    import torch
    lens = [1000, 700]
    H, D = 4, 128
    q, k, v, cu = _attn_inputs(lens, H=H, D=D, seed=777)
    q[:, :, :64] = (q[:, :, :64].float() * 0.5 + 2.0).to(torch.bfloat16)
    k[:, :, :64] = (k[:, :, :64].float() * 0.5).to(torch.bfloat16)
    for s, (a0, L) in enumerate(zip(cu[:-1], lens)):
        for h in range(H):
            j = int(a0) + 100 + 37 * h + 151 * s          # key tiles 3.. of the sequence
            assert j < a0 + L - 32
            k[j, h, :64] = 16.0
    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    O_ref, L_ref = R.attention(f(q), f(k), f(v), cu)
    assert L_ref.max() > 150.0                             # the spikes dominate
    G.say("score spike redo, grid", grid)
    O, lse, _ = _run_attn(q, k, v, cu, grid)
    G.check_attention(O, O_ref, f"spike_grid{grid}", lse, L_ref)


def test_prologue_schedule_exact():
    """Packs of more than 64 sequences take their work schedule from the
    prologue kernel, in the caller's workspace: sequences ranked by
    descending octave of their 32-key step count (empty sequences last),
    ties by index, with tiles = ceil(L/256), steps = ceil(L/32) and the
    exclusive prefix of tiles*H*steps.  Read back, it equals this host
    computation exactly."""
    rng = np.random.default_rng(2718)
    lens = [int(x) for x in rng.integers(0, 3000, size=150)]
    lens[7] = lens[40] = 0
    H, D = 2, 64
    q, k, v, cu = _attn_inputs(lens, H=H, D=D, seed=11)
    G.say("prologue schedule, n", len(lens))
    _, _, ws = _run_attn(q, k, v, cu, 0)
    raw = ws.cpu().numpy()
    n = len(lens)
    W_got = int(raw[0:8].view(np.int64)[0])
    ints = raw[8:8 + 4 * (1 + 3 * n)].view(np.int32)
    assert ints[0] == n
    seq, tiles, nkv = ints[1:1 + n], ints[1 + n:1 + 2 * n], ints[1 + 2 * n:1 + 3 * n]
    off = (12 + 12 * n + 7) // 8 * 8
    it_start = raw[off:off + 8 * (n + 1)].view(np.int64)
    steps = [(L + 31) // 32 for L in lens]
    octave = [0 if s == 0 else int(s).bit_length() for s in steps]
    order = sorted(range(n), key=lambda i: (-octave[i], i))
    np.testing.assert_array_equal(seq, order)
    np.testing.assert_array_equal(tiles, [(lens[i] + 255) // 256 for i in order])
    np.testing.assert_array_equal(nkv, [steps[i] for i in order])
    work = [((lens[i] + 255) // 256) * H * steps[i] for i in order]
    np.testing.assert_array_equal(it_start, np.concatenate([[0], np.cumsum(work)]))
    assert W_got == sum(work)


def test_side_stream_without_workspace():
    """stream= given and no workspace: the binding allocates the call's
    workspace on that stream, so memory allocated and filled on the current
    stream right after the call cannot land on it while the kernels run."""
    import torch
    lens = [2000, 900]
    q, k, v, cu = _attn_inputs(lens, H=8, D=128, seed=99)
    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    O_ref, L_ref = R.attention(f(q), f(k), f(v), cu)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((8, int(sum(lens))), float("nan"), dtype=torch.float32, device="cuda")
    cud = torch.from_numpy(cu).cuda()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    G.say("attention on a side stream without a workspace")
    for _ in range(3):
        native.varlen_attn_fwd(qd, kd, vd, o, cud, max(lens), lse=lse, stream=side)
        junk = [torch.full((1 << 22,), 3.0, device="cuda") for _ in range(8)]   # current stream
        del junk
        side.synchronize()
        torch.cuda.synchronize()
        G.check_attention(G.f64(o), O_ref, "side_stream", lse.cpu().numpy().astype(np.float64), L_ref)


def test_rows_outside_table_read_as_zero():
    """An adaLN row outside [0, n_rows) reads no table memory and acts as a
    row of zeros: every forward entry point gives, bit for bit, what it gives
    with a third, all-zero table row that those tokens select."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    T, H, D = 100, 2, 64
    C = H * D
    bf = lambda *s: torch.randn(*s, generator=g, device="cuda").to(torch.bfloat16)
    pos = torch.zeros((T, 3), dtype=torch.int32, device="cuda")
    pos[:, 1] = torch.arange(T, device="cuda", dtype=torch.int32) // 10
    pos[:, 2] = torch.arange(T, device="cuda", dtype=torch.int32) % 10
    rows = torch.zeros(T, dtype=torch.int32, device="cuda")
    rows[40:] = 1
    rows[7], rows[55], rows[99] = 2, -1, 1 << 30       # outside a 2-row table
    rows_ref = torch.where((rows < 0) | (rows >= 2), torch.full_like(rows, 2), rows)
    zero_row = torch.zeros((1, C), dtype=torch.bfloat16, device="cuda")
    shift, scale, gate = bf(2, C), bf(2, C), bf(2, C)
    shift3, scale3, gate3 = (torch.cat([t, zero_row]) for t in (shift, scale, gate))
    q, k, x, o = bf(T, H, D), bf(T, H, D), bf(T, C), bf(T, C)
    dims = (0, 32, 32)

    def same(a, b, name):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name

    outs = [torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    native.modulate_rope(q, k, outs[0], outs[1], pos, dims, 10000.0, shift, scale, rows)
    native.modulate_rope(q, k, outs[2], outs[3], pos, dims, 10000.0, shift3, scale3, rows_ref)
    torch.cuda.synchronize()
    same(outs[0], outs[2], "modulate_rope q")
    same(outs[1], outs[3], "modulate_rope k")

    y, z, y3, z3 = (torch.empty((T, C), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    native.gated_residual(x, o, y, gate, rows, shift, scale, z)
    native.gated_residual(x, o, y3, gate3, rows_ref, shift3, scale3, z3)
    torch.cuda.synchronize()
    same(y, y3, "gated_residual y")
    same(z, z3, "gated_residual z")
    same(y[7], x[7], "gated_residual: zero gate keeps x")

    w_qkv, w_o = (bf(3 * C, C) * 0.1).to(torch.bfloat16), (bf(C, C) * 0.1).to(torch.bfloat16)
    qkv, qkv3 = (torch.empty((T, 3 * C), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    native.block_qkv(x, w_qkv, qkv, pos, H, dims, 10000.0, shift, scale, rows)
    native.block_qkv(x, w_qkv, qkv3, pos, H, dims, 10000.0, shift3, scale3, rows_ref)
    yo, yo3 = (torch.empty((T, C), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    native.block_out(o, w_o, x, gate, rows, yo)
    native.block_out(o, w_o, x, gate3, rows_ref, yo3)
    torch.cuda.synchronize()
    same(qkv, qkv3, "block_qkv")
    same(yo, yo3, "block_out")
    same(yo[55], x[55], "block_out: zero gate keeps x")
