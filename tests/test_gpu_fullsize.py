"""HIP path vs the fp64 oracle at the workloads' full sizes, in the same
launch configuration the benchmark times (runner.run_chain), on sampled
outputs the oracle computes one by one:
  * tables: every entry, exact;
  * modulate+RoPE and the gated residual: whole rows of sampled tokens
    (per kernel: the oracle is fed the kernel's own bf16 inputs);
  * attention: sampled (token, head) rows, each against its whole sequence;
  * end to end (1024^2 sample): oracle chain in fp64 from the seeded inputs
    at sampled rows.
"""
import numpy as np
import pytest

import gpu_common as G
from oracle import reference as R
from packed_attention_amd import native, runner, workloads as W

pytestmark = pytest.mark.gpu

N_TOKENS = 192       # sampled tokens for the row-wise kernels
N_ROWS = 384         # sampled (token, head) attention rows
N_ROWS_BIG = 1536    # the same for the ~34k-token packs


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    native.lib()


def _sample_tokens(rng, cu, n):
    """Sampled tokens, always including each sequence's first and last token."""
    T = int(cu[-1])
    edges = [int(c) for c in cu[:-1] if c < T] + [int(c) - 1 for c in cu[1:] if c > 0]
    pick = rng.choice(T, size=min(n, T), replace=False)
    return np.unique(np.concatenate([pick, np.asarray(edges, dtype=np.int64)]))


def check_full(w, e2e=False, n_rows=N_ROWS):
    import torch
    G.say(w.name, "T", w.T, "n_seq", w.n_seq, "descs", w.descs)
    b = runner.to_device(w)
    cu, pos, sid, mr = R.pack_tables(w.descs)
    np.testing.assert_array_equal(b.cu_host, cu)
    np.testing.assert_array_equal(b.pos_host, pos)
    np.testing.assert_array_equal(b.mod_row_host, mr)
    runner.run_chain(b)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 99)
    toks = _sample_tokens(rng, cu, N_TOKENS)
    tk = torch.as_tensor(toks, device="cuda")
    a = G.wl_f64(w)

    # modulate + RoPE on sampled rows
    qr_ref, kr_ref = R.modulate_rope(a["q"][toks], a["k"][toks], pos[toks], w.rope_dims,
                                     w.rope_base, a["shift"], a["scale"], mr[toks], w.eps)
    qr_s, kr_s = G.f64(b.qr[tk]), G.f64(b.kr[tk])
    G.check_bar(qr_s, qr_ref, w.name + ".q'")
    G.check_bar(kr_s, kr_ref, w.name + ".k'")
    G.check_rounded(qr_s, qr_ref, w.name + ".q'")
    G.check_rounded(kr_s, kr_ref, w.name + ".k'")

    # attention on sampled (token, head) rows, per kernel
    qr32 = runner.bf16_to_f64(b.qr).astype(np.float32)
    kr32 = runner.bf16_to_f64(b.kr).astype(np.float32)
    v32 = runner.bf16_to_f64(b.v).astype(np.float32)
    rows = _sample_tokens(rng, cu, n_rows)
    heads = rng.integers(0, w.H, size=len(rows))
    O_ref, L_ref = R.attention_rows(qr32, kr32, v32, cu, rows, heads)
    O_all = b.o.cpu()
    O_s = G.f64(O_all[torch.as_tensor(rows), torch.as_tensor(heads)])
    lse_s = b.lse.cpu().numpy()[heads, rows].astype(np.float64)
    G.check_attention(O_s, O_ref, w.name, lse_s, L_ref)

    # gated residual on sampled rows, fed the kernel's own O
    O_rows = G.f64(O_all[torch.as_tensor(toks)]).reshape(len(toks), -1)
    y_ref, z_ref = R.gated_residual(a["x"][toks], O_rows, a["gate"], mr[toks], a["shift2"],
                                    a["scale2"], w.eps)
    y_s, z_s = G.f64(b.y[tk]), G.f64(b.z[tk])
    G.check_bar(y_s, y_ref, w.name + ".y")
    G.check_rounded(y_s, y_ref, w.name + ".y")
    G.check_bar(z_s, z_ref, w.name + ".z")
    G.check_rounded(z_s, z_ref, w.name + ".z", slack=1e-5)

    if e2e:
        qf, kf = R.modulate_rope(a["q"], a["k"], pos, w.rope_dims, w.rope_base, a["shift"],
                                 a["scale"], mr, w.eps)
        O_e, L_e = R.attention_rows(qf, kf, a["v"], cu, rows, heads)
        G.check_attention(O_s, O_e, w.name + ".e2e", lse_s, L_e, G.LSE_ABS_E2E)


def test_single_1024_full():
    check_full(W.single_1024(), e2e=True)


@pytest.mark.parametrize("seed", range(2000, 2008))
def test_native_budget_pack(seed):
    check_full(W.native_pack(seed))


def test_cfg_pack():
    check_full(W.cfg_pack(), n_rows=N_ROWS_BIG)


def test_edit_pack_3d_rope():
    check_full(W.edit_pack(), n_rows=N_ROWS_BIG)
