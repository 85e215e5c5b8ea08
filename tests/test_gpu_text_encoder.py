"""Text-encoder variant (mf_qk_norm_rope, mf_varlen_attn_causal_fwd) vs the
fp64 text-encoder oracle.

qk-norm + RoPE is elementwise from exact bf16 inputs in fp32: within one bf16
ulp of the oracle per element (plus 1e-6 absolute near zero).  The causal
attention is fed the kernel's own bf16 q', k', v (as the forward's tests do),
with the forward's bars: relative RMS of O <= 1e-2, max-abs <= 2e-2 *
max|ref|, LSE within 1e-3.  Small and ragged packs are compared element by
element; the 16-prompt pack at full size as well (the oracle handles it).
"""
import numpy as np
import pytest

import gpu_common as G
from oracle import text_encoder as TE
from packed_attention_amd import native, runner, workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    native.lib()


def run_norm_rope(tp):
    import torch
    G.say(tp.name, "qk_norm_rope", "T", tp.T, "Hq", tp.Hq, "Hkv", tp.Hkv, "D", tp.D)
    cu, pos = native.prompt_tables(tp.lens)
    q, k = runner.bf16_tensor(tp.q), runner.bf16_tensor(tp.k)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    native.qk_norm_rope(q, k, qo, ko, runner.bf16_tensor(tp.wq), runner.bf16_tensor(tp.wk),
                        torch.from_numpy(pos).cuda(), tp.rope_base, tp.eps)
    torch.cuda.synchronize()
    f = W.bf16_bits_to_f64
    rq, rk = TE.qk_norm_rope(f(tp.q), f(tp.k), f(tp.wq), f(tp.wk), pos, tp.rope_base, tp.eps)
    for name, got, ref in (("q'", qo, rq), ("k'", ko, rk)):
        g = G.f64(got)
        assert np.all(np.abs(g - ref) <= G.bf16_ulp(ref) + 1e-6), (tp.name, name, float(np.abs(g - ref).max()))
    return cu, qo, ko


def run_causal(tp, cu, q, k, v):
    import torch
    G.say(tp.name, "causal attention", "T", tp.T, "prompts", len(tp.lens))
    T, Hq, D = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")
    native.varlen_attn_causal_fwd(q, k, v, o, torch.from_numpy(cu).cuda(), lse=lse)
    torch.cuda.synchronize()
    ref, rl = TE.causal_attention(G.f64(q), G.f64(k), G.f64(v), cu)
    g = G.f64(o)
    assert np.all(np.isfinite(g))
    rel = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
    assert rel <= 1e-2, (tp.name, rel)
    assert np.abs(g - ref).max() <= 2e-2 * np.abs(ref).max(), tp.name
    assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3, (tp.name, float(np.abs(lse.cpu().numpy() - rl).max()))


def check_pack(tp):
    cu, qo, ko = run_norm_rope(tp)
    run_causal(tp, cu, qo, ko, runner.bf16_tensor(tp.v))


def test_tiny_grouped():
    check_pack(W.text_pack(seed=51, Hq=4, Hkv=2, D=64, lens=[5, 1, 9, 3], name="text_tiny"))


# lengths around the 64-key and 128-query tiles, an empty prompt, one token
@pytest.mark.parametrize("D", [64, 128])
def test_ragged(D):
    lens = [1, 2, 63, 64, 65, 0, 127, 128, 129, 300]
    check_pack(W.text_pack(seed=52 + D, Hq=8, Hkv=2, D=D, lens=lens, name=f"text_ragged_d{D}"))


# group sizes 8 (four heads per workgroup, two workgroups per key/value head
# and slab) and 3 (one head per workgroup, 128-query slabs)
@pytest.mark.parametrize("Hq,Hkv,D", [(16, 2, 128), (6, 2, 64), (8, 1, 64)])
def test_group_sizes(Hq, Hkv, D):
    check_pack(W.text_pack(seed=60 + Hq, Hq=Hq, Hkv=Hkv, D=D, lens=[33, 129, 1, 200, 64],
                           name=f"text_g{Hq // Hkv}_d{D}"))


def test_no_grouping():
    check_pack(W.text_pack(seed=57, Hq=4, Hkv=4, D=128, lens=[70, 200, 3], name="text_mha"))


def test_text_pack_full():
    """16 prompts U{64..512}, 32 query / 8 key-value heads of 128 dims."""
    check_pack(W.text_pack())


def test_text_pack_bench_size():
    """The 64-prompt pack the benchmark times, every element."""
    check_pack(W.text_pack(seed=W.TEXT_BENCH_SEED, n_prompts=W.TEXT_BENCH_PROMPTS, name="text_pack_64"))


def test_long_prompt_sampled():
    """A 66 000-token prompt (units of more than 1023 key tiles, past the
    prologue's largest work class) beside a short one: q', k' element by
    element, O and LSE on sampled rows against the row-at-a-time oracle."""
    import torch
    tp = W.text_pack(seed=71, Hq=2, Hkv=1, D=64, lens=[66000, 300], name="text_long")
    cu, qo, ko = run_norm_rope(tp)
    G.say(tp.name, "causal attention, sampled rows")
    o = torch.full_like(qo, float("nan"))
    lse = torch.empty((tp.Hq, tp.T), dtype=torch.float32, device="cuda")
    native.varlen_attn_causal_fwd(qo, ko, runner.bf16_tensor(tp.v), o, torch.from_numpy(cu).cuda(), lse=lse)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 65471, 65472, 65535, 65999, 66000, 66001, 66299],
                                     np.random.default_rng(72).choice(tp.T, 24, replace=False)]))
    ref, rl = TE.causal_attention_rows(G.f64(qo), G.f64(ko), W.bf16_bits_to_f64(tp.v), cu, rows)
    g = G.f64(o)[rows]
    assert np.all(np.isfinite(g))
    rel = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
    assert rel <= 1e-2, rel
    assert np.abs(g - ref).max() <= 2e-2 * np.abs(ref).max()
    assert np.abs(lse.cpu().numpy()[:, rows] - rl).max() <= 1e-3


def test_first_token_attends_to_itself():
    """Closed form on the GPU: every prompt's first token outputs its own v."""
    import torch
    tp = W.text_pack(seed=58, Hq=4, Hkv=1, D=128, lens=[40, 1, 90])
    cu, _ = native.prompt_tables(tp.lens)
    q, k, v = (runner.bf16_tensor(a) for a in (tp.q, tp.k, tp.v))
    o = torch.empty_like(q)
    native.varlen_attn_causal_fwd(q, k, v, o, torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    for a in cu[:-1]:
        for h in range(4):
            assert torch.equal(o[a, h], v[a, 0])
