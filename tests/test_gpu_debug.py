"""MF_DEBUG=1: the library copies the index tables to the host and rejects
invalid contents with MF_ERR_TABLE before anything is launched.

MF_DEBUG is read once per process, so the calls run in a child process with
it set.  Each case breaks exactly one table entry of an otherwise valid call:
  * attention (forward, allocation-free forward, backward): cu_seqlens not
    starting at 0, not ending at T, decreasing, or a sequence longer than
    max_seqlen;
  * modulate + RoPE (forward and backward): a negative position; an adaLN
    row that is negative (forward) or >= n_rows;
  * gated residual (forward and backward): a negative row, or a row >= n_rows;
  * block projections (QKV with modulation, out with the gate): a negative
    row, or a row >= n_rows.
Every rejected call must leave its NaN-filled output untouched (nothing ran),
and the same calls with valid tables must succeed."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import json, math
import torch
from packed_attention_amd import native

MF_ERR_TABLE = -6
out = {}

def status(fn):
    try:
        fn()
        torch.cuda.synchronize()
        return 0
    except native.MFError as e:
        return e.code

def i32(xs):
    return torch.tensor(xs, dtype=torch.int32, device="cuda")

def record(name, fn, outputs):
    before = [t.clone() for t in outputs]
    s = status(fn)
    untouched = all(torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                                b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))
                    for a, b in zip(outputs, before))
    out[name] = {"status": s, "untouched": untouched}

g = torch.Generator(device="cuda")
g.manual_seed(5)
T, H, D = 100, 2, 64
C = H * D
bf = lambda *s: torch.randn(*s, generator=g, device="cuda").to(torch.bfloat16)
nan_bf = lambda *s: torch.full(s, float("nan"), dtype=torch.bfloat16, device="cuda")
nan_f = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")

# ---- attention
q, k, v = bf(T, H, D), bf(T, H, D), bf(T, H, D)
good = i32([0, 60, 100])
bad = {"cu_start": i32([4, 60, 100]), "cu_end": i32([0, 60, 90]), "cu_decreasing": i32([0, 70, 60, 100])}
o, lse = nan_bf(T, H, D), nan_f(H, T)
record("attn_fwd_ok", lambda: native.varlen_attn_fwd(q, k, v, o, good, 60, lse=lse), [])
for name, cu in bad.items():
    o2, l2 = nan_bf(T, H, D), nan_f(H, T)
    record("attn_fwd_" + name, lambda: native.varlen_attn_fwd(q, k, v, o2, cu, 70, lse=l2), [o2, l2])
    o3 = nan_bf(T, H, D)
    record("attn_noalloc_" + name, lambda: native.varlen_attn_fwd_noalloc(q, k, v, o3, cu, 70), [o3])
o2 = nan_bf(T, H, D)
record("attn_fwd_max_seqlen", lambda: native.varlen_attn_fwd(q, k, v, o2, good, 50), [o2])
dout = bf(T, H, D)
dq, dk, dv = nan_bf(T, H, D), nan_bf(T, H, D), nan_bf(T, H, D)
record("attn_bwd_ok", lambda: native.varlen_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, good, 60), [])
for name, cu in list(bad.items()) + [("max_seqlen", good)]:
    a, b_, c = nan_bf(T, H, D), nan_bf(T, H, D), nan_bf(T, H, D)
    ms = 50 if name == "max_seqlen" else 70
    record("attn_bwd_" + name, lambda: native.varlen_attn_bwd(q, k, v, o, dout, lse, a, b_, c, cu, ms),
           [a, b_, c])

# ---- modulate + RoPE
pos = torch.zeros((T, 3), dtype=torch.int32, device="cuda")
pos[:, 1] = torch.arange(T, device="cuda", dtype=torch.int32) // 10
pos[:, 2] = torch.arange(T, device="cuda", dtype=torch.int32) % 10
rows = torch.zeros(T, dtype=torch.int32, device="cuda")
rows[50:] = 1
shift, scale = bf(2, C), bf(2, C)
dims = (0, 32, 32)
qo, ko = nan_bf(T, H, D), nan_bf(T, H, D)
record("modrope_ok", lambda: native.modulate_rope(q, k, qo, ko, pos, dims, 10000.0, shift, scale, rows), [])
bad_pos = pos.clone(); bad_pos[37, 2] = -1
bad_row = rows.clone(); bad_row[80] = -1
big_row = rows.clone(); big_row[99] = 2        # n_rows = 2
for name, p, r in (("pos", bad_pos, rows), ("row", pos, bad_row), ("big_row", pos, big_row)):
    a, b_ = nan_bf(T, H, D), nan_bf(T, H, D)
    record("modrope_" + name, lambda: native.modulate_rope(q, k, a, b_, p, dims, 10000.0, shift, scale, r), [a, b_])
dqo, dko = bf(T, H, D), bf(T, H, D)
dsh, dsc = nan_f(2, C), nan_f(2, C)
a, b_ = nan_bf(T, H, D), nan_bf(T, H, D)
record("modrope_bwd_ok", lambda: native.modulate_rope_bwd(q, k, dqo, dko, a, b_, pos, dims, 10000.0, scale, rows,
                                                          dsh, dsc), [])
for name, p, r in (("pos", bad_pos, rows), ("row", pos, big_row)):
    a, b_, s1, s2 = nan_bf(T, H, D), nan_bf(T, H, D), nan_f(2, C), nan_f(2, C)
    record("modrope_bwd_" + name, lambda: native.modulate_rope_bwd(q, k, dqo, dko, a, b_, p, dims, 10000.0, scale, r,
                                                                   s1, s2), [a, b_, s1, s2])

# ---- gated residual
x, og, gate = bf(T, C), bf(T, C), bf(2, C)
y, z = nan_bf(T, C), nan_bf(T, C)
record("gres_ok", lambda: native.gated_residual(x, og, y, gate, rows, shift, scale, z), [])
for name, r in (("row", bad_row), ("big_row", big_row)):
    a, b_ = nan_bf(T, C), nan_bf(T, C)
    record("gres_" + name, lambda: native.gated_residual(x, og, a, gate, r, shift, scale, b_), [a, b_])
dy, dz = bf(T, C), bf(T, C)
dx, do = nan_bf(T, C), nan_bf(T, C)
dg, ds2, dc2 = nan_f(2, C), nan_f(2, C), nan_f(2, C)
record("gres_bwd_ok", lambda: native.gated_residual_bwd(x, og, gate, rows, dy, dx, do, dg, scale, dz, ds2, dc2), [])
for name, r in (("neg_row", bad_row), ("big_row", big_row)):
    a, b_, c1, c2, c3 = nan_bf(T, C), nan_bf(T, C), nan_f(2, C), nan_f(2, C), nan_f(2, C)
    record("gres_bwd_" + name, lambda: native.gated_residual_bwd(x, og, gate, r, dy, a, b_, c1, scale, dz, c2, c3),
           [a, b_, c1, c2, c3])

# ---- block projections
w_qkv, w_o = bf(3 * C, C), bf(C, C)
qkv = nan_bf(T, 3 * C)
record("bqkv_ok", lambda: native.block_qkv(x, w_qkv, qkv, pos, H, dims, 10000.0, shift, scale, rows), [])
yo = nan_bf(T, C)
record("bout_ok", lambda: native.block_out(og, w_o, x, gate, rows, yo), [])
for name, r in (("neg_row", bad_row), ("big_row", big_row)):
    a = nan_bf(T, 3 * C)
    record("bqkv_" + name, lambda: native.block_qkv(x, w_qkv, a, pos, H, dims, 10000.0, shift, scale, r), [a])
    b_ = nan_bf(T, C)
    record("bout_" + name, lambda: native.block_out(og, w_o, x, gate, r, b_), [b_])
print("RESULT " + json.dumps(out), flush=True)
'''


def test_debug_table_checks():
    env = dict(os.environ, MF_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=240)
    lines = [l for l in r.stdout.splitlines() if l.startswith("RESULT ")]
    assert r.returncode == 0 and lines, r.stdout[-3000:]
    res = json.loads(lines[-1][len("RESULT "):])
    for name, v in res.items():
        if name.endswith("_ok"):
            assert v["status"] == 0, (name, v)
        else:
            assert v["status"] == -6, (name, v)          # MF_ERR_TABLE
            assert v["untouched"], (name, "a rejected call wrote its outputs")
    assert len([n for n in res if not n.endswith("_ok")]) == 24
