"""The C-ABI library loads, exports every symbol include/mf.h declares, and
rejects bad arguments on the host before any HIP call (no GPU needed: every
call here fails validation, so nothing reaches the device)."""
import ctypes
import os
import re

import pytest

from packed_attention_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

NULL, SHAPE, ALIGN, UNSUP, WS = -1, -2, -3, -4, -5
P = 0x10000          # a 16-byte-aligned stand-in address; never dereferenced
PODD = 0x10002       # misaligned


def header_symbols():
    src = open(os.path.join(ROOT, "include", "mf.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mf_[a-z0-9_]+)\s*\(", src)))


def test_exports_match_header():
    syms = header_symbols()
    assert syms == sorted(native.EXPORTS)
    lib = native.lib()
    for s in syms:
        assert hasattr(lib, s), s


def test_version_and_strings():
    lib = native.lib()
    assert lib.mf_abi_version() == 2
    for code in range(-7, 1):
        s = lib.mf_status_string(code).decode()
        assert s.startswith(native.STATUS_NAMES[code])
    assert lib.mf_status_string(-99).decode() == "MF_ERR_UNKNOWN"


def modrope(**kw):
    a = dict(stream=None, q_in=P, k_in=P, q_out=P, k_out=P, T=4, H=2, D=64, ld_in=128, ld_out=128,
             shift=None, scale=None, mod_row=None, n_rows=2, pos=P, f=0, r=32, c=32, base=10000.0,
             eps=1e-6)
    a.update(kw)
    return native.lib().mf_modulate_rope(*a.values())


def test_modulate_rope_validation():
    assert modrope(D=96) == UNSUP
    assert modrope(H=0) == SHAPE
    assert modrope(T=-1) == SHAPE
    assert modrope(H=128, D=128, ld_in=16384, ld_out=16384, r=64, c=64) == UNSUP   # C > 8192
    assert modrope(r=20, c=44) == SHAPE          # not multiples of 8
    assert modrope(r=32, c=24) == SHAPE          # sum != D
    assert modrope(f=-8, r=40, c=32) == SHAPE
    assert modrope(base=0.0) == SHAPE
    assert modrope(ld_in=120) == SHAPE
    assert modrope(shift=P) == NULL              # shift without scale
    assert modrope(shift=P, scale=P, mod_row=P, n_rows=2, eps=0.0) == SHAPE
    assert modrope(shift=P, scale=P, mod_row=P, n_rows=0) == SHAPE         # no rows for 4 tokens
    assert modrope(shift=P, scale=P, mod_row=P, n_rows=-1) == SHAPE
    assert modrope(shift=P, scale=P, mod_row=P, n_rows=(1 << 31) // 128 + 1) == SHAPE
    assert modrope(T=0, shift=P, scale=P, mod_row=P, n_rows=0) == 0          # no tokens, no rows
    assert modrope(q_in=None) == NULL
    assert modrope(pos=None) == NULL
    assert modrope(shift=P, scale=P, mod_row=None) == NULL
    assert modrope(ld_in=132, ld_out=136) == ALIGN
    assert modrope(k_out=PODD) == ALIGN
    assert modrope(shift=PODD, scale=P, mod_row=P) == ALIGN
    assert modrope(T=0, q_in=None, k_in=None, q_out=None, k_out=None, pos=None) == 0   # no-op


def attn(**kw):
    a = dict(stream=None, q=P, k=P, v=P, o=P, lse=None, cu=P, n_seq=1, max_seqlen=4, T=4, H=2,
             D=128, ld=256, ld_o=256, scale=0.088, ws=P, ws_bytes=1 << 31)
    a.update(kw)
    return native.lib().mf_varlen_attn_fwd(*a.values())


def test_attention_validation():
    assert attn(D=96) == UNSUP
    assert attn(H=0) == SHAPE
    assert attn(n_seq=0) == SHAPE
    assert attn(max_seqlen=5) == SHAPE
    assert attn(max_seqlen=0) == SHAPE
    assert attn(ld=200) == SHAPE
    assert attn(scale=0.0) == SHAPE
    assert attn(scale=float("inf")) == SHAPE
    assert attn(q=None) == NULL
    assert attn(cu=None) == NULL
    assert attn(ld=264, ld_o=260) == ALIGN
    assert attn(v=PODD) == ALIGN
    assert attn(lse=PODD) == ALIGN
    assert attn(ws=None) == WS
    assert attn(ws_bytes=8) == WS
    assert attn(ws=P + 16) == ALIGN
    # one sequence's rows must be addressable with 32-bit byte offsets
    assert attn(T=2_000_000, max_seqlen=2_000_000, ld=4096, ld_o=256) == UNSUP
    assert attn(T=0, n_seq=0, max_seqlen=0, q=None, k=None, v=None, o=None, cu=None) == 0


def test_workspace_query():
    lib = native.lib()
    a = lib.mf_varlen_attn_workspace_bytes(1, 4352, 24, 128)
    b = lib.mf_varlen_attn_workspace_bytes(1000, 4352, 24, 128)
    assert a > 0 and a % 256 == 0 and b % 256 == 0 and b >= (3 + 3 * 1000) * 4


def attn_bwd(**kw):
    a = dict(stream=None, q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, cu=P, n_seq=1,
             max_seqlen=4, T=4, H=2, D=128, ld=256, ld_o=256, ld_d=256, scale=0.088, ws=P,
             ws_bytes=1 << 31)
    a.update(kw)
    return native.lib().mf_varlen_attn_bwd(*a.values())


def test_attention_bwd_validation():
    assert attn_bwd(D=96) == UNSUP
    assert attn_bwd(H=0) == SHAPE
    assert attn_bwd(n_seq=0) == SHAPE
    assert attn_bwd(max_seqlen=5) == SHAPE
    assert attn_bwd(ld_d=128) == SHAPE
    assert attn_bwd(scale=-1.0) == SHAPE
    for name in ("q", "o", "dout", "lse", "dq", "dk", "dv", "cu"):
        assert attn_bwd(**{name: None}) == NULL, name
    assert attn_bwd(ld_d=260) == ALIGN
    assert attn_bwd(dk=PODD) == ALIGN
    assert attn_bwd(lse=P + 2) == ALIGN
    assert attn_bwd(ws=None) == WS
    assert attn_bwd(ws_bytes=64) == WS
    assert attn_bwd(ws=P + 16) == ALIGN
    assert attn_bwd(T=2_000_000, max_seqlen=2_000_000, ld=256, ld_o=4096) == UNSUP
    assert attn_bwd(T=0, n_seq=0, max_seqlen=0, q=None, k=None, v=None, o=None, dout=None,
                    lse=None, dq=None, dk=None, dv=None, cu=None) == 0
    lib = native.lib()
    a = lib.mf_varlen_attn_bwd_workspace_bytes(1, 4352, 24, 128)
    assert a % 256 == 0 and a >= 4352 * 24 * 4


def modrope_bwd(**kw):
    a = dict(stream=None, q_in=P, k_in=P, ld_in=128, dq_out=P, dk_out=P, ld_gout=128, dq_in=P,
             dk_in=P, ld_gin=128, T=4, H=2, D=64, scale=None, mod_row=None, n_rows=0, dshift=None,
             dscale=None, pos=P, f=0, r=32, c=32, base=10000.0, eps=1e-6, ws=P, ws_bytes=1 << 31)
    a.update(kw)
    return native.lib().mf_modulate_rope_bwd(*a.values())


def test_modulate_rope_bwd_validation():
    mod = dict(scale=P, mod_row=P, n_rows=2, dshift=P, dscale=P)
    assert modrope_bwd(D=96) == UNSUP
    assert modrope_bwd(H=0) == SHAPE
    assert modrope_bwd(r=20, c=44) == SHAPE
    assert modrope_bwd(ld_gin=100) == SHAPE
    assert modrope_bwd(**{**mod, "n_rows": 0}) == SHAPE
    assert modrope_bwd(**{**mod, "eps": 0.0}) == SHAPE
    for name in ("q_in", "dq_out", "dk_in", "pos"):
        assert modrope_bwd(**{name: None}) == NULL, name
    assert modrope_bwd(**{**mod, "dscale": None}) == NULL
    assert modrope_bwd(**{**mod, "mod_row": None}) == NULL
    assert modrope_bwd(ld_in=132) == ALIGN
    assert modrope_bwd(dk_out=PODD) == ALIGN
    assert modrope_bwd(**{**mod, "dshift": P + 2}) == ALIGN
    assert modrope_bwd(**{**mod, "ws": None}) == WS
    assert modrope_bwd(**{**mod, "ws_bytes": 64}) == WS
    assert modrope_bwd(**{**mod, "ws": P + 16}) == ALIGN
    assert modrope_bwd(T=0, q_in=None, k_in=None, dq_out=None, dk_out=None, dq_in=None, dk_in=None,
                       pos=None) == 0


def gres_bwd(**kw):
    a = dict(stream=None, x=P, o=P, gate=P, mod_row=P, n_rows=2, dy=P, scale2=None, dz=None, dx=P,
             dout=P, dgate=P, dshift2=None, dscale2=None, T=4, C=256, eps=1e-6, ws=P,
             ws_bytes=1 << 31)
    a.update(kw)
    return native.lib().mf_gated_residual_bwd(*a.values())


def test_gated_residual_bwd_validation():
    assert gres_bwd(C=100) == SHAPE
    assert gres_bwd(n_rows=0) == SHAPE
    assert gres_bwd(dz=P) == NULL                      # fused set incomplete
    assert gres_bwd(scale2=P, dz=P, dshift2=P, dscale2=P, eps=0.0) == SHAPE
    for name in ("x", "o", "gate", "mod_row", "dx", "dout", "dgate"):
        assert gres_bwd(**{name: None}) == NULL, name
    assert gres_bwd(o=PODD) == ALIGN
    assert gres_bwd(dy=PODD) == ALIGN
    assert gres_bwd(dgate=P + 2) == ALIGN
    assert gres_bwd(ws=None) == WS
    assert gres_bwd(ws_bytes=16) == WS
    assert gres_bwd(ws=P + 32) == ALIGN
    lib = native.lib()
    assert lib.mf_gated_residual_bwd_workspace_bytes(4352, 3072) >= 3 * 4352 * 3072
    assert lib.mf_modulate_rope_bwd_workspace_bytes(4352, 24, 128) >= 2 * 4352 * 3072


def gres(**kw):
    a = dict(stream=None, x=P, o=P, y=P, gate=P, mod_row=P, n_rows=2, shift2=None, scale2=None, z=None,
             T=4, C=256, eps=1e-6)
    a.update(kw)
    return native.lib().mf_gated_residual(*a.values())


def test_gated_residual_validation():
    assert gres(C=100) == SHAPE
    assert gres(C=16384) == SHAPE
    assert gres(T=-3) == SHAPE
    assert gres(shift2=P) == NULL
    assert gres(shift2=P, scale2=P, z=P, eps=-1.0) == SHAPE
    assert gres(x=None) == NULL
    assert gres(mod_row=None) == NULL
    assert gres(o=PODD) == ALIGN
    assert gres(shift2=P, scale2=P, z=PODD) == ALIGN
    assert gres(T=0, x=None, o=None, y=None, gate=None, mod_row=None) == 0
    assert gres(T=0, x=None, o=None, y=None, gate=None, mod_row=None, n_rows=0) == 0
    assert gres(n_rows=0) == SHAPE
    assert gres(n_rows=-2) == SHAPE
    assert gres(n_rows=(1 << 31) // 256 + 1) == SHAPE


def bqkv(**kw):
    a = dict(stream=None, x=P, ld_x=128, w=P, qkv=P, ld_qkv=384, shift=None, scale=None, mod_row=None,
             n_rows=2, pos=P, T=4, H=2, D=64, f=0, r=32, c=32, base=10000.0, eps=1e-6, ws=None, ws_bytes=0)
    a.update(kw)
    return native.lib().mf_block_qkv(*a.values())


def bout(**kw):
    a = dict(stream=None, o=P, ld_o=256, w=P, x=P, gate=P, mod_row=P, n_rows=2, y=P, T=4, C=256)
    a.update(kw)
    return native.lib().mf_block_out(*a.values())


def test_block_projection_validation():
    assert bqkv(D=96) == UNSUP
    assert bqkv(H=72, D=128, ld_x=9216, ld_qkv=27648) == UNSUP          # C > 8192
    assert bqkv(r=20, c=44) == SHAPE
    assert bqkv(ld_x=64) == SHAPE
    assert bqkv(ld_qkv=256) == SHAPE
    assert bqkv(shift=P) == NULL
    assert bqkv(shift=P, scale=P, mod_row=P, eps=0.0) == SHAPE
    assert bqkv(shift=P, scale=P, mod_row=P, n_rows=0) == SHAPE
    assert bqkv(shift=P, scale=P, mod_row=P, n_rows=(1 << 31) // 128 + 1) == SHAPE
    assert bqkv(x=None) == NULL
    assert bqkv(pos=None) == NULL
    assert bqkv(shift=P, scale=P, mod_row=None) == NULL
    assert bqkv(ld_x=132) == ALIGN
    assert bqkv(w=PODD) == ALIGN
    assert bqkv(shift=P, scale=P, mod_row=P) == WS
    assert bqkv() == WS                                                  # required without modulation too
    assert bqkv(shift=P, scale=P, mod_row=P, ws=P, ws_bytes=16) == WS
    assert bqkv(shift=P, scale=P, mod_row=P, ws=P + 16, ws_bytes=1 << 20) == ALIGN
    assert bqkv(T=1 << 20, ld_x=4096) == UNSUP                           # 32-bit offsets
    assert bqkv(T=0, x=None, w=None, qkv=None, pos=None) == 0
    assert bout(C=100) == SHAPE
    assert bout(ld_o=128) == SHAPE
    assert bout(ld_o=260) == ALIGN
    assert bout(o=None) == NULL
    assert bout(gate=None) == NULL
    assert bout(n_rows=0) == SHAPE
    assert bout(n_rows=(1 << 31) // 256 + 1) == SHAPE
    assert bout(y=PODD) == ALIGN
    assert bout(T=1 << 22, C=1024, ld_o=1024) == UNSUP
    assert bout(T=0, o=None, w=None, x=None, gate=None, mod_row=None, y=None) == 0
    # the modulated rows (T C bf16), then the rotation table (T D/2 pairs of
    # fp32 cos, sin); no part depends on the device
    assert native.lib().mf_block_qkv_workspace_bytes(4352, 24, 128) == 4352 * 3072 * 2 + 4352 * 128 * 4
    assert native.lib().mf_block_qkv_workspace_bytes(4096, 24, 128) == 4096 * 3072 * 2 + 4096 * 128 * 4
    assert native.lib().mf_block_qkv_workspace_bytes(16384, 24, 128) == 16384 * 3072 * 2 + 16384 * 128 * 4
    # the table rows are 256-byte aligned: T D 4 = 3 * 64 * 4 rounds up to 768
    assert native.lib().mf_block_qkv_workspace_bytes(3, 1, 64) % 256 == 0


def cfg_step(**kw):
    a = dict(stream=None, v=P, ld_v=128, rows=P, z=P, z_out=P, x=None, ld_x=0, N=16, Cl=128, w=4.5, t=0.75,
             tn=0.5)
    a.update(kw)
    return native.lib().mf_cfg_euler_step(*a.values())


def test_cfg_euler_validation():
    assert cfg_step(Cl=100) == SHAPE
    assert cfg_step(Cl=8192) == SHAPE
    assert cfg_step(N=-1) == SHAPE
    assert cfg_step(ld_v=64) == SHAPE
    assert cfg_step(x=P, ld_x=64) == SHAPE
    assert cfg_step(w=float("nan")) == SHAPE
    assert cfg_step(t=float("inf")) == SHAPE
    assert cfg_step(v=None) == NULL
    assert cfg_step(rows=None) == NULL
    assert cfg_step(z_out=None) == NULL
    assert cfg_step(ld_v=132) == ALIGN
    assert cfg_step(rows=P + 4) == ALIGN
    assert cfg_step(z=PODD) == ALIGN
    assert cfg_step(x=PODD, ld_x=128) == ALIGN
    assert cfg_step(N=0, v=None, rows=None, z=None, z_out=None) == 0


def qknr(**kw):
    a = dict(stream=None, q=P, ld_q=256, k=P, ld_k=128, qo=P, ld_qo=256, ko=P, ld_ko=128, wq=P, wk=P, pos=P,
             T=4, Hq=4, Hkv=2, D=64, base=10000.0, eps=1e-6)
    a.update(kw)
    return native.lib().mf_qk_norm_rope(*a.values())


def causal(**kw):
    a = dict(stream=None, q=P, ld_q=256, k=P, v=P, ld_kv=128, o=P, ld_o=256, lse=None, cu=P, n=2, T=4, Hq=4,
             Hkv=2, D=64, scale=0.125, ws=None, ws_bytes=0)
    a.update(kw)
    return native.lib().mf_varlen_attn_causal_fwd(*a.values())


def test_text_encoder_validation():
    assert qknr(D=96) == UNSUP
    assert qknr(Hq=160, ld_q=10240, ld_qo=10240) == UNSUP
    assert qknr(ld_q=128) == SHAPE
    assert qknr(ld_ko=64) == SHAPE
    assert qknr(eps=0.0) == SHAPE
    assert qknr(base=-1.0) == SHAPE
    assert qknr(wq=None) == NULL
    assert qknr(pos=None) == NULL
    assert qknr(ld_k=132) == ALIGN
    assert qknr(ko=PODD) == ALIGN
    assert qknr(T=0, q=None, k=None, qo=None, ko=None, wq=None, wk=None, pos=None) == 0
    assert causal(Hq=3) == SHAPE                 # Hq not a multiple of Hkv
    assert causal(D=80) == UNSUP
    assert causal(ld_kv=64) == SHAPE
    assert causal(scale=0.0) == SHAPE
    assert causal(T=1 << 24, ld_q=256) == UNSUP
    assert causal(q=None) == NULL
    assert causal(cu=None) == NULL
    assert causal(ld_o=260) == ALIGN
    assert causal(lse=P + 2) == ALIGN
    assert causal() == WS
    assert causal(ws=P, ws_bytes=32) == WS       # T=4, n=2: (0 + 2 + 1) descriptors of 16 bytes
    assert causal(ws=P + 8, ws_bytes=64) == ALIGN
    assert causal(n=0, q=None) == 0
    assert native.lib().mf_varlen_attn_causal_workspace_bytes(16, 4096) == (128 + 16 + 1) * 16
    assert native.lib().mf_varlen_attn_causal_workspace_bytes(-1, 4) == 0


def test_library_has_no_oracle_dependency():
    """The product path never touches the oracle: no module of the package
    imports it, and the native sources do not mention it."""
    pkg = os.path.join(ROOT, "packed_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_library_resolves_every_symbol():
    """Load with immediate binding: an undefined symbol (e.g. a kernel stub the
    host pass failed to emit) fails here instead of at the first GPU call."""
    ctypes.CDLL(native.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)
