"""ctypes binding of libmf.so (include/mf.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module only
turns torch tensors into device pointers, strides and the current stream.
If libmf.so is missing the first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmf.so")

MF_OK = 0
STATUS_NAMES = {0: "MF_OK", -1: "MF_ERR_NULL", -2: "MF_ERR_SHAPE", -3: "MF_ERR_ALIGN",
                -4: "MF_ERR_UNSUPPORTED", -5: "MF_ERR_WORKSPACE", -6: "MF_ERR_TABLE",
                -7: "MF_ERR_HIP"}

# Every symbol include/mf.h declares.
EXPORTS = ("mf_status_string", "mf_abi_version", "mf_pack_count", "mf_pack_tables",
           "mf_modulate_rope", "mf_varlen_attn_workspace_bytes", "mf_varlen_attn_fwd",
           "mf_gated_residual", "mf_varlen_attn_bwd_workspace_bytes", "mf_varlen_attn_bwd",
           "mf_modulate_rope_bwd", "mf_gated_residual_bwd", "mf_modulate_rope_bwd_workspace_bytes",
           "mf_gated_residual_bwd_workspace_bytes", "mf_block_qkv_workspace_bytes", "mf_block_qkv",
           "mf_block_out", "mf_cfg_pair_count", "mf_cfg_pair_rows", "mf_cfg_euler_step", "mf_qk_norm_rope",
           "mf_varlen_attn_causal_workspace_bytes", "mf_varlen_attn_causal_fwd", "mf_prompt_tables",
           "mf_set_attn_fwd_grid", "mf_varlen_attn_fwd_noalloc")


class MFError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (status {code})")
        self.code = code


class SampleDesc(ctypes.Structure):
    _fields_ = [("text_len", ctypes.c_int32), ("n_frames", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("mod_row_text", ctypes.c_int32), ("mod_row_image", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmf.so (built in-tree by packed_attention_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run packed_attention_amd.build.build() "
                           "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    L.mf_status_string.argtypes = [i32]
    L.mf_status_string.restype = ctypes.c_char_p
    L.mf_abi_version.argtypes = []
    L.mf_abi_version.restype = i32
    L.mf_pack_count.argtypes = [vp, i32, ctypes.POINTER(i64)]
    L.mf_pack_count.restype = i32
    L.mf_pack_tables.argtypes = [vp, i32, vp, vp, vp, vp]
    L.mf_pack_tables.restype = i32
    L.mf_modulate_rope.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i64, i64, vp, vp, vp, i32, vp,
                                   i32, i32, i32, f32, f32]
    L.mf_modulate_rope.restype = i32
    L.mf_varlen_attn_workspace_bytes.argtypes = [i32, i64, i32, i32]
    L.mf_varlen_attn_workspace_bytes.restype = sz
    L.mf_varlen_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i64, i64,
                                     f32, vp, sz]
    L.mf_varlen_attn_fwd.restype = i32
    L.mf_varlen_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i64, i64, f32]
    L.mf_varlen_attn_fwd_noalloc.restype = i32
    L.mf_set_attn_fwd_grid.argtypes = [i32]
    L.mf_set_attn_fwd_grid.restype = i32
    L.mf_gated_residual.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, i64, i32, f32]
    L.mf_gated_residual.restype = i32
    L.mf_varlen_attn_bwd_workspace_bytes.argtypes = [i32, i64, i32, i32]
    L.mf_varlen_attn_bwd_workspace_bytes.restype = sz
    L.mf_varlen_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, i32,
                                     i32, i64, i64, i64, f32, vp, sz]
    L.mf_varlen_attn_bwd.restype = i32
    L.mf_modulate_rope_bwd.argtypes = [vp, vp, vp, i64, vp, vp, i64, vp, vp, i64, i64, i32, i32, vp, vp,
                                       i32, vp, vp, vp, i32, i32, i32, f32, f32, vp, sz]
    L.mf_modulate_rope_bwd_workspace_bytes.argtypes = [i64, i32, i32]
    L.mf_modulate_rope_bwd_workspace_bytes.restype = sz
    L.mf_gated_residual_bwd_workspace_bytes.argtypes = [i64, i32]
    L.mf_gated_residual_bwd_workspace_bytes.restype = sz
    L.mf_modulate_rope_bwd.restype = i32
    L.mf_gated_residual_bwd.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                        i32, f32, vp, sz]
    L.mf_gated_residual_bwd.restype = i32
    L.mf_block_qkv_workspace_bytes.argtypes = [i64, i32, i32]
    L.mf_block_qkv_workspace_bytes.restype = sz
    L.mf_block_qkv.argtypes = [vp, vp, i64, vp, vp, i64, vp, vp, vp, i32, vp, i64, i32, i32, i32, i32,
                               i32, f32, f32, vp, sz]
    L.mf_block_qkv.restype = i32
    L.mf_block_out.argtypes = [vp, vp, i64, vp, vp, vp, vp, i32, vp, i64, i32]
    L.mf_block_out.restype = i32
    L.mf_cfg_pair_count.argtypes = [vp, i32, vp, vp, i32, ctypes.POINTER(i64)]
    L.mf_cfg_pair_count.restype = i32
    L.mf_cfg_pair_rows.argtypes = [vp, i32, vp, vp, i32, vp]
    L.mf_cfg_pair_rows.restype = i32
    L.mf_cfg_euler_step.argtypes = [vp, vp, i64, vp, vp, vp, vp, i64, i64, i32, f32, f32, f32]
    L.mf_cfg_euler_step.restype = i32
    L.mf_qk_norm_rope.argtypes = [vp, vp, i64, vp, i64, vp, i64, vp, i64, vp, vp, vp, i64, i32, i32, i32, f32, f32]
    L.mf_qk_norm_rope.restype = i32
    L.mf_varlen_attn_causal_workspace_bytes.argtypes = [i32, i64]
    L.mf_varlen_attn_causal_workspace_bytes.restype = sz
    L.mf_varlen_attn_causal_fwd.argtypes = [vp, vp, i64, vp, vp, i64, vp, i64, vp, vp, i32, i64, i32, i32, i32, f32,
                                            vp, sz]
    L.mf_varlen_attn_causal_fwd.restype = i32
    L.mf_prompt_tables.argtypes = [vp, i32, vp, vp]
    L.mf_prompt_tables.restype = i32
    _lib = L
    return L


def check(code: int) -> None:
    if code != MF_OK:
        msg = lib().mf_status_string(code).decode()
        raise MFError(code, msg)


# ---------------------------------------------------------------------------
# Host tables
# ---------------------------------------------------------------------------

def _desc_array(descs: Sequence[Tuple[int, ...]]):
    arr = (SampleDesc * max(1, len(descs)))()
    for i, d in enumerate(descs):
        arr[i] = SampleDesc(*[int(x) for x in d])
    return arr


def pack_count(descs) -> int:
    out = ctypes.c_int64(0)
    check(lib().mf_pack_count(_desc_array(descs), len(descs), ctypes.byref(out)))
    return int(out.value)


def pack_tables(descs):
    """Host C++ tables: (cu_seqlens[n+1], pos[T][3], seq_id[T], mod_row[T]) as int32 numpy."""
    n = len(descs)
    T = pack_count(descs)
    cu = np.zeros(n + 1, dtype=np.int32)
    pos = np.zeros((T, 3), dtype=np.int32)
    sid = np.zeros(T, dtype=np.int32)
    mr = np.zeros(T, dtype=np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    check(lib().mf_pack_tables(_desc_array(descs), n, p(cu), p(pos), p(sid), p(mr)))
    return cu, pos, sid, mr


# ---------------------------------------------------------------------------
# Device calls (torch tensors)
# ---------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _temp_workspace(nbytes: int, device, stream):
    """A workspace for one call when the caller passed none.  It is allocated
    on the stream the kernels run on, so the caching allocator hands its bytes
    to later work only in that stream's order (a block allocated on another
    stream could be reused while the kernels still read it)."""
    import torch
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _check_bf16_rows(name, t, cols):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{name}: expected a bfloat16 CUDA tensor")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")


def _table_rows(name, t, cols, rows=None):
    """Row count of a contiguous bf16 [n_rows][cols] adaLN table (0 for None);
    with rows given, the table must have that many."""
    if t is None:
        return 0 if rows is None else rows
    _check_bf16_rows(name, t, cols)
    if not t.is_contiguous() or t.numel() % cols:
        raise ValueError(f"{name}: expected a contiguous [n_rows][{cols}] tensor")
    n = t.numel() // cols
    if rows is not None and n != rows:
        raise ValueError(f"{name}: {n} rows, expected {rows}")
    return n


def _token_stride(t, inner):
    """Token stride (elements) of a [T][H][D] or [T][C] view whose inner dims are packed."""
    if t.dim() == 3:
        if t.stride(1) != t.shape[2]:
            raise ValueError("head dimension must be packed (stride(1) == D)")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), inner)


def modulate_rope(q_in, k_in, q_out, k_out, pos, rope_dims, rope_base=10000.0,
                  shift=None, scale=None, mod_row=None, eps=1e-6, stream=None):
    """mf_modulate_rope on [T][H][D] bf16 tensors (q_out/k_out may alias the inputs)."""
    T, H, D = q_in.shape
    for n, t in (("q_in", q_in), ("k_in", k_in), ("q_out", q_out), ("k_out", k_out)):
        _check_bf16_rows(n, t, H * D)
        if tuple(t.shape) != (T, H, D):
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {(T, H, D)}")
    ld_in = _token_stride(q_in, H * D)
    if _token_stride(k_in, H * D) != ld_in:
        raise ValueError("q_in and k_in must share a token stride")
    ld_out = _token_stride(q_out, H * D)
    if _token_stride(k_out, H * D) != ld_out:
        raise ValueError("q_out and k_out must share a token stride")
    f, r, c = (int(x) for x in rope_dims)
    n_rows = _table_rows("scale", scale, H * D, _table_rows("shift", shift, H * D) if shift is not None else None)
    check(lib().mf_modulate_rope(_stream(stream), _ptr(q_in), _ptr(k_in), _ptr(q_out), _ptr(k_out),
                                 T, H, D, ld_in, ld_out, _ptr(shift), _ptr(scale), _ptr(mod_row), n_rows,
                                 _ptr(pos), f, r, c, float(rope_base), float(eps)))


def set_attn_fwd_grid(g: int) -> None:
    """Test hook: run the attention forward on g persistent workgroups (0 =
    one per CU).  Process-wide; size workspaces after setting it."""
    check(lib().mf_set_attn_fwd_grid(int(g)))


def attn_workspace_bytes(n_seq: int, T: int, H: int, D: int) -> int:
    return int(lib().mf_varlen_attn_workspace_bytes(n_seq, T, H, D))


def varlen_attn_fwd(q, k, v, o, cu_seqlens, max_seqlen, lse=None, softmax_scale=None,
                    workspace=None, stream=None):
    """mf_varlen_attn_fwd on [T][H][D] bf16 q, k, v (sharing one token stride) into o."""
    import torch
    T, H, D = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_bf16_rows(n, t, H * D)
        if tuple(t.shape) != (T, H, D):
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {(T, H, D)}")
    ld = _token_stride(q, H * D)
    if _token_stride(k, H * D) != ld or _token_stride(v, H * D) != ld:
        raise ValueError("q, k and v must share a token stride")
    ld_o = _token_stride(o, H * D)
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
        raise TypeError("cu_seqlens: expected an int32 CUDA tensor")
    n_seq = cu_seqlens.numel() - 1
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (H, T)):
        raise ValueError("lse: expected float32 [H][T]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    need = attn_workspace_bytes(n_seq, T, H, D)
    if workspace is None:
        workspace = _temp_workspace(need, q.device, stream)
    check(lib().mf_varlen_attn_fwd(_stream(stream), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   _ptr(cu_seqlens), n_seq, int(max_seqlen), T, H, D, ld, ld_o,
                                   float(softmax_scale), _ptr(workspace), workspace.numel()))


def varlen_attn_fwd_noalloc(q, k, v, o, cu_seqlens, max_seqlen, lse=None, softmax_scale=None, stream=None):
    """mf_varlen_attn_fwd_noalloc: mf_varlen_attn_fwd with the library's
    per-GPU scratch array as its workspace (nothing is allocated; calls that
    overlap on one GPU race)."""
    import torch
    T, H, D = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_bf16_rows(n, t, H * D)
        if tuple(t.shape) != (T, H, D):
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {(T, H, D)}")
    ld = _token_stride(q, H * D)
    if _token_stride(k, H * D) != ld or _token_stride(v, H * D) != ld:
        raise ValueError("q, k and v must share a token stride")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
        raise TypeError("cu_seqlens: expected an int32 CUDA tensor")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (H, T)):
        raise ValueError("lse: expected float32 [H][T]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    check(lib().mf_varlen_attn_fwd_noalloc(_stream(stream), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                           _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen), T, H, D,
                                           ld, _token_stride(o, H * D), float(softmax_scale)))


def gated_residual(x, o, y, gate, mod_row, shift2=None, scale2=None, z=None, eps=1e-6, stream=None):
    """mf_gated_residual on contiguous [T][C] bf16 rows (o may be given as [T][H][D])."""
    T = x.shape[0]
    C = x.numel() // max(T, 1) if T else x.shape[-1]
    for n, t in (("x", x), ("o", o), ("y", y), ("z", z)):
        if t is None:
            continue
        _check_bf16_rows(n, t, C)
        if not t.is_contiguous() or t.numel() != T * C:
            raise ValueError(f"{n}: expected a contiguous [T][C] tensor")
    n_rows = _table_rows("gate", gate, C)
    _table_rows("shift2", shift2, C, n_rows)
    _table_rows("scale2", scale2, C, n_rows)
    check(lib().mf_gated_residual(_stream(stream), _ptr(x), _ptr(o), _ptr(y), _ptr(gate),
                                  _ptr(mod_row), n_rows, _ptr(shift2), _ptr(scale2), _ptr(z), T, C,
                                  float(eps)))


def attn_bwd_workspace_bytes(n_seq: int, T: int, H: int, D: int) -> int:
    return int(lib().mf_varlen_attn_bwd_workspace_bytes(n_seq, T, H, D))


def varlen_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, max_seqlen, softmax_scale=None,
                    workspace=None, stream=None):
    """mf_varlen_attn_bwd: dq, dk, dv ([T][H][D] bf16, one token stride) from the forward's
    q, k, v (one token stride), o and dout (one token stride) and lse (float32 [H][T])."""
    import torch
    T, H, D = q.shape
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk),
                 ("dv", dv)):
        _check_bf16_rows(n, t, H * D)
        if tuple(t.shape) != (T, H, D):
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {(T, H, D)}")
    ld = _token_stride(q, H * D)
    if _token_stride(k, H * D) != ld or _token_stride(v, H * D) != ld:
        raise ValueError("q, k and v must share a token stride")
    ld_o = _token_stride(o, H * D)
    if _token_stride(dout, H * D) != ld_o:
        raise ValueError("o and dout must share a token stride")
    ld_d = _token_stride(dq, H * D)
    if _token_stride(dk, H * D) != ld_d or _token_stride(dv, H * D) != ld_d:
        raise ValueError("dq, dk and dv must share a token stride")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
        raise TypeError("cu_seqlens: expected an int32 CUDA tensor")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (H, T) or not lse.is_contiguous():
        raise ValueError("lse: expected contiguous float32 [H][T]")
    n_seq = cu_seqlens.numel() - 1
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    need = attn_bwd_workspace_bytes(n_seq, T, H, D)
    if workspace is None:
        workspace = _temp_workspace(need, q.device, stream)
    check(lib().mf_varlen_attn_bwd(_stream(stream), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                   _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), n_seq,
                                   int(max_seqlen), T, H, D, ld, ld_o, ld_d, float(softmax_scale),
                                   _ptr(workspace), workspace.numel()))


def modulate_rope_bwd(q_in, k_in, dq_out, dk_out, dq_in, dk_in, pos, rope_dims, rope_base=10000.0,
                      scale=None, mod_row=None, dshift=None, dscale=None, eps=1e-6, workspace=None,
                      stream=None):
    """mf_modulate_rope_bwd on [T][H][D] bf16 tensors; dshift/dscale float32 [n_rows][H*D]."""
    import torch
    T, H, D = q_in.shape
    for n, t in (("q_in", q_in), ("k_in", k_in), ("dq_out", dq_out), ("dk_out", dk_out),
                 ("dq_in", dq_in), ("dk_in", dk_in)):
        _check_bf16_rows(n, t, H * D)
        if tuple(t.shape) != (T, H, D):
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {(T, H, D)}")
    ld_in = _token_stride(q_in, H * D)
    ld_gout = _token_stride(dq_out, H * D)
    ld_gin = _token_stride(dq_in, H * D)
    if (_token_stride(k_in, H * D) != ld_in or _token_stride(dk_out, H * D) != ld_gout
            or _token_stride(dk_in, H * D) != ld_gin):
        raise ValueError("q and k tensors of each pair must share a token stride")
    n_rows = 0
    if scale is not None:
        n_rows = scale.shape[0]
        for n, t in (("dshift", dshift), ("dscale", dscale)):
            if t is None or t.dtype != torch.float32 or tuple(t.shape) != (n_rows, H * D):
                raise ValueError(f"{n}: expected float32 [n_rows][H*D]")
    f, r, c = (int(x) for x in rope_dims)
    if workspace is None and scale is not None:
        workspace = _temp_workspace(int(lib().mf_modulate_rope_bwd_workspace_bytes(T, H, D)), q_in.device,
                                    stream)
    check(lib().mf_modulate_rope_bwd(_stream(stream), _ptr(q_in), _ptr(k_in), ld_in, _ptr(dq_out),
                                     _ptr(dk_out), ld_gout, _ptr(dq_in), _ptr(dk_in), ld_gin, T, H, D,
                                     _ptr(scale), _ptr(mod_row), n_rows, _ptr(dshift), _ptr(dscale),
                                     _ptr(pos), f, r, c, float(rope_base), float(eps), _ptr(workspace),
                                     0 if workspace is None else workspace.numel()))


def gated_residual_bwd(x, o, gate, mod_row, dy, dx, dout, dgate, scale2=None, dz=None, dshift2=None,
                       dscale2=None, eps=1e-6, workspace=None, stream=None):
    """mf_gated_residual_bwd on contiguous [T][C] bf16 rows; row sums float32 [n_rows][C]."""
    import torch
    T = x.shape[0]
    C = x.shape[-1]
    for n, t in (("x", x), ("o", o), ("dy", dy), ("dz", dz), ("dx", dx), ("dout", dout)):
        if t is None:
            continue
        _check_bf16_rows(n, t, C)
        if not t.is_contiguous() or t.numel() != T * C:
            raise ValueError(f"{n}: expected a contiguous [T][C] tensor")
    n_rows = gate.shape[0]
    for n, t in (("dgate", dgate), ("dshift2", dshift2), ("dscale2", dscale2)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (n_rows, C)):
            raise ValueError(f"{n}: expected float32 [n_rows][C]")
    if workspace is None:
        workspace = _temp_workspace(int(lib().mf_gated_residual_bwd_workspace_bytes(T, C)), x.device, stream)
    check(lib().mf_gated_residual_bwd(_stream(stream), _ptr(x), _ptr(o), _ptr(gate), _ptr(mod_row),
                                      n_rows, _ptr(dy), _ptr(scale2), _ptr(dz), _ptr(dx), _ptr(dout),
                                      _ptr(dgate), _ptr(dshift2), _ptr(dscale2), T, C, float(eps),
                                      _ptr(workspace), workspace.numel()))


def block_qkv_workspace_bytes(T: int, H: int, D: int) -> int:
    return int(lib().mf_block_qkv_workspace_bytes(T, H, D))


def block_qkv(x, w_qkv, qkv, pos, H, rope_dims, rope_base=10000.0, shift=None, scale=None, mod_row=None,
              eps=1e-6, workspace=None, stream=None):
    """mf_block_qkv: qkv [T][3C] bf16 (q', k', v) from the residual stream x [T][C] bf16 and
    W_qkv [3C][C] bf16 (modulated by shift/scale rows when given)."""
    import torch
    T, C = x.shape
    D = C // H
    _check_bf16_rows("x", x, C)
    _check_bf16_rows("qkv", qkv, 3 * C)
    _check_bf16_rows("w_qkv", w_qkv, C)
    if tuple(w_qkv.shape) != (3 * C, C) or not w_qkv.is_contiguous():
        raise ValueError("w_qkv: expected a contiguous [3C][C] tensor")
    if qkv.dim() != 2 or qkv.shape[0] != T or qkv.shape[1] != 3 * C:
        raise ValueError("qkv: expected [T][3C]")
    if workspace is None:
        workspace = _temp_workspace(block_qkv_workspace_bytes(T, H, D), x.device, stream)
    f, r, c = (int(v) for v in rope_dims)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    n_rows = _table_rows("scale", scale, C, _table_rows("shift", shift, C) if shift is not None else None)
    check(lib().mf_block_qkv(_stream(stream), _ptr(x), _token_stride(x, C), _ptr(w_qkv), _ptr(qkv),
                             _token_stride(qkv, 3 * C), _ptr(shift), _ptr(scale), _ptr(mod_row), n_rows, _ptr(pos),
                             T, H, D, f, r, c, float(rope_base), float(eps), _ptr(workspace), nbytes))


def block_out(o, w_o, x, gate, mod_row, y, stream=None):
    """mf_block_out: y = x + gate[m] * (o W_o^T) on [T][C] bf16 rows (o may be [T][H][D])."""
    T, C = x.shape
    _check_bf16_rows("o", o, C)
    for n, t in (("x", x), ("y", y), ("w_o", w_o)):
        _check_bf16_rows(n, t, C)
        if not t.is_contiguous():
            raise ValueError(f"{n}: expected a contiguous tensor")
    if tuple(w_o.shape) != (C, C):
        raise ValueError("w_o: expected [C][C]")
    n_rows = _table_rows("gate", gate, C)
    check(lib().mf_block_out(_stream(stream), _ptr(o), _token_stride(o, C), _ptr(w_o), _ptr(x), _ptr(gate),
                             _ptr(mod_row), n_rows, _ptr(y), T, C))


def cfg_pair_rows(descs, cond, uncond) -> np.ndarray:
    """mf_cfg_pair_count + mf_cfg_pair_rows: int32 [N][2] packed rows of the
    conditional and unconditional copy of every evolving latent token."""
    arr = _desc_array(descs)
    P = len(cond)
    ca = np.ascontiguousarray(cond, dtype=np.int32)
    ua = np.ascontiguousarray(uncond, dtype=np.int32)
    n = ctypes.c_int64(0)
    check(lib().mf_cfg_pair_count(arr, len(descs), ca.ctypes.data, ua.ctypes.data, P, ctypes.byref(n)))
    rows = np.zeros((max(n.value, 1), 2), dtype=np.int32)
    check(lib().mf_cfg_pair_rows(arr, len(descs), ca.ctypes.data, ua.ctypes.data, P, rows.ctypes.data))
    return rows[:n.value]


def cfg_euler_step(v, rows, z, z_out, guidance, t, t_next, x_next=None, stream=None):
    """mf_cfg_euler_step: v bf16 [T][Cl] rows, rows int32 [N][2] (device), z/z_out fp32 [N][Cl]."""
    import torch
    T, Cl = v.shape
    _check_bf16_rows("v", v, Cl)
    if rows.dtype != torch.int32 or not rows.is_contiguous() or rows.dim() != 2 or rows.shape[1] != 2:
        raise ValueError("rows: expected a contiguous int32 [N][2] tensor")
    N = rows.shape[0]
    for n_, t_ in (("z", z), ("z_out", z_out)):
        if t_.dtype != torch.float32 or not t_.is_contiguous() or tuple(t_.shape) != (N, Cl):
            raise ValueError(f"{n_}: expected a contiguous float32 [N][Cl] tensor")
    ld_x = 0
    if x_next is not None:
        _check_bf16_rows("x_next", x_next, Cl)
        ld_x = _token_stride(x_next, Cl)
    check(lib().mf_cfg_euler_step(_stream(stream), _ptr(v), _token_stride(v, Cl), _ptr(rows), _ptr(z), _ptr(z_out),
                                  _ptr(x_next), ld_x, N, Cl, float(guidance), float(t), float(t_next)))


def qk_norm_rope(q_in, k_in, q_out, k_out, wq, wk, pos, rope_base=10000.0, eps=1e-6, stream=None):
    """mf_qk_norm_rope on q [T][Hq][D] and k [T][Hkv][D] bf16 (outputs may alias inputs)."""
    T, Hq, D = q_in.shape
    Hkv = k_in.shape[1]
    for n, t, H in (("q_in", q_in, Hq), ("q_out", q_out, Hq), ("k_in", k_in, Hkv), ("k_out", k_out, Hkv)):
        _check_bf16_rows(n, t, H * D)
        if tuple(t.shape) != (T, H, D):
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {(T, H, D)}")
    check(lib().mf_qk_norm_rope(_stream(stream), _ptr(q_in), _token_stride(q_in, Hq * D), _ptr(k_in),
                                _token_stride(k_in, Hkv * D), _ptr(q_out), _token_stride(q_out, Hq * D),
                                _ptr(k_out), _token_stride(k_out, Hkv * D), _ptr(wq), _ptr(wk), _ptr(pos), T, Hq,
                                Hkv, D, float(rope_base), float(eps)))


def varlen_attn_causal_fwd(q, k, v, o, cu_seqlens, lse=None, softmax_scale=None, workspace=None, stream=None):
    """mf_varlen_attn_causal_fwd: q, o [T][Hq][D], k, v [T][Hkv][D] bf16 (k, v sharing a token stride)."""
    import torch
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    for n, t, H in (("q", q, Hq), ("o", o, Hq), ("k", k, Hkv), ("v", v, Hkv)):
        _check_bf16_rows(n, t, H * D)
        if tuple(t.shape) != (T, H, D):
            raise ValueError(f"{n}: shape {tuple(t.shape)} != {(T, H, D)}")
    ld_kv = _token_stride(k, Hkv * D)
    if _token_stride(v, Hkv * D) != ld_kv:
        raise ValueError("k and v must share a token stride")
    n_seq = cu_seqlens.numel() - 1
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    need = int(lib().mf_varlen_attn_causal_workspace_bytes(n_seq, T))
    if workspace is None:
        workspace = _temp_workspace(max(need, 16), q.device, stream)
    check(lib().mf_varlen_attn_causal_fwd(_stream(stream), _ptr(q), _token_stride(q, Hq * D), _ptr(k), _ptr(v),
                                          ld_kv, _ptr(o), _token_stride(o, Hq * D), _ptr(lse), _ptr(cu_seqlens),
                                          n_seq, T, Hq, Hkv, D, float(softmax_scale), _ptr(workspace),
                                          workspace.numel() * workspace.element_size()))


def prompt_tables(lens):
    """mf_prompt_tables: (cu_seqlens[n+1], pos[T]) int32 numpy for packed prompts of the given lengths."""
    la = np.ascontiguousarray(lens, dtype=np.int32)
    n = len(la)
    T = int(la.astype(np.int64).sum()) if n else 0
    cu = np.zeros(n + 1, dtype=np.int32)
    # the library rejects T > INT32_MAX before writing: no buffer that large
    pos = np.zeros(max(T, 1) if T <= 2 ** 31 - 1 else 1, dtype=np.int32)
    check(lib().mf_prompt_tables(la.ctypes.data if n else None, n, cu.ctypes.data, pos.ctypes.data))
    return cu, pos[:T]
