"""Run the hot path of a workload on one GPU through the C-ABI binding.

Moves a seeded workload (bf16 bit patterns from ``workloads``) into HBM,
builds the integer tables with the library's host table builder, and chains
mf_modulate_rope -> mf_varlen_attn_fwd -> mf_gated_residual on the current
stream.  Used by the GPU tests, the smoke check and the benchmark.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import native, workloads
from .workloads import Workload


def bf16_tensor(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_to_f64(t) -> np.ndarray:
    """Exact widening of a bf16 torch tensor (any device) to float64 numpy."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class DeviceBatch:
    w: Workload
    cu_host: np.ndarray
    pos_host: np.ndarray
    mod_row_host: np.ndarray
    cu: object
    pos: object
    mod_row: object
    q: object
    k: object
    v: object
    x: Optional[object]
    shift: Optional[object]
    scale: Optional[object]
    gate: Optional[object]
    shift2: Optional[object]
    scale2: Optional[object]
    # outputs / intermediates
    qr: object
    kr: object
    o: object
    lse: object
    y: Optional[object]
    z: Optional[object]
    workspace: object
    max_seqlen: int


def to_device(w: Workload, device="cuda", with_lse=True) -> DeviceBatch:
    import torch
    cu, pos, _sid, mr = native.pack_tables(w.descs)
    T, H, D = w.T, w.H, w.D
    dev = lambda a: None if a is None else bf16_tensor(a, device)  # noqa: E731
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    lens = np.diff(cu)
    max_seqlen = int(lens.max()) if len(lens) else 0
    return DeviceBatch(
        w=w, cu_host=cu, pos_host=pos, mod_row_host=mr,
        cu=torch.from_numpy(cu).to(device), pos=torch.from_numpy(pos).to(device),
        mod_row=torch.from_numpy(mr).to(device),
        q=q, k=k, v=v, x=dev(w.x), shift=dev(w.shift), scale=dev(w.scale), gate=dev(w.gate),
        shift2=dev(w.shift2), scale2=dev(w.scale2),
        # attention outputs start as NaN, so that a row the kernels never
        # write cannot pass a check on values left in reused memory
        qr=torch.empty_like(q), kr=torch.empty_like(k), o=torch.full_like(q, float("nan")),
        lse=torch.full((H, T), float("nan"), dtype=torch.float32, device=device) if with_lse else None,
        y=torch.empty((T, H * D), dtype=torch.bfloat16, device=device) if w.x is not None else None,
        z=torch.empty((T, H * D), dtype=torch.bfloat16, device=device) if w.x is not None else None,
        workspace=torch.empty(native.attn_workspace_bytes(len(w.descs), T, H, D), dtype=torch.uint8,
                              device=device),
        max_seqlen=max_seqlen,
    )


def to_device_synthetic(shape: "workloads.Shape", device="cuda", seed: int = 0) -> DeviceBatch:
    """A device batch of the given shape whose tensors are drawn on the GPU
    from a seeded generator with the workloads' distributions (q, k, v, x
    ~ N(0,1), adaLN rows ~ N(0,0.1), bf16): for timing the large packs
    without building them on the host; tables from the library's builder."""
    import torch
    cu, pos, _sid, mr = native.pack_tables(shape.descs)
    T, H, D, n = shape.T, shape.H, shape.D, len(shape.descs)
    C = H * D
    g = torch.Generator(device=device)
    g.manual_seed(int(shape.seed) * 7919 + seed)
    rn = lambda *sz, s=1.0: (torch.randn(*sz, generator=g, device=device) * s).to(torch.bfloat16)  # noqa: E731
    q, k, v = rn(T, H, D), rn(T, H, D), rn(T, H, D)
    x = rn(T, C) if shape.residual else None
    shift = rn(n, C, s=0.1) if shape.modulate else None
    scale = rn(n, C, s=0.1) if shape.modulate else None
    gate = rn(n, C, s=0.1) if shape.residual else None
    shift2 = rn(n, C, s=0.1) if shape.residual else None
    scale2 = rn(n, C, s=0.1) if shape.residual else None
    lens = np.diff(cu)
    return DeviceBatch(
        w=shape, cu_host=cu, pos_host=pos, mod_row_host=mr,
        cu=torch.from_numpy(cu).to(device), pos=torch.from_numpy(pos).to(device),
        mod_row=torch.from_numpy(mr).to(device),
        q=q, k=k, v=v, x=x, shift=shift, scale=scale, gate=gate, shift2=shift2, scale2=scale2,
        qr=torch.empty_like(q), kr=torch.empty_like(k), o=torch.empty_like(q),
        lse=torch.empty((H, T), dtype=torch.float32, device=device),
        y=torch.empty((T, C), dtype=torch.bfloat16, device=device) if x is not None else None,
        z=torch.empty((T, C), dtype=torch.bfloat16, device=device) if x is not None else None,
        workspace=torch.empty(native.attn_workspace_bytes(n, T, H, D), dtype=torch.uint8, device=device),
        max_seqlen=int(lens.max()) if len(lens) else 0,
    )


def run_modulate_rope(b: DeviceBatch, stream=None):
    w = b.w
    native.modulate_rope(b.q, b.k, b.qr, b.kr, b.pos, w.rope_dims, w.rope_base,
                         b.shift, b.scale, b.mod_row if b.shift is not None else None, w.eps,
                         stream=stream)


def run_attention(b: DeviceBatch, stream=None):
    native.varlen_attn_fwd(b.qr, b.kr, b.v, b.o, b.cu, b.max_seqlen, lse=b.lse,
                           workspace=b.workspace, stream=stream)


def run_gated_residual(b: DeviceBatch, stream=None):
    if b.x is None:
        return
    native.gated_residual(b.x, b.o.view(b.w.T, -1), b.y, b.gate, b.mod_row, b.shift2, b.scale2,
                          b.z, b.w.eps, stream=stream)


def run_gated_residual_y(b: DeviceBatch, stream=None):
    """The gated residual alone (y = x + gate * o, no fused next adaLN)."""
    if b.x is None:
        return
    native.gated_residual(b.x, b.o.view(b.w.T, -1), b.y, b.gate, b.mod_row, stream=stream)


def run_chain(b: DeviceBatch, stream=None):
    """One pass of the whole hot path."""
    run_modulate_rope(b, stream)
    run_attention(b, stream)
    run_gated_residual(b, stream)


def capture_chain(b: DeviceBatch):
    """Record one pass of the hot path on `b` into a HIP graph (torch's
    CUDAGraph wrapper); ``g.replay()`` then re-runs the three calls with one
    submission.  The path enqueues kernels only (no memsets, no allocation),
    so the graph holds exactly the eager kernels.  Run the chain eagerly once
    before capturing so that one-time set-up happens outside the capture."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_chain(b)
    return g


@dataclasses.dataclass
class GradBatch:
    """Upstream gradients and backward outputs for one DeviceBatch."""
    dy: object
    dz: object
    dx: object
    do: object
    dgate: object
    dshift2: object
    dscale2: object
    dqr: object
    dkr: object
    dv: object
    dq: object
    dk: object
    dshift: object
    dscale: object
    workspace: object
    ws_mod: object
    ws_gres: object


def grads_to_device(b: DeviceBatch, device="cuda") -> GradBatch:
    """Seeded upstream gradients dy, dz (bf16 [T][C]) and every backward
    output, allocated once."""
    import torch
    from .workloads import upstream_grads
    w = b.w
    g = upstream_grads(w)
    T, H, D = w.T, w.H, w.D
    C = H * D
    n_rows = len(w.descs)
    rows = lambda: torch.empty((n_rows, C), dtype=torch.float32, device=device)  # noqa: E731
    return GradBatch(
        dy=bf16_tensor(g["dy"], device), dz=bf16_tensor(g["dz"], device),
        dx=torch.empty((T, C), dtype=torch.bfloat16, device=device),
        do=torch.empty((T, C), dtype=torch.bfloat16, device=device),
        dgate=rows(), dshift2=rows(), dscale2=rows(),
        dqr=torch.empty_like(b.q), dkr=torch.empty_like(b.k), dv=torch.empty_like(b.v),
        dq=torch.empty_like(b.q), dk=torch.empty_like(b.k),
        dshift=rows() if w.modulate else None, dscale=rows() if w.modulate else None,
        workspace=torch.empty(native.attn_bwd_workspace_bytes(len(w.descs), T, H, D),
                              dtype=torch.uint8, device=device),
        ws_mod=torch.empty(int(native.lib().mf_modulate_rope_bwd_workspace_bytes(T, H, D)),
                           dtype=torch.uint8, device=device),
        ws_gres=torch.empty(int(native.lib().mf_gated_residual_bwd_workspace_bytes(T, C)),
                            dtype=torch.uint8, device=device))


def run_gated_residual_bwd(b: DeviceBatch, gb: GradBatch, stream=None):
    T, C = b.w.T, b.w.H * b.w.D
    native.gated_residual_bwd(b.x, b.o.view(T, C), b.gate, b.mod_row, gb.dy, gb.dx, gb.do, gb.dgate,
                              b.scale2, gb.dz, gb.dshift2, gb.dscale2, b.w.eps, workspace=gb.ws_gres,
                              stream=stream)


def run_attention_bwd(b: DeviceBatch, gb: GradBatch, stream=None):
    w = b.w
    native.varlen_attn_bwd(b.qr, b.kr, b.v, b.o, gb.do.view(w.T, w.H, w.D), b.lse, gb.dqr, gb.dkr,
                           gb.dv, b.cu, b.max_seqlen, workspace=gb.workspace, stream=stream)


def run_modulate_rope_bwd(b: DeviceBatch, gb: GradBatch, stream=None):
    w = b.w
    native.modulate_rope_bwd(b.q, b.k, gb.dqr, gb.dkr, gb.dq, gb.dk, b.pos, w.rope_dims, w.rope_base,
                             b.scale, b.mod_row if b.scale is not None else None, gb.dshift,
                             gb.dscale, w.eps, workspace=gb.ws_mod, stream=stream)


def run_backward_chain(b: DeviceBatch, gb: GradBatch, stream=None):
    """One backward pass of the hot path (after run_chain on the same batch):
    gated residual -> attention -> modulate+RoPE."""
    run_gated_residual_bwd(b, gb, stream)
    run_attention_bwd(b, gb, stream)
    run_modulate_rope_bwd(b, gb, stream)


# ---------------------------------------------------------------------------
# Block projections around the attention
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class BlockBatch:
    x: object          # residual stream [T][C]
    w_qkv: object      # [3C][C]
    w_o: object        # [C][C]
    gate: object       # [n_rows][C]
    qkv: object        # [T][3C] output
    y: object          # [T][C] output
    workspace: object


def block_to_device(b: DeviceBatch, device="cuda") -> BlockBatch:
    """Seeded residual stream and random-init projection weights for b's workload."""
    import torch
    w = b.w
    T, C = w.T, w.H * w.D
    bi = workloads.block_inputs(w)
    gate = b.gate if b.gate is not None else torch.zeros((len(w.descs), C), dtype=torch.bfloat16, device=device)
    return BlockBatch(x=bf16_tensor(bi["x"], device), w_qkv=bf16_tensor(bi["w_qkv"], device),
                      w_o=bf16_tensor(bi["w_o"], device), gate=gate,
                      qkv=torch.empty((T, 3 * C), dtype=torch.bfloat16, device=device),
                      y=torch.empty((T, C), dtype=torch.bfloat16, device=device),
                      workspace=torch.empty(native.block_qkv_workspace_bytes(T, w.H, w.D), dtype=torch.uint8,
                                            device=device))


def run_block_qkv(b: DeviceBatch, bb: BlockBatch, stream=None):
    w = b.w
    native.block_qkv(bb.x, bb.w_qkv, bb.qkv, b.pos, w.H, w.rope_dims, w.rope_base, b.shift, b.scale,
                     b.mod_row if b.shift is not None else None, w.eps, workspace=bb.workspace, stream=stream)


def run_block_out(b: DeviceBatch, bb: BlockBatch, stream=None):
    native.block_out(b.o.view(b.w.T, -1), bb.w_o, bb.x, bb.gate, b.mod_row, bb.y, stream=stream)
