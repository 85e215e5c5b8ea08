"""Packed varlen RoPE joint-attention forward for MI355X (gfx950).

The hot path is a C-ABI library, libmf.so (include/mf.h), built from the
HIP kernels under csrc/; ``native`` is its ctypes binding and ``workloads``
draws the seeded synthetic packs.  Importing the package loads nothing; the
first binding call loads libmf.so and fails loudly if it is not built.
"""
from . import native, workloads  # noqa: F401
from .native import (MFError, attn_workspace_bytes, gated_residual, modulate_rope,  # noqa: F401
                     pack_count, pack_tables, varlen_attn_fwd)
