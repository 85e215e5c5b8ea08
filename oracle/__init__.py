"""Oracle for the packed varlen RoPE joint-attention forward.

TEST INFRASTRUCTURE ONLY: the fp64 numpy definition (``reference``), a
pure-Python loop version for tiny packs (``brute``), the block projections
around the attention (``block``), the packed-CFG sampler step (``sampler``)
the text-encoder variant (``text_encoder``) and the exact gradients of
the forward steps for the backward pass (``backward``).  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import this package; the
HIP library and its binding never do, and this package imports nothing from
them.
"""
from . import backward, block, brute, reference, sampler, text_encoder  # noqa: F401
