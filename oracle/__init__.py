"""Oracle for the packed varlen RoPE joint-attention forward.

TEST INFRASTRUCTURE ONLY: the fp64 numpy definition (``reference``) and a
pure-Python loop version for tiny packs (``brute``).  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import this package; the
HIP library and its binding never do, and this package imports nothing from
them.
"""
from . import brute, reference  # noqa: F401
