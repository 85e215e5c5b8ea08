"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import math
import sys

import numpy as np

from packed_attention_amd import runner
from packed_attention_amd.workloads import bf16_bits_to_f64

# Bar on bf16 outputs against the fp64 oracle (max-abs, mean-abs), plus the
# stricter internal checks on the attention output.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
O_REL_RMS = 1e-2
LSE_ABS = 1e-3
# End to end the kernel attends over bf16-rounded q', k' while the oracle keeps
# them in fp64: each score moves by about scale * sqrt(d) * 2^-9 * |q||k| / sqrt(3)
# (~2e-3 at d=128 with unit rows), and the LSE by at most the largest score shift.
LSE_ABS_E2E = 2e-2


def say(*a):
    """Name the case before each GPU step, flushed, so a failing run tells which."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def f64(t) -> np.ndarray:
    return runner.bf16_to_f64(t)


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_bar(got: np.ndarray, ref: np.ndarray, name: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - ref)
    assert err.max() <= max_abs, f"{name}: max-abs {err.max():.3e} > {max_abs}"
    assert err.mean() <= mean_abs, f"{name}: mean-abs {err.mean():.3e} > {mean_abs}"
    return float(err.max()), float(err.mean())


def check_rounded(got: np.ndarray, ref: np.ndarray, name: str, slack=1e-6):
    """Elementwise kernels compute in fp32 and round once to bf16: every
    output is within one bf16 ulp of the exact value (half an ulp from the
    rounding, the rest from fp32 arithmetic near a rounding boundary)."""
    err = np.abs(got - ref)
    lim = bf16_ulp(ref) + slack
    bad = err > lim
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements beyond one bf16 ulp; worst err "
                           f"{err[bad].max():.3e} at ref {ref[bad][np.argmax(err[bad])]:.4e}")


def check_attention(got_O: np.ndarray, ref_O: np.ndarray, name: str, got_lse=None, ref_lse=None,
                    lse_abs=LSE_ABS):
    check_bar(got_O, ref_O, name + ".O")
    rel = np.linalg.norm(got_O - ref_O) / max(np.linalg.norm(ref_O), 1e-30)
    assert rel <= O_REL_RMS, f"{name}: O relative RMS {rel:.3e}"
    if got_lse is not None:
        e = np.abs(got_lse - ref_lse).max()
        assert e <= lse_abs, f"{name}: LSE max-abs {e:.3e}"


def wl_f64(w):
    f = bf16_bits_to_f64
    g = lambda a: None if a is None else f(a)  # noqa: E731
    return dict(q=f(w.q), k=f(w.k), v=f(w.v), x=g(w.x), shift=g(w.shift), scale=g(w.scale),
                gate=g(w.gate), shift2=g(w.shift2), scale2=g(w.scale2))


def softmax_scale(w):
    return 1.0 / math.sqrt(w.D)
