"""Seeded synthetic packs for the packed varlen RoPE-attention path.

This module only draws inputs: per-sample descriptors and bf16 tensors.  It
holds none of the method's arithmetic (no tables, no normalisation, no
rotary embedding, no attention); both the fp64 oracle and the HIP path
consume exactly what it returns, so the two sides see the same bits.

Workload shapes follow the Mage-Flow pages:
  * 16x spatial downsampling of the latent grid, so a 1024x1024 image is a
    64x64 token grid (picx.dev summary, Methodology > Mage-VAE);
  * native resolutions from 512 to 2048 per side with aspect ratios up to
    4:1 (molayo1419.me post, key-features list, native-resolution item);
  * variable-length image and text sequences packed under a fixed token
    budget, packed CFG with conditional and unconditional sequences in one
    forward, and edit samples whose source and target latents are told apart
    by a frame coordinate (picx.dev summary, Methodology > Native-Resolution
    MMDiT).

A descriptor is a tuple
    (text_len, n_frames, grid_h, grid_w, mod_row_text, mod_row_image)
with the modulation row equal to the sample index for both modalities (one
adaLN row per packed sequence).

Random numbers: numpy PCG64 (``default_rng(seed)``).  Draw order is the
descriptors, then q, k, v, x, shift, scale, gate, shift2, scale2.  Normals are
drawn in float32, multiplied by their standard deviation and rounded to bf16
with round-to-nearest-even; tensors are returned as uint16 bf16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

Desc = Tuple[int, int, int, int, int, int]

ROPE_BASE = 10000.0
LN_EPS = 1e-6


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def sample_len(d: Desc) -> int:
    """Token count of one sample: its text plus every frame of its latent grid."""
    t, f, h, w = d[0], d[1], d[2], d[3]
    return int(t + f * h * w)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    descs: List[Desc]
    H: int
    D: int
    rope_dims: Tuple[int, int, int]      # (frame, row, col) dims per head
    modulate: bool                       # adaLN modulation before RoPE
    q: np.ndarray                        # uint16 bf16 bits [T][H][D]
    k: np.ndarray
    v: np.ndarray
    x: Optional[np.ndarray] = None       # residual stream [T][C]
    shift: Optional[np.ndarray] = None   # [n_rows][C]
    scale: Optional[np.ndarray] = None
    gate: Optional[np.ndarray] = None
    shift2: Optional[np.ndarray] = None
    scale2: Optional[np.ndarray] = None
    rope_base: float = ROPE_BASE
    eps: float = LN_EPS

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def C(self) -> int:
        return self.H * self.D

    @property
    def n_seq(self) -> int:
        return len(self.descs)

    @property
    def seq_lens(self) -> List[int]:
        return [sample_len(d) for d in self.descs]

    @property
    def sum_sq_len(self) -> int:
        return int(sum(L * L for L in self.seq_lens))

    def attn_flops(self) -> float:
        """QK^T plus PV multiply-adds counted as 2 flops each: 4 * d * H * sum L^2."""
        return 4.0 * self.D * self.H * self.sum_sq_len


def _normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return f32_to_bf16_bits(a)


def _draw_tensors(name, seed, rng, descs, H, D, rope_dims, modulate, with_residual,
                  qk_sigma=1.0) -> Workload:
    T = sum(sample_len(d) for d in descs)
    C = H * D
    n_rows = len(descs)
    q = _normal_bf16(rng, (T, H, D), qk_sigma)
    k = _normal_bf16(rng, (T, H, D), qk_sigma)
    v = _normal_bf16(rng, (T, H, D), 1.0)
    w = Workload(name=name, seed=seed, descs=list(descs), H=H, D=D,
                 rope_dims=tuple(rope_dims), modulate=modulate, q=q, k=k, v=v)
    if with_residual:
        w.x = _normal_bf16(rng, (T, C), 1.0)
    if modulate:
        w.shift = _normal_bf16(rng, (n_rows, C), 0.1)
        w.scale = _normal_bf16(rng, (n_rows, C), 0.1)
    if with_residual:
        w.gate = _normal_bf16(rng, (n_rows, C), 0.1)
        w.shift2 = _normal_bf16(rng, (n_rows, C), 0.1)
        w.scale2 = _normal_bf16(rng, (n_rows, C), 0.1)
    return w


def _desc(s: int, text: int, frames: int, h: int, w: int) -> Desc:
    return (int(text), int(frames), int(h), int(w), int(s), int(s))


# ---------------------------------------------------------------------------
# Descriptor recipes
# ---------------------------------------------------------------------------

def descs_tiny() -> List[Desc]:
    """Two samples: 8 text + 4x6 latent grid, and 5 text + 8x4 grid (rows x cols)."""
    return [_desc(0, 8, 1, 4, 6), _desc(1, 5, 1, 8, 4)]


def descs_1024() -> List[Desc]:
    """One 1024x1024 image: 256 text tokens and a 64x64 latent grid."""
    return [_desc(0, 256, 1, 64, 64)]


def descs_native_budget(rng: np.random.Generator, budget: int = 16384) -> List[Desc]:
    """Native-resolution training pack filled up to a token budget.

    Image sides are drawn independently from {512, 528, ..., 2048} (latent
    side 32..128, so aspect ratios stay within 4:1) and text length from
    U{32..512}.  A drawn sample is appended when it fits the remaining budget
    and rejected otherwise; filling stops once the remaining budget is below
    the smallest possible sample (32 text + 32x32 latents) or after 100
    rejections in a row.
    """
    out: List[Desc] = []
    used = 0
    rejects = 0
    smallest = 32 + 32 * 32
    while budget - used >= smallest and rejects < 100:
        h = int(rng.integers(32, 129))
        w = int(rng.integers(32, 129))
        t = int(rng.integers(32, 513))
        L = t + h * w
        if used + L <= budget:
            out.append(_desc(len(out), t, 1, h, w))
            used += L
            rejects = 0
        else:
            rejects += 1
    return out


def descs_cfg(rng: np.random.Generator, prompts: int = 4) -> List[Desc]:
    """Packed CFG at 1024^2: per prompt a conditional sequence (text U{64..512}
    plus 64x64 latents) followed by its unconditional one (16 text plus the
    same 64x64 latent grid)."""
    out: List[Desc] = []
    for _ in range(prompts):
        t = int(rng.integers(64, 513))
        out.append(_desc(len(out), t, 1, 64, 64))
        out.append(_desc(len(out), 16, 1, 64, 64))
    return out


def descs_edit(rng: np.random.Generator) -> List[Desc]:
    """Edit pack: two edit samples (text U{64..512}, source frame 0 and target
    frame 1 of 64x64 latents each) plus one 2048x2048 generation sample (512
    text + 128x128 latents at frame 0)."""
    out: List[Desc] = []
    for _ in range(2):
        t = int(rng.integers(64, 513))
        out.append(_desc(len(out), t, 2, 64, 64))
    out.append(_desc(len(out), 512, 1, 128, 128))
    return out


def upstream_grads(w: Workload) -> dict:
    """Seeded stand-ins for the gradients a training loss sends back into the
    hot path: dO [T][H][D] (attention output), dy and dz [T][C] (residual
    stream and next adaLN output), dq and dk [T][H][D] (q', k' of the
    modulate+RoPE step), all N(0, 1) bf16 bits.  Drawn from their
    own generator (seed + 1000003), so the forward tensors of a workload do not
    change."""
    rng = np.random.default_rng(w.seed + 1000003)
    T, H, D = w.T, w.H, w.D
    g = dict(dO=_normal_bf16(rng, (T, H, D), 1.0), dy=_normal_bf16(rng, (T, H * D), 1.0),
             dz=_normal_bf16(rng, (T, H * D), 1.0))
    # gradients of the modulate+RoPE outputs q', k' (for that kernel alone)
    g["dq"] = _normal_bf16(rng, (T, H, D), 1.0)
    g["dk"] = _normal_bf16(rng, (T, H, D), 1.0)
    return g


def block_inputs(w: Workload) -> dict:
    """Seeded stand-ins for the block around the attention: the residual
    stream x [T][C] (the workload's own x when it has one, else N(0, 1)), the
    projection weights W_qkv [3C][C] and W_o [C][C] (output x input, as a
    random initialisation: N(0, 1/C) entries) -- there are no trained weights
    here.  bf16 bits from their own generator (seed + 2000003)."""
    rng = np.random.default_rng(w.seed + 2000003)
    T, C = w.T, w.H * w.D
    x = w.x if w.x is not None else _normal_bf16(rng, (T, C), 1.0)
    sig = 1.0 / np.sqrt(C)
    return dict(x=x, w_qkv=_normal_bf16(rng, (3 * C, C), sig), w_o=_normal_bf16(rng, (C, C), sig))


LATENT_CHANNELS = 128   # Mage-VAE latents: 16x downsampling, 128 channels per token


def cfg_prompts(w: Workload) -> Tuple[List[int], List[int]]:
    """(cond, uncond) sample indices of a packed-CFG workload: the packs here
    place each prompt's conditional sample right before its unconditional one."""
    n = len(w.descs)
    return list(range(0, n - 1, 2)), list(range(1, n, 2))


def sampler_inputs(w: Workload, n_tokens: int, Cl: int = LATENT_CHANNELS) -> dict:
    """Seeded stand-ins for one sampler step: the model's velocity output for
    every packed token v [T][Cl] (N(0, 1), bf16 bits) and the fp32 latent
    state of the n_tokens evolving tokens z [N][Cl] (N(0, 1)); own generator
    (seed + 3000003)."""
    rng = np.random.default_rng(w.seed + 3000003)
    v = _normal_bf16(rng, (w.T, Cl), 1.0)
    z = rng.standard_normal((n_tokens, Cl)).astype(np.float32)
    return dict(v=v, z=z)


@dataclasses.dataclass
class TextPack:
    """Packed prompts for the text-encoder variant (bf16 bit patterns)."""
    name: str
    seed: int
    lens: List[int]
    Hq: int
    Hkv: int
    D: int
    q: np.ndarray       # [T][Hq][D]
    k: np.ndarray       # [T][Hkv][D]
    v: np.ndarray       # [T][Hkv][D]
    wq: np.ndarray      # [D] per-head norm weights
    wk: np.ndarray
    rope_base: float = ROPE_BASE
    eps: float = LN_EPS

    @property
    def T(self) -> int:
        return int(sum(self.lens))

    def causal_flops(self) -> float:
        """QK^T and PV over the unmasked pairs: 4 * D * Hq * sum L (L + 1) / 2."""
        return 4.0 * self.D * self.Hq * sum(L * (L + 1) / 2 for L in self.lens)


TEXT_BENCH_SEED = 1006
TEXT_BENCH_PROMPTS = 64


def text_pack(seed: int = 1005, n_prompts: int = 16, Hq: int = 32, Hkv: int = 8, D: int = 128,
              lens: Optional[Sequence[int]] = None, name: str = "text_pack") -> TextPack:
    """Packed prompts: lengths U{64..512} (the prompt lengths of the packed
    CFG workload), q, k, v ~ N(0, 1), norm weights 1 + N(0, 0.1); default
    heads 32 query / 8 key-value of 128 dims."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = [int(x) for x in rng.integers(64, 513, size=n_prompts)]
    T = int(sum(lens))
    q = _normal_bf16(rng, (T, Hq, D), 1.0)
    k = _normal_bf16(rng, (T, Hkv, D), 1.0)
    v = _normal_bf16(rng, (T, Hkv, D), 1.0)
    wq = f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    wk = f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    return TextPack(name, seed, list(lens), Hq, Hkv, D, q, k, v, wq, wk)


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

def tiny(seed: int = 1000) -> Workload:
    """Tiny pack, H=2, d=64, 2D RoPE split (0, 32, 32), no modulation."""
    rng = np.random.default_rng(seed)
    descs = descs_tiny()
    return _draw_tensors("tiny", seed, rng, descs, 2, 64, (0, 32, 32), False, False)


def tiny_mod(seed: int = 1001) -> Workload:
    """The tiny pack with modulation, residual stream and gates present."""
    rng = np.random.default_rng(seed)
    descs = descs_tiny()
    return _draw_tensors("tiny_mod", seed, rng, descs, 2, 64, (0, 32, 32), True, True)


def single_1024(seed: int = 1002) -> Workload:
    """Single 1024x1024 sample: 256 + 64x64 tokens, H=24, d=128."""
    rng = np.random.default_rng(seed)
    descs = descs_1024()
    return _draw_tensors("single_1024", seed, rng, descs, 24, 128, (0, 64, 64), True, True)


def native_pack(seed: int = 2000, budget: int = 16384) -> Workload:
    """Native-resolution pack under a 16384-token budget, H=24, d=128."""
    rng = np.random.default_rng(seed)
    descs = descs_native_budget(rng, budget)
    return _draw_tensors(f"native_pack_{seed}", seed, rng, descs, 24, 128, (0, 64, 64), True, True)


CFG_SEED = 1003


def cfg_pack(seed: int = CFG_SEED) -> Workload:
    """Packed CFG inference at 1024^2: 8 sequences, H=24, d=128."""
    rng = np.random.default_rng(seed)
    descs = descs_cfg(rng)
    return _draw_tensors("cfg_pack", seed, rng, descs, 24, 128, (0, 64, 64), True, True)


def edit_pack(seed: int = 1004) -> Workload:
    """Edit pack with 3D RoPE split (16, 56, 56), H=24, d=128."""
    rng = np.random.default_rng(seed)
    descs = descs_edit(rng)
    return _draw_tensors("edit_pack", seed, rng, descs, 24, 128, (16, 56, 56), True, True)


@dataclasses.dataclass
class Shape:
    """A workload's shape without its tensors: descriptors and parameters."""
    name: str
    seed: int
    descs: List[Desc]
    H: int
    D: int
    rope_dims: Tuple[int, int, int]
    modulate: bool
    residual: bool
    rope_base: float = ROPE_BASE
    eps: float = LN_EPS

    @property
    def T(self) -> int:
        return int(sum(sample_len(d) for d in self.descs))

    @property
    def C(self) -> int:
        return self.H * self.D

    @property
    def n_seq(self) -> int:
        return len(self.descs)

    @property
    def sum_sq_len(self) -> int:
        return int(sum(sample_len(d) ** 2 for d in self.descs))

    def attn_flops(self) -> float:
        return 4.0 * self.D * self.H * self.sum_sq_len


def shapes_of_configs() -> List[Shape]:
    """The measured configurations other than the 1024^2 pack, with the same
    seeded descriptor draws as their named workloads: the tiny pack, the
    eight native-resolution budget packs (seeds 2000..2007), packed CFG and
    the edit pack with 3D RoPE."""
    out = [Shape("tiny", 1000, descs_tiny(), 2, 64, (0, 32, 32), False, False)]
    for seed in range(2000, 2008):
        out.append(Shape(f"native_pack_{seed}", seed, descs_native_budget(np.random.default_rng(seed)),
                         24, 128, (0, 64, 64), True, True))
    out.append(Shape("cfg_pack", CFG_SEED, descs_cfg(np.random.default_rng(CFG_SEED)), 24, 128, (0, 64, 64),
                     True, True))
    out.append(Shape("edit_pack", 1004, descs_edit(np.random.default_rng(1004)), 24, 128, (16, 56, 56),
                     True, True))
    return out


def custom(descs: Sequence[Desc], H: int, D: int, rope_dims=(0, 0, 0), modulate=False,
           residual=False, seed: int = 0, qk_sigma: float = 1.0, name: str = "custom") -> Workload:
    """Arbitrary descriptor list (edge cases, stress packs)."""
    rng = np.random.default_rng(seed)
    if rope_dims == (0, 0, 0):
        rope_dims = (0, D // 2, D // 2)
    return _draw_tensors(name, seed, rng, list(descs), H, D, rope_dims, modulate, residual,
                         qk_sigma=qk_sigma)


def random_descs(rng: np.random.Generator, n_max: int = 4, max_text: int = 12,
                 max_side: int = 6, max_frames: int = 2) -> List[Desc]:
    """Small random descriptor lists for exhaustive table tests (empty grids and
    empty text allowed)."""
    n = int(rng.integers(1, n_max + 1))
    out = []
    for s in range(n):
        t = int(rng.integers(0, max_text + 1))
        f = int(rng.integers(1, max_frames + 1))
        h = int(rng.integers(0, max_side + 1))
        w = int(rng.integers(0, max_side + 1)) if h > 0 else 0
        mt = int(rng.integers(0, n + 1))
        mi = int(rng.integers(0, n + 1))
        out.append((t, f, h, w, mt, mi))
    return out


NAMED = {
    "tiny": tiny,
    "tiny_mod": tiny_mod,
    "single_1024": single_1024,
    "native_pack": native_pack,
    "cfg_pack": cfg_pack,
    "edit_pack": edit_pack,
}
