"""Seeded synthetic workloads for the DCNv4 forward operator.

This module only draws random inputs of the shapes, value distributions and
dtypes of the pages' workloads.  It holds none of the operator's arithmetic:
the output size (Ho, Wo) is passed in by the caller, who takes it from the
library under test or from the oracle.

Inputs stand in for the pages' workloads (no dataset or trained weights are
used): InternImage-like stages and latent-diffusion U-Net blocks
([DCNv4 digest] = CSDN "（论文速读）DCNv4：高效可变形卷积算子", abstract; the
U-Net tutorial at framerc.cn "从ConvNet到Diffusion：手把手把DCNv4塞进Stable
Diffusion的U-Net里试试效果", section 2.2, for the 1280-channel blocks) and
FlowDCN tokens ([FlowDCN] = kler.cn "NeurIPS'24 | FlowDCN：基于可变形卷积的任意
分辨率图像生成模型", section 3.1, per-group scale priors).

Recipe (every workload): draws in float32 from numpy's PCG64 seeded with the
workload seed, in the order input, offsets, weights (then, for FlowDCN's
predicted scales, the per-pixel scales); x ~ N(0,1); weights m ~ N(0, 1/9)
(standard deviation 1/3); offsets per workload (uniform U[-a,a] or normal with
the given variance); values are then rounded to the I/O dtype with
round-to-nearest-even (torch's CPU cast for bf16, numpy's for fp16).  Group
scale priors and predicted per-pixel scales stay fp32; the predicted scales
are U[lo, hi] (the pages give no distribution: a band around 1, so that with
the clamp Smax some groups of every pixel hit the maximum).
The offset/weight tensor om has layout [N,Ho,Wo,G,3K]: per group the K
interleaved (dx, dy) pairs first, then the K weights.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" | "bf16" | "f16": input, om and output
    N: int
    H: int
    W: int
    C: int
    G: int
    kh: int = 3
    kw: int = 3
    sh: int = 1
    sw: int = 1
    ph: int = 1
    pw: int = 1
    dh: int = 1
    dw: int = 1
    offset_scale: float = 1.0
    multiscale: bool = False
    offset_dist: str = "uniform"   # "uniform": U[-a,a]; "normal": N(0, a)
    offset_param: float = 2.0      # a (half-width, or variance)
    seed: int = 0
    pixel_scales: bool = False     # FlowDCN predicted scale per (pixel, group)
    pixel_scale_range: tuple = (0.5, 1.5)
    max_scale: float = 0.0         # > 0: Smax clamp of the effective scale

    @property
    def K(self) -> int:
        return self.kh * self.kw

    @property
    def D(self) -> int:
        return self.C // self.G

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def describe(self) -> str:
        off = (f"U[-{self.offset_param:g},{self.offset_param:g}]"
               if self.offset_dist == "uniform"
               else f"N(0,{self.offset_param:g})")
        mode = "multi-scale" if self.multiscale else "standard"
        if self.pixel_scales:
            lo, hi = self.pixel_scale_range
            mode += f" pixel scales U[{lo:g},{hi:g}] Smax {self.max_scale:g}"
        return (f"{self.name}: {self.dtype} N={self.N} {self.H}x{self.W} "
                f"C={self.C} G={self.G} k={self.kh}x{self.kw} "
                f"s={self.sh},{self.sw} p={self.ph},{self.pw} "
                f"d={self.dh},{self.dw} {mode} offsets {off} seed {self.seed}")


# The pages' workloads, at their full sizes.
WORKLOADS = {
    # tiny fp32 case: 1x16x16x64, 4 groups of 16 channels
    "dcn4_small_f32": Workload("dcn4_small_f32", "f32", 1, 16, 16, 64, 4,
                               offset_dist="uniform", offset_param=2.0),
    # InternImage-stage-like: 64 images of 56x56x64, 4 groups
    "internimage_stage_f32": Workload("internimage_stage_f32", "f32", 64, 56,
                                      56, 64, 4, offset_dist="uniform",
                                      offset_param=3.0),
    "internimage_stage_bf16": Workload("internimage_stage_bf16", "bf16", 64,
                                       56, 56, 64, 4, offset_dist="uniform",
                                       offset_param=3.0),
    # latent-diffusion U-Net block: 8 x 128x128x320, 20 groups of 16
    "ldm_unet_block_bf16": Workload("ldm_unet_block_bf16", "bf16", 8, 128,
                                    128, 320, 20, offset_dist="normal",
                                    offset_param=2.0),
    # wide low-resolution block, dilation 2: 16 x 32x32x1280, 40 groups of 32
    "wide_lowres_dil2_f16": Workload("wide_lowres_dil2_f16", "f16", 16, 32,
                                     32, 1280, 40, dh=2, dw=2,
                                     offset_dist="uniform", offset_param=8.0),
    # FlowDCN groupwise multi-scale: 32 x 32x32 tokens x 1152, 16 groups of 72
    "flowdcn_multiscale_bf16": Workload("flowdcn_multiscale_bf16", "bf16", 32,
                                        32, 32, 1152, 16, multiscale=True,
                                        offset_dist="uniform",
                                        offset_param=1.0),
    # the same tokens with FlowDCN's predicted per-pixel scale times the group
    # prior and the maximum scale Smax = 4 (the largest prior)
    "flowdcn_pixelscale_bf16": Workload("flowdcn_pixelscale_bf16", "bf16", 32,
                                        32, 32, 1152, 16, multiscale=True,
                                        offset_dist="uniform", offset_param=1.0,
                                        pixel_scales=True, max_scale=4.0),
}

# The workload the headline throughput is quoted on.
HEADLINE = "ldm_unet_block_bf16"


def to_raw(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> raw storage of the I/O dtype (round to nearest even).
    f32 stays float32; bf16 and f16 become uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(a).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def from_raw(a: np.ndarray, dtype: str) -> np.ndarray:
    """raw storage -> float32 values (exact)."""
    if dtype == "f32":
        return np.asarray(a, np.float32)
    if dtype == "f16":
        return np.asarray(a, np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def group_scales(G: int) -> np.ndarray:
    """FlowDCN per-group scale priors, log-spaced from 1 to 4:
    s_g = 4**(g/(G-1)) evaluated in float64, stored as float32."""
    if G == 1:
        return np.ones(1, np.float32)
    g = np.arange(G, dtype=np.float64)
    return (4.0 ** (g / (G - 1))).astype(np.float32)


@dataclass
class Inputs:
    x: np.ndarray                 # raw [N,H,W,C]
    om: np.ndarray                # raw [N,Ho,Wo,G,3K]
    scales: Optional[np.ndarray]  # float32 [G] or None
    pscales: Optional[np.ndarray] = None  # float32 [N,Ho,Wo,G] or None


def make_inputs(w: Workload, Ho: int, Wo: int, seed: Optional[int] = None,
                n_images: Optional[int] = None) -> Inputs:
    """Draw one batch of the workload.  ``seed`` overrides the workload seed
    and ``n_images`` the batch size (a smaller batch drawn with the same
    recipe, not a slice of the full batch)."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    N = w.N if n_images is None else n_images
    K, G = w.K, w.G
    x = rng.standard_normal((N, w.H, w.W, w.C), dtype=np.float32)
    if w.offset_dist == "uniform":
        a = np.float32(w.offset_param)
        off = rng.random((N, Ho, Wo, G, 2 * K), dtype=np.float32) * (2 * a) - a
    elif w.offset_dist == "normal":
        sd = np.float32(np.sqrt(w.offset_param))
        off = rng.standard_normal((N, Ho, Wo, G, 2 * K), dtype=np.float32) * sd
    else:
        raise ValueError(w.offset_dist)
    m = rng.standard_normal((N, Ho, Wo, G, K), dtype=np.float32) * np.float32(1.0 / 3.0)
    om = np.concatenate([off, m], axis=-1)
    scales = group_scales(G) if w.multiscale else None
    pscales = None
    if w.pixel_scales:
        lo, hi = (np.float32(v) for v in w.pixel_scale_range)
        pscales = rng.random((N, Ho, Wo, G), dtype=np.float32) * (hi - lo) + lo
    return Inputs(to_raw(x, w.dtype), to_raw(om, w.dtype), scales, pscales)


def make_linear_inputs(M: int, Cin: int, Nout: int, dtype: str, seed: int = 7,
                       with_bias: bool = True):
    """Inputs of the merged offset/weight layer: features ~ N(0, 1) (a
    normalised token), weights ~ N(0, 1/Cin) so every output has unit
    variance, bias ~ N(0, 0.25) in fp32.  Returns raw feat [M, Cin], raw
    weight [Nout, Cin] in the I/O dtype and the fp32 bias (or None)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    feat = rng.standard_normal((M, Cin), dtype=np.float32)
    weight = rng.standard_normal((Nout, Cin), dtype=np.float32) * np.float32(1.0 / np.sqrt(Cin))
    bias = (rng.standard_normal(Nout, dtype=np.float32) * np.float32(0.5)) if with_bias else None
    return to_raw(feat, dtype), to_raw(weight, dtype), bias
