"""Seeded synthetic inputs for the p4 EQ-Linear workloads.

This module draws random numbers and casts them to the storage dtype; it holds
none of the layer's arithmetic.  The same arrays feed both the HIP library and
the fp64 oracle, so a parity comparison never depends on how they were drawn.

Workloads stand in for the ViT-B / ViT-H layers that the Flash EQ-Linear
summary evaluates (gist.science 2607.21271, "Network-level results"): token
counts are batch x (patches + 1), 197 = 14*14 + 1 and 257 = 16*16 + 1.  The
"narrow" workload (16 group channels over 16 ViT-B batches of tokens) is the
small-width regime, where the layer moves far more bytes than it multiplies
and HBM bandwidth rather than the matrix cores bounds it.
No dataset or trained weight is involved: X ~ N(0, 1), dY ~ N(0, 1) and the
circulant vectors w ~ N(0, 1/C), C being the layer's full input width.

Recipe: numpy.random.default_rng(seed) (PCG64) with seed = [base_seed, layer],
draws in the order X, w, dY as float64 standard normals, scaled, then cast
round-to-nearest-even to the storage dtype.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

T_P4 = 4


@dataclass(frozen=True)
class Layer:
    name: str
    N: int
    C: int
    D: int


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    dtypes: tuple
    layers: tuple = field(default_factory=tuple)
    backward: bool = False


WORKLOADS = {
    "tiny": Workload(
        "tiny", "tiny p4 EQ-Linear, N=64, C=D=32 (8 group channels in and out)",
        ("f32",), (Layer("tiny", 64, 32, 32),)),
    "vitb_attn": Workload(
        "vitb_attn", "ViT-B-shaped attention projection, N=64*197=12608, C=D=768",
        ("f32",), (Layer("attn", 12608, 768, 768),)),
    "vitb_mlp": Workload(
        "vitb_mlp", "ViT-B-shaped MLP pair, N=12608, fc1 768->3072 and fc2 3072->768",
        ("f16",), (Layer("fc1", 12608, 768, 3072), Layer("fc2", 12608, 3072, 768))),
    "vith_mlp": Workload(
        "vith_mlp", "ViT-H-shaped MLP pair, N=32*257=8224, fc1 1280->5120 and fc2 5120->1280",
        ("f32", "f16"), (Layer("fc1", 8224, 1280, 5120), Layer("fc2", 8224, 5120, 1280))),
    "narrow": Workload(
        "narrow", "narrow p4 EQ-Linear over many rows, N=16*12608=201728, C=D=64 (16 group channels in and out)",
        ("f32", "f16"), (Layer("narrow", 201728, 64, 64),)),
    "vitb_attn_bwd": Workload(
        "vitb_attn_bwd", "backward of the ViT-B attention projection shapes (dX and dw)",
        ("f16", "f32"), (Layer("attn", 12608, 768, 768),), backward=True),
}

NP_DTYPE = {"f32": np.float32, "f16": np.float16}


def make_layer_inputs(N: int, C: int, D: int, dtype: str = "f32", seed: int = 0,
                      layer: int = 0, T: int = T_P4, with_dy: bool = True):
    """Return (X [N][C], w [D/T][C/T][T], dY [N][D] or None) in the storage dtype."""
    if C % T or D % T:
        raise ValueError("C and D must be multiples of T")
    rng = np.random.default_rng([seed, layer])
    npdt = NP_DTYPE[dtype]
    X = rng.standard_normal((N, C)).astype(npdt)
    w = (rng.standard_normal((D // T, C // T, T)) / np.sqrt(C)).astype(npdt)
    dY = rng.standard_normal((N, D)).astype(npdt) if with_dy else None
    return X, w, dY


# f16 range cases: values at the top of binary16 (|x| in [3e4, 6e4], the
# largest finite value being 65504) and just above its smallest normal
# (|x| in [2^-14, 2^-12]).  Within every group of T channels of the first
# half of the group channels all T values share one sign, so that a sum of
# the T values (the zero frequency of a group transform) reaches T max|x|;
# the other half draw their signs independently.  Weights are scaled so that
# the exact outputs stay finite in binary16: large regime w ~ U(-1, 1) /
# max(C, D) (every output is a sum of at most max(C, D) terms of |w x| <
# 6e4 / max(C, D)), small regime w ~ U(-1, 1).
RANGE_REGIMES = {"large": (3.0e4, 6.0e4), "small": (2.0 ** -14, 2.0 ** -12)}


def _range_values(rng, shape, T, lo, hi):
    mag = rng.uniform(lo, hi, size=shape)
    n, cg = shape[0], shape[1] // T
    sign = rng.choice([-1.0, 1.0], size=shape).reshape(n, cg, T)
    coherent = rng.choice([-1.0, 1.0], size=(n, cg, 1))
    sign[:, : cg // 2, :] = coherent[:, : cg // 2, :]
    return mag * sign.reshape(shape)


def make_range_inputs(N: int, C: int, D: int, regime: str, seed: int = 0, T: int = T_P4):
    """f16 (X [N][C], w [D/T][C/T][T], dY [N][D]) at one end of the binary16 range (RANGE_REGIMES)."""
    if C % T or D % T:
        raise ValueError("C and D must be multiples of T")
    lo, hi = RANGE_REGIMES[regime]
    rng = np.random.default_rng([seed, 7])
    X = _range_values(rng, (N, C), T, lo, hi).astype(np.float16)
    wscale = 1.0 / max(C, D) if regime == "large" else 1.0
    w = (rng.uniform(-1.0, 1.0, size=(D // T, C // T, T)) * wscale).astype(np.float16)
    dY = _range_values(rng, (N, D), T, lo, hi).astype(np.float16)
    return X, w, dY


def workload_inputs(name: str, dtype: str | None = None, seed: int = 0, with_dy: bool = True):
    """Inputs for every layer of a named workload: list of (Layer, X, w, dY)."""
    wl = WORKLOADS[name]
    dt = dtype or wl.dtypes[0]
    out = []
    for i, L in enumerate(wl.layers):
        X, w, dY = make_layer_inputs(L.N, L.C, L.D, dt, seed=seed, layer=i, with_dy=with_dy)
        out.append((L, X, w, dY))
    return out


# ------------------------------------------------------------ p4 group convolution
#
# The summary names equivariant convolution as future work ("Limitations and
# future work") and measures none, so its workload is a stand-in: one 3 x 3
# p4 group convolution of a ResNet-stage shape, 32 images of 56 x 56 pixels,
# C = D = 256 channels (64 group channels x 4 rotations).
# Recipe: default_rng([seed, layer]), draws in the order X, psi, dY as float64
# standard normals, psi scaled by 1/sqrt(C K^2) (a dense conv's fan-in), cast
# round-to-nearest-even to the storage dtype.

@dataclass(frozen=True)
class ConvLayer:
    name: str
    N: int
    H: int
    W: int
    C: int
    D: int
    K: int


CONV_WORKLOADS = {
    "p4conv": Workload(
        "p4conv", "p4 group convolution 3x3, 32 images of 56x56, C=D=256 (64 group channels in and out)",
        ("f32", "f16"), (ConvLayer("conv3x3", 32, 56, 56, 256, 256, 3),)),
    "p4conv_tiny": Workload(
        "p4conv_tiny", "tiny p4 group convolution 3x3, 2 images of 8x8, C=D=16",
        ("f32",), (ConvLayer("tiny", 2, 8, 8, 16, 16, 3),)),
}


def make_conv_inputs(N: int, H: int, W: int, C: int, D: int, K: int, dtype: str = "f32", seed: int = 0,
                     layer: int = 0, with_dy: bool = True):
    """Return (X [N][H][W][C], psi [D/4][C/4][K][K][4], dY [N][H][W][D] or None) in the storage dtype."""
    if C % 4 or D % 4:
        raise ValueError("C and D must be multiples of 4")
    rng = np.random.default_rng([seed, layer])
    npdt = NP_DTYPE[dtype]
    X = rng.standard_normal((N, H, W, C)).astype(npdt)
    psi = (rng.standard_normal((D // 4, C // 4, K, K, 4)) / np.sqrt(C * K * K)).astype(npdt)
    dY = rng.standard_normal((N, H, W, D)).astype(npdt) if with_dy else None
    return X, psi, dY


def make_conv_range_inputs(N: int, H: int, W: int, C: int, D: int, K: int, regime: str, seed: int = 0):
    """f16 (X [N][H][W][C], psi [D/4][C/4][K][K][4], dY [N][H][W][D]) at one end of the binary16
    range, drawn as make_range_inputs draws a layer over the N H W pixels (equal-sign groups of
    rotations in the first half of the group channels); psi ~ U(-1, 1) / max(C K^2, D K^2) in the
    large regime (every output a sum of at most that many terms), U(-1, 1) in the small one."""
    if C % 4 or D % 4:
        raise ValueError("C and D must be multiples of 4")
    lo, hi = RANGE_REGIMES[regime]
    rng = np.random.default_rng([seed, 8])
    P = N * H * W
    X = _range_values(rng, (P, C), 4, lo, hi).astype(np.float16).reshape(N, H, W, C)
    scale = 1.0 / (max(C, D) * K * K) if regime == "large" else 1.0
    psi = (rng.uniform(-1.0, 1.0, size=(D // 4, C // 4, K, K, 4)) * scale).astype(np.float16)
    dY = _range_values(rng, (P, D), 4, lo, hi).astype(np.float16).reshape(N, H, W, D)
    return X, psi, dY
