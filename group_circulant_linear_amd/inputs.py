"""Seeded synthetic inputs for the p4 EQ-Linear workloads.

This module draws random numbers and casts them to the storage dtype; it holds
none of the layer's arithmetic.  The same arrays feed both the HIP library and
the fp64 oracle, so a parity comparison never depends on how they were drawn.

Workloads stand in for the ViT-B / ViT-H layers that the Flash EQ-Linear
summary evaluates (gist.science 2607.21271, "Network-level results"): token
counts are batch x (patches + 1), 197 = 14*14 + 1 and 257 = 16*16 + 1.
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


def workload_inputs(name: str, dtype: str | None = None, seed: int = 0, with_dy: bool = True):
    """Inputs for every layer of a named workload: list of (Layer, X, w, dY)."""
    wl = WORKLOADS[name]
    dt = dtype or wl.dtypes[0]
    out = []
    for i, L in enumerate(wl.layers):
        X, w, dY = make_layer_inputs(L.N, L.C, L.D, dt, seed=seed, layer=i, with_dy=with_dy)
        out.append((L, X, w, dY))
    return out
