"""The f16 operand scales of the HIP library, pinned on the CPU.

In f16 every Fourier operand plane p (the transformed input, dY and the
prepared weights) is multiplied by a power of two s_p before it is rounded to
binary16 (kF16Scale in the library's device code, stated in include/eqlin.h).
The claim: for any input with |z| <= M, |s_p plane_p(z)| <= M, so no finite
binary16 input can overflow an operand, and s_p is the largest power of two
that does this.  The planes are linear in z, so the largest |plane_p| over the
cube |z| <= 1 is reached at a vertex z in {-1, +1}^T: every vertex is checked,
with the planes computed by the oracle's own definitions (the DFT for the
cyclic groups, the irreducible representations for p4m).
"""
import itertools
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEVICE = os.path.join(ROOT, "group_circulant_linear_amd", "csrc", "eqlin_device.h")
HEADER = os.path.join(ROOT, "include", "eqlin.h")


def device_scales():
    """kF16Scale of every Grp specialisation in the device code, by group code."""
    text = open(DEVICE).read()
    out = {}
    for m in re.finditer(r"struct Grp<(\w+)>\s*\{(.*?)\n\};", text, re.S):
        code = {"4": 4, "8": 8, "kP4M": "p4m"}[m.group(1)]
        arr = re.search(r"kF16Scale\[kOrder\]\s*=\s*\{([^}]*)\}", m.group(2))
        out[code] = [float(v.strip().rstrip("f")) for v in arr.group(1).split(",")]
    return out


def planes(z, g):
    w = np.asarray(z, dtype=np.float64)[None, None, :]
    return (oracle.p4m_planes(w) if g == "p4m" else oracle.kept_planes(w))[0, 0]


@pytest.mark.parametrize("g", [4, 8, "p4m"])
def test_scales_are_the_largest_powers_of_two_that_bound_every_plane(g):
    scales = np.array(device_scales()[g])
    T = 8 if g == "p4m" else g
    assert len(scales) == T
    bound = np.zeros(T)
    for z in itertools.product((-1.0, 1.0), repeat=T):
        bound = np.maximum(bound, np.abs(planes(z, g)))
    # every scaled plane within max|z| ...
    assert np.all(scales * bound <= 1 + 1e-12), (scales, bound)
    # ... by the largest power of two
    assert np.all(np.log2(scales) == np.round(np.log2(scales)))
    assert np.all(2 * scales * bound > 1 + 1e-12), (scales, bound)


@pytest.mark.parametrize("g", [4, 8, "p4m"])
def test_products_of_an_output_plane_share_one_scale(g):
    # the epilogue multiplies output plane p by 1 / s_p^2: valid when every
    # product into plane p multiplies two operand planes of scale s_p
    text = open(DEVICE).read()
    name = {4: "4", 8: "8", "p4m": "kP4M"}[g]
    body = re.search(r"struct Grp<%s>\s*\{(.*?)\n\};" % name, text, re.S).group(1)
    scales = device_scales()[g]
    for lst in ("kFwd", "kDw"):
        m = re.search(lst + r"\[kProducts\]\s*=\s*\{(.*?)\};", body, re.S)
        if m is None:
            continue
        for out, a, b in re.findall(r"\{(\d+),\s*(\d+),\s*(\d+),\s*(?:true|false)\}", m.group(1)):
            assert scales[int(a)] == scales[int(b)] == scales[int(out)], (lst, out, a, b)


def test_header_states_the_device_scales():
    text = open(HEADER).read()
    scales = device_scales()
    frac = {0.25: "1/4", 0.5: "1/2", 0.125: "1/8"}
    for g, label in ((4, "T = 4"), (8, "T = 8"), ("p4m", "EQLIN_P4M")):
        line = re.search(r"f16 operand scales, %s:\s*\(([^)]*)\)" % re.escape(label), text)
        assert line, label
        assert [s.strip() for s in line.group(1).split(",")] == [frac[v] for v in scales[g]], label


def test_p4_scaled_route_in_float16_emulation_stays_finite():
    # an emulation of the f16 route at the top of the range: inputs whose
    # groups sum past 65504 give finite scaled operands and, after the
    # products in float64 and the inverse scale, the exact layer output
    s = np.array(device_scales()[4])
    rng = np.random.default_rng(0)
    X = (rng.uniform(3e4, 6e4, size=(16, 8, 4)) * rng.choice([-1.0, 1.0], size=(16, 8, 1))).astype(np.float16)
    w = (rng.uniform(-1, 1, size=(6, 8, 4)) / 32).astype(np.float16)
    Xh = oracle.kept_planes(X.astype(np.float64))
    assert np.max(np.abs(Xh)) > 65504                       # unscaled operands would overflow
    Xs = (Xh * s).astype(np.float16)
    Ws = (oracle.kept_planes(w.astype(np.float64)) * s).astype(np.float16)
    assert np.all(np.isfinite(Xs)) and np.all(np.isfinite(Ws))
    # planes back to the spectrum (the inverse scale), products per frequency, inverse DFT
    F = Xs.astype(np.float64) / s
    G = Ws.astype(np.float64) / s
    Xc = np.stack([F[..., 0], F[..., 2] + 1j * F[..., 3], F[..., 1], F[..., 2] - 1j * F[..., 3]], -1)
    Wc = np.stack([G[..., 0], G[..., 2] + 1j * G[..., 3], G[..., 1], G[..., 2] - 1j * G[..., 3]], -1)
    Yc = np.einsum("nck,dck->ndk", Xc, Wc)
    Y = np.fft.ifft(Yc, axis=-1).real.reshape(16, 24)
    ref = oracle.forward_direct(X.reshape(16, 32), w)
    assert np.max(np.abs(Y - ref)) / np.max(np.abs(ref)) < 3e-3
