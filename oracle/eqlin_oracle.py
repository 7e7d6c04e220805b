"""fp64 CPU oracle for the p4 group-circulant (EQ-)linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code, table or helper with the HIP
library; both sides receive the same arrays from a seeded generator that holds
none of the layer's arithmetic.

Source: "Technical summary: Flash EQ-Linear" (gist.science, arXiv 2607.21271),
sections "Key insight", "Algorithmic approach" (items 1-3), "Specialisation for
the p4 rotation group" and "Main contributions" (item 2).

What the layer computes (plain definition, no Fourier tricks)
-------------------------------------------------------------
The page ("Key insight") states that the EQ-Linear weight is group-circulant:
it is built by cyclically shifting and replicating a learnable parameter set,
so the layer is a circular convolution along the group axis combined with a
linear map along the channel axis.  With group size T, C = C'*T input and
D = D'*T output channels, channel index = group_channel*T + group_element
(group element fastest), and learnable w[d', c', u] (u = 0..T-1):

    W[d'T + t, c'T + s] = w[d', c', (t - s) mod T]
    Y = X W^T,   i.e.   Y[n, d'T+t] = sum_{c', s} w[d', c', (t-s) mod T] X[n, c'T+s]

The page only says "cyclically shifting"; the orientation (t - s) is a
reading (the opposite orientation conjugates the weight spectrum and is the
transpose pass used for dX below).  The Fourier algorithm the page describes is
exact (DFT invertibility + convolution theorem, "Main contributions" item 2),
so the oracle is the plain definition above, not the Fourier algorithm.

Backward pass (plain calculus on the same definition):
    dX = dY W                      (transposed group-circulant)
    dw[d', c', u] = sum_n sum_t dY[n, d'T+t] X[n, c'T + (t-u) mod T]

Every routine here is T-generic and runs in float64 with NumPy.  The only
library primitive used as a step is a dense matrix product.

The group spectrum routine (``group_spectrum``) is the plain DFT definition
F[k] = sum_u z[u] exp(-2 pi i k u / T) along the group axis, used to check the
prepared weight planes ("Algorithmic approach" item 1, conjugate symmetry in
item 2, p4 specialisation).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "forward_bias_act",
    "gelu_erf",
    "dense_expand",
    "forward_direct",
    "backward_direct",
    "dx_direct",
    "dw_direct",
    "group_spectrum",
    "kept_p4_planes",
    "kept_planes",
    "forward_rows",
    "dw_entries",
    "cyclic_table",
    "p4m_table",
    "p4m_irreps",
    "dense_expand_group",
    "forward_group",
    "dx_group",
    "dw_group",
    "p4m_planes",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _split_groups(A: np.ndarray, T: int) -> np.ndarray:
    """[rows][G*T] -> [rows][G][T] (group element fastest)."""
    rows, width = A.shape
    if width % T:
        raise ValueError(f"width {width} is not a multiple of T={T}")
    return A.reshape(rows, width // T, T)


def dense_expand(w) -> np.ndarray:
    """Dense D x C weight of the group-circulant layer ("Key insight").

    W[d'T + t, c'T + s] = w[d', c', (t - s) mod T], built entry by entry from
    the definition with explicit index arithmetic.
    """
    w = _f64(w)
    Dp, Cp, T = w.shape
    W = np.empty((Dp * T, Cp * T), dtype=np.float64)
    for t in range(T):
        for s in range(T):
            W[t::T, s::T] = w[:, :, (t - s) % T]
    return W


def forward_direct(X, w) -> np.ndarray:
    """Y = X W^T by the direct circular-convolution formula ("Key insight").

    Y3[n, d', t] = sum_u sum_c' w[d', c', u] * X3[n, c', (t - u) mod T]
    (u = t - s).  For each shift u this is one dense contraction over c'
    against the group-rolled input X3[..., (t-u) mod T] = roll(X3, u)[..., t].
    """
    X = _f64(X)
    w = _f64(w)
    Dp, Cp, T = w.shape
    N = X.shape[0]
    X3 = _split_groups(X, T)
    if X3.shape[1] != Cp:
        raise ValueError("X width does not match w")
    Y3 = np.zeros((N, Dp, T), dtype=np.float64)
    for u in range(T):
        Xs = np.roll(X3, u, axis=2)            # Xs[n, c', t] = X3[n, c', (t-u) mod T]
        # [N*T, C'] @ [C', D'] -> [N, T, D']
        prod = Xs.transpose(0, 2, 1).reshape(N * T, Cp) @ w[:, :, u].T
        Y3 += prod.reshape(N, T, Dp).transpose(0, 2, 1)
    return Y3.reshape(N, Dp * T)


def dx_direct(dY, w) -> np.ndarray:
    """dX = dY W (transposed group-circulant), by the direct formula.

    dX3[n, c', s] = sum_u sum_d' w[d', c', u] * dY3[n, d', (s + u) mod T]
    """
    dY = _f64(dY)
    w = _f64(w)
    Dp, Cp, T = w.shape
    N = dY.shape[0]
    G3 = _split_groups(dY, T)
    if G3.shape[1] != Dp:
        raise ValueError("dY width does not match w")
    dX3 = np.zeros((N, Cp, T), dtype=np.float64)
    for u in range(T):
        Gs = np.roll(G3, -u, axis=2)           # Gs[n, d', s] = G3[n, d', (s+u) mod T]
        prod = Gs.transpose(0, 2, 1).reshape(N * T, Dp) @ w[:, :, u]
        dX3 += prod.reshape(N, T, Cp).transpose(0, 2, 1)
    return dX3.reshape(N, Cp * T)


def dw_direct(dY, X, T: int = 4) -> np.ndarray:
    """Gradient with respect to the learnable circulant vectors w.

    dw[d', c', u] = sum_n sum_t dY3[n, d', t] * X3[n, c', (t - u) mod T],
    i.e. the dense gradient dY^T X summed along each circulant diagonal.
    """
    dY = _f64(dY)
    X = _f64(X)
    G3 = _split_groups(dY, T)
    X3 = _split_groups(X, T)
    N, Dp, _ = G3.shape
    Cp = X3.shape[1]
    dw = np.empty((Dp, Cp, T), dtype=np.float64)
    Gm = G3.transpose(1, 0, 2).reshape(Dp, N * T)         # [D', (n,t)]
    for u in range(T):
        Xs = np.roll(X3, u, axis=2)                        # Xs[n, c', t] = X3[n, c', (t-u)]
        Xm = Xs.transpose(0, 2, 1).reshape(N * T, Cp)      # [(n,t), C']
        dw[:, :, u] = Gm @ Xm
    return dw


def backward_direct(dY, X, w):
    """(dX, dw) of the layer for upstream gradient dY, autograd-free."""
    w = _f64(w)
    return dx_direct(dY, w), dw_direct(dY, X, w.shape[2])


def group_spectrum(z) -> np.ndarray:
    """DFT along the last (group) axis by its definition, complex128.

    F[..., k] = sum_u z[..., u] * exp(-2 pi i k u / T)
    ("Algorithmic approach" item 1: the group convolution becomes a pointwise
    product per frequency).
    """
    z = _f64(z)
    T = z.shape[-1]
    k = np.arange(T).reshape(T, 1)
    u = np.arange(T).reshape(1, T)
    F = np.exp(-2j * np.pi * k * u / T)                   # F[k, u]
    return z.astype(np.complex128) @ F.T


def kept_p4_planes(w) -> np.ndarray:
    """The non-redundant real planes of the p4 (T=4) weight spectrum.

    Real input gives a conjugate-symmetric spectrum ("Algorithmic approach"
    item 2), F[3] = conj(F[1]); F[0] and F[2] are real.  Returns, per
    (d', c'), the four reals (Re F0, Re F2, Re F1, Im F1), shape [D'][C'][4].
    """
    w = _f64(w)
    if w.shape[-1] != 4:
        raise ValueError("p4 planes need T = 4")
    F = group_spectrum(w)
    return np.stack([F[..., 0].real, F[..., 2].real, F[..., 1].real, F[..., 1].imag], axis=-1)


def kept_planes(w) -> np.ndarray:
    """The T non-redundant real planes of the group spectrum, for even T.

    For real circulant vectors the spectrum is conjugate symmetric
    ("Algorithmic approach" item 2): F[T-k] = conj(F[k]), and F[0], F[T/2] are
    real.  Returns, per (d', c'), the T reals
    (Re F0, Re F[T/2], Re F1, Im F1, ..., Re F[T/2-1], Im F[T/2-1]),
    shape [D'][C'][T]; for T = 4 this is kept_p4_planes.
    """
    w = _f64(w)
    T = w.shape[-1]
    if T % 2 or T < 2:
        raise ValueError("kept planes need an even T")
    F = group_spectrum(w)
    planes = [F[..., 0].real, F[..., T // 2].real]
    for k in range(1, T // 2):
        planes += [F[..., k].real, F[..., k].imag]
    return np.stack(planes, axis=-1)


def forward_rows(X, w, rows) -> np.ndarray:
    """Selected output rows of forward_direct, for spot checks of huge shapes."""
    X = _f64(X)
    rows = np.asarray(rows, dtype=np.int64)
    return forward_direct(X[rows], w)


def dw_entries(dY, X, idx, T: int = 4) -> np.ndarray:
    """Selected dw[d', c', :] vectors (idx = [(d', c'), ...]) by the definition."""
    G3 = _split_groups(_f64(dY), T)
    X3 = _split_groups(_f64(X), T)
    out = np.empty((len(idx), T), dtype=np.float64)
    for i, (d, c) in enumerate(idx):
        g = G3[:, d, :]                                    # [N, T]
        x = X3[:, c, :]                                    # [N, T]
        for u in range(T):
            out[i, u] = float(np.sum(g * np.roll(x, u, axis=1)))
    return out


def gelu_erf(z) -> np.ndarray:
    """GELU by its definition z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)), float64."""
    from math import erf, sqrt
    z = _f64(z)
    verf = np.vectorize(erf, otypes=[np.float64])
    return 0.5 * z * (1.0 + verf(z / sqrt(2.0)))


def forward_bias_act(X, w, bias=None, act: str = "none", residual=None) -> np.ndarray:
    """act(X W^T + b) (+ R) with a group-invariant bias b[d'] added to the T
    outputs of output group d' (reading: the summary is silent on bias; a bias
    shared by the group elements keeps the layer equivariant), an optional GELU,
    and an optional residual R [N][D] added after the activation (reading: the
    skip connection around the MLP of the ViT blocks of "Network-level
    results", which the summary does not spell out)."""
    Y = forward_direct(X, w)
    T = _f64(w).shape[2]
    if bias is not None:
        Y = Y + np.repeat(_f64(bias), T)[None, :]
    if act == "gelu":
        Y = gelu_erf(Y)
    elif act != "none":
        raise ValueError(act)
    if residual is not None:
        Y = Y + _f64(residual)
    return Y


# ---------------------------------------------------------------------------
# Finite groups given by their multiplication (Cayley) table.
#
# The summary's method is specialised to p4; its "Limitations" section names
# other groups (reflections) as future work without formulas.  The plain
# reading for a group G of order T with elements 0..T-1 is the group
# convolution that the cyclic case already is:
#
#     W[d'T + g, c'T + h] = w[d', c', h^-1 g]
#     Y3[n, d', g] = sum_{c', h} w[d', c', h^-1 g] X3[n, c', h]
#
# (for C_T, h^-1 g = g - h, which is the circulant above).  table[i, j] is the
# index of the product g_i g_j.

def cyclic_table(T: int) -> np.ndarray:
    """Cayley table of the cyclic group C_T: i * j = (i + j) mod T."""
    i = np.arange(T)
    return (i[:, None] + i[None, :]) % T


def p4m_table() -> np.ndarray:
    """Cayley table of p4m (the dihedral group of order 8).

    Element index u = k + 4 m stands for r^k s^m: r the rotation by 90 degrees,
    s a reflection, with s r s = r^-1.  Hence r^k1 s^m1 r^k2 s^m2 =
    r^(k1 + (-1)^m1 k2) s^(m1 + m2).
    """
    t = np.empty((8, 8), dtype=np.int64)
    for i in range(8):
        k1, m1 = i % 4, i // 4
        for j in range(8):
            k2, m2 = j % 4, j // 4
            t[i, j] = (k1 + (k2 if m1 == 0 else -k2)) % 4 + 4 * (m1 ^ m2)
    return t


def _inverse(table: np.ndarray) -> np.ndarray:
    e = int(np.nonzero(np.all(table == np.arange(len(table))[None, :], axis=1))[0][0])   # identity row
    return np.array([int(np.nonzero(table[i] == e)[0][0]) for i in range(len(table))])


def dense_expand_group(w, table) -> np.ndarray:
    """Dense D x C weight W[d'T + g, c'T + h] = w[d', c', h^-1 g], entry by entry."""
    w = _f64(w)
    Dp, Cp, T = w.shape
    inv = _inverse(table)
    W = np.empty((Dp * T, Cp * T), dtype=np.float64)
    for g in range(T):
        for h in range(T):
            W[g::T, h::T] = w[:, :, table[inv[h], g]]
    return W


def forward_group(X, w, table) -> np.ndarray:
    """Y3[n, d', g] = sum_u sum_c' w[d', c', u] X3[n, c', g u^-1] (u = h^-1 g)."""
    X = _f64(X)
    w = _f64(w)
    Dp, Cp, T = w.shape
    inv = _inverse(table)
    X3 = _split_groups(X, T)
    N = X.shape[0]
    Y3 = np.zeros((N, Dp, T), dtype=np.float64)
    for u in range(T):
        src = [table[g, inv[u]] for g in range(T)]          # h = g u^-1
        Xs = X3[:, :, src]                                  # Xs[n, c', g] = X3[n, c', g u^-1]
        prod = Xs.transpose(0, 2, 1).reshape(N * T, Cp) @ w[:, :, u].T
        Y3 += prod.reshape(N, T, Dp).transpose(0, 2, 1)
    return Y3.reshape(N, Dp * T)


def dx_group(dY, w, table) -> np.ndarray:
    """dX = dY W:  dX3[n, c', h] = sum_u sum_d' w[d', c', u] dY3[n, d', h u]."""
    dY = _f64(dY)
    w = _f64(w)
    Dp, Cp, T = w.shape
    G3 = _split_groups(dY, T)
    N = dY.shape[0]
    dX3 = np.zeros((N, Cp, T), dtype=np.float64)
    for u in range(T):
        src = [table[h, u] for h in range(T)]               # g = h u
        Gs = G3[:, :, src]
        prod = Gs.transpose(0, 2, 1).reshape(N * T, Dp) @ w[:, :, u]
        dX3 += prod.reshape(N, T, Cp).transpose(0, 2, 1)
    return dX3.reshape(N, Cp * T)


def dw_group(dY, X, table) -> np.ndarray:
    """dw[d', c', u] = sum_n sum_h dY3[n, d', h u] X3[n, c', h]  (= d<dY, Y>/dw)."""
    T = len(table)
    G3 = _split_groups(_f64(dY), T)
    X3 = _split_groups(_f64(X), T)
    N, Dp, _ = G3.shape
    Cp = X3.shape[1]
    dw = np.empty((Dp, Cp, T), dtype=np.float64)
    Xm = X3.transpose(0, 2, 1).reshape(N * T, Cp)           # [(n, h), c']
    for u in range(T):
        src = [table[h, u] for h in range(T)]
        Gm = G3[:, :, src].transpose(1, 0, 2).reshape(Dp, N * T)   # [d', (n, h)] = dY3[n, d', h u]
        dw[:, :, u] = Gm @ Xm
    return dw


def p4m_irreps():
    """The irreducible real representations of p4m, element by element.

    Four one-dimensional characters A1, A2, B1, B2 with r -> (1, 1, -1, -1) and
    s -> (1, -1, 1, -1), and the two-dimensional representation E with
    r -> [[0, -1], [1, 0]] (rotation by 90 degrees) and s -> diag(1, -1).
    Returns (chars [8][4], E [8][2][2]) for the elements u = k + 4 m.
    """
    R = np.array([[0.0, -1.0], [1.0, 0.0]])
    S = np.diag([1.0, -1.0])
    chars = np.empty((8, 4))
    E = np.empty((8, 2, 2))
    for u in range(8):
        k, m = u % 4, u // 4
        chars[u] = [1.0, (-1.0) ** m, (-1.0) ** k, (-1.0) ** (k + m)]
        E[u] = np.linalg.matrix_power(R, k) @ np.linalg.matrix_power(S, m)
    return chars, E


def p4m_planes(w) -> np.ndarray:
    """Group Fourier transform of p4m signals by its definition, as 8 real planes.

    f_hat(rho) = sum_g f(g) rho(g): the four characters, then the 2 x 2 block
    of E row-major: (A1, A2, B1, B2, E00, E01, E10, E11), shape [..., 8].
    With this convention the group convolution above becomes
    Y_hat(rho) = X_hat(rho) w_hat(rho) per representation.
    """
    w = _f64(w)
    if w.shape[-1] != 8:
        raise ValueError("p4m signals have 8 values")
    chars, E = p4m_irreps()
    return np.concatenate([w @ chars, (w @ E.reshape(8, 4))], axis=-1)
