"""fp64 CPU oracle for the p4 group convolution (test infrastructure only).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code, table or helper with the HIP
library.

Source: "Technical summary: Flash EQ-Linear" (gist.science, arXiv 2607.21271),
section "Limitations and future work": the authors name the extension of the
Fourier principle to other equivariant operators, equivariant convolution
being their example.  The page gives no formula for it, so this module takes
the plain reading, the p4 group convolution of regular feature maps whose
1 x 1 case is exactly the EQ-Linear layer of the page ("Key insight"):

  feature map   f[n, i, j, c'*4 + s]     (image n, pixel (i, j), channel c',
                                          rotation s = 0..3, rotation fastest)
  filter        psi[d', c', a, b, u]     (spatial tap (a - p, b - p) of a
                                          K x K window, K = 2p + 1 odd, and
                                          group offset u)

  y[n, x, d'*4 + r] = sum_{c', s, delta} f[n, x + delta, c'*4 + s]
                                        * psi[d', c', R^-r delta, (r - s) mod 4]

with delta running over the K x K offsets {-p..p}^2, zero padding outside the
image, and R the quarter turn of offsets R(di, dj) = (-dj, di), which is the
turn numpy.rot90 applies to the (i, j) axes.  At K = 1 this is
Y[d'T + t] = sum w[d', c', (t - s) mod T] X[c'T + s], the page's layer.  The
map is equivariant: turning the image by R^g and shifting the rotation index
by g (f(R^-g x, s - g)) turns and shifts the output the same way.

Backward pass (plain calculus on the same definition):
  dX[n, x + delta, c'*4 + s] += dY[n, x, d'*4 + r] psi[d', c', R^-r delta, (r - s) mod 4]
  dpsi[d', c', R^-r delta, (r - s) mod 4] += dY[n, x, d'*4 + r] f[n, x + delta, c'*4 + s]

Everything runs in float64 with NumPy; the only library step is a dense
matrix product per (r, delta).
"""
from __future__ import annotations

import numpy as np

from .eqlin_oracle import gelu_erf

__all__ = [
    "rot_offset",
    "conv_forward",
    "conv_forward_bias_act",
    "conv_dx",
    "conv_dw",
    "conv_dense_filter",
    "conv_forward_pixels",
    "conv_dx_pixels",
    "conv_dw_entries",
]

T4 = 4


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rot_offset(r: int, di: int, dj: int):
    """R^r (di, dj) with R(di, dj) = (-dj, di); r may be negative."""
    for _ in range(r % 4):
        di, dj = -dj, di
    return di, dj


def _shapes(f, psi):
    N, H, W, C = f.shape
    Dp, Cp, K, K2, T = psi.shape
    if T != T4 or K != K2 or K % 2 != 1 or C != Cp * T4:
        raise ValueError("f [N][H][W][4C'] and psi [D'][C'][K][K][4] with odd K expected")
    return N, H, W, Cp, Dp, K


def _taps(K: int):
    p = K // 2
    return [(di, dj) for di in range(-p, p + 1) for dj in range(-p, p + 1)]


def _kernel_for(psi, r: int, di: int, dj: int) -> np.ndarray:
    """[D'][C'][s] = psi[d', c', R^-r delta, (r - s) mod 4]."""
    p = psi.shape[2] // 2
    ai, aj = rot_offset(-r, di, dj)
    ker = psi[:, :, ai + p, aj + p, :]
    return ker[:, :, [(r - s) % T4 for s in range(T4)]]


def conv_forward(f, psi) -> np.ndarray:
    """y = p4 group convolution of f with psi, by the definition above."""
    f, psi = _f64(f), _f64(psi)
    N, H, W, Cp, Dp, K = _shapes(f, psi)
    p = K // 2
    fp = np.zeros((N, H + 2 * p, W + 2 * p, Cp * T4))
    fp[:, p:p + H, p:p + W] = f
    y = np.zeros((N, H, W, Dp, T4))
    for r in range(T4):
        for di, dj in _taps(K):
            kr = _kernel_for(psi, r, di, dj).reshape(Dp, Cp * T4)
            sh = fp[:, p + di:p + di + H, p + dj:p + dj + W]          # f(x + delta)
            y[..., r] += (sh.reshape(-1, Cp * T4) @ kr.T).reshape(N, H, W, Dp)
    return y.reshape(N, H, W, Dp * T4)


def conv_forward_bias_act(f, psi, bias=None, act: str = "none") -> np.ndarray:
    """act(conv(f, psi) + b) with the group-invariant bias b[d'] of the linear
    layer added to the four rotations of output channel d'."""
    y = conv_forward(f, psi)
    if bias is not None:
        y = y + np.repeat(_f64(bias), T4)
    if act == "gelu":
        y = gelu_erf(y)
    elif act != "none":
        raise ValueError(act)
    return y


def conv_forward_pixels(f, psi, pix) -> np.ndarray:
    """Rows of conv_forward at the flat pixel indices pix (n*H*W + i*W + j),
    computed one by one from the definition (for spot checks at full size)."""
    f, psi = _f64(f), _f64(psi)
    N, H, W, Cp, Dp, K = _shapes(f, psi)
    out = np.zeros((len(pix), Dp * T4))
    for row, q in enumerate(pix):
        n, rem = divmod(int(q), H * W)
        i, j = divmod(rem, W)
        y = np.zeros((Dp, T4))
        for r in range(T4):
            for di, dj in _taps(K):
                if 0 <= i + di < H and 0 <= j + dj < W:
                    kr = _kernel_for(psi, r, di, dj).reshape(Dp, Cp * T4)
                    y[:, r] += kr @ f[n, i + di, j + dj]
        out[row] = y.reshape(-1)
    return out


def conv_dx(dy, psi, H: int, W: int) -> np.ndarray:
    """dX = adjoint of conv_forward in f, applied to dy [N][H][W][4D']."""
    dy, psi = _f64(dy), _f64(psi)
    Dp, Cp, K = psi.shape[0], psi.shape[1], psi.shape[2]
    N = dy.shape[0]
    p = K // 2
    dY = dy.reshape(N, H, W, Dp, T4)
    dxp = np.zeros((N, H + 2 * p, W + 2 * p, Cp * T4))
    for r in range(T4):
        for di, dj in _taps(K):
            kr = _kernel_for(psi, r, di, dj).reshape(Dp, Cp * T4)
            contrib = (dY[..., r].reshape(-1, Dp) @ kr).reshape(N, H, W, Cp * T4)
            dxp[:, p + di:p + di + H, p + dj:p + dj + W] += contrib
    return dxp[:, p:p + H, p:p + W].copy()


def conv_dw(dy, f, K: int) -> np.ndarray:
    """dpsi [D'][C'][K][K][4]: gradient of <dy, conv_forward(f, psi)> in psi."""
    dy, f = _f64(dy), _f64(f)
    N, H, W, C = f.shape
    Cp = C // T4
    Dp = dy.shape[3] // T4
    p = K // 2
    dY = dy.reshape(N, H, W, Dp, T4)
    fp = np.zeros((N, H + 2 * p, W + 2 * p, C))
    fp[:, p:p + H, p:p + W] = f
    dpsi = np.zeros((Dp, Cp, K, K, T4))
    for r in range(T4):
        for di, dj in _taps(K):
            sh = fp[:, p + di:p + di + H, p + dj:p + dj + W].reshape(-1, Cp, T4)
            G = np.einsum("xd,xcs->dcs", dY[..., r].reshape(-1, Dp), sh)
            ai, aj = rot_offset(-r, di, dj)
            for s in range(T4):
                dpsi[:, :, ai + p, aj + p, (r - s) % T4] += G[:, :, s]
    return dpsi


def conv_dense_filter(psi) -> np.ndarray:
    """The ordinary K x K filter bank [4D'][4C'][K][K] of the same map (output
    channel d'*4 + r, input channel c'*4 + s, cross-correlation taps), entry by
    entry from the definition."""
    psi = _f64(psi)
    Dp, Cp, K = psi.shape[0], psi.shape[1], psi.shape[2]
    p = K // 2
    Wd = np.zeros((Dp * T4, Cp * T4, K, K))
    for r in range(T4):
        for di, dj in _taps(K):
            kr = _kernel_for(psi, r, di, dj)                       # [D'][C'][s]
            for s in range(T4):
                Wd[r::T4, s::T4, di + p, dj + p] = kr[:, :, s]
    return Wd


def conv_dx_pixels(dy, psi, H: int, W: int, pix) -> np.ndarray:
    """Rows of conv_dx at the flat pixel indices pix, one by one from the
    adjoint's definition: dX[y, c'*4 + s] = sum_{r, delta} dY[y - delta, d'*4 + r]
    psi[d', c', R^-r delta, (r - s) mod 4]."""
    dy, psi = _f64(dy), _f64(psi)
    Dp, Cp, K = psi.shape[0], psi.shape[1], psi.shape[2]
    N = dy.shape[0]
    dY = dy.reshape(N, H, W, Dp, T4)
    out = np.zeros((len(pix), Cp * T4))
    for row, q in enumerate(pix):
        n, rem = divmod(int(q), H * W)
        i, j = divmod(rem, W)
        for r in range(T4):
            for di, dj in _taps(K):
                if 0 <= i - di < H and 0 <= j - dj < W:
                    kr = _kernel_for(psi, r, di, dj).reshape(Dp, Cp * T4)
                    out[row] += dY[n, i - di, j - dj, :, r] @ kr
    return out


def conv_dw_entries(dy, f, K: int, idx) -> np.ndarray:
    """Entries dpsi[d', c', a, b, v] for idx rows (d', c', a, b, v), one by one:
    sum_{x, r} dY[x, d'*4 + r] f[x + R^r (a - p, b - p), c'*4 + (r - v) mod 4]."""
    dy, f = _f64(dy), _f64(f)
    N, H, W, C = f.shape
    Cp, p = C // T4, K // 2
    Dp = dy.shape[3] // T4
    dY = dy.reshape(N, H, W, Dp, T4)
    f5 = f.reshape(N, H, W, Cp, T4)
    out = np.zeros(len(idx))
    for e, (d, c, a, b, v) in enumerate(idx):
        acc = 0.0
        for r in range(T4):
            di, dj = rot_offset(r, a - p, b - p)
            i0, i1 = max(0, -di), min(H, H - di)
            j0, j1 = max(0, -dj), min(W, W - dj)
            if i0 >= i1 or j0 >= j1:
                continue
            acc += float(np.sum(dY[:, i0:i1, j0:j1, d, r] *
                                f5[:, i0 + di:i1 + di, j0 + dj:j1 + dj, c, (r - v) % T4]))
        out[e] = acc
    return out
