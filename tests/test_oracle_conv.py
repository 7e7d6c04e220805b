"""Pins for the oracle's p4 group convolution, independent of its own code.

The summary names equivariant convolution as future work ("Limitations and
future work") without formulas.  The oracle's reading is the p4 group
convolution whose 1 x 1 case is the page's EQ-Linear layer.  It is pinned by:
the reduction to the (already pinned) linear layer at K = 1, a library
convolution (torch conv2d in float64) with numpy.rot90-turned filters, exact
equivariance under numpy.rot90 plus a shift of the rotation axis (and a
planted wrong turn that breaks it), brute-force loops on a tiny case, the
adjoint identities and torch autograd.  The last test checks the reading the
HIP path is built on (the convolution as one EQ-Linear over a rotation-aware
gather) against the oracle.
"""
import numpy as np
import pytest

import oracle
from oracle import eqconv_oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _turn(z, g):
    """(L_g z)(x, s) = z(R^-g x, s - g) on [N][H][W][4C]: numpy.rot90 on the
    pixel axes and a roll of the rotation axis."""
    N, H, W, C = z.shape
    z5 = z.reshape(N, H, W, C // 4, 4)
    z5 = np.roll(np.rot90(z5, g, axes=(1, 2)), g, axis=4)
    return np.ascontiguousarray(z5).reshape(N, H, W, C)


def test_rot_offset_is_the_turn_of_numpy_rot90():
    # rot90 moves the entry at centred offset v to R v
    n, c = 5, 2
    for di in range(-2, 3):
        for dj in range(-2, 3):
            A = np.zeros((n, n))
            A[c + di, c + dj] = 1
            B = np.rot90(A)
            ii, jj = np.argwhere(B == 1)[0]
            assert (ii - c, jj - c) == oracle.rot_offset(1, di, dj)
            assert oracle.rot_offset(4, di, dj) == (di, dj)
            assert oracle.rot_offset(-1, *oracle.rot_offset(1, di, dj)) == (di, dj)


def test_one_by_one_is_the_linear_layer():
    N, H, W, Cp, Dp = 2, 3, 4, 3, 5
    f = _rand((N, H, W, 4 * Cp), 1)
    psi = _rand((Dp, Cp, 1, 1, 4), 2)
    y = oracle.conv_forward(f, psi)
    ref = oracle.forward_direct(f.reshape(-1, 4 * Cp), psi[:, :, 0, 0, :]).reshape(N, H, W, 4 * Dp)
    assert _rel(y, ref) < 1e-14


@pytest.mark.parametrize("K", [3, 5])
def test_library_convolution_with_turned_filters(K):
    # f constant over the rotation axis and psi supported on u = 0: output
    # rotation r is conv2d of the channel image with the filter turned r times
    torch = pytest.importorskip("torch")
    N, H, W, Cp, Dp = 2, 7, 6, 3, 2
    g = _rand((N, H, W, Cp), 3)
    f = np.repeat(g, 4, axis=3)                       # f[.., c'*4+s] = g[.., c']
    psi = np.zeros((Dp, Cp, K, K, 4))
    psi[..., 0] = _rand((Dp, Cp, K, K), 4)
    y = oracle.conv_forward(f, psi).reshape(N, H, W, Dp, 4)
    gt = torch.tensor(g).permute(0, 3, 1, 2)
    for r in range(4):
        ker = torch.tensor(np.ascontiguousarray(np.rot90(psi[..., 0], r, axes=(2, 3))))
        ref = torch.nn.functional.conv2d(gt, ker, padding=K // 2).permute(0, 2, 3, 1).numpy()
        assert _rel(y[..., r], ref) < 1e-13


def test_dense_filter_bank_through_library_convolution():
    torch = pytest.importorskip("torch")
    N, H, W, Cp, Dp, K = 2, 6, 5, 2, 3, 3
    f = _rand((N, H, W, 4 * Cp), 5)
    psi = _rand((Dp, Cp, K, K, 4), 6)
    Wd = torch.tensor(oracle.conv_dense_filter(psi))
    ref = torch.nn.functional.conv2d(torch.tensor(f).permute(0, 3, 1, 2), Wd, padding=1)
    assert _rel(oracle.conv_forward(f, psi), ref.permute(0, 2, 3, 1).numpy()) < 1e-13


@pytest.mark.parametrize("K", [1, 3, 5])
def test_equivariance_under_every_turn(K):
    N, S, Cp, Dp = 2, 7, 3, 2
    f = _rand((N, S, S, 4 * Cp), 7)
    psi = _rand((Dp, Cp, K, K, 4), 8)
    y = oracle.conv_forward(f, psi)
    for g in range(1, 4):
        assert _rel(oracle.conv_forward(_turn(f, g), psi), _turn(y, g)) < 1e-13


def test_planted_wrong_turn_breaks_equivariance(monkeypatch):
    # turning the filter taps with R^r instead of R^-r is not equivariant
    N, S, Cp, Dp, K = 1, 6, 2, 2, 3
    f = _rand((N, S, S, 4 * Cp), 9)
    psi = _rand((Dp, Cp, K, K, 4), 10)
    good = oracle.conv_forward(f, psi)
    real = eqconv_oracle.rot_offset
    monkeypatch.setattr(eqconv_oracle, "rot_offset", lambda r, di, dj: real(-r, di, dj))
    bad = eqconv_oracle.conv_forward(f, psi)
    assert _rel(bad, good) > 1e-3
    err = max(_rel(eqconv_oracle.conv_forward(_turn(f, g), psi), _turn(bad, g)) for g in (1, 3))
    assert err > 1e-3


def test_brute_force_loops_tiny():
    N, H, W, Cp, Dp, K = 1, 3, 4, 2, 2, 3
    f = _rand((N, H, W, 4 * Cp), 11)
    psi = _rand((Dp, Cp, K, K, 4), 12)
    y = np.zeros((N, H, W, 4 * Dp))
    for i in range(H):
        for j in range(W):
            for d in range(Dp):
                for r in range(4):
                    acc = 0.0
                    for c in range(Cp):
                        for s in range(4):
                            for a in range(K):
                                for b in range(K):
                                    di, dj = a - 1, b - 1
                                    if not (0 <= i + di < H and 0 <= j + dj < W):
                                        continue
                                    # R^-r (di, dj) written out: (dj, -di) per inverse quarter turn
                                    ti, tj = di, dj
                                    for _ in range(r):
                                        ti, tj = tj, -ti
                                    acc += f[0, i + di, j + dj, 4 * c + s] * psi[d, c, ti + 1, tj + 1, (r - s) % 4]
                    y[0, i, j, 4 * d + r] = acc
    assert _rel(oracle.conv_forward(f, psi), y) < 1e-14
    pix = [0, 5, 11]
    assert _rel(oracle.conv_forward_pixels(f, psi, pix), y.reshape(-1, 4 * Dp)[pix]) < 1e-14


def test_adjoint_identities():
    N, H, W, Cp, Dp, K = 2, 5, 6, 3, 2, 3
    f = _rand((N, H, W, 4 * Cp), 13)
    psi = _rand((Dp, Cp, K, K, 4), 14)
    dy = _rand((N, H, W, 4 * Dp), 15)
    y = oracle.conv_forward(f, psi)
    a = float(np.sum(dy * y))
    assert abs(a - float(np.sum(oracle.conv_dx(dy, psi, H, W) * f))) < 1e-12 * abs(a)
    assert abs(a - float(np.sum(oracle.conv_dw(dy, f, K) * psi))) < 1e-12 * abs(a)


def test_gradients_match_torch_autograd():
    torch = pytest.importorskip("torch")
    N, H, W, Cp, Dp, K = 2, 5, 4, 2, 3, 3
    f = _rand((N, H, W, 4 * Cp), 16)
    psi = _rand((Dp, Cp, K, K, 4), 17)
    dy = _rand((N, H, W, 4 * Dp), 18)
    # dense filter bank gathered from psi with an index table built from np.rot90
    idx = np.zeros((4 * Dp, 4 * Cp, K, K), dtype=np.int64)
    flat = np.arange(Dp * Cp * K * K * 4).reshape(Dp, Cp, K, K, 4)
    for r in range(4):
        # tap delta of rotation r reads psi at R^-r delta: rot90 of the tap grid r times
        turned = np.rot90(flat, r, axes=(2, 3))
        for s in range(4):
            idx[r::4, s::4] = turned[..., (r - s) % 4]
    pt = torch.tensor(psi, requires_grad=True)
    Wd = pt.reshape(-1)[torch.tensor(idx)]
    ft = torch.tensor(f, requires_grad=True)
    yt = torch.nn.functional.conv2d(ft.permute(0, 3, 1, 2), Wd, padding=K // 2).permute(0, 2, 3, 1)
    yt.backward(torch.tensor(dy))
    assert _rel(oracle.conv_forward(f, psi), yt.detach().numpy()) < 1e-13
    assert _rel(oracle.conv_dx(dy, psi, H, W), ft.grad.numpy()) < 1e-13
    assert _rel(oracle.conv_dw(dy, f, K), pt.grad.numpy()) < 1e-13


def test_bias_and_gelu():
    N, H, W, Cp, Dp, K = 1, 4, 4, 2, 2, 3
    f = _rand((N, H, W, 4 * Cp), 19)
    psi = _rand((Dp, Cp, K, K, 4), 20)
    b = _rand((Dp,), 21)
    y = oracle.conv_forward(f, psi)
    yb = oracle.conv_forward_bias_act(f, psi, b, "gelu")
    z = y + np.repeat(b, 4)
    assert _rel(yb, oracle.gelu_erf(z)) < 1e-15


# ------------------------------------------ the reading the GPU path uses

def test_convolution_is_one_linear_layer_over_a_turned_gather():
    """Taps split into the centre and the quarter-turn orbits of the offsets
    (a, b) with a > 0, b >= 0.  For orbit o the four taps R^m delta_o gather
    x_lin[(c', o, b)][m] = f[x + R^m delta_o, c'*4 + (m + b) mod 4]; the centre
    gathers f[x, c'*4 + m].  The convolution is then the page's group-
    circulant layer on x_lin with w_lin[(c', o, b)][u] = psi[c', R^-u delta_o,
    (u - b) mod 4] (centre: psi[c', 0, u]), each psi entry used once."""
    N, H, W, Cp, Dp, K = 2, 5, 6, 3, 2, 5
    p = K // 2
    f = _rand((N, H, W, 4 * Cp), 22)
    psi = _rand((Dp, Cp, K, K, 4), 23)
    orbits = [(a, b) for a in range(1, p + 1) for b in range(0, p + 1)]
    assert 1 + 4 * len(orbits) == K * K
    fp = np.zeros((N, H + 2 * p, W + 2 * p, Cp, 4))
    fp[:, p:p + H, p:p + W] = f.reshape(N, H, W, Cp, 4)
    cols, wcols = [], []
    cols.append(fp[:, p:p + H, p:p + W])                          # centre [N,H,W,C',4]
    wcols.append(psi[:, :, p, p, :])                              # [D',C',4]
    used = np.zeros(psi.shape, dtype=int)
    used[:, :, p, p, :] += 1
    for (a, b0) in orbits:
        for bb in range(4):
            g = np.zeros((N, H, W, Cp, 4))
            wl = np.zeros((Dp, Cp, 4))
            for m in range(4):
                di, dj = oracle.rot_offset(m, a, b0)
                g[..., m] = fp[:, p + di:p + di + H, p + dj:p + dj + W, :, (m + bb) % 4]
            for u in range(4):
                ti, tj = oracle.rot_offset(-u, a, b0)
                wl[:, :, u] = psi[:, :, ti + p, tj + p, (u - bb) % 4]
                used[:, :, ti + p, tj + p, (u - bb) % 4] += 1
            cols.append(g)
            wcols.append(wl)
    assert np.all(used == 1)
    X_lin = np.concatenate(cols, axis=3).reshape(N * H * W, -1)
    w_lin = np.concatenate(wcols, axis=1)
    y = oracle.forward_direct(X_lin, w_lin).reshape(N, H, W, 4 * Dp)
    assert _rel(y, oracle.conv_forward(f, psi)) < 1e-13


def test_input_gradient_is_a_convolution_of_dy():
    """dX is the same kind of convolution of dy with
    psi'[c', d', delta, u] = psi[d', c', -R^u delta, -u mod 4] (the reading
    the GPU path uses to run dX through the forward kernel)."""
    N, H, W, Cp, Dp, K = 2, 5, 5, 3, 2, 3
    p = K // 2
    psi = _rand((Dp, Cp, K, K, 4), 24)
    dy = _rand((N, H, W, 4 * Dp), 25)
    psi_t = np.zeros((Cp, Dp, K, K, 4))
    for a in range(K):
        for b in range(K):
            for u in range(4):
                ti, tj = oracle.rot_offset(u, a - p, b - p)
                psi_t[:, :, a, b, u] = psi[:, :, -ti + p, -tj + p, (-u) % 4].T
    assert _rel(oracle.conv_forward(dy, psi_t), oracle.conv_dx(dy, psi, H, W)) < 1e-13


def test_per_pixel_and_per_entry_routines_match_the_whole_tensor_ones():
    N, H, W, Cp, Dp, K = 2, 5, 4, 2, 3, 3
    f = _rand((N, H, W, 4 * Cp), 26)
    psi = _rand((Dp, Cp, K, K, 4), 27)
    dy = _rand((N, H, W, 4 * Dp), 28)
    pix = [0, 3, 7, 19, 39]
    dx = oracle.conv_dx(dy, psi, H, W).reshape(-1, 4 * Cp)
    assert _rel(oracle.conv_dx_pixels(dy, psi, H, W, pix), dx[pix]) < 1e-14
    dw = oracle.conv_dw(dy, f, K)
    idx = [(0, 0, 0, 0, 0), (2, 1, 1, 2, 3), (1, 0, 2, 1, 1), (2, 1, 1, 1, 2)]
    assert _rel(oracle.conv_dw_entries(dy, f, K, idx), np.array([dw[i] for i in idx])) < 1e-13
