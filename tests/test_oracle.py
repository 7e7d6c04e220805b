"""Pins for the fp64 oracle, independent of the oracle's own code paths.

Each test checks the oracle against something the page or mathematics fixes:
library routines (scipy's circulant matrix, numpy's FFT, torch autograd),
brute force on tiny inputs, closed-form special cases, invariants (group
equivariance, adjoint identities) and the numeric facts the Flash EQ-Linear
summary states (tests/golden/p4_facts.json).
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from group_circulant_linear_amd.inputs import make_layer_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p4_facts.json")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _dense_by_scipy(w):
    """Dense weight assembled from scipy.linalg.circulant blocks.

    scipy's circulant(c) has C[i, j] = c[(i - j) mod n]: block (d', c') of the
    layer is the circulant of w[d', c', :].
    """
    Dp, Cp, T = w.shape
    return np.block([[scipy.linalg.circulant(w[d, c]) for c in range(Cp)] for d in range(Dp)])


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8])
def test_forward_matches_scipy_circulant_dense(T):
    N, Cp, Dp = 7, 3, 5
    X = _rand((N, Cp * T), 1)
    w = _rand((Dp, Cp, T), 2)
    Y = oracle.forward_direct(X, w)
    Yref = X @ _dense_by_scipy(w).T
    assert _rel(Y, Yref) < 1e-13
    # the oracle's own expansion must be that same matrix
    assert np.array_equal(oracle.dense_expand(w), _dense_by_scipy(w))


def test_forward_brute_force_tiny_config():
    # the tiny p4 workload: N=64, C=D=32, fp32 storage
    X, w, _ = make_layer_inputs(64, 32, 32, "f32", seed=0, with_dy=False)
    X = X.astype(np.float64)
    w = w.astype(np.float64)
    Dp, Cp, T = w.shape
    Y = oracle.forward_direct(X, w)
    Yb = np.zeros_like(Y)
    Xl = X.tolist()
    wl = w.tolist()
    for n in range(X.shape[0]):
        row = Xl[n]
        for d in range(Dp):
            for t in range(T):
                acc = 0.0
                for c in range(Cp):
                    for s in range(T):
                        acc += wl[d][c][(t - s) % T] * row[c * T + s]
                Yb[n, d * T + t] = acc
    assert _rel(Y, Yb) < 1e-13


@pytest.mark.parametrize("T", [2, 3, 4, 8])
def test_forward_matches_fft_convolution_theorem(T):
    # independent route: circular convolution along the group axis = ifft(fft * fft)
    N, Cp, Dp = 6, 4, 3
    X = _rand((N, Cp * T), 3)
    w = _rand((Dp, Cp, T), 4)
    X3 = X.reshape(N, Cp, T)
    Fx = np.fft.fft(X3, axis=2)                      # [N, C', T]
    Fw = np.fft.fft(w, axis=2)                       # [D', C', T]
    Fy = np.einsum("dck,nck->ndk", Fw, Fx)
    Yref = np.fft.ifft(Fy, axis=2).real.reshape(N, Dp * T)
    assert _rel(oracle.forward_direct(X, w), Yref) < 1e-13


def test_T1_is_plain_gemm():
    X = _rand((9, 5), 5)
    w = _rand((4, 5, 1), 6)
    assert _rel(oracle.forward_direct(X, w), X @ w[:, :, 0].T) < 1e-14


def test_identity_shift_only_gives_four_strided_gemms():
    X = _rand((8, 24), 7)
    w = np.zeros((5, 6, 4))
    w[:, :, 0] = _rand((5, 6), 8)
    Y = oracle.forward_direct(X, w)
    for t in range(4):
        assert _rel(Y[:, t::4], X[:, t::4] @ w[:, :, 0].T) < 1e-14


def test_constant_over_group_collapses_to_f0():
    X = _rand((8, 24), 9)
    base = _rand((5, 6), 10)
    w = np.repeat(base[:, :, None], 4, axis=2)
    Y = oracle.forward_direct(X, w).reshape(8, 5, 4)
    expect = X.reshape(8, 6, 4).sum(axis=2) @ base.T
    for t in range(4):
        assert _rel(Y[:, :, t], expect) < 1e-13


def test_one_hot_row_returns_weight_column():
    w = _rand((3, 2, 4), 11)
    W = _dense_by_scipy(w)
    for j in range(8):
        x = np.zeros((1, 8))
        x[0, j] = 1.0
        assert np.allclose(oracle.forward_direct(x, w)[0], W[:, j], rtol=0, atol=1e-15)


@pytest.mark.parametrize("T", [4, 3, 8])
def test_equivariance_group_shift(T):
    # rolling the group index of every input block by one rolls every output block by one
    N, Cp, Dp = 5, 4, 6
    X = _rand((N, Cp * T), 12)
    w = _rand((Dp, Cp, T), 13)
    Xr = np.roll(X.reshape(N, Cp, T), 1, axis=2).reshape(N, Cp * T)
    Y = oracle.forward_direct(X, w).reshape(N, Dp, T)
    Yr = oracle.forward_direct(Xr, w).reshape(N, Dp, T)
    assert _rel(Yr, np.roll(Y, 1, axis=2)) < 1e-14


def test_linearity():
    X1, X2 = _rand((6, 16), 14), _rand((6, 16), 15)
    w1, w2 = _rand((3, 4, 4), 16), _rand((3, 4, 4), 17)
    a, b = 0.7, -1.3
    f = oracle.forward_direct
    assert _rel(f(a * X1 + b * X2, w1), a * f(X1, w1) + b * f(X2, w1)) < 1e-13
    assert _rel(f(X1, a * w1 + b * w2), a * f(X1, w1) + b * f(X1, w2)) < 1e-13


def test_forward_rows_subset():
    X = _rand((20, 16), 18)
    w = _rand((3, 4, 4), 19)
    rows = [0, 7, 19]
    assert _rel(oracle.forward_rows(X, w, rows), oracle.forward_direct(X, w)[rows]) < 1e-15


# --------------------------------------------------------------- backward pins

@pytest.mark.parametrize("T", [4, 3, 8])
def test_gradients_by_directional_derivatives(T):
    # L(X, w) = <dY, Y(X, w)> is linear in X and in w separately, so
    # dL/dX[i] = L(e_i, w) and dL/dw[j] = L(X, e_j) exactly.
    N, Cp, Dp = 3, 2, 3
    X = _rand((N, Cp * T), 20)
    w = _rand((Dp, Cp, T), 21)
    dY = _rand((N, Dp * T), 22)
    dX, dw = oracle.backward_direct(dY, X, w)

    def L(Xv, wv):
        return float(np.sum(dY * (Xv @ _dense_by_scipy(wv).T)))

    gX = np.zeros_like(X)
    for i in np.ndindex(*X.shape):
        e = np.zeros_like(X)
        e[i] = 1.0
        gX[i] = L(e, w)
    gw = np.zeros_like(w)
    for j in np.ndindex(*w.shape):
        e = np.zeros_like(w)
        e[j] = 1.0
        gw[j] = L(X, e)
    assert _rel(dX, gX) < 1e-13
    assert _rel(dw, gw) < 1e-13


@pytest.mark.parametrize("T", [4, 8])
def test_gradients_match_torch_autograd(T):
    torch = pytest.importorskip("torch")
    Cp, Dp, N = 8, 6, 11
    X = _rand((N, Cp * T), 23)
    w = _rand((Dp, Cp, T), 24)
    dY = _rand((N, Dp * T), 25)
    # dense weight assembled by torch from the circulant blocks via gather of
    # scipy-built index pattern: idx[t, s] = (t - s) mod T
    idx = torch.tensor(scipy.linalg.circulant(np.arange(T)), dtype=torch.long)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    blocks = wt[:, :, idx]                               # [D', C', T, T]
    Wd = blocks.permute(0, 2, 1, 3).reshape(Dp * T, Cp * T)
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Yt = torch.nn.functional.linear(Xt, Wd)
    Yt.backward(torch.tensor(dY))
    dX, dw = oracle.backward_direct(dY, X, w)
    assert _rel(Yt.detach().numpy(), oracle.forward_direct(X, w)) < 1e-14
    assert _rel(dX, Xt.grad.numpy()) < 1e-13
    assert _rel(dw, wt.grad.numpy()) < 1e-13


def test_adjoint_identities():
    X, w, dY = make_layer_inputs(40, 64, 48, "f32", seed=3)
    X, w, dY = X.astype(float), w.astype(float), dY.astype(float)
    Y = oracle.forward_direct(X, w)
    dX, dw = oracle.backward_direct(dY, X, w)
    a = np.sum(dY * Y)
    assert abs(np.sum(dX * X) - a) < 1e-11 * abs(a) + 1e-12
    assert abs(np.sum(dw * w) - a) < 1e-11 * abs(a) + 1e-12


def test_dw_entries_subset():
    X = _rand((30, 16), 26)
    dY = _rand((30, 12), 27)
    dw = oracle.dw_direct(dY, X, 4)
    idx = [(0, 0), (2, 3), (1, 2)]
    sub = oracle.dw_entries(dY, X, idx)
    for i, (d, c) in enumerate(idx):
        assert _rel(sub[i], dw[d, c]) < 1e-13


def test_dx_equivariance():
    N, Cp, Dp, T = 5, 3, 4, 4
    dY = _rand((N, Dp * T), 28)
    w = _rand((Dp, Cp, T), 29)
    dYr = np.roll(dY.reshape(N, Dp, T), 1, axis=2).reshape(N, Dp * T)
    dX = oracle.dx_direct(dY, w).reshape(N, Cp, T)
    dXr = oracle.dx_direct(dYr, w).reshape(N, Cp, T)
    assert _rel(dXr, np.roll(dX, 1, axis=2)) < 1e-14


# ------------------------------------------------------------ spectrum pins

def test_group_spectrum_matches_numpy_fft():
    z = _rand((5, 7, 4), 30)
    assert np.max(np.abs(oracle.group_spectrum(z) - np.fft.fft(z, axis=-1))) < 1e-13
    z8 = _rand((3, 8), 31)
    assert np.max(np.abs(oracle.group_spectrum(z8) - np.fft.fft(z8, axis=-1))) < 1e-13


def test_kept_planes_conjugate_symmetry_and_values():
    w = _rand((4, 6, 4), 32)
    F = np.fft.fft(w, axis=-1)
    P = oracle.kept_p4_planes(w)
    # real signal -> F3 = conj(F1), F0 and F2 real
    assert np.max(np.abs(F[..., 3] - np.conj(F[..., 1]))) < 1e-13
    assert np.max(np.abs(F[..., 0].imag)) < 1e-13 and np.max(np.abs(F[..., 2].imag)) < 1e-13
    assert np.max(np.abs(P[..., 0] - F[..., 0].real)) < 1e-13
    assert np.max(np.abs(P[..., 1] - F[..., 2].real)) < 1e-13
    assert np.max(np.abs(P[..., 2] - F[..., 1].real)) < 1e-13
    assert np.max(np.abs(P[..., 3] - F[..., 1].imag)) < 1e-13


@pytest.mark.parametrize("T", [2, 4, 6, 8])
def test_kept_planes_general_even_T(T):
    w = _rand((3, 5, T), 33 + T)
    P = oracle.kept_planes(w)
    assert P.shape == (3, 5, T)
    # numpy's real inverse FFT of the half spectrum rebuilt from the planes gives w back
    half = np.zeros((3, 5, T // 2 + 1), dtype=complex)
    half[..., 0] = P[..., 0]
    half[..., T // 2] = P[..., 1]
    for k in range(1, T // 2):
        half[..., k] = P[..., 2 * k] + 1j * P[..., 2 * k + 1]
    assert np.max(np.abs(np.fft.irfft(half, n=T, axis=-1) - w)) < 1e-13
    # and the planes are numpy's forward FFT values
    F = np.fft.rfft(w, axis=-1)
    assert np.max(np.abs(P[..., 0] - F[..., 0].real)) < 1e-13
    if T >= 4:
        assert np.max(np.abs(P[..., 3] - F[..., 1].imag)) < 1e-13
    if T == 4:
        assert np.array_equal(P, oracle.kept_p4_planes(w))


# ------------------------------------------------------ page facts (golden)

def _facts():
    with open(GOLDEN) as f:
        return json.load(f)["facts"]


def _real_dft4():
    """Real form of the kept p4 spectrum: x -> (F0, F2, Re F1, Im F1), from group_spectrum."""
    R = np.zeros((4, 4))
    for s in range(4):
        e = np.zeros(4)
        e[s] = 1.0
        F = oracle.group_spectrum(e)
        R[:, s] = [F[0].real, F[2].real, F[1].real, F[1].imag]
    return R


def test_p4_transform_coefficients_are_dyadic():
    facts = _facts()
    allowed = set(facts["p4_dft_coefficients"]["value"])
    R = _real_dft4()
    Rinv = np.linalg.inv(R)
    # unnormalised forward has entries in {0, +-1}; the inverse carries 1/4 and 1/2.
    assert set(np.round(R, 12).ravel().tolist()) <= {0.0, 1.0, -1.0}
    assert set(np.round(Rinv, 12).ravel().tolist()) <= {0.0, 0.25, -0.25, 0.5, -0.5}
    # with the normalisation split as 1/2 on each side both matrices use exactly
    # the page's coefficient set {0, +-1, +-1/2}
    both = set(np.round(R / 2, 12).ravel().tolist()) | set(np.round(2 * Rinv, 12).ravel().tolist())
    assert both <= allowed


def test_p4_six_real_products_instead_of_sixteen():
    facts = _facts()
    R = _real_dft4()
    Rinv = np.linalg.inv(R)
    c = _rand(4, 33)
    B = R @ scipy.linalg.circulant(c) @ Rinv
    nonzero = int(np.sum(np.abs(B) > 1e-12))
    assert nonzero == facts["p4_real_gemms_fourier"]["value"]
    assert B.size == facts["p4_real_gemms_naive"]["value"]
    assert round(B.size / nonzero, 2) == facts["p4_theoretical_speedup"]["value"]
    # the surviving pattern: f0 and f2 scalars, f1 a 2x2 rotation-scaling block
    F = np.fft.fft(c)
    assert abs(B[0, 0] - F[0].real) < 1e-12 and abs(B[1, 1] - F[2].real) < 1e-12
    assert abs(B[2, 2] - F[1].real) < 1e-12 and abs(B[3, 3] - F[1].real) < 1e-12
    assert abs(B[2, 3] + F[1].imag) < 1e-12 and abs(B[3, 2] - F[1].imag) < 1e-12


def test_mac_count_and_parameter_facts():
    facts = _facts()
    T = facts["p4_group_size"]["value"]
    # exact kept-spectrum real MACs per (n, d', c') for even T: 1 + 1 + 4*(T/2 - 1)
    for TT in (4, 8, 16, 64):
        macs = 2 + 4 * (TT // 2 - 1)
        naive = TT * TT
        if TT == T:
            assert macs == facts["p4_real_gemms_fourier"]["value"]
        # ratio to the naive count tends to 2/T (page: NDC -> about 2NDC/T)
        assert abs(macs / naive - 2 / TT) <= 2 / TT ** 2 + 1e-15
    # parameters: w holds D*C/T values against D*C dense
    D, C = 3072, 768
    assert (D * C) / (D * C // T) == facts["parameter_reduction_T4"]["value"]


def test_fp32_rounding_scale_matches_page():
    # the page reports ~1e-7 differences in FP32; an fp32 evaluation of the
    # same definition lands at that scale against the fp64 oracle
    facts = _facts()
    X, w, _ = make_layer_inputs(256, 768, 768, "f32", seed=1, with_dy=False)
    W32 = oracle.dense_expand(w).astype(np.float32)
    Y32 = (X @ W32.T).astype(np.float64)
    err = _rel(Y32, oracle.forward_direct(X, w))
    assert facts["fp32_numerical_difference"]["value"] / 100 < err < facts["fp32_numerical_difference"]["value"] * 100


# --------------------------------------------------- a planted mistake fails

def test_pins_catch_planted_mistakes():
    """Plausible oracle mistakes (wrong orientation, dropped term) break the pins."""
    X = _rand((5, 16), 34)
    w = _rand((3, 4, 4), 35)
    ref = X @ _dense_by_scipy(w).T

    def wrong_orientation(Xv, wv):
        # block (d', c') = w[(s - t) mod T] instead of w[(t - s) mod T]
        Wt = np.block([[scipy.linalg.circulant(wv[d, c]).T for c in range(4)] for d in range(3)])
        return Xv @ Wt.T

    def dropped_shift(Xv, wv):
        w2 = wv.copy()
        w2[:, :, 3] = 0.0
        return oracle.forward_direct(Xv, w2)

    assert _rel(wrong_orientation(X, w), ref) > 1e-3
    assert _rel(dropped_shift(X, w), ref) > 1e-3


# ------------------------------------------------- fused epilogue (bias, GELU)

def test_gelu_matches_torch_and_closed_forms():
    torch = pytest.importorskip("torch")
    z = np.linspace(-8, 8, 1001)
    ref = torch.nn.functional.gelu(torch.tensor(z, dtype=torch.float64)).numpy()
    assert np.max(np.abs(oracle.gelu_erf(z) - ref)) < 1e-15
    assert oracle.gelu_erf(np.array([0.0]))[0] == 0.0
    # GELU(z) - GELU(-z) = z (Phi(z) + Phi(-z) = 1)
    assert np.max(np.abs(oracle.gelu_erf(z) - oracle.gelu_erf(-z) - z)) < 1e-14


def test_bias_act_forward_is_equivariant_and_reduces_to_forward():
    X = _rand((7, 24), 40)
    w = _rand((5, 6, 4), 41)
    b = _rand(5, 42)
    assert np.array_equal(oracle.forward_bias_act(X, w), oracle.forward_direct(X, w))
    Y = oracle.forward_bias_act(X, w, b, "gelu").reshape(7, 5, 4)
    Xr = np.roll(X.reshape(7, 6, 4), 1, axis=2).reshape(7, 24)
    Yr = oracle.forward_bias_act(Xr, w, b, "gelu").reshape(7, 5, 4)
    assert _rel(Yr, np.roll(Y, 1, axis=2)) < 1e-14
    # the bias is one value per output group, the same for all four elements
    Z = oracle.forward_bias_act(X, w, b) - oracle.forward_direct(X, w)
    assert np.allclose(Z.reshape(7, 5, 4), b[None, :, None], rtol=0, atol=1e-14)


def test_residual_forward_adds_after_the_activation_and_stays_equivariant():
    X = _rand((7, 24), 43)
    w = _rand((5, 6, 4), 44)
    b = _rand(5, 45)
    R = _rand((7, 20), 46)
    # a zero residual changes nothing; the residual is added after GELU, not inside it
    assert np.array_equal(oracle.forward_bias_act(X, w, b, "gelu", np.zeros((7, 20))),
                          oracle.forward_bias_act(X, w, b, "gelu"))
    Y = oracle.forward_bias_act(X, w, b, "gelu", R)
    assert _rel(Y - R, oracle.gelu_erf(oracle.forward_bias_act(X, w, b))) < 1e-14
    # the dense expansion, written out on this tiny case: Y = GELU(X Wd^T + b) + R
    Wd = np.zeros((20, 24))
    for d in range(5):
        for c in range(6):
            for t in range(4):
                for s in range(4):
                    Wd[4 * d + t, 4 * c + s] = w[d, c, (t - s) % 4]
    assert _rel(Y, oracle.gelu_erf(X @ Wd.T + np.repeat(b, 4)[None, :]) + R) < 1e-14
    # shifting the group index of the input and of the residual shifts the output
    Xr = np.roll(X.reshape(7, 6, 4), 1, axis=2).reshape(7, 24)
    Rr = np.roll(R.reshape(7, 5, 4), 1, axis=2).reshape(7, 20)
    Yr = oracle.forward_bias_act(Xr, w, b, "gelu", Rr).reshape(7, 5, 4)
    assert _rel(Yr, np.roll(Y.reshape(7, 5, 4), 1, axis=2)) < 1e-14

