"""Pins for the oracle's group-convolution routines (any Cayley table) and the
p4m (dihedral, order 8) transform, independent of the oracle's own code paths.

The summary gives no formulas for groups other than p4 ("Limitations" names
them as future work).  The oracle takes the plain reading: the group
convolution W[d'T + g, c'T + h] = w[d', c', h^-1 g], which for C_T is the
circulant of the pinned cyclic routines.  The pins below fix it by
mathematics: a faithful matrix realisation of the dihedral group, the cyclic
case (already pinned to scipy / numpy FFT), group equivariance, the reduction
of rotation-only weights to p4, torch autograd, and the representation theory
of p4m (homomorphisms, Schur orthogonality, Fourier inversion, convolution
theorem).
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _inv(table):
    return np.array([int(np.nonzero(table[i] == 0)[0][0]) for i in range(len(table))])


# ------------------------------------------------------------ the group

def test_p4m_table_is_the_symmetry_group_of_the_square():
    t = oracle.p4m_table()
    # faithful realisation: the integer 2 x 2 matrices of the square's symmetries
    R = np.array([[0, -1], [1, 0]])
    S = np.array([[1, 0], [0, -1]])
    M = [np.linalg.matrix_power(R, u % 4) @ np.linalg.matrix_power(S, u // 4) for u in range(8)]
    assert len({m.tobytes() for m in M}) == 8
    for i in range(8):
        for j in range(8):
            assert np.array_equal(M[i] @ M[j], M[t[i, j]])
    # presentation r^4 = s^2 = e, s r s = r^-1; non-abelian; element orders 1, 2 (x5), 4 (x2)
    r, s = 1, 4
    assert t[t[t[r, r], r], r] == 0 and t[s, s] == 0 and t[t[s, r], s] == 3
    assert not np.array_equal(t, t.T)
    orders = []
    for g in range(8):
        k, x = 1, g
        while x != 0:
            x, k = t[x, g], k + 1
        orders.append(k)
    assert sorted(orders) == [1, 2, 2, 2, 2, 2, 4, 4]


def test_cyclic_table():
    t = oracle.cyclic_table(5)
    assert t[3, 4] == 2 and np.array_equal(t, t.T) and np.array_equal(t[0], np.arange(5))


# ------------------------------------------- group convolution routines

@pytest.mark.parametrize("T", [3, 4, 8])
def test_group_routines_with_cyclic_table_are_the_circulant_layer(T):
    N, Cp, Dp = 6, 3, 4
    X, w, dY = _rand((N, Cp * T), 1), _rand((Dp, Cp, T), 2), _rand((N, Dp * T), 3)
    t = oracle.cyclic_table(T)
    assert _rel(oracle.forward_group(X, w, t), oracle.forward_direct(X, w)) < 1e-14
    assert _rel(oracle.dx_group(dY, w, t), oracle.dx_direct(dY, w)) < 1e-14
    assert _rel(oracle.dw_group(dY, X, t), oracle.dw_direct(dY, X, T)) < 1e-14
    assert np.array_equal(oracle.dense_expand_group(w, t), oracle.dense_expand(w))


def _left_translate(Z, a, table):
    """(L_a z)(g) = z(a^-1 g) on every group block of Z [N][G*T]."""
    T = len(table)
    inv = _inv(table)
    N = Z.shape[0]
    Z3 = Z.reshape(N, -1, T)
    src = [table[inv[a], g] for g in range(T)]
    return Z3[:, :, src].reshape(N, -1)


def test_p4m_forward_is_equivariant_under_every_element():
    t = oracle.p4m_table()
    X, w = _rand((5, 3 * 8), 4), _rand((2, 3, 8), 5)
    Y = oracle.forward_group(X, w, t)
    for a in range(8):
        Ya = oracle.forward_group(_left_translate(X, a, t), w, t)
        assert _rel(Ya, _left_translate(Y, a, t)) < 1e-14


def test_planted_right_multiplication_breaks_equivariance():
    # the same layer with g u^-1 and u^-1 g confused is not left-equivariant
    t = oracle.p4m_table()
    inv = _inv(t)
    X, w = _rand((4, 2 * 8), 6), _rand((3, 2, 8), 7)

    def wrong(Xm):
        X3 = Xm.reshape(Xm.shape[0], 2, 8)
        Y3 = np.zeros((Xm.shape[0], 3, 8))
        for u in range(8):
            src = [t[inv[u], g] for g in range(8)]
            Y3 += np.einsum("nch,dc->ndh", X3[:, :, src], w[:, :, u])
        return Y3.reshape(Xm.shape[0], -1)
    Yw = wrong(X)
    errs = [_rel(wrong(_left_translate(X, a, t)), _left_translate(Yw, a, t)) for a in range(8)]
    assert max(errs) > 1e-3
    assert _rel(Yw, oracle.forward_group(X, w, t)) > 1e-3


def test_p4m_rotation_only_weights_reduce_to_p4():
    # w supported on rotations: the rotation coset sees the p4 circulant of w,
    # the reflection coset the p4 circulant of w reversed (s r^k s = r^-k)
    t = oracle.p4m_table()
    N, Cp, Dp = 7, 3, 2
    X = _rand((N, Cp * 8), 8)
    w4 = _rand((Dp, Cp, 4), 9)
    w = np.concatenate([w4, np.zeros_like(w4)], axis=2)
    Y3 = oracle.forward_group(X, w, t).reshape(N, Dp, 8)
    X3 = X.reshape(N, Cp, 8)
    Yrot = oracle.forward_direct(X3[:, :, :4].reshape(N, -1), w4).reshape(N, Dp, 4)
    wrev = w4[:, :, [0, 3, 2, 1]]
    Yref = oracle.forward_direct(X3[:, :, 4:].reshape(N, -1), wrev).reshape(N, Dp, 4)
    assert _rel(Y3[:, :, :4], Yrot) < 1e-14
    assert _rel(Y3[:, :, 4:], Yref) < 1e-14


def test_p4m_gradients_match_torch_autograd():
    torch = pytest.importorskip("torch")
    t = oracle.p4m_table()
    inv = _inv(t)
    N, Cp, Dp = 9, 4, 3
    X, w, dY = _rand((N, Cp * 8), 10), _rand((Dp, Cp, 8), 11), _rand((N, Dp * 8), 12)
    idx = torch.tensor([[t[inv[h], g] for h in range(8)] for g in range(8)], dtype=torch.long)
    wt = torch.tensor(w, requires_grad=True)
    Wd = wt[:, :, idx].permute(0, 2, 1, 3).reshape(Dp * 8, Cp * 8)
    Xt = torch.tensor(X, requires_grad=True)
    Yt = torch.nn.functional.linear(Xt, Wd)
    Yt.backward(torch.tensor(dY))
    assert _rel(Yt.detach().numpy(), oracle.forward_group(X, w, t)) < 1e-14
    assert _rel(oracle.dx_group(dY, w, t), Xt.grad.numpy()) < 1e-13
    assert _rel(oracle.dw_group(dY, X, t), wt.grad.numpy()) < 1e-13
    assert np.array_equal(oracle.dense_expand_group(w, t), Wd.detach().numpy())


def test_p4m_adjoint_identities():
    t = oracle.p4m_table()
    X, w, dY = _rand((11, 16), 13), _rand((3, 2, 8), 14), _rand((11, 24), 15)
    Y = oracle.forward_group(X, w, t)
    dX = oracle.dx_group(dY, w, t)
    dw = oracle.dw_group(dY, X, t)
    a = float(np.sum(dY * Y))
    assert abs(a - float(np.sum(dX * X))) < 1e-12 * abs(a) + 1e-12
    assert abs(a - float(np.sum(dw * w))) < 1e-12 * abs(a) + 1e-12


# ------------------------------------------------------- the transform

def test_p4m_irreps_homomorphisms_and_schur_orthogonality():
    t = oracle.p4m_table()
    chars, E = oracle.p4m_irreps()
    for i in range(8):
        for j in range(8):
            assert np.allclose(chars[i] * chars[j], chars[t[i, j]])
            assert np.allclose(E[i] @ E[j], E[t[i, j]])
    # characters: sum_g chi_a chi_b = 8 delta_ab; matrix coefficients of E: 8/2 delta delta
    assert np.allclose(chars.T @ chars, 8 * np.eye(4))
    Ef = E.reshape(8, 4)
    assert np.allclose(Ef.T @ Ef, 4 * np.eye(4))
    assert np.allclose(chars.T @ Ef, 0)
    # dimensions: 4 * 1^2 + 2^2 = |G|
    assert 4 * 1 + 2 * 2 == 8


def _p4m_inverse(P):
    """f(g) = (1/8) [sum_chi chi(g) f_chi + 2 tr(E(g)^T F)]  (Fourier inversion)."""
    chars, E = oracle.p4m_irreps()
    return (P[..., :4] @ chars.T + 2 * P[..., 4:] @ E.reshape(8, 4).T) / 8


def _irrep_product(A, B):
    """Per representation: 1-D pointwise, 2 x 2 block A @ B."""
    out = np.empty(np.broadcast(A, B).shape)
    out[..., :4] = A[..., :4] * B[..., :4]
    out[..., 4:] = np.einsum("...ik,...kj->...ij", A[..., 4:].reshape(A.shape[:-1] + (2, 2)),
                             B[..., 4:].reshape(B.shape[:-1] + (2, 2))).reshape(out.shape[:-1] + (4,))
    return out


def test_p4m_planes_inversion_and_convolution_theorem():
    t = oracle.p4m_table()
    N, Cp, Dp = 5, 3, 2
    X, w = _rand((N, Cp * 8), 16), _rand((Dp, Cp, 8), 17)
    Pw = oracle.p4m_planes(w)
    assert _rel(_p4m_inverse(Pw), w) < 1e-14
    Y3 = oracle.forward_group(X, w, t).reshape(N, Dp, 8)
    PX = oracle.p4m_planes(X.reshape(N, Cp, 8))                   # [N][C'][8]
    PY = np.zeros((N, Dp, 8))
    for d in range(Dp):
        for c in range(Cp):
            PY[:, d] += _irrep_product(PX[:, c], Pw[d, c][None, :])   # Y_hat = X_hat w_hat
    assert _rel(_p4m_inverse(PY), Y3) < 1e-13
    assert _rel(oracle.p4m_planes(Y3), PY) < 1e-13


def test_p4m_backward_spectra():
    # dX uses the spectrum of w'(u) = w(u^-1): the 2 x 2 block transposed;
    # dw_hat = X_hat^T dY_hat per (n, d', c') summed over n
    t = oracle.p4m_table()
    inv = _inv(t)
    w = _rand((2, 3, 8), 18)
    P = oracle.p4m_planes(w)
    Pinv = oracle.p4m_planes(w[:, :, inv])
    PT = P.copy()
    PT[..., 5], PT[..., 6] = P[..., 6], P[..., 5]
    assert _rel(Pinv, PT) < 1e-14
    N = 6
    X, dY = _rand((N, 3 * 8), 19), _rand((N, 2 * 8), 20)
    dw = oracle.dw_group(dY, X, t)
    PX = oracle.p4m_planes(X.reshape(N, 3, 8))
    PG = oracle.p4m_planes(dY.reshape(N, 2, 8))
    PXT = PX.copy()
    PXT[..., 5], PXT[..., 6] = PX[..., 6], PX[..., 5]
    Pdw = np.zeros((2, 3, 8))
    for d in range(2):
        for c in range(3):
            Pdw[d, c] = _irrep_product(PXT[:, c], PG[:, d]).sum(axis=0)
    assert _rel(oracle.p4m_planes(dw), Pdw) < 1e-13
