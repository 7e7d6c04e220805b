"""Seeded randomized GPU parity against the fp64 oracle.

Shapes, groups, dtypes, forward tiles, the tail split, bias and activation
are drawn from a fixed seed, so every run checks the same cases.  Row counts
and channel counts are mostly ragged against every tile, group-channel
counts run from one upwards, and one case in four is a narrow layer over
16k-40k rows (launches of more than 256 tiles).  Every case checks
forward_ex (with the drawn epilogue), dX and dw through the C ABI (the
convolution: forward, dX and dpsi); bars as in the other parity tests
(max|gpu - ref| / max|ref| <= 1e-5 fp32, 3e-3 f16 storage).
"""
import numpy as np
import pytest

import oracle
from group_circulant_linear_amd.inputs import make_conv_inputs, make_layer_inputs

torch = pytest.importorskip("torch")
eq = pytest.importorskip("group_circulant_linear_amd.eqlin")

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 3e-3}
DEV = "cuda"
P4M_TABLE = oracle.p4m_table()

P4_TILES = ["112221", "111221", "112121", "222221", "212421", "112411", "212211", "122211", "112211", "112212",
            "112412", "111211", "2124211", "1122111", "1122211", "1112111", "112111", "1121111"]
ORDER8_TILES = ["112211", "112221", "111221", "212211", "122211", "1122111", "1222111", "2122111", "122241"]
CONV_TILES = ["112211", "112221", "111211", "212421", "111221"]


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.double().cpu().numpy()


def _linear_cases(n=96, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        g = [4, 8, "p4m"][i % 3]
        dt = ["f32", "f16"][(i // 3) % 2]
        T = 8 if g == "p4m" else g
        step = 2 if (dt == "f16" and T == 4) else 1          # f16 p4 needs even group-channel counts
        if i % 4 == 3:
            # many rows, narrow layers: launches of more than 256 tiles (the tail split's range)
            Cg = int(rng.integers(1, 12)) * step
            Dg = int(rng.integers(1, 12)) * step
            N = int(rng.integers(16000, 40000))
        else:
            Cg = int(rng.integers(1, 100)) * step
            Dg = int(rng.integers(1, 100)) * step
            N = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 3000))]))
        tiles = P4_TILES if T == 4 else ORDER8_TILES
        tile = "auto" if rng.random() < 0.3 else str(rng.choice(tiles))
        act = ["none", "gelu"][int(rng.integers(0, 2))]
        bias = bool(rng.integers(0, 2))
        split = str(int(rng.integers(0, 2)))
        cases.append((i, g, dt, N, T * Cg, T * Dg, tile, bias, act, split))
    return cases


def _conv_cases(n=30, seed=2025):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = ["f32", "f16"][i % 2]
        blk = 4 if dt == "f32" else 8                         # C' and D' multiples of this
        C = 4 * blk * int(rng.integers(1, 5))
        D = 4 * blk * int(rng.integers(1, 5))
        K = int(rng.choice([1, 3, 5, 7]))
        N, H, W = int(rng.integers(1, 4)), int(rng.integers(1, 21)), int(rng.integers(1, 21))
        tile = "auto" if rng.random() < 0.3 else str(rng.choice(CONV_TILES))
        act = ["none", "gelu"][int(rng.integers(0, 2))]
        bias = bool(rng.integers(0, 2))
        cases.append((i, dt, N, H, W, C, D, K, tile, bias, act))
    return cases


@pytest.mark.parametrize("i,g,dt,N,C,D,tile,bias,act,split", _linear_cases())
def test_random_linear(i, g, dt, N, C, D, tile, bias, act, split, monkeypatch):
    T = 8 if g == "p4m" else g
    print(f"random linear {i}: group={g} {dt} N={N} C={C} D={D} tile={tile} bias={bias} act={act} split={split}",
          flush=True)
    if tile != "auto":
        monkeypatch.setenv("EQLIN_FWD_TILE", tile)
    monkeypatch.setenv("EQLIN_FWD_SPLIT", split)
    X, w, dY = make_layer_inputs(N, C, D, dt, seed=100 + i, T=T)
    b = np.random.default_rng(200 + i).standard_normal(D // T).astype(X.dtype) if bias else None
    Wh = eq.eqlin_prepare_weights(dev(w), group="p4m" if g == "p4m" else None)
    Y = host(eq.eqlin_forward_ex(dev(X), Wh, dev(b) if bias else None, act))
    if g == "p4m":
        Z = oracle.forward_group(X, w, P4M_TABLE)
        dXr, dwr = oracle.dx_group(dY, w, P4M_TABLE), oracle.dw_group(dY, X, P4M_TABLE)
    else:
        Z = oracle.forward_direct(X, w)
        dXr, dwr = oracle.dx_direct(dY, w), oracle.dw_direct(dY, X, T)
    if bias:
        Z = Z + np.repeat(b.astype(np.float64), T)[None, :]
    ref = oracle.gelu_erf(Z) if act == "gelu" else Z
    assert rel_err(Y, ref) <= TOL[dt]
    dX, dw = eq.eqlin_backward(dev(dY), dev(X), Wh)
    assert rel_err(host(dX), dXr) <= TOL[dt]
    assert rel_err(host(dw), dwr) <= TOL[dt]


@pytest.mark.parametrize("i,dt,N,H,W,C,D,K,tile,bias,act", _conv_cases())
def test_random_conv(i, dt, N, H, W, C, D, K, tile, bias, act, monkeypatch):
    print(f"random conv {i}: {dt} N={N} H={H} W={W} C={C} D={D} K={K} tile={tile} bias={bias} act={act}", flush=True)
    if tile != "auto":
        monkeypatch.setenv("EQCONV_FWD_TILE", tile)
    X, psi, dY = make_conv_inputs(N, H, W, C, D, K, dt, seed=300 + i)
    b = np.random.default_rng(400 + i).standard_normal(D // 4).astype(X.dtype) if bias else None
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = host(eq.eqconv_forward(dev(X), P, bias=dev(b) if bias else None, act=act))
    assert rel_err(Y, oracle.conv_forward_bias_act(X, psi, b, act)) <= TOL[dt]
    dX, dpsi = eq.eqconv_backward(dev(dY), dev(X), P)
    assert rel_err(host(dX), oracle.conv_dx(dY, psi, H, W)) <= TOL[dt]
    assert rel_err(host(dpsi), oracle.conv_dw(dY, X, K)) <= TOL[dt]
