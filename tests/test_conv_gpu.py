"""GPU parity of the p4 group convolution (through the C ABI) against the fp64
oracle.

Metric: max|gpu - ref| / max|ref|; bars 1e-5 (fp32) and 3e-3 (f16 storage with
fp32 accumulation), as for the linear layer.  Small maps span several tiles
with ragged pixel and channel tails, every compiled tile and K = 1, 3, 5, 7;
the full-size workload is checked on sampled pixels (forward, dX) and sampled
filter-gradient entries, computed one by one by the oracle.
"""

import numpy as np
import pytest

import oracle
from group_circulant_linear_amd.inputs import CONV_WORKLOADS, make_conv_inputs, make_conv_range_inputs

torch = pytest.importorskip("torch")
eq = pytest.importorskip("group_circulant_linear_amd.eqlin")

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 3e-3}
DEV = "cuda"
TILES = ["112211", "112221", "111211", "212421", "212431", "112241", "111221"]


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.double().cpu().numpy()


def say(*a):
    print(*a, flush=True)


# (dtype, N, H, W, C, D, K): pixel counts off every tile height, C' and D' at
# the smallest legal multiples and above, output widths off the tile widths
CASES = [
    ("f32", 2, 7, 9, 16, 32, 3),
    ("f32", 1, 13, 11, 32, 16, 5),
    ("f32", 3, 5, 6, 16, 16, 1),
    ("f32", 1, 20, 19, 64, 48, 3),
    ("f32", 2, 9, 9, 48, 80, 7),
    ("f32", 1, 3, 4, 16, 16, 5),          # filter wider than the image
    ("f16", 2, 7, 9, 32, 64, 3),
    ("f16", 1, 12, 10, 64, 32, 5),
    ("f16", 2, 6, 6, 32, 32, 1),
    ("f16", 1, 17, 15, 96, 160, 3),
]


@pytest.mark.parametrize("dt,N,H,W,C,D,K", CASES)
def test_forward_matches_oracle(dt, N, H, W, C, D, K):
    say(f"conv forward {dt} N={N} H={H} W={W} C={C} D={D} K={K}")
    X, psi, _ = make_conv_inputs(N, H, W, C, D, K, dt, seed=1, with_dy=False)
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = eq.eqconv_forward(dev(X), P)
    assert rel_err(host(Y), oracle.conv_forward(X, psi)) < TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("tile", TILES)
def test_forward_every_tile(dt, tile, monkeypatch):
    N, H, W, C, D, K = 2, 11, 13, 32, 96, 3
    say(f"conv forward tile {tile} {dt}")
    X, psi, _ = make_conv_inputs(N, H, W, C, D, K, dt, seed=2, with_dy=False)
    ref = oracle.conv_forward(X, psi)
    monkeypatch.setenv("EQCONV_FWD_TILE", tile)
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = eq.eqconv_forward(dev(X), P)
    assert rel_err(host(Y), ref) < TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_forward_bias_gelu(dt):
    N, H, W, C, D, K = 1, 9, 7, 32, 64, 3
    say(f"conv forward bias+gelu {dt}")
    X, psi, _ = make_conv_inputs(N, H, W, C, D, K, dt, seed=3, with_dy=False)
    b = (np.random.default_rng(4).standard_normal(D // 4) * 0.5).astype(X.dtype)
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = eq.eqconv_forward(dev(X), P, bias=dev(b), act="gelu")
    assert rel_err(host(Y), oracle.conv_forward_bias_act(X, psi, b, "gelu")) < TOL[dt]


@pytest.mark.parametrize("dt,N,H,W,C,D,K", CASES)
def test_backward_matches_oracle(dt, N, H, W, C, D, K):
    say(f"conv backward {dt} N={N} H={H} W={W} C={C} D={D} K={K}")
    X, psi, dY = make_conv_inputs(N, H, W, C, D, K, dt, seed=5)
    P = eq.eqconv_prepare_weights(dev(psi))
    dX, dpsi = eq.eqconv_backward(dev(dY), dev(X), P)
    assert rel_err(host(dX), oracle.conv_dx(dY, psi, H, W)) < TOL[dt]
    assert rel_err(host(dpsi), oracle.conv_dw(dY, X, K)) < TOL[dt]
    # each output alone gives the same values
    dX2, none = eq.eqconv_backward(dev(dY), None, P, need_dpsi=False)
    none2, dpsi2 = eq.eqconv_backward(dev(dY), dev(X), P, need_dx=False)
    assert none is None and none2 is None
    assert torch.equal(dX2, dX) and torch.equal(dpsi2, dpsi)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_equivariance_on_the_gpu(dt):
    # turning the input image by R^g and rolling the rotation axis by g turns
    # and rolls the output (to the summation-order rounding of the kernel)
    N, S, C, D, K = 2, 15, 32, 32, 3
    say(f"conv equivariance {dt}")
    X, psi, _ = make_conv_inputs(N, S, S, C, D, K, dt, seed=6, with_dy=False)
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = host(eq.eqconv_forward(dev(X), P))

    def turn(z, g):
        z5 = z.reshape(N, S, S, -1, 4)
        return np.ascontiguousarray(np.roll(np.rot90(z5, g, axes=(1, 2)), g, axis=4)).reshape(N, S, S, -1)

    for g in (1, 2, 3):
        Yg = host(eq.eqconv_forward(dev(turn(X, g)), P))
        assert rel_err(Yg, turn(Y, g)) < TOL[dt]


def test_empty_batch():
    X, psi, dY = make_conv_inputs(1, 4, 4, 16, 16, 3, "f32", seed=7)
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = eq.eqconv_forward(dev(X[:0]), P)
    assert tuple(Y.shape) == (0, 4, 4, 16)
    dX, dpsi = eq.eqconv_backward(dev(dY[:0]), dev(X[:0]), P)
    assert dX.shape[0] == 0
    assert torch.count_nonzero(dpsi).item() == 0


def test_one_by_one_equals_the_linear_layer():
    # K = 1 runs the gathered layer with the centre blocks only: the same
    # values as the linear layer's forward on the flattened map
    X, psi, _ = make_conv_inputs(2, 9, 7, 32, 48, 1, "f32", seed=8, with_dy=False)
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = host(eq.eqconv_forward(dev(X), P))
    Wl = eq.eqlin_prepare_weights(dev(np.ascontiguousarray(psi[:, :, 0, 0, :])))
    Yl = host(eq.eqlin_forward(dev(X.reshape(-1, 32)), Wl))
    assert rel_err(Y.reshape(-1, 48), Yl) < 1e-6


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_full_size_workload_sampled(dt):
    L = CONV_WORKLOADS["p4conv"].layers[0]
    say(f"conv full size {dt} N={L.N} H={L.H} W={L.W} C={L.C} D={L.D} K={L.K}")
    X, psi, dY = make_conv_inputs(L.N, L.H, L.W, L.C, L.D, L.K, dt, seed=0)
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = eq.eqconv_forward(dev(X), P)
    dX, dpsi = eq.eqconv_backward(dev(dY), dev(X), P)
    rng = np.random.default_rng(9)
    npix = L.N * L.H * L.W
    # image corners and edges plus random pixels
    corners = [0, L.W - 1, (L.H - 1) * L.W, L.H * L.W - 1, npix - 1, npix - L.W]
    pix = np.concatenate([corners, rng.integers(0, npix, 40)])
    Yh = host(Y.reshape(npix, -1)[torch.from_numpy(pix).to(DEV)])
    assert rel_err(Yh, oracle.conv_forward_pixels(X, psi, pix)) < TOL[dt]
    dXh = host(dX.reshape(npix, -1)[torch.from_numpy(pix).to(DEV)])
    assert rel_err(dXh, oracle.conv_dx_pixels(dY, psi, L.H, L.W, pix)) < TOL[dt]
    idx = [tuple(int(v) for v in (rng.integers(0, L.D // 4), rng.integers(0, L.C // 4), rng.integers(0, L.K),
                                  rng.integers(0, L.K), rng.integers(0, 4))) for _ in range(24)]
    got = host(dpsi)[tuple(np.array(idx).T)]
    ref = oracle.conv_dw_entries(dY, X, L.K, idx)
    # the sampled entries are compared against the largest sampled magnitude
    assert rel_err(got, ref) < TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_wide_filter_on_a_small_map(dt):
    # C = 1024, K = 5: 6400 gathered group channels (200 f32 / 100 f16 stages), D' = 72
    N, H, W, C, D, K = 1, 6, 7, 1024, 288, 5
    say(f"conv wide {dt}")
    X, psi, dY = make_conv_inputs(N, H, W, C, D, K, dt, seed=12)
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = eq.eqconv_forward(dev(X), P)
    dX, dpsi = eq.eqconv_backward(dev(dY), dev(X), P)
    assert rel_err(host(Y), oracle.conv_forward(X, psi)) < TOL[dt]
    assert rel_err(host(dX), oracle.conv_dx(dY, psi, H, W)) < TOL[dt]
    assert rel_err(host(dpsi), oracle.conv_dw(dY, X, K)) < TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("K", [9, 11, 13, 15])
def test_large_filters(dt, K):
    # the largest filters the header allows (odd K <= 15: (K^2 - 1) / 4 orbits,
    # up to 56), on maps narrower and shorter than the filter
    N, H, W, C, D = 2, 9, 18, 32, 32
    say(f"conv large filter {dt} K={K}")
    X, psi, dY = make_conv_inputs(N, H, W, C, D, K, dt, seed=20 + K)
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = eq.eqconv_forward(dev(X), P)
    dX, dpsi = eq.eqconv_backward(dev(dY), dev(X), P)
    assert rel_err(host(Y), oracle.conv_forward(X, psi)) < TOL[dt]
    assert rel_err(host(dX), oracle.conv_dx(dY, psi, H, W)) < TOL[dt]
    assert rel_err(host(dpsi), oracle.conv_dw(dY, X, K)) < TOL[dt]


@pytest.mark.parametrize("tile", ["112211", "112221", "212421"])
def test_tail_split(tile, monkeypatch):
    # fp32: 301 row tiles over the 256 CUs, so the last 45 run as half-height
    # workgroups; the last tile has rows in its first half only.  Forward, the
    # separate dX launch and the fused backward (dX and dpsi), split and
    # whole, against the oracle.
    BM = 128 if tile == "212421" else 64
    N, H, W = (4 if BM == 128 else 2), 97, 99
    C, D, K = 32, 4 * BM, 3
    say(f"conv tail split tile {tile} N={N} H={H} W={W} C={C} D={D}")
    X, psi, dY = make_conv_inputs(N, H, W, C, D, K, "f32", seed=18)
    monkeypatch.setenv("EQCONV_FWD_TILE", tile)
    P = eq.eqconv_prepare_weights(dev(psi))
    ref, dref = oracle.conv_forward(X, psi), oracle.conv_dx(dY, psi, H, W)
    pref = oracle.conv_dw(dY, X, K)
    for split in ("1", "0"):
        monkeypatch.setenv("EQLIN_FWD_SPLIT", split)
        Y = eq.eqconv_forward(dev(X), P)
        dX, _ = eq.eqconv_backward(dev(dY), None, P, need_dpsi=False)
        assert rel_err(host(Y), ref) < TOL["f32"]
        assert rel_err(host(dX), dref) < TOL["f32"]
        dX2, dpsi = eq.eqconv_backward(dev(dY), dev(X), P)
        assert rel_err(host(dX2), dref) < TOL["f32"]
        assert rel_err(host(dpsi), pref) < TOL["f32"]


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_module_autograd_matches_oracle(dt):
    from group_circulant_linear_amd.module import FlashEQConv2d
    N, H, W, C, D, K = 2, 8, 10, 32, 32, 3
    tdt, tol = (torch.float32, TOL["f32"]) if dt == "f32" else (torch.float16, TOL["f16"])
    say(f"conv module autograd {dt}")
    torch.manual_seed(0)
    m = FlashEQConv2d(C, D, K, device=DEV, dtype=tdt)
    X = torch.randn(N, H, W, C, device=DEV).to(tdt).requires_grad_(True)
    Y = m(X)
    dY = torch.randn_like(Y)
    Y.backward(dY)
    psi = m.psi.detach().double().cpu().numpy()
    Xn, dYn = X.detach().double().cpu().numpy(), dY.double().cpu().numpy()
    assert rel_err(host(Y.detach()), oracle.conv_forward(Xn, psi)) < tol
    assert rel_err(host(X.grad), oracle.conv_dx(dYn, psi, H, W)) < tol
    assert rel_err(host(m.psi.grad), oracle.conv_dw(dYn, Xn, K)) < tol
    # the cached spectra follow an in-place update of the filter
    with torch.no_grad():
        m.psi.mul_(2.0)
    Y2 = m(X.detach())
    assert rel_err(host(Y2.detach()), 2.0 * oracle.conv_forward(Xn, psi)) < tol


@pytest.mark.parametrize("regime", ["large", "small"])
def test_f16_operand_range(regime):
    # binary16 inputs up to 6e4 (rotation groups of equal sign, whose plain
    # zero-frequency sums pass 65504) and just above the smallest normal; the
    # f16 Fourier operands are scaled into range before rounding
    N, H, W, C, D, K = 2, 9, 11, 32, 64, 3
    say(f"conv f16 range {regime}")
    X, psi, dY = make_conv_range_inputs(N, H, W, C, D, K, regime, seed=3)
    Yr, dXr, dpr = oracle.conv_forward(X, psi), oracle.conv_dx(dY, psi, H, W), oracle.conv_dw(dY, X, K)
    assert np.max(np.abs(Yr)) < 65504 and np.max(np.abs(dXr)) < 65504
    P = eq.eqconv_prepare_weights(dev(psi))
    Y = host(eq.eqconv_forward(dev(X), P))
    dX, dpsi = eq.eqconv_backward(dev(dY), dev(X), P)
    dX, dpsi = host(dX), host(dpsi)
    errs = (rel_err(Y, Yr), rel_err(dX, dXr), rel_err(dpsi, dpr))
    say(f"  Y {errs[0]:.2e}  dX {errs[1]:.2e}  dpsi {errs[2]:.2e}")
    assert all(np.all(np.isfinite(a)) for a in (Y, dX, dpsi))
    assert max(errs) <= TOL["f16"], errs
