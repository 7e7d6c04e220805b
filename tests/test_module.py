"""FlashEQLinear: the plug-and-play module over the C ABI (GPU), and its host-side
pieces (CPU): construction, state-dict conversion, dense view, no CPU fallback."""
import numpy as np
import pytest

import oracle
from group_circulant_linear_amd.inputs import make_layer_inputs

torch = pytest.importorskip("torch")
from group_circulant_linear_amd.module import FlashEQLinear, convert_state_dict  # noqa: E402


@pytest.mark.parametrize("g", [4, 8, "p4m"])
def test_dense_view_matches_oracle_expansion(g):
    m = FlashEQLinear(3 * 8, 5 * 8, group=g)
    W = m.dense_weight().detach().double().numpy()
    w = m.w.detach().double().numpy()
    ref = oracle.dense_expand_group(w, oracle.p4m_table()) if g == "p4m" else oracle.dense_expand(w)
    assert np.array_equal(W, ref)


def test_from_naive_copies_parameters_and_rejects_other_groups():
    w = torch.randn(5, 3, 4)
    m = FlashEQLinear.from_naive(w)
    assert (m.in_features, m.out_features, m.group_size) == (12, 20, 4)
    assert torch.equal(m.w.detach(), w)
    m8 = FlashEQLinear.from_naive(torch.randn(5, 3, 8))
    assert (m8.in_features, m8.out_features, m8.group_size) == (24, 40, 8)
    mm = FlashEQLinear.from_naive(torch.randn(5, 3, 8), group="p4m")
    assert (mm.group, mm.group_size) == (108, 8) and "p4m" in mm.extra_repr()
    with pytest.raises(ValueError):
        FlashEQLinear.from_naive(torch.randn(5, 3, 6))
    with pytest.raises(ValueError):
        FlashEQLinear.from_naive(torch.randn(5, 3, 4), group="p4m")
    with pytest.raises(ValueError):
        FlashEQLinear(10, 8)
    with pytest.raises(ValueError):
        FlashEQLinear(12, 16, group=8)


def test_convert_state_dict_renames_only_keys():
    sd = {"blocks.0.mlp.fc1.weight_vec": torch.ones(2, 2, 4), "blocks.0.norm.weight": torch.ones(3)}
    out = convert_state_dict(sd, {"weight_vec": "w"})
    assert set(out) == {"blocks.0.mlp.fc1.w", "blocks.0.norm.weight"}
    assert out["blocks.0.mlp.fc1.w"] is sd["blocks.0.mlp.fc1.weight_vec"]


def test_no_cpu_fallback():
    m = FlashEQLinear(16, 16)
    with pytest.raises(ValueError):
        m(torch.randn(3, 16))


@pytest.mark.gpu
@pytest.mark.parametrize("g", [4, 8, "p4m"])
@pytest.mark.parametrize("dt,tol", [("f32", 1e-5), ("f16", 3e-3)])
def test_module_forward_backward_matches_oracle(dt, tol, g):
    B, S, C, D = 3, 197, 96, 160
    X, w, dY = make_layer_inputs(B * S, C, D, dt, seed=11, T=8 if g == "p4m" else g)
    m = FlashEQLinear.from_naive(torch.from_numpy(w).cuda(), group=g)
    Xt = torch.from_numpy(X).cuda().reshape(B, S, C).requires_grad_(True)
    Y = m(Xt)
    assert Y.shape == (B, S, D)
    Y.backward(torch.from_numpy(dY).cuda().reshape(B, S, D))
    torch.cuda.synchronize()
    if g == "p4m":
        t = oracle.p4m_table()
        Yr, dXr, dwr = oracle.forward_group(X, w, t), oracle.dx_group(dY, w, t), oracle.dw_group(dY, X, t)
    else:
        Yr = oracle.forward_direct(X, w)
        dXr, dwr = oracle.backward_direct(dY, X, w)

    def rel(a, b):
        return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
    assert rel(Y.detach().double().cpu().numpy().reshape(-1, D), Yr) <= tol
    assert rel(Xt.grad.double().cpu().numpy().reshape(-1, C), dXr) <= tol
    # the parameter gradient is cast to the parameter dtype; f16 adds one rounding
    assert rel(m.w.grad.double().cpu().numpy(), dwr) <= tol


@pytest.mark.gpu
def test_spectra_cache_follows_weight_updates():
    X, w, _ = make_layer_inputs(300, 64, 64, "f32", seed=12, with_dy=False)
    m = FlashEQLinear.from_naive(torch.from_numpy(w).cuda())
    Xt = torch.from_numpy(X).cuda()
    Y1 = m(Xt).detach().clone()
    p1 = m._cache.prepared
    Y1b = m(Xt)
    assert m._cache.prepared is p1            # reused: same weight version
    assert torch.equal(Y1, Y1b)
    with torch.no_grad():
        m.w.mul_(2.0)                         # in-place update bumps the version
    Y2 = m(Xt)
    assert m._cache.prepared is not p1
    torch.cuda.synchronize()
    assert torch.allclose(Y2, 2 * Y1, rtol=1e-6, atol=1e-6)


@pytest.mark.gpu
def test_sgd_step_through_module():
    torch.manual_seed(0)
    m = FlashEQLinear(128, 64).cuda()
    opt = torch.optim.SGD(m.parameters(), lr=0.1)
    X = torch.randn(512, 128, device="cuda")
    target = torch.randn(512, 64, device="cuda")
    losses = []
    for _ in range(5):
        opt.zero_grad()
        loss = torch.nn.functional.mse_loss(m(X), target)
        loss.backward()
        opt.step()
        losses.append(loss.item())
    assert losses[-1] < losses[0]


def test_conv_dense_filter_matches_the_oracle_cpu():
    # the dense filter bank of the p4 convolution (used by the benchmark's
    # dense comparator) is the oracle's, entry for entry
    import numpy as np
    import oracle
    torch = pytest.importorskip("torch")
    from group_circulant_linear_amd.module import conv_dense_filter
    psi = np.random.default_rng(0).standard_normal((3, 2, 5, 5, 4))
    got = conv_dense_filter(torch.from_numpy(psi)).numpy()
    assert np.array_equal(got, oracle.conv_dense_filter(psi))
