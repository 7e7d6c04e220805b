"""The allocation-free backward (eqlin_backward_noalloc) against eqlin_backward.

eqlin_backward_noalloc keeps the dw split partials in the library's static
per-device scratch instead of a caller workspace.  Its outputs are checked
against eqlin_backward's on the same inputs (bit for bit where its split
plan is not capped by the scratch size, else to the tolerance) and against
the fp64 oracle, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's partials).
"""
import numpy as np
import pytest

import oracle
from group_circulant_linear_amd.inputs import make_layer_inputs

torch = pytest.importorskip("torch")
eq = pytest.importorskip("group_circulant_linear_amd.eqlin")

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 3e-3}
DEV = "cuda"


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


def host(t):
    torch.cuda.synchronize()
    return t.double().cpu().numpy()


def say(*a):
    print(*a, flush=True)


def ref_dx_dw(dY, X, w, g):
    if g == "p4m":
        t = oracle.p4m_table()
        return oracle.dx_group(dY, w, t), oracle.dw_group(dY, X, t)
    return oracle.backward_direct(dY, X, w)


def capped(N, C, D, T, dt, lib):
    # eqlin_backward's workspace holds more than the scratch: the no-alloc plan has fewer splits
    n = 8 if T == "p4m" else T
    code = eq.group_code(T)
    need = lib.eqlin_backward_workspace_bytes(N, C, D, code, 0 if dt == "f32" else 1)
    return need > eq.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("g", [4, 8, "p4m"])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_noalloc_backward_matches_backward_twice(dt, g):
    lib = eq.load_library()
    n = 8 if g == "p4m" else g
    # first a ViT-B attention layer, then a smaller ragged one on the same scratch
    for (N, C, D) in ((12608, 768, 768), (1001, 8 * 20, 8 * 12)):
        say(f"noalloc group={g} {dt} N={N} C={C} D={D}")
        X, w, dY = make_layer_inputs(N, C, D, dt, seed=31, T=n)
        tX, tw, tdY = (torch.from_numpy(a).to(DEV) for a in (X, w, dY))
        Wh = eq.eqlin_prepare_weights(tw, group=None if g != "p4m" else "p4m")
        dX_ref, dw_ref = eq.eqlin_backward(tdY, tX, Wh)
        dX = torch.full((N, C), float("nan"), dtype=tX.dtype, device=DEV)
        dw = torch.full((D // n, C // n, n), float("nan"), dtype=torch.float32, device=DEV)
        eq.eqlin_backward_noalloc(tdY, tX, Wh, dX, dw)
        torch.cuda.synchronize()
        e_dx = rel_err(host(dX), host(dX_ref).astype(np.float64))
        e_dw = rel_err(host(dw), host(dw_ref).astype(np.float64))
        say(f"  vs eqlin_backward: dX {e_dx:.2e}  dw {e_dw:.2e}  capped={capped(N, C, D, g, dt, lib)}")
        assert torch.equal(dX, dX_ref)                       # dX never uses the scratch
        if not capped(N, C, D, g, dt, lib):
            assert torch.equal(dw, dw_ref)
        assert e_dw <= TOL[dt]
        dXr, dwr = ref_dx_dw(dY, X, w, g)
        assert rel_err(host(dX), dXr) <= TOL[dt] and rel_err(host(dw), dwr) <= TOL[dt]


def test_noalloc_dx_only_and_empty_batch():
    X, w, dY = make_layer_inputs(300, 64, 96, "f32", seed=32)
    tX, tw, tdY = (torch.from_numpy(a).to(DEV) for a in (X, w, dY))
    Wh = eq.eqlin_prepare_weights(tw)
    dX = torch.empty((300, 64), device=DEV)
    eq.eqlin_backward_noalloc(tdY, None, Wh, dX, None)
    assert torch.equal(dX, eq.eqlin_backward_dx(tdY, Wh))
    # empty batch: dw written as zeros, no partials read
    dw = torch.full((24, 16, 4), float("nan"), device=DEV)
    eq.eqlin_backward_noalloc(tdY[:0], tX[:0], Wh, None, dw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0
