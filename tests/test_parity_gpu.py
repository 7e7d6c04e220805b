"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every group the library implements is covered: the p4 rotation group
(cyclic, order 4), the cyclic group C8 and the dihedral group p4m (order 8).

Metric: max|gpu - ref| / max|ref| over the compared outputs.  Bars: 1e-5 for
fp32, 3e-3 for f16 storage with fp32 accumulation.  Small shapes span several
tiles plus ragged row / column / k tails and are compared element by element;
the full-size workloads are compared whole where the oracle takes seconds
(ViT-B attention forward and backward) and on sampled rows otherwise.
"""
import numpy as np
import pytest

import oracle
from group_circulant_linear_amd.inputs import WORKLOADS, make_layer_inputs, make_range_inputs

torch = pytest.importorskip("torch")
eq = pytest.importorskip("group_circulant_linear_amd.eqlin")

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 3e-3}
DEV = "cuda"


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


P4M_TABLE = oracle.p4m_table()
GROUPS = [4, 8, "p4m"]


def order(g):
    return 8 if g == "p4m" else g


def prep(w, g):
    return eq.eqlin_prepare_weights(dev(w), group=None if g != "p4m" else "p4m")


def ref_forward(X, w, g):
    return oracle.forward_group(X, w, P4M_TABLE) if g == "p4m" else oracle.forward_direct(X, w)


def ref_dx(dY, w, g):
    return oracle.dx_group(dY, w, P4M_TABLE) if g == "p4m" else oracle.dx_direct(dY, w)


def ref_dw(dY, X, g):
    return oracle.dw_group(dY, X, P4M_TABLE) if g == "p4m" else oracle.dw_direct(dY, X, g)


# --------------------------------------------------------------------- a1

def slot_group(s, dt, T):
    """Group channel held by slot s of a 64-byte stage block (the header's g(s))."""
    V = 4 if dt == "f32" else 8
    gb = T * (4 if dt == "f32" else 2)
    G = 1 if gb >= 16 else 16 // gb
    return G * (s // V + 4 * ((s % V) // G)) + (s % V) % G


def test_slot_group_formula_matches_header_for_p4():
    # the general formula reduces to the two p4 formulas the header spells out
    for s in range(16):
        assert slot_group(s, "f32", 4) == (s >> 2) + 4 * (s & 3)
    for s in range(32):
        assert slot_group(s, "f16", 4) == 2 * ((s >> 3) + 4 * ((s >> 1) & 3)) + (s & 1)
    for dt, S in (("f32", 16), ("f16", 32)):
        for T in (4, 8):
            assert sorted(slot_group(s, dt, T) for s in range(S)) == list(range(S))


# per-plane scales of the f16 Fourier operands, as include/eqlin.h states them
F16_PLANE_SCALE = {4: [1 / 4, 1 / 4, 1 / 2, 1 / 2],
                   8: [1 / 8, 1 / 8, 1 / 8, 1 / 8, 1 / 4, 1 / 4, 1 / 8, 1 / 8],
                   "p4m": [1 / 8, 1 / 8, 1 / 8, 1 / 8, 1 / 4, 1 / 4, 1 / 4, 1 / 4]}


def decode_planes(flat, rows, groups, dt, T):
    """[rows][ceil(groups/S)][T][S] stage blocks -> [rows][groups][T]; checks zero padding."""
    S = 16 if dt == "f32" else 32
    nks = -(-groups // S)
    blk = flat[: rows * nks * T * S].reshape(rows, nks, T, S)
    out = np.zeros((rows, groups, T))
    for ks in range(nks):
        for s in range(S):
            g = ks * S + slot_group(s, dt, T)
            if g < groups:
                out[:, g, :] = blk[:, ks, :, s]
            else:
                assert np.all(blk[:, ks, :, s] == 0)
    return out


@pytest.mark.parametrize("g,dt,Dp,Cp", [(4, "f32", 5, 3), (4, "f32", 20, 36), (4, "f32", 192, 192),
                                         (4, "f16", 6, 4), (4, "f16", 40, 70), (4, "f16", 768, 192),
                                         (8, "f32", 5, 3), (8, "f32", 96, 40), (8, "f16", 7, 5),
                                         (8, "f16", 96, 384), ("p4m", "f32", 5, 3), ("p4m", "f32", 96, 40),
                                         ("p4m", "f16", 7, 5), ("p4m", "f16", 96, 384)])
def test_prepared_planes_match_group_spectrum(g, dt, Dp, Cp):
    T = order(g)
    say(f"prepare group={g} {dt} D'={Dp} C'={Cp}")
    _, w, _ = make_layer_inputs(4, T * Cp, T * Dp, dt, seed=1, T=T, with_dy=False)
    Wh = prep(w, g)
    tdt = torch.float32 if dt == "f32" else torch.float16
    buf = Wh.buf
    off = eq.eqlin_prepared_transpose_offset(T * Cp, T * Dp, tdt, g)
    wf = decode_planes(host(buf[:off].view(tdt)), Dp, Cp, dt, T)
    wb = decode_planes(host(buf[off:].view(tdt)), Cp, Dp, dt, T)
    tol = 1e-6 if dt == "f32" else 1e-3
    if g == "p4m":
        ref = oracle.p4m_planes(w.astype(np.float64))
        adj = ref.copy()
        adj[..., 5], adj[..., 6] = ref[..., 6], ref[..., 5]     # transposed 2 x 2 block
    else:
        ref = oracle.kept_planes(w.astype(np.float64))
        adj = ref.copy()
        adj[..., 3::2] = -adj[..., 3::2]      # imaginary planes
    if dt == "f16":
        # f16 planes are stored scaled into the operand range (include/eqlin.h)
        sc = np.array(F16_PLANE_SCALE[g])
        ref, adj = ref * sc, adj * sc
    assert rel_err(wf, ref) < tol
    assert rel_err(wb, adj.transpose(1, 0, 2)) < tol


# ----------------------------------------------------------------- forward

SMALL_SHAPES = {
    "f32": [(64, 32, 32), (1, 4, 4), (131, 12, 20), (1000, 160, 96), (257, 64 * 4 + 4 * 20, 4 * 70),
            (333, 4 * 200, 4 * 130)],
    "f16": [(64, 32, 32), (1, 8, 8), (131, 8 * 3, 8 * 5), (1000, 8 * 20, 8 * 12), (257, 4 * 34, 4 * 70),
            (333, 4 * 200, 4 * 130)],
}


SMALL_SHAPES_C8 = {
    "f32": [(64, 64, 64), (1, 8, 8), (131, 24, 40), (1000, 160, 96), (257, 8 * 34, 8 * 70),
            (333, 8 * 100, 8 * 65)],
    "f16": [(64, 64, 64), (1, 8, 8), (131, 24, 40), (1000, 8 * 21, 8 * 13), (257, 8 * 34, 8 * 70),
            (333, 8 * 100, 8 * 65)],
}


def _forward_case(dt, N, C, D, seed=0, g=4):
    X, w, _ = make_layer_inputs(N, C, D, dt, seed=seed, T=order(g), with_dy=False)
    Wh = prep(w, g)
    Y = eq.eqlin_forward(dev(X), Wh)
    return X, w, host(Y)


@pytest.mark.parametrize("tile", ["auto", "112221", "111221", "112121", "222221", "212421", "212431", "122241",
                                  "112241", "112411", "212211", "122211", "112211", "112212", "112412", "111211",
                                  "2124211", "1122111", "1122211", "1112111", "112111", "1121111"])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_forward_small_shapes_all_tiles(dt, tile, monkeypatch):
    if tile != "auto":
        monkeypatch.setenv("EQLIN_FWD_TILE", tile)
    for (N, C, D) in SMALL_SHAPES[dt]:
        say(f"forward {dt} tile={tile} N={N} C={C} D={D}")
        X, w, Y = _forward_case(dt, N, C, D)
        err = rel_err(Y, oracle.forward_direct(X, w))
        assert err <= TOL[dt], (N, C, D, err)


@pytest.mark.parametrize("tile", ["auto", "112211", "112221", "111221", "212211", "122211", "1122111", "1222111",
                                  "2122111", "122241"])
@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("g", [8, "p4m"])
def test_forward_order8_small_shapes_all_tiles(g, dt, tile, monkeypatch):
    if tile != "auto":
        monkeypatch.setenv("EQLIN_FWD_TILE", tile)
    for (N, C, D) in SMALL_SHAPES_C8[dt]:
        say(f"forward group={g} {dt} tile={tile} N={N} C={C} D={D}")
        X, w, Y = _forward_case(dt, N, C, D, g=g)
        err = rel_err(Y, ref_forward(X, w, g))
        assert err <= TOL[dt], (N, C, D, err)


# Tail split (fp32 tiles): when the last round of tiles over the 256 CUs
# fills at most half of them, each of those tiles runs as two half-height
# workgroups whose wave rows split every stage's k range; EQLIN_FWD_SPLIT=0
# runs every tile whole.  Shapes: one column of 300 tiles
# whose last tile has rows in its first half only, then in both halves, and
# three columns of 99 row tiles (the split starts inside a row of tiles).
SPLIT_TILES = [(4, "112211"), (4, "112221"), (4, "112121"), (4, "212421"), (4, "112212"), (8, "112211"),
               (8, "112221"), ("p4m", "112211"), ("p4m", "112221")]


def _split_shapes(tile):
    FM, FN, WM, WN = (int(c) for c in tile[:4])
    BM, BN = 32 * FM * WM, 32 * FN * WN
    return [(299 * BM + BM // 4 + 3, BN), (299 * BM + BM // 2 + 5, BN), (98 * BM + BM // 2 + 5, 3 * BN)]


@pytest.mark.parametrize("g,tile", SPLIT_TILES)
def test_forward_tail_split(g, tile, monkeypatch):
    dt = "f32"
    T = order(g)
    monkeypatch.setenv("EQLIN_FWD_TILE", tile)
    for (N, mg) in _split_shapes(tile):
        C, D = T * 42, T * mg
        say(f"tail split group={g} {dt} tile={tile} N={N} C={C} D={D}")
        X, w, _ = make_layer_inputs(N, C, D, dt, seed=15, T=T, with_dy=False)
        Wh = prep(w, g)
        ref = ref_forward(X, w, g)
        # halves (no workspace: eqlin_forward), the K split (the binding's
        # workspace: eqlin_forward_ws), every tile whole
        monkeypatch.setenv("EQLIN_FWD_SPLIT", "1")
        Ys = host(eq.eqlin_forward(dev(X), Wh, workspace=None))
        Yk = host(eq.eqlin_forward(dev(X), Wh))
        monkeypatch.setenv("EQLIN_FWD_SPLIT", "0")
        Yw = host(eq.eqlin_forward(dev(X), Wh))
        es, ek, ew = rel_err(Ys, ref), rel_err(Yk, ref), rel_err(Yw, ref)
        say(f"  split {es:.2e} k split {ek:.2e} whole {ew:.2e}")
        assert es <= TOL[dt] and ek <= TOL[dt] and ew <= TOL[dt]
    # bias and GELU in the halves' epilogue, and dX through the same launch
    monkeypatch.setenv("EQLIN_FWD_SPLIT", "1")
    N, mg = _split_shapes(tile)[1]
    C, D = T * 42, T * mg
    X, w, dY = make_layer_inputs(N, C, D, dt, seed=16, T=T)
    b = np.random.default_rng(17).standard_normal(D // T).astype(X.dtype)
    Wh = prep(w, g)
    Y = host(eq.eqlin_forward_ex(dev(X), Wh, dev(b), "gelu", workspace=None))
    Z = ref_forward(X, w, g) + np.repeat(b.astype(np.float64), T)[None, :]
    assert rel_err(Y, oracle.gelu_erf(Z)) <= TOL[dt]
    dX = host(eq.eqlin_backward_dx(dev(dY), Wh))
    assert rel_err(dX, ref_dx(dY, w, g)) <= TOL[dt]


def test_rows_and_batch_size(monkeypatch):
    # a row's output does not depend on the other rows of the call: bit for
    # bit with the tail split off, and for rows of whole tiles with it on;
    # rows of split tiles (partial sums over k) agree to the tolerance.  With
    # the K-split workspace a launch of fewer tiles than CUs splits every
    # tile, so there the rows agree to the tolerance too.
    monkeypatch.setenv("EQLIN_FWD_TILE", "112211")
    N, C, D = 299 * 64 + 50, 4 * 42, 256          # 300 tiles: the last 44 run split
    X, w, _ = make_layer_inputs(N, C, D, "f32", seed=19, with_dy=False)
    Wh = prep(w, 4)
    whole_rows = 256 * 64
    for split in ("0", "1"):
        monkeypatch.setenv("EQLIN_FWD_SPLIT", split)
        for ws in (None, "auto"):
            Y = host(eq.eqlin_forward(dev(X), Wh, workspace=ws))
            Ya = host(eq.eqlin_forward(dev(X[:6400]), Wh, workspace=ws))          # 100 tiles
            Yb = host(eq.eqlin_forward(dev(X[whole_rows:]), Wh, workspace=ws))    # 44 tiles
            if ws is None or split == "0":
                assert np.array_equal(Y[:6400], Ya)
            else:
                assert rel_err(Y[:6400], Ya) <= 1e-6
            if split == "0":
                assert np.array_equal(Y[whole_rows:], Yb)
            else:
                assert rel_err(Y[whole_rows:], Yb) <= 1e-6


# (N, C, D, group) -> parts of the K split (p4 only): the ViT-B attention
# projection (591 tiles of 64 x 64, 79 in the last round: 3 parts, dispatched
# before the whole tiles), the ViT-B fc1 shape with a ragged last row tile (4
# parts), a launch of fewer tiles than CUs (204 tiles of 32 x 64 in 2 parts:
# more parts than CUs, dispatched after the whole tiles), and the ViT-H fc2
# shape (133 tail tiles in 3 parts of 27 stages, after the whole tiles)
KSPLIT_CASES = [(12608, 768, 768, 4, 3), (12608 - 37, 768, 3072, 4, 4), (2176 - 5, 768, 768, 4, 2),
                (8224, 5120, 1280, 4, 3)]


@pytest.mark.parametrize("N,C,D,g,parts", KSPLIT_CASES)
def test_forward_k_split(N, C, D, g, parts):
    """The K split of the last round's tiles (eqlin_forward_ws): against the
    oracle, against the launch without a workspace, the same bits on a
    second call, the arrival counters back at zero, and the fused epilogue
    (bias, GELU, residual) run by the part that finishes last."""
    T = order(g)
    nbytes, got_parts = eq.eqlin_forward_workspace_bytes(N, C, D, torch.float32, T=g)
    assert got_parts == parts and nbytes > 0
    say(f"k split group={g} N={N} C={C} D={D} parts={parts} workspace={nbytes}")
    X, w, _ = make_layer_inputs(N, C, D, "f32", seed=31, T=T, with_dy=False)
    Wh = prep(w, g)
    tX = dev(X)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    Y1 = eq.eqlin_forward(tX, Wh, workspace=ws).clone()
    Y2 = eq.eqlin_forward(tX, Wh, workspace=ws)
    Y0 = eq.eqlin_forward(tX, Wh, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    assert torch.count_nonzero(ws[:1024]).item() == 0
    ref = ref_forward(X, w, g)
    e1, e0 = rel_err(host(Y1), ref), rel_err(host(Y0), ref)
    say(f"  rel err k split {e1:.2e} without workspace {e0:.2e}")
    assert e1 <= TOL["f32"] and e0 <= TOL["f32"]
    # epilogue after the reduction
    rng = np.random.default_rng(32)
    b = rng.standard_normal(D // T).astype(np.float32)
    R = rng.standard_normal((N, D)).astype(np.float32)
    Yr = host(eq.eqlin_forward_ex(tX, Wh, dev(b), "gelu", residual=dev(R), workspace=ws))
    Z = oracle.gelu_erf(ref + np.repeat(b.astype(np.float64), T)[None, :]) + R
    assert rel_err(Yr, Z) <= TOL["f32"]
    assert torch.count_nonzero(ws[:1024]).item() == 0
    # the residual updated in place (R is the output): only the part that
    # arrives last reads R and writes Y
    tR = dev(R)
    eq.eqlin_forward_ex(tX, Wh, dev(b), "gelu", out=tR, residual=tR, workspace=ws)
    assert rel_err(host(tR), Z) <= TOL["f32"]
    # a workspace one byte short is refused before any launch
    with pytest.raises(ValueError):
        eq.eqlin_forward(tX, Wh, workspace=ws[:nbytes - 1])


def test_forward_k_split_not_for_order_8():
    for g in (8, "p4m"):
        assert eq.eqlin_forward_workspace_bytes(12608, 768, 768, torch.float32, T=g) == (0, 0)


def _sample_rows(N, rng, k=96):
    rows = set(range(8)) | set(range(N - 8, N))
    rows |= set(rng.choice(N, size=k, replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name,dt,g", [("tiny", "f32", 4), ("vitb_attn", "f32", 4), ("vitb_mlp", "f16", 4),
                                       ("vith_mlp", "f32", 4), ("vith_mlp", "f16", 4), ("tiny", "f32", 8),
                                       ("vitb_attn", "f32", 8), ("vitb_mlp", "f16", 8), ("vith_mlp", "f32", 8),
                                       ("vith_mlp", "f16", 8), ("tiny", "f32", "p4m"), ("vitb_attn", "f32", "p4m"),
                                       ("vitb_mlp", "f16", "p4m"), ("vith_mlp", "f32", "p4m"),
                                       ("vith_mlp", "f16", "p4m"), ("narrow", "f32", 4), ("narrow", "f16", 4)])
def test_forward_workloads(name, dt, g):
    # the p4 workloads (the layer shapes the method is measured on) whole;
    # the order-8 groups' largest layers on sampled rows (rows are independent)
    wl = WORKLOADS[name]
    for li, L in enumerate(wl.layers):
        say(f"forward workload {name} {L.name} {dt} group={g} N={L.N} C={L.C} D={L.D}")
        X, w, _ = make_layer_inputs(L.N, L.C, L.D, dt, seed=0, layer=li, T=order(g), with_dy=False)
        Wh = prep(w, g)
        Y = host(eq.eqlin_forward(dev(X), Wh))
        if g == 4 or L.N * L.C * L.D <= 12608 * 768 * 768:
            err = rel_err(Y, ref_forward(X, w, g))
        else:
            rows = _sample_rows(L.N, np.random.default_rng(li))
            err = rel_err(Y[rows], ref_forward(X[rows], w, g))
        say(f"  rel err {err:.3e}")
        assert err <= TOL[dt]


# ---------------------------------------------------------------- backward

# (64, 32, 32): rows read in chunks of 4 by the dw tile; (1002, 64, 32) and
# (2000, 112, 128): chunks of 2 (N = 2 mod 4; 32 group channels)
BWD_SHAPES = {
    "f32": [(64, 32, 32), (1, 4, 4), (77, 12, 20), (1000, 160, 96), (3001, 4 * 70, 4 * 130), (1002, 64, 32),
            (2000, 112, 128)],
    "f16": [(64, 32, 32), (1, 8, 8), (77, 8 * 3, 8 * 5), (1000, 8 * 20, 8 * 12), (3001, 4 * 70, 4 * 130),
            (1002, 64, 32), (2000, 112, 128)],
}


BWD_SHAPES_C8 = [(64, 64, 64), (1, 8, 8), (77, 24, 40), (1000, 160, 96), (3001, 8 * 70, 8 * 130)]


@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_backward_small_shapes(dt, g):
    for (N, C, D) in (BWD_SHAPES[dt] if g == 4 else BWD_SHAPES_C8):
        say(f"backward group={g} {dt} N={N} C={C} D={D}")
        X, w, dY = make_layer_inputs(N, C, D, dt, seed=2, T=order(g))
        Wh = prep(w, g)
        dX, dw = eq.eqlin_backward(dev(dY), dev(X), Wh)
        dXr, dwr = ref_dx(dY, w, g), ref_dw(dY, X, g)
        e1, e2 = rel_err(host(dX), dXr), rel_err(host(dw), dwr)
        assert e1 <= TOL[dt], ("dX", N, C, D, e1)
        assert e2 <= TOL[dt], ("dw", N, C, D, e2)


@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_backward_workload_vitb(dt, g):
    L = WORKLOADS["vitb_attn_bwd"].layers[0]
    say(f"backward workload vitb_attn_bwd {dt} group={g} N={L.N} C={L.C} D={L.D}")
    X, w, dY = make_layer_inputs(L.N, L.C, L.D, dt, seed=0, T=order(g))
    Wh = prep(w, g)
    dX, dw = eq.eqlin_backward(dev(dY), dev(X), Wh)
    e1 = rel_err(host(dX), ref_dx(dY, w, g))
    e2 = rel_err(host(dw), ref_dw(dY, X, g))
    say(f"  dX rel err {e1:.3e}  dw rel err {e2:.3e}")
    assert e1 <= TOL[dt] and e2 <= TOL[dt]


def test_backward_wide_f16_layers():
    """f16 p4 layers with 256 or more group channels in and out run dX through
    the forward's tile choice and dw alone with the 128-wide tile: a ragged
    wide layer whole, and the ViT-H fc1 layer (dX on sampled rows, dw whole)."""
    for (N, C, D) in ((3001, 4 * 300, 4 * 260), (8224, 1280, 5120)):
        say(f"backward wide f16 N={N} C={C} D={D}")
        X, w, dY = make_layer_inputs(N, C, D, "f16", seed=26)
        Wh = prep(w, 4)
        dX, dw = eq.eqlin_backward(dev(dY), dev(X), Wh)
        dX = host(dX)
        if N * C * D <= 3001 * 1200 * 1040:
            e1 = rel_err(dX, oracle.dx_direct(dY, w))
        else:
            rows = _sample_rows(N, np.random.default_rng(27))
            e1 = rel_err(dX[rows], oracle.dx_direct(dY[rows], w))
        e2 = rel_err(host(dw), oracle.dw_direct(dY, X, 4))
        say(f"  dX rel err {e1:.3e}  dw rel err {e2:.3e}")
        assert e1 <= TOL["f16"] and e2 <= TOL["f16"]


@pytest.mark.parametrize("C,D", [(1280, 5120), (5120, 1280)])
def test_backward_fused_fallback_f32(C, D):
    """fp32 p4 layers of the ViT-H widths over 2056 rows: one dw split per CU
    would run 65 stages against 26100 stage units of work (over 1.75 x the
    average per resident workgroup), so the fused launch takes its two-per-CU
    fallback, whose split count rounds up (512 / 100 dw tiles -> 6 splits of
    352 rows, the last 296)."""
    N = 2056
    say(f"backward fused fallback f32 N={N} C={C} D={D}")
    X, w, dY = make_layer_inputs(N, C, D, "f32", seed=28)
    Wh = prep(w, 4)
    dX, dw = eq.eqlin_backward(dev(dY), dev(X), Wh)
    dXr, dwr = oracle.backward_direct(dY, X, w)
    e1, e2 = rel_err(host(dX), dXr), rel_err(host(dw), dwr)
    say(f"  dX rel err {e1:.3e}  dw rel err {e2:.3e}")
    assert e1 <= TOL["f32"] and e2 <= TOL["f32"]


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_backward_workload_narrow(dt):
    """The HBM-bound narrow layer (16 group channels, 201728 rows): dw reduces
    over every row through many split partials."""
    L = WORKLOADS["narrow"].layers[0]
    say(f"backward workload narrow {dt} N={L.N} C={L.C} D={L.D}")
    X, w, dY = make_layer_inputs(L.N, L.C, L.D, dt, seed=0)
    Wh = prep(w, 4)
    dX, dw = eq.eqlin_backward(dev(dY), dev(X), Wh)
    e1 = rel_err(host(dX), ref_dx(dY, w, 4))
    e2 = rel_err(host(dw), ref_dw(dY, X, 4))
    say(f"  dX rel err {e1:.3e}  dw rel err {e2:.3e}")
    assert e1 <= TOL[dt] and e2 <= TOL[dt]


@pytest.mark.parametrize("width", ["128", "64"])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_dw_tile_widths(dt, width, monkeypatch):
    """The stand-alone dw launch with the 128 x 128 partial tile (eight waves,
    two fragments each) and the 64 x 64 one: ragged rows, group channels past
    the tile, the ViT shapes whole."""
    monkeypatch.setenv("EQLIN_DW_WIDTH", width)
    shapes = [(77, 8 * 20, 8 * 12), (1000, 4 * 130, 4 * 70), (3001, 4 * 300, 4 * 260), (12608, 768, 768),
              (8224, 1280, 5120), (8224, 5120, 1280)]
    for (N, C, D) in shapes:
        say(f"dw tile width {width} {dt} N={N} C={C} D={D}")
        X, w, dY = make_layer_inputs(N, C, D, dt, seed=25)
        dw = host(eq.eqlin_backward_dw(dev(dY), dev(X)))
        err = rel_err(dw, oracle.dw_direct(dY, X, 4))
        say(f"  rel err {err:.2e}")
        assert err <= TOL[dt], (N, C, D, err)


@pytest.mark.parametrize("g", GROUPS)
def test_backward_separate_entry_points_agree(g):
    X, w, dY = make_layer_inputs(500, 64, 96, "f32", seed=4, T=order(g))
    Wh = prep(w, g)
    dX, dw = eq.eqlin_backward(dev(dY), dev(X), Wh)
    dX2 = eq.eqlin_backward_dx(dev(dY), Wh)
    dw2 = eq.eqlin_backward_dw(dev(dY), dev(X), T=g)
    assert torch.equal(dX, dX2) and torch.equal(dw, dw2)


# -------------------------------------------------------------- edge cases

@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_extreme_widths_and_heights(dt, g):
    # a very wide layer (C = 2^17: 512 KiB rows in fp32, 8192 pipeline stages),
    # then a tall thin one (about a million rows: many dw splits, ragged last split)
    T = order(g)
    for (N, C, D) in ((40, 1 << 17, 64), ((1 << 20) + 37, 16, 32)):
        say(f"extreme group={g} {dt} N={N} C={C} D={D}")
        X, w, dY = make_layer_inputs(N, C, D, dt, seed=11, T=T)
        Wh = prep(w, g)
        Y = eq.eqlin_forward(dev(X), Wh)
        dX, dw = eq.eqlin_backward(dev(dY), dev(X), Wh)
        e = (rel_err(host(Y), ref_forward(X, w, g)), rel_err(host(dX), ref_dx(dY, w, g)),
             rel_err(host(dw), ref_dw(dY, X, g)))
        say(f"  Y {e[0]:.2e} dX {e[1]:.2e} dw {e[2]:.2e}")
        assert max(e) <= TOL[dt], e
        del X, dY, Y, dX, dw


@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_empty_batch(dt, g):
    T = order(g)
    tdt = torch.float32 if dt == "f32" else torch.float16
    _, w, _ = make_layer_inputs(1, 32, 48, dt, seed=5, T=T, with_dy=False)
    Wh = prep(w, g)
    X = torch.empty((0, 32), dtype=tdt, device=DEV)
    dY = torch.empty((0, 48), dtype=tdt, device=DEV)
    assert eq.eqlin_forward(X, Wh).shape == (0, 48)
    dw = torch.full((48 // T, 32 // T, T), float("nan"), device=DEV)
    dX, dw = eq.eqlin_backward(dY, X, Wh, dw_out=dw)
    torch.cuda.synchronize()
    assert dX.shape == (0, 32)
    assert torch.count_nonzero(dw).item() == 0


@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_determinism(dt, g):
    X, w, dY = make_layer_inputs(2000, 256, 384, dt, seed=6, T=order(g))
    Wh = prep(w, g)
    tX, tdY = dev(X), dev(dY)
    Y1 = eq.eqlin_forward(tX, Wh).clone()
    Y2 = eq.eqlin_forward(tX, Wh)
    dX1, dw1 = eq.eqlin_backward(tdY, tX, Wh)
    dX2, dw2 = eq.eqlin_backward(tdY, tX, Wh)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(dX1, dX2) and torch.equal(dw1, dw2)


@pytest.mark.parametrize("pair", [("112211", "112221"), ("111211", "111221"), ("112211", "112212"),
                                  ("112411", "112412"), ("212421", "212431"), ("122211", "122241"),
                                  ("112211", "112241")])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_lds_buffering_is_bitwise_invisible(dt, pair, monkeypatch):
    """Race check: one fragment layout run single-buffered (NBUF = 1: two
    barriers per stage, the stage stored into the buffer just read) and
    double-buffered (NBUF = 2: one barrier, the next stage stored into the
    other buffer while this one is read), or with one and with two stages of
    global loads in flight, multiplies the same operands in the same order:
    the outputs must agree bit for bit.  A missing wait or barrier shows up
    as a difference.  The last three pairs copy the weight operand straight
    from memory into LDS (NBUF = 3: three weight buffers beside two of the
    input; NBUF = 4: two beside one) instead of through registers.
    The first shape has one k stage (the copies of the idle stages only)."""
    a, b = pair
    if max(int(a[4]), int(b[4])) >= 3:
        # the DMA tiles run no tail split, whose halves add their k ranges
        # in another order: compare whole tiles with whole tiles
        monkeypatch.setenv("EQLIN_FWD_SPLIT", "0")
    shapes = [(200, 64, 136), (1000, 160, 96), (333, 800, 520), (299 * 64 + 37, 4 * 42, 256)]
    for (N, C, D) in shapes:
        say(f"buffering {dt} tiles {a} / {b} N={N} C={C} D={D}")
        X, w, _ = make_layer_inputs(N, C, D, dt, seed=24, with_dy=False)
        Wh = prep(w, 4)
        tX = dev(X)
        out = {}
        for tile in (a, b):
            monkeypatch.setenv("EQLIN_FWD_TILE", tile)
            out[tile] = eq.eqlin_forward(tX, Wh)
        torch.cuda.synchronize()
        assert torch.equal(out[a], out[b]), (N, C, D)
        assert rel_err(host(out[a]), oracle.forward_direct(X, w)) <= TOL[dt]


@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_row_isolation(dt, g):
    # a NaN in row r of X may only reach row r of Y (checks tail masking and row mapping)
    N, C, D = 300, 128, 160
    X, w, _ = make_layer_inputs(N, C, D, dt, seed=7, T=order(g), with_dy=False)
    Wh = prep(w, g)
    Y0 = host(eq.eqlin_forward(dev(X), Wh))
    Xn = X.copy()
    for r in (0, 131, N - 1):
        Xn[r, 5] = np.nan
    Y1 = host(eq.eqlin_forward(dev(Xn), Wh))
    bad = np.isnan(Y1).any(axis=1)
    assert set(np.nonzero(bad)[0].tolist()) == {0, 131, N - 1}
    assert np.array_equal(Y1[~bad], Y0[~bad])


def _left_translate(Z, a, table):
    """(L_a z)(g) = z(a^-1 g) on every group block of Z [N][G*n]."""
    n = len(table)
    inv = [int(np.nonzero(table[i] == 0)[0][0]) for i in range(n)]
    src = [table[inv[a], h] for h in range(n)]
    return Z.reshape(Z.shape[0], -1, n)[:, :, src].reshape(Z.shape)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_p4m_equivariance_under_every_element(dt):
    N, C, D = 256, 128, 192
    X, w, _ = make_layer_inputs(N, C, D, dt, seed=8, T=8, with_dy=False)
    Wh = prep(w, "p4m")
    Y = host(eq.eqlin_forward(dev(X), Wh))
    for a in range(8):
        Ya = host(eq.eqlin_forward(dev(_left_translate(X, a, P4M_TABLE)), Wh))
        assert rel_err(Ya, _left_translate(Y, a, P4M_TABLE)) <= TOL[dt], a


@pytest.mark.parametrize("T", [4, 8])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_group_shift_equivariance(dt, T):
    N, C, D = 512, 256, 192
    X, w, _ = make_layer_inputs(N, C, D, dt, seed=8, T=T, with_dy=False)
    Xr = np.roll(X.reshape(N, C // T, T), 1, axis=2).reshape(N, C)
    Wh = eq.eqlin_prepare_weights(dev(w))
    Y = host(eq.eqlin_forward(dev(X), Wh)).reshape(N, D // T, T)
    Yr = host(eq.eqlin_forward(dev(Xr), Wh)).reshape(N, D // T, T)
    assert rel_err(Yr, np.roll(Y, 1, axis=2)) <= TOL[dt]


def test_non_default_stream():
    X, w, dY = make_layer_inputs(700, 96, 64, "f32", seed=9)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tX, tw, tdY = dev(X), dev(w), dev(dY)
        Wh = eq.eqlin_prepare_weights(tw)
        Y = eq.eqlin_forward(tX, Wh)
        dX, dw = eq.eqlin_backward(tdY, tX, Wh)
    s.synchronize()
    assert rel_err(host(Y), oracle.forward_direct(X, w)) <= 1e-5
    dXr, dwr = oracle.backward_direct(dY, X, w)
    assert rel_err(host(dX), dXr) <= 1e-5 and rel_err(host(dw), dwr) <= 1e-5


# ------------------------------------------------- fused bias + GELU epilogue

@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("with_bias,act", [(True, "none"), (False, "gelu"), (True, "gelu")])
def test_forward_ex_bias_gelu(dt, with_bias, act, g):
    T = order(g)
    for (N, C, D) in [(131, 8 * 3, 8 * 5), (1000, 160, 96), (333, 8 * 100, 8 * 65)]:
        say(f"forward_ex group={g} {dt} bias={with_bias} act={act} N={N} C={C} D={D}")
        X, w, _ = make_layer_inputs(N, C, D, dt, seed=13, T=T, with_dy=False)
        b = (np.random.default_rng(14).standard_normal(D // T)).astype(X.dtype) if with_bias else None
        Wh = prep(w, g)
        Y = host(eq.eqlin_forward_ex(dev(X), Wh, dev(b) if with_bias else None, act))
        if g == "p4m":
            # the oracle's bias/act step applied to the p4m group convolution
            Z = ref_forward(X, w, g) + (np.repeat(b.astype(np.float64), T)[None, :] if with_bias else 0.0)
            ref = oracle.gelu_erf(Z) if act == "gelu" else Z
        else:
            ref = oracle.forward_bias_act(X, w, b, act)
        assert rel_err(Y, ref) <= TOL[dt]


@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("with_bias,act,inplace", [(False, "none", False), (True, "gelu", False),
                                                   (True, "none", True)])
def test_forward_residual(dt, with_bias, act, inplace, g):
    """Y = act(X W^T + b) + R, R added in float32 after the activation; R may be Y."""
    T = order(g)
    for (N, C, D) in [(131, 8 * 3, 8 * 5), (1000, 160, 96), (333, 8 * 100, 8 * 65), (3001, 64, 64)]:
        say(f"forward_residual group={g} {dt} bias={with_bias} act={act} inplace={inplace} N={N} C={C} D={D}")
        X, w, R = make_layer_inputs(N, C, D, dt, seed=17, T=T)
        b = (np.random.default_rng(18).standard_normal(D // T)).astype(X.dtype) if with_bias else None
        Wh = prep(w, g)
        tR = dev(R)
        Y = eq.eqlin_forward_ex(dev(X), Wh, dev(b) if with_bias else None, act, out=tR if inplace else None,
                                residual=tR)
        Z = ref_forward(X, w, g) + (np.repeat(b.astype(np.float64), T)[None, :] if with_bias else 0.0)
        ref = (oracle.gelu_erf(Z) if act == "gelu" else Z) + R.astype(np.float64)
        if g != "p4m":
            assert np.array_equal(ref, oracle.forward_bias_act(X, w, b, act, R))
        err = rel_err(host(Y), ref)
        say(f"  rel err {err:.3e}")
        assert err <= TOL[dt]


def test_forward_residual_mlp_block_vitb_f16_sampled():
    # the ViT block's MLP with its skip connection: X + fc2(GELU(fc1(X) + b1)) + b2
    wl = WORKLOADS["vitb_mlp"]
    (L1, L2) = wl.layers
    X, w1, _ = make_layer_inputs(L1.N, L1.C, L1.D, "f16", seed=0, layer=0, with_dy=False)
    _, w2, _ = make_layer_inputs(8, L2.C, L2.D, "f16", seed=0, layer=1, with_dy=False)
    rng = np.random.default_rng(19)
    b1 = rng.standard_normal(L1.D // 4).astype(np.float16)
    b2 = rng.standard_normal(L2.D // 4).astype(np.float16)
    W1, W2 = eq.eqlin_prepare_weights(dev(w1)), eq.eqlin_prepare_weights(dev(w2))
    tX = dev(X)
    H = eq.eqlin_forward_ex(tX, W1, dev(b1), "gelu")
    Y = host(eq.eqlin_forward_ex(H, W2, dev(b2), "none", residual=tX))
    rows = _sample_rows(L1.N, np.random.default_rng(20), k=48)
    Hh = host(H)[rows]
    err = rel_err(Y[rows], oracle.forward_bias_act(Hh.astype(np.float16), w2, b2, "none", X[rows]))
    say(f"  block rel err {err:.3e}")
    assert err <= 3e-3


def test_forward_ex_mlp_block_vitb_f16_sampled():
    # fc1 768->3072 (+bias, GELU) then fc2 3072->768 (+bias), f16 storage
    wl = WORKLOADS["vitb_mlp"]
    (L1, L2) = wl.layers
    X, w1, _ = make_layer_inputs(L1.N, L1.C, L1.D, "f16", seed=0, layer=0, with_dy=False)
    _, w2, _ = make_layer_inputs(8, L2.C, L2.D, "f16", seed=0, layer=1, with_dy=False)
    rng = np.random.default_rng(15)
    b1 = rng.standard_normal(L1.D // 4).astype(np.float16)
    b2 = rng.standard_normal(L2.D // 4).astype(np.float16)
    W1, W2 = eq.eqlin_prepare_weights(dev(w1)), eq.eqlin_prepare_weights(dev(w2))
    H = eq.eqlin_forward_ex(dev(X), W1, dev(b1), "gelu")
    Y = host(eq.eqlin_forward_ex(H, W2, dev(b2), "none"))
    rows = _sample_rows(L1.N, np.random.default_rng(16), k=48)
    Hh = host(H)[rows]
    # stage-wise parity: the second layer is checked on the GPU's own (f16) hidden rows
    err1 = rel_err(Hh, oracle.forward_bias_act(X[rows], w1, b1, "gelu"))
    err2 = rel_err(Y[rows], oracle.forward_bias_act(Hh.astype(np.float16), w2, b2, "none"))
    say(f"  fc1 rel err {err1:.3e}  fc2 rel err {err2:.3e}")
    assert err1 <= 3e-3 and err2 <= 3e-3


# ------------------------------------------- f16 range of the Fourier operands

# The f16 route rounds every Fourier operand (transformed X, dY and the
# prepared weights) to binary16.  A zero-frequency plane sums all T values of
# a group, so each plane is scaled by a power of two that keeps it within
# max|input| before the rounding: no finite input overflows an operand.
# Inputs at |x| up to 6e4 (groups of equal sign, whose plain sums pass
# 65504) and just above the smallest normal 2^-14; the exact outputs are
# finite binary16 numbers (dw is float32).
RANGE_SHAPES = {4: [(257, 160, 96), (1000, 64, 64)], 8: [(257, 320, 192)], "p4m": [(257, 320, 192)]}


@pytest.mark.parametrize("regime", ["large", "small"])
@pytest.mark.parametrize("g", GROUPS)
def test_f16_operand_range(g, regime):
    T = order(g)
    for (N, C, D) in RANGE_SHAPES[g]:
        say(f"f16 range {regime} group={g} N={N} C={C} D={D}")
        X, w, dY = make_range_inputs(N, C, D, regime, seed=21, T=T)
        Yr, dXr, dwr = ref_forward(X, w, g), ref_dx(dY, w, g), ref_dw(dY, X, g)
        assert np.max(np.abs(Yr)) < 65504 and np.max(np.abs(dXr)) < 65504
        Wh = prep(w, g)
        tX, tdY = dev(X), dev(dY)
        Y = host(eq.eqlin_forward(tX, Wh))
        dX, dw = eq.eqlin_backward(tdY, tX, Wh)
        dX, dw = host(dX), host(dw)
        dX2 = host(eq.eqlin_backward_dx(tdY, Wh))
        dw2 = host(eq.eqlin_backward_dw(tdY, tX, T=g))
        errs = {"Y": rel_err(Y, Yr), "dX": rel_err(dX, dXr), "dw": rel_err(dw, dwr), "dX alone": rel_err(dX2, dXr),
                "dw alone": rel_err(dw2, dwr)}
        say("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
        for a in (Y, dX, dw, dX2, dw2):
            assert np.all(np.isfinite(a))
        assert max(errs.values()) <= TOL["f16"], errs


@pytest.mark.parametrize("tile", ["212421", "122211", "112211", "111221", "2124211", "1121111"])
def test_f16_operand_range_forward_tiles(tile, monkeypatch):
    # every p4 f16 tile, with the bias + GELU epilogue (the general inverse
    # transform) beside the plain one
    monkeypatch.setenv("EQLIN_FWD_TILE", tile)
    N, C, D = 333, 4 * 40, 4 * 70
    X, w, _ = make_range_inputs(N, C, D, "large", seed=22)
    b = (np.random.default_rng(23).uniform(-1e3, 1e3, size=D // 4)).astype(np.float16)
    Wh = prep(w, 4)
    Y = host(eq.eqlin_forward(dev(X), Wh))
    Yg = host(eq.eqlin_forward_ex(dev(X), Wh, dev(b), "gelu"))
    e1 = rel_err(Y, oracle.forward_direct(X, w))
    e2 = rel_err(Yg, oracle.forward_bias_act(X, w, b, "gelu"))
    say(f"  tile {tile}: Y {e1:.2e}  bias+GELU {e2:.2e}")
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(Yg))
    assert e1 <= TOL["f16"] and e2 <= TOL["f16"]


def test_stage_trace_program_runs():
    """The stage-timeline diagnostic (csrc/stage_trace.hip, built beside the
    library) traces one launch of each of its layer shapes: every line has
    its rounds, each with a positive stage time, within the launch."""
    import json
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(eq.LIB), "eqlin_stage_trace")
    assert os.path.exists(exe), "stage trace program not built"
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120, check=True).stdout
    lines = [json.loads(l) for l in out.splitlines() if l.startswith("{")]
    assert [l["layer"] for l in lines] == ["vith_fc1", "vith_fc2", "vitb_fc2", "vitb_attn", "vitb_attn_ksplit",
                                           "vith_fc2_f32_ksplit"]
    # the K-split launches: three parts per tail tile, a group of their own,
    # and the dispatcher's placement (XCC = workgroup id mod 8, every CU used)
    for l in lines[4:]:
        assert l["ksplit_parts"] == 3 and l["groups"][-1]["group"] == "k-split parts"
        assert l["placement"]["cus"] == 256 and l["placement"]["xcc_is_workgroup_id_mod_8"]
    for l in lines:
        say(f"  {l['layer']} {l['dtype']}: {l['launch_us']} us, clock {l['shader_clock_ghz']} GHz")
        assert l["launch_us"] > 0 and l["groups"]
        assert sum(g["workgroups"] for g in l["groups"]) == l["workgroups"]
        for g in l["groups"]:
            assert 0 < g["stage_us"] < l["launch_us"] and g["end_us"][1] <= 2 * l["launch_us"]


def test_dma_check_program_runs():
    """The check of the direct global-to-LDS load that the f16 forward tiles
    use for their weight operand (csrc/dma_check.hip, built beside the
    library, calling the library's dma16): lane l's 16 bytes land at
    16 l past the wave's LDS address, and lanes reading out of the buffer's
    range write zeros."""
    import json
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(eq.LIB), "eqlin_dma_check")
    assert os.path.exists(exe), "DMA check program not built"
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    say(f"  {run.stdout.strip()}")
    assert run.returncode == 0, run.stdout + run.stderr
    res = json.loads([l for l in run.stdout.splitlines() if l.startswith("{")][-1])
    assert res["mismatched"] == 0
    assert res["out_of_range_words"] == 64 and res["out_of_range_zero"] == 64
