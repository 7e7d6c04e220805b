"""Host logic of bench.py (no GPU): the executed-FLOP fractions and the
roofline bound it reports for each workload's forward."""
import bench
from group_circulant_linear_amd.inputs import WORKLOADS


def test_executed_flop_fractions():
    # real products per dense-equivalent product: p4 6 of 16, C8 14 of 64, p4m 12 of 64
    assert bench.group_args("4")[1:] == (4, 6 / 16)
    assert bench.group_args("8")[1:] == (8, 14 / 64)
    assert bench.group_args("p4m")[1:] == (8, 12 / 64)


def _bound(name, dt, g="4"):
    _, T, frac = bench.group_args(g)
    return bench.layer_roofline(WORKLOADS[name].layers, 4 if dt == "f32" else 2, T, frac, bench.PEAK_TFLOPS[dt])


def test_roofline_bound_of_the_workloads():
    b, nbytes, flops = _bound("vitb_attn", "f32")
    assert b == "mfma"
    assert nbytes == 4 * 12608 * (768 + 768) + 4 * 768 * 768 / 4     # X, Y and the four spectra planes
    assert flops == 0.75 * 12608 * 768 * 768                          # six real products of N x 192 x 192
    assert _bound("vith_mlp", "f32")[0] == "mfma"
    assert _bound("vith_mlp", "f16")[0] == "mfma"                     # 373 FLOP/B, above the f16 ridge of 312
    assert _bound("vitb_mlp", "f16")[0] == "hbm"                      # 228 FLOP/B, below it
    assert _bound("narrow", "f32")[0] == "hbm"                        # 6 FLOP/B
    assert _bound("narrow", "f16")[0] == "hbm"
    assert _bound("vitb_attn", "f32", "8")[0] == "mfma"
