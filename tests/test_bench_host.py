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


def test_backward_roofline_of_the_attention_shapes():
    # dX and dw: X and dY read once, dX written once, the transpose spectra read once, dw (float32)
    # written once; twice the forward's executed FLOPs
    L = WORKLOADS["vitb_attn_bwd"].layers
    _, T, frac = bench.group_args("4")
    b16, n16, f16 = bench.backward_roofline(L, 2, T, frac, bench.PEAK_TFLOPS["f16"])
    b32, n32, f32 = bench.backward_roofline(L, 4, T, frac, bench.PEAK_TFLOPS["f32"])
    N, C, D = 12608, 768, 768
    assert n16 == 2 * N * (2 * C + D) + 2 * C * D / 4 + 4 * C * D / 4
    assert n32 == 4 * N * (2 * C + D) + 4 * C * D / 4 + 4 * C * D / 4
    assert f16 == f32 == 1.5 * N * C * D
    assert b16 == "hbm" and b32 == "mfma"     # 189 FLOP/B below the f16 ridge; 95 above the fp32 ridge of 20


def test_per_config_entries_name_measured_workloads():
    # every entry beside the headline is a linear workload the bench runs, in a dtype it declares
    assert len(bench.PER_CONFIG) == len(set(bench.PER_CONFIG))
    for name, dt in bench.PER_CONFIG:
        assert name in WORKLOADS and dt in WORKLOADS[name].dtypes, (name, dt)
    assert ("vith_mlp", "f32") in bench.PER_CONFIG and ("vith_mlp", "f16") in bench.PER_CONFIG


def test_profiled_traffic_sums_one_row_per_layer(tmp_path, monkeypatch):
    # a summary keeps one row per grid size: one launch per layer sums them, a
    # row count other than the layer count (grids that coincide) gives no figure,
    # and a summary of other kernel sources gives none either
    import json
    (tmp_path / "profiles").mkdir()
    rows = {"eqlin::fwd_kernel<_Float16, 4>": [{"grid": 1, "bytes": 10.0}, {"grid": 2, "bytes": 32.0}],
            "eqlin::dw_finalize_kernel<4, true>": [{"grid": 3, "bytes": 5.0}]}
    doc = {"source_sha256": "1" * 64, "kernels": rows}
    (tmp_path / "profiles" / "traffic_pair.json").write_text(json.dumps(doc))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "1" * 64)
    assert bench.profiled_traffic("pair", "eqlin::fwd_kernel", 2) == 42.0
    assert bench.profiled_traffic("pair", "eqlin::fwd_kernel", 3) is None
    assert bench.profiled_traffic("pair", "eqlin::fwd_kernel") == 32.0
    doc["source_sha256"] = "0" * 64
    (tmp_path / "profiles" / "traffic_pair.json").write_text(json.dumps(doc))
    assert bench.profiled_traffic("pair", "eqlin::fwd_kernel", 2) is None


def test_kernel_source_sha_ignores_comment_lines(tmp_path, monkeypatch):
    # the profiles' key changes with the kernels' code, not with comments, blank
    # lines or the standalone diagnostic programs beside the sources
    csrc = tmp_path / "group_circulant_linear_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (csrc / "k.hip").write_text("int f() {\n  return 1;   // one\n}\n")
    base = bench.kernel_source_sha256()
    (csrc / "k.hip").write_text("// a comment\nint f() {\n\n  return 1;   // one\n}\n")
    assert bench.kernel_source_sha256() == base
    (csrc / "stage_trace.hip").write_text("int main() { return 0; }\n")
    (csrc / "dma_check.hip").write_text("int main() { return 0; }\n")
    assert bench.kernel_source_sha256() == base
    (csrc / "k.hip").write_text("int f() {\n  return 2;   // one\n}\n")
    assert bench.kernel_source_sha256() != base
