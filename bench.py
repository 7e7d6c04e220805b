"""Benchmark of the group-circulant linear layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for every layer of the workload, prepare the weight spectra, run the forward
(Y = X W^T), and the backward (dX = dY W, then dw).  Inputs live in HBM before
the timed region starts; R rotating buffer sets (more than the 256 MB
Infinity Cache) keep consecutive steps from being served by the cache.  The
K timed steps run phase by phase (all K prepares of a layer, then its K
forwards, then its K backwards), each phase between one pair of HIP events on
the launch stream, so a phase's per-launch time is its event time / K.

The reported metric is the forward dense-equivalent throughput
2*N*D*C / t_forward (the same N x D x C dense GEMM counts 2NDC FLOPs), summed
over the workload's layers, with t_forward the forward kernel time measured by
HIP events on the launch stream inside the timed steps.  The fraction of the
MFMA peak counts the FLOPs the kernel executes: for the p4 group (T = 4) six
real products of N x D/4 x C/4, i.e. 0.75 NDC; for C8 (--group 8) fourteen of
N x D/8 x C/8, i.e. 0.4375 NDC (in general 2NDC (2T - 2) / T^2); for p4m
(--group p4m) twelve of N x D/8 x C/8, i.e. 0.375 NDC.

The roofline object names the forward kernel's bound by the roofline model:
HBM when its algorithmic bytes (X read once, Y written once, the weight
spectra read once) take longer at 8 TB/s than its executed FLOPs at the
dtype's MFMA peak, else MFMA; both fractions are reported beside it.  The
"narrow" workload (C = D = 64 over 201728 rows) is the HBM-bound case.

The p4 group convolution workloads (--workload p4conv | p4conv_tiny) time
the convolution's prepare, forward and backward the same way and print their
own JSON line (metric: dense-equivalent K x K convolution TFLOP/s).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--dtype f32|f16] [--group 4|8|p4m]
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "EQ-Linear fwd dense-equiv TFLOP/s (2NDC) + % MFMA peak, p4 ViT-B/H shapes"
PEAK_TFLOPS = {"f32": 157.3, "f16": 2500.0}      # MI355X dense MFMA peaks
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="vitb_attn")
    p.add_argument("--dtype", default=None)
    p.add_argument("--group", default="4", choices=("4", "8", "p4m"),
                   help="group: 4 (p4 rotations), 8 (cyclic C8) or p4m (dihedral, order 8)")
    p.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0 = enough to exceed 600 MB)")
    p.add_argument("--settle", type=float, default=0.5,
                   help="seconds of untimed steps before the warmup steps (GPU clock ramp)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-per-config", action="store_true",
                   help="the headline line only (no per-configuration entries)")
    p.add_argument("--forward-only", action="store_true",
                   help="time only the forward (for profiling the forward kernel); not a valid bench line")
    p.add_argument("--mlp-block", action="store_true",
                   help="time the EQ-MLP block fc1(+bias, GELU) -> fc2(+bias) of a two-layer workload with the "
                        "fused epilogue, next to the dense torch block; prints its own JSON line")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="also run one plain device copy of this many MB (counter calibration)")
    return p.parse_args()


# standalone diagnostic programs beside the library's sources (not in its kernels)
_NOT_LIBRARY = ("ceilings.hip", "stage_trace.hip", "dma_check.hip")


def kernel_source_sha256():
    """sha256 over the library's HIP sources and headers (sorted by name), without
    their blank and whole-line comment lines, so that a profile stays matched to
    the kernels it measured across edits of comments only."""
    import hashlib
    csrc = os.path.join(ROOT, "group_circulant_linear_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")) and name not in _NOT_LIBRARY:
            with open(os.path.join(csrc, name), "rb") as f:
                code = [l.rstrip() for l in f.read().split(b"\n")]
            code = [l for l in code if l.strip() and not l.lstrip().startswith(b"//")]
            h.update(name.encode() + b"\0" + b"\n".join(code))
    return h.hexdigest()


def group_args(group):
    """(group argument for the binding, group order, executed MFMA FLOPs per dense-equivalent FLOP)."""
    if group == "p4m":
        return "p4m", 8, 12 / 64            # 4 characters + the 2 x 2 block: 12 of 64 real products
    T = int(group)
    return T, T, (2 * T - 2) / T ** 2       # cyclic: F0, F_{T/2} and T/2 - 1 complex frequencies


def layer_roofline(layers, es, T, exec_frac, peak_tflops):
    """(bound, algorithmic bytes, executed FLOPs) of the forward over `layers`
    (objects with N, C, D): X read once, Y written once, the T-plane weight
    spectra (C D / T values) read once; executed FLOPs 2 NCD exec_frac.  The
    bound is the roofline model's: "hbm" when the bytes at the HBM peak take
    longer than the FLOPs at the MFMA peak, else "mfma"."""
    alg_bytes = sum(es * L.N * (L.C + L.D) + es * L.C * L.D / T for L in layers)
    exec_flops = 2.0 * exec_frac * sum(L.N * L.C * L.D for L in layers)
    bound = "hbm" if alg_bytes / (HBM_PEAK_GBS * 1e9) > exec_flops / (peak_tflops * 1e12) else "mfma"
    return bound, alg_bytes, exec_flops


def backward_roofline(layers, es, T, exec_frac, peak_tflops):
    """(bound, algorithmic bytes, executed FLOPs) of the backward (dX and dw) over
    `layers`: X and dY read once, dX written once, the transpose spectra read
    once, dw (float32, C D / T values) written once; executed FLOPs twice the
    forward's (the dX and the dw products)."""
    alg_bytes = sum(es * L.N * (2 * L.C + L.D) + es * L.C * L.D / T + 4 * L.C * L.D / T for L in layers)
    exec_flops = 4.0 * exec_frac * sum(L.N * L.C * L.D for L in layers)
    bound = "hbm" if alg_bytes / (HBM_PEAK_GBS * 1e9) > exec_flops / (peak_tflops * 1e12) else "mfma"
    return bound, alg_bytes, exec_flops


def profile_tag(workload, dt, group):
    return f"{workload}_{dt}" + {"4": "", "8": "_c8", "p4m": "_p4m"}[str(group)]


def profiled_traffic(tag, kernel_name, nlayers=1):
    """HBM bytes per launch of `kernel_name` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is no
    summary for this workload or the kernel sources changed since it was taken.
    The summary keeps one row per grid size; with nlayers > 1 (one launch per
    layer, the layers' grids distinct) the rows are summed, and a count other
    than nlayers gives None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    try:
        with open(path) as f:
            d = json.load(f)
        if kernel_source_sha256() != d["source_sha256"]:
            return None
        rows = [r for k, v in d["kernels"].items() if k.startswith(kernel_name) for r in v]
        if nlayers > 1:
            return sum(r["bytes"] for r in rows) if len(rows) == nlayers else None
        return max(r["bytes"] for r in rows) if rows else None
    except (OSError, KeyError, ValueError):
        return None


def dense_weight(torch, w, group):
    """Dense D x C weight of the group-circulant blocks for the dense-GEMM comparator."""
    from group_circulant_linear_amd.module import dense_expansion
    return dense_expansion(w, group).contiguous()


def cpu_baseline(layers, budget_s=12.0):
    """Time the fp64 oracle forward on the host cores (reported baseline only)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    flops = 0.0
    elapsed = 0.0
    samples = []
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < budget_s:
        for (L, X, w, _) in layers:
            n = min(L.N, 2048)
            t0 = time.perf_counter()
            oracle.forward_direct(X[:n], w)
            dt = time.perf_counter() - t0
            elapsed += dt
            flops += 2.0 * n * L.C * L.D
            samples.append(f"{L.name}:{n}x{L.C}->{L.D}")
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 oracle forward_direct on the first rows of each layer "
                      f"({', '.join(sorted(set(samples)))}), repeated for {elapsed:.1f} s"}


def mlp_block(args):
    """EQ-MLP block timing: fc1 (+bias, GELU fused) then fc2 (+bias and the block's skip connection fused:
    Y = X + fc2(GELU(fc1(X)))), against the same block in torch on the dense weights."""
    import torch
    from group_circulant_linear_amd import eqlin
    from group_circulant_linear_amd.inputs import WORKLOADS, make_layer_inputs

    wl = WORKLOADS[args.workload]
    if len(wl.layers) != 2:
        raise SystemExit("--mlp-block needs a two-layer workload (vitb_mlp, vith_mlp)")
    dt = args.dtype or wl.dtypes[0]
    G, T, _ = group_args(args.group)
    tdt = torch.float32 if dt == "f32" else torch.float16
    dev = torch.device("cuda:0")
    L1, L2 = wl.layers
    X, w1, _ = make_layer_inputs(L1.N, L1.C, L1.D, dt, seed=0, layer=0, T=T, with_dy=False)
    _, w2, _ = make_layer_inputs(8, L2.C, L2.D, dt, seed=0, layer=1, T=T, with_dy=False)
    rng = np.random.default_rng(1)
    nsets = 3
    Xs = [torch.from_numpy(X).to(dev) for _ in range(nsets)]
    tw1, tw2 = torch.from_numpy(w1).to(dev), torch.from_numpy(w2).to(dev)
    b1 = torch.from_numpy(rng.standard_normal(L1.D // T).astype(X.dtype)).to(dev)
    b2 = torch.from_numpy(rng.standard_normal(L2.D // T).astype(X.dtype)).to(dev)
    W1, W2 = eqlin.eqlin_prepare_weights(tw1, group=G), eqlin.eqlin_prepare_weights(tw2, group=G)
    Hs = [torch.empty((L1.N, L1.D), dtype=tdt, device=dev) for _ in range(nsets)]
    Ys = [torch.empty((L1.N, L2.D), dtype=tdt, device=dev) for _ in range(nsets)]

    def eq_block(i):
        eqlin.eqlin_forward_ex(Xs[i % nsets], W1, b1, "gelu", out=Hs[i % nsets])
        eqlin.eqlin_forward_ex(Hs[i % nsets], W2, b2, "none", out=Ys[i % nsets], residual=Xs[i % nsets])

    D1, D2 = dense_weight(torch, tw1, G), dense_weight(torch, tw2, G)
    db1, db2 = b1.repeat_interleave(T), b2.repeat_interleave(T)
    F = torch.nn.functional

    def dense_block(i):
        h = F.gelu(F.linear(Xs[i % nsets], D1, db1))
        return torch.addmm(Xs[i % nsets] + db2, h, D2.t())

    def timeit(fn, reps):
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < args.settle:
            for i in range(4):
                fn(i)
            torch.cuda.synchronize()
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    eq_us = timeit(eq_block, args.steps)
    dense_us = timeit(dense_block, args.steps)
    flops = 2.0 * L1.N * (L1.C * L1.D + L2.C * L2.D)
    print(json.dumps({"mode": "mlp_block", "workload": wl.name, "dtype": dt, "group": str(args.group),
                      "block": f"fc1 {L1.C}->{L1.D} +bias+GELU, fc2 {L2.C}->{L2.D} +bias +residual, N={L1.N}",
                      "eq_us": round(eq_us, 2), "dense_us": round(dense_us, 2),
                      "speedup": round(dense_us / eq_us, 3),
                      "eq_tflops_dense_equiv": round(flops / (eq_us * 1e-6) / 1e12, 2),
                      "dense_what": "torch F.linear + F.gelu + addmm (bias and residual) on the pre-expanded "
                                    "dense weights"}),
          flush=True)


def conv_bench(args):
    """p4 group convolution: prepare, forward and backward (dX and dpsi) of one
    layer per step, timed phase by phase as the linear workloads; prints one
    JSON line.  The metric is the forward dense-equivalent throughput
    2 * P * (C K^2) * D / t_forward (P = N H W pixels: the FLOPs of the dense
    K x K convolution with the expanded filter bank); the executed MFMA FLOPs
    are those of the gathered group-circulant layer, 0.75 * P * C K^2 * D."""
    import torch
    from group_circulant_linear_amd import eqlin
    from group_circulant_linear_amd.inputs import CONV_WORKLOADS, make_conv_inputs
    from group_circulant_linear_amd.module import conv_dense_filter

    wl = CONV_WORKLOADS[args.workload]
    L = wl.layers[0]
    dt = args.dtype or wl.dtypes[0]
    tdt = torch.float32 if dt == "f32" else torch.float16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    eqlin.load_library()
    X, psi, dY = make_conv_inputs(L.N, L.H, L.W, L.C, L.D, L.K, dt, seed=0)
    es = X.itemsize
    P = L.N * L.H * L.W
    ws_bytes = eqlin.eqconv_backward_workspace_bytes(L.N, L.H, L.W, L.C, L.D, L.K, tdt)
    set_bytes = es * P * (2 * L.C + 2 * L.D) + ws_bytes
    nsets = args.sets or max(2, int(np.ceil(600e6 / set_bytes)))
    sets = []
    for r in range(nsets):
        sets.append(dict(X=torch.from_numpy(X).to(dev), psi=torch.from_numpy(psi).to(dev),
                         dY=torch.from_numpy(dY).to(dev),
                         buf=torch.empty(eqlin.eqconv_prepared_weight_bytes(L.C, L.D, L.K, tdt), dtype=torch.uint8,
                                         device=dev),
                         Y=torch.empty((L.N, L.H, L.W, L.D), dtype=tdt, device=dev),
                         ws=torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()
    phases = ("prepare", "forward") if args.forward_only else ("prepare", "forward", "backward")
    prepared = [None] * nsets

    def run_phase(ph, i0, count):
        for i in range(i0, i0 + count):
            b = sets[i % nsets]
            if ph == "prepare":
                prepared[i % nsets] = eqlin.eqconv_prepare_weights(b["psi"], out=b["buf"])
            elif ph == "forward":
                eqlin.eqconv_forward(b["X"], prepared[i % nsets], out=b["Y"])
            else:
                eqlin.eqconv_backward(b["dY"], b["X"], prepared[i % nsets], workspace=b["ws"])

    def run_steps(i0, count, events=None):
        for ph in phases:
            if events is not None:
                events[ph][0].record()
            run_phase(ph, i0, count)
            if events is not None:
                events[ph][1].record()

    K = args.steps
    evs = {ph: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for ph in phases}
    with NoGC():
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < args.settle:
            run_steps(0, 2)
            torch.cuda.synchronize()
        if args.warmup:
            run_steps(0, args.warmup)
        torch.cuda.synchronize()
        print(f"# warmup done ({args.warmup} steps after {args.settle} s of clock settle, {nsets} buffer sets)",
              file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        run_steps(0, K, evs)
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / K
    us = {ph: evs[ph][0].elapsed_time(evs[ph][1]) * 1e3 / K for ph in phases}

    ck = L.C * L.K * L.K
    dense_flops = 2.0 * P * ck * L.D
    value = dense_flops / (us["forward"] * 1e-6) / 1e12
    exec_flops = 0.75 * P * ck * L.D
    peak = PEAK_TFLOPS[dt]
    achieved = exec_flops / (us["forward"] * 1e-6) / 1e12
    alg_bytes = es * P * (L.C + L.D) + es * ck * L.D / 4
    traffic = profiled_traffic(f"{wl.name}_{dt}", "eqlin::conv_fwd_kernel")
    roofline = {"bound": "mfma", "kernel": "eqlin::conv_fwd_kernel", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": (round(traffic) if traffic else None), "traffic_algorithmic": round(alg_bytes),
                "traffic_unit": "bytes per launch", "flops_per_launch": exec_flops}
    layer = {"layer": L.name, "N": P, "C": ck, "D": L.D, "images": L.N, "H": L.H, "W": L.W, "C_in": L.C, "K": L.K}
    for ph in phases:
        layer[f"{ph}_us"] = round(us[ph], 2)
    layer["fwd_tflops_dense_equiv"] = round(value, 2)
    layer["fwd_mfma_frac"] = round(achieved / peak, 4)
    if not args.forward_only:
        layer["bwd_tflops_dense_equiv"] = round(2 * dense_flops / (us["backward"] * 1e-6) / 1e12, 2)

    dense = None
    if not args.no_dense:
        # the dense K x K convolution with the expanded filter bank (MIOpen through torch), channels last
        Wd = conv_dense_filter(sets[0]["psi"]).contiguous(memory_format=torch.channels_last)
        xs = [sets[r]["X"].permute(0, 3, 1, 2) for r in range(nsets)]         # NCHW views, channels-last memory
        gs = [sets[r]["dY"].permute(0, 3, 1, 2) for r in range(nsets)]
        pad = L.K // 2
        F = torch.nn.functional

        def dfwd(i):
            return F.conv2d(xs[i % nsets], Wd, padding=pad)

        def dbwd(i):
            return torch.ops.aten.convolution_backward(gs[i % nsets], xs[i % nsets], Wd, None, [1, 1], [pad, pad],
                                                       [1, 1], False, [0, 0], 1, [True, True, False])

        for i in range(3):
            dfwd(i)
            dbwd(i)
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        reps = max(5, K)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            dfwd(i)
        e1.record()
        for i in range(reps):
            dbwd(i)
        e2.record()
        torch.cuda.synchronize()
        tf = e0.elapsed_time(e1) * 1e3 / reps
        tb = e1.elapsed_time(e2) * 1e3 / reps
        dense = {"fwd_us": round(tf, 2), "fwd_tflops": round(dense_flops / (tf * 1e-6) / 1e12, 2),
                 "fwd_speedup": round(tf / us["forward"], 3), "bwd_us": round(tb, 2),
                 "bwd_speedup": (round(tb / us["backward"], 3) if not args.forward_only else None),
                 "what": "torch conv2d / convolution_backward (MIOpen) with the expanded K x K filter bank, "
                         "channels-last, same dtype"}
        del Wd

    if args.copy_calibration_mb:
        nb = args.copy_calibration_mb * (1 << 20)
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = os.cpu_count() or 1
        flops, elapsed, n = 0.0, 0.0, 0
        while elapsed < 10.0:
            t = time.perf_counter()
            oracle.conv_forward(X[n % L.N:n % L.N + 1], psi)
            elapsed += time.perf_counter() - t
            flops += 2.0 * L.H * L.W * ck * L.D
            n += 1
        cpu = {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
               "sample": f"fp64 oracle conv_forward on single {L.H}x{L.W} images ({n} images, {elapsed:.1f} s)"}

    out = {
        "metric": "p4 group conv fwd dense-equiv TFLOP/s (2 P C K^2 D) + % MFMA peak", "value": round(value, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "dtype": dt,
                   "layers": [{"name": L.name, "N": L.N, "H": L.H, "W": L.W, "C": L.C, "D": L.D, "K": L.K}],
                   "group": "4", "T": 4,
                   "step": "prepare+forward" if args.forward_only else "prepare+forward+dX+dpsi",
                   "buffer_sets": nsets},
        "fwd_mfma_frac": round(achieved / peak, 4), "roofline": roofline, "cpu_baseline": cpu,
        "dense_gemm": dense, "per_layer": [layer],
    }
    if args.forward_only:
        out["note"] = "forward-only profiling run, not a bench line"
    print(json.dumps(out), flush=True)


class NoGC:
    """No garbage-collector pass from the clock settle to the end of the timed
    steps: a pass over the objects of earlier workloads can stall the
    launching thread long enough to starve the GPU in phases of short
    launches.  The collection runs before the settle, never between warmup
    and timing: an idle GPU drops its clocks within milliseconds (measured:
    a collection there made every timed kernel about 15% slower)."""

    def __enter__(self):
        gc.collect()
        self.was_enabled = gc.isenabled()
        gc.disable()

    def __exit__(self, *exc):
        if self.was_enabled:
            gc.enable()


def run_linear(args, workload, dtype, group, with_cpu):
    """One linear-layer workload: inputs to HBM, the timed steps, the dense
    comparator; returns the bench dictionary (not printed)."""
    import torch
    from group_circulant_linear_amd import eqlin
    from group_circulant_linear_amd.inputs import WORKLOADS, make_layer_inputs

    wl = WORKLOADS[workload]
    dt = dtype or wl.dtypes[0]
    G, T, exec_frac = group_args(group)
    tdt = torch.float32 if dt == "f32" else torch.float16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    eqlin.load_library()

    # ---- inputs (host, seeded) -> HBM, rotating sets
    layers = []
    for li, L in enumerate(wl.layers):
        X, w, dY = make_layer_inputs(L.N, L.C, L.D, dt, seed=0, layer=li, T=T)
        layers.append((L, X, w, dY))
    set_bytes = 0
    for (L, X, w, dY) in layers:
        es = X.itemsize
        set_bytes += es * L.N * (2 * L.C + 2 * L.D) + eqlin.eqlin_backward_workspace_bytes(L.N, L.C, L.D, tdt, G)
    nsets = args.sets or max(2, int(np.ceil(600e6 / set_bytes)))

    sets = []
    for r in range(nsets):
        S = []
        for (L, X, w, dY) in layers:
            tX = torch.from_numpy(X).to(dev)
            tw = torch.from_numpy(w).to(dev)
            tdY = torch.from_numpy(dY).to(dev)
            Wbuf = torch.empty(eqlin.eqlin_prepared_weight_bytes(L.C, L.D, tdt, G), dtype=torch.uint8, device=dev)
            Y = torch.empty((L.N, L.D), dtype=tdt, device=dev)
            dX = torch.empty((L.N, L.C), dtype=tdt, device=dev)
            dw = torch.empty((L.D // T, L.C // T, T), dtype=torch.float32, device=dev)
            ws = torch.empty(max(1, eqlin.eqlin_backward_workspace_bytes(L.N, L.C, L.D, tdt, G)), dtype=torch.uint8,
                             device=dev)
            S.append(dict(L=L, X=tX, w=tw, dY=tdY, Wbuf=Wbuf, Y=Y, dX=dX, dw=dw, ws=ws))
        sets.append(S)
    torch.cuda.synchronize()

    phases = ("prepare", "forward") if args.forward_only else ("prepare", "forward", "backward")
    prepared = [[None] * len(layers) for _ in range(nsets)]

    def run_phase(p, li, i0, count):
        for i in range(i0, i0 + count):
            b = sets[i % nsets][li]
            if p == "prepare":
                prepared[i % nsets][li] = eqlin.eqlin_prepare_weights(b["w"], out=b["Wbuf"], group=G)
            elif p == "forward":
                eqlin.eqlin_forward(b["X"], prepared[i % nsets][li], out=b["Y"])
            else:
                eqlin.eqlin_backward(b["dY"], b["X"], prepared[i % nsets][li], workspace=b["ws"], dX_out=b["dX"],
                                     dw_out=b["dw"])

    def run_steps(i0, count, events=None):
        """`count` steps (batches i0, i0+1, ...): for each layer, each phase runs for
        all the batches back to back between one event pair, so the per-launch time
        carries no event overhead (an event pair around a single launch adds a few
        microseconds to it)."""
        for li in range(len(layers)):
            for p in phases:
                if events is not None:
                    events[li][p][0].record()
                run_phase(p, li, i0, count)
                if events is not None:
                    events[li][p][1].record()

    K = args.steps
    evs = [{p: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for p in phases}
           for _ in layers]
    with NoGC():
        # untimed clock settle: the GPU ramps its clocks over the first tens of
        # milliseconds of work, longer than a few warmup steps take
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < args.settle:
            run_steps(0, 4)
            torch.cuda.synchronize()
        if args.warmup:
            run_steps(0, args.warmup)
        torch.cuda.synchronize()
        print(f"# warmup done ({args.warmup} steps after {args.settle} s of clock settle, {nsets} buffer sets)",
              file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        run_steps(0, K, evs)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    ph_us = {p: [0.0] * len(layers) for p in ("prepare", "forward", "backward")}
    for li in range(len(layers)):
        for p in phases:
            a, b = evs[li][p]
            ph_us[p][li] = a.elapsed_time(b) * 1e3 / K

    fwd_flops = sum(2.0 * L.N * L.C * L.D for (L, _, _, _) in layers)
    fwd_us = sum(ph_us["forward"])
    value = fwd_flops / (fwd_us * 1e-6) / 1e12
    exec_flops = 2.0 * exec_frac * sum(L.N * L.C * L.D for (L, _, _, _) in layers)

    # roofline of the forward kernel (one launch per layer; summed over layers)
    achieved = exec_flops / (fwd_us * 1e-6) / 1e12
    peak = PEAK_TFLOPS[dt]
    es_b = 4 if dt == "f32" else 2
    bound, alg_bytes, _ = layer_roofline([L for (L, _, _, _) in layers], es_b, T, exec_frac, peak)
    traffic = profiled_traffic(profile_tag(wl.name, dt, group), "eqlin::fwd_kernel", len(layers))
    gbs = alg_bytes / (fwd_us * 1e-6) / 1e9
    hbm_bound = bound == "hbm"
    roofline = {"bound": "hbm" if hbm_bound else "mfma", "kernel": "eqlin::fwd_kernel",
                "achieved": round(gbs, 1) if hbm_bound else round(achieved, 2),
                "peak": HBM_PEAK_GBS if hbm_bound else peak,
                "unit": "GB/s" if hbm_bound else "TFLOP/s",
                "frac": round(gbs / HBM_PEAK_GBS if hbm_bound else achieved / peak, 4),
                "traffic": (round(traffic) if traffic else None),
                "traffic_algorithmic": round(alg_bytes), "traffic_unit": "bytes per launch",
                "flops_per_launch": exec_flops,
                "mfma_tflops": round(achieved, 2), "mfma_frac": round(achieved / peak, 4),
                "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}

    per_layer = []
    for li, (L, _, _, _) in enumerate(layers):
        nd = L.N * L.C * L.D
        es = 4 if dt == "f32" else 2
        d = {"layer": L.name, "N": L.N, "C": L.C, "D": L.D}
        for p in phases:
            d[f"{p}_us"] = round(ph_us[p][li], 2)
        d["fwd_tflops_dense_equiv"] = round(2 * nd / (ph_us["forward"][li] * 1e-6) / 1e12, 2)
        d["fwd_mfma_frac"] = round(2 * exec_frac * nd / (ph_us["forward"][li] * 1e-6) / 1e12 / peak, 4)
        d["fwd_hbm_gbs_algorithmic"] = round(
            (es * L.N * (L.C + L.D) + es * L.C * L.D / T) / (ph_us["forward"][li] * 1e-6) / 1e9, 1)
        if not args.forward_only:
            d["bwd_tflops_dense_equiv"] = round(4 * nd / (ph_us["backward"][li] * 1e-6) / 1e12, 2)
            d["bwd_mfma_frac"] = round(4 * exec_frac * nd / (ph_us["backward"][li] * 1e-6) / 1e12 / peak, 4)
        per_layer.append(d)

    # dense GEMM comparator: F.linear on the pre-expanded weight, same dtype, same stream
    dense = None
    if not args.no_dense:
        F = torch.nn.functional
        tot_f, tot_b = 0.0, 0.0
        for li, (L, X, w, dY) in enumerate(layers):
            b = sets[0][li]
            Wd = dense_weight(torch, b["w"], G)
            Xs = [sets[r][li]["X"] for r in range(nsets)]
            dYs = [sets[r][li]["dY"] for r in range(nsets)]
            Yd = torch.empty((L.N, L.D), dtype=tdt, device=dev)
            dXd = torch.empty((L.N, L.C), dtype=tdt, device=dev)
            dWd = torch.empty((L.D, L.C), dtype=tdt, device=dev)
            for i in range(3):
                torch.mm(Xs[i % nsets], Wd.t(), out=Yd)
                torch.mm(dYs[i % nsets], Wd, out=dXd)
                torch.mm(dYs[i % nsets].t(), Xs[i % nsets], out=dWd)
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            reps = max(10, K)
            torch.cuda.synchronize()
            e0.record()
            for i in range(reps):
                torch.mm(Xs[i % nsets], Wd.t(), out=Yd)
            e1.record()
            for i in range(reps):
                torch.mm(dYs[i % nsets], Wd, out=dXd)
                torch.mm(dYs[i % nsets].t(), Xs[i % nsets], out=dWd)
            e2.record()
            torch.cuda.synchronize()
            tot_f += e0.elapsed_time(e1) * 1e3 / reps
            tot_b += e1.elapsed_time(e2) * 1e3 / reps
            del Wd
        eq_b = sum(ph_us["backward"])
        dense = {"fwd_us": round(tot_f, 2), "fwd_tflops": round(fwd_flops / (tot_f * 1e-6) / 1e12, 2),
                 "fwd_speedup": round(tot_f / fwd_us, 3), "bwd_us": round(tot_b, 2),
                 "bwd_speedup": (round(tot_b / eq_b, 3) if not args.forward_only else None),
                 "what": "torch.matmul (hipBLASLt) on the pre-expanded dense weight, same dtype"}

    if args.copy_calibration_mb:
        nb = args.copy_calibration_mb * (1 << 20)
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    if hbm_bound and not args.no_dense:
        # practical streaming ceiling beside the HBM peak: a device copy moving
        # the forward's algorithmic bytes (half read, half written), rotating
        # over buffer sets as the layer's launches do
        half = int(alg_bytes) // 2 // 4
        cps = [(torch.empty(half, dtype=torch.float32, device=dev).fill_(1.0),
                torch.empty(half, dtype=torch.float32, device=dev)) for _ in range(nsets)]
        for (a, b) in cps:
            b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(10, K)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            cps[i % nsets][1].copy_(cps[i % nsets][0])
        e1.record()
        torch.cuda.synchronize()
        cp_us = e0.elapsed_time(e1) * 1e3 / reps
        roofline["copy_gbs"] = round(2 * half * 4 / (cp_us * 1e-6) / 1e9, 1)
        roofline["copy_us"] = round(cp_us, 2)
        del cps

    roofline_bwd = None
    if not args.forward_only:
        bwd_us = sum(ph_us["backward"])
        bbound, bbytes, bflops = backward_roofline([L for (L, _, _, _) in layers], es_b, T, exec_frac, peak)
        b_hbm = bbound == "hbm"
        b_tf = bflops / (bwd_us * 1e-6) / 1e12
        b_gbs = bbytes / (bwd_us * 1e-6) / 1e9
        roofline_bwd = {"bound": bbound, "kernel": "eqlin::bwd_fused_kernel (+ dw finalize)",
                        "achieved": round(b_gbs, 1) if b_hbm else round(b_tf, 2),
                        "peak": HBM_PEAK_GBS if b_hbm else peak, "unit": "GB/s" if b_hbm else "TFLOP/s",
                        "frac": round(b_gbs / HBM_PEAK_GBS if b_hbm else b_tf / peak, 4),
                        "traffic": None, "traffic_algorithmic": round(bbytes), "flops_per_launch": bflops,
                        "mfma_tflops": round(b_tf, 2), "mfma_frac": round(b_tf / peak, 4),
                        "hbm_gbs": round(b_gbs, 1), "hbm_frac": round(b_gbs / HBM_PEAK_GBS, 4)}
        if len(layers) == 1:
            t = profiled_traffic(profile_tag(wl.name, dt, group), "eqlin::bwd_fused_kernel")
            roofline_bwd["traffic"] = round(t) if t else None

    cpu = None
    if with_cpu:
        cpu = cpu_baseline(layers)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "dtype": dt,
                   "layers": [{"name": L.name, "N": L.N, "C": L.C, "D": L.D} for (L, _, _, _) in layers],
                   "group": str(group), "T": T,
                   "step": ("prepare+forward" if args.forward_only else "prepare+forward+dX+dw"),
                   "buffer_sets": nsets},
        "fwd_mfma_frac": round(achieved / peak, 4),
        "roofline": roofline,
        "roofline_backward": roofline_bwd,
        "cpu_baseline": cpu,
        "dense_gemm": dense,
        "per_layer": per_layer,
    }
    if args.forward_only:
        out["note"] = "forward-only profiling run, not a bench line"
    del sets, prepared
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# The configurations beside the headline (the ViT-B attention projection in
# fp32), each with its own timing, roofline and dense comparison: the layer
# shapes at which the method's speed-up is stated (large widths, ViT-H), the
# f16 MLP pair and the backward of the attention shapes.
PER_CONFIG = (("vith_mlp", "f32"), ("vith_mlp", "f16"), ("vitb_mlp", "f16"), ("vitb_attn_bwd", "f16"),
              ("vitb_attn_bwd", "f32"))


def config_summary(r):
    """The per-configuration entry of the bench line."""
    keys = ("value", "unit", "ms_per_step", "dtype", "fwd_mfma_frac", "roofline", "roofline_backward",
            "dense_gemm", "per_layer")
    d = {"workload": r["config"]["workload"], "description": r["config"]["description"]}
    d.update({k: r[k] for k in keys})
    d["metric"] = "forward dense-equivalent TFLOP/s (2NDC), summed over the layers"
    return d


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures a single GPU; --gpus must be 1"}))
        sys.exit(2)
    if args.mlp_block:
        mlp_block(args)
        return
    from group_circulant_linear_amd.inputs import CONV_WORKLOADS
    if args.workload in CONV_WORKLOADS:
        conv_bench(args)
        return
    out = run_linear(args, args.workload, args.dtype, args.group, not args.no_cpu_baseline)
    headline = (args.workload == "vitb_attn" and args.dtype in (None, "f32") and str(args.group) == "4"
                and not args.forward_only)
    if headline and not args.no_per_config:
        out["per_config"] = []
        for (wl, dt) in PER_CONFIG:
            print(f"# per-config {wl} {dt}", file=sys.stderr, flush=True)
            out["per_config"].append(config_summary(run_linear(args, wl, dt, "4", False)))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
