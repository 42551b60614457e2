#!/usr/bin/env python3
"""Benchmark of the routed FP8 block-scaled MoE layer on one MI355X.

One step = one forward of the whole layer (router top-k, 1x128 activation
quantisation, grouping, gate/up GEMM, SiLU-mul requantisation, down GEMM,
fixed-order combine) over one batch of synthetic input already resident in
HBM.  The default workload is the one-token decode layer
(M=1, h=2048, i=768, E=128, top-8).

Timing: the forwards of C rotation copies (distinct weight copies and
inputs, together far larger than the 256 MB Infinity Cache, so every step
streams its experts from HBM) are captured in one HIP graph; W warm-up steps,
then exactly K timed steps between a synchronisation and HIP events on both
sides.  A second pass times graph replays of the same forwards cut after
their first j stages (j = 1..n, HIP events around the replays); the
differences give each stage's mean duration, and the dominant stage is
reported against its roofline.  The CPU baseline is the oracle (plain C, all host
threads) on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
MALL_BYTES = 256 << 20         # Infinity Cache
METRIC = "MoE-layer tokens/s; %HBM peak at M=1/12 and %FP8 MFMA peak at M=8192"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=1, help="layer shape index (0..5); 1 = decode M=1")
    ap.add_argument("--copies", type=int, default=0, help="rotation copies (0 = enough to exceed 4x the Infinity Cache)")
    ap.add_argument("--timing-replays", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device-to-device copies of MIB MiB (counter calibration) and exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output folders of FETCH_SIZE / WRITE_SIZE runs of a workload and of "
                         "the copy calibration: record the kernel's HBM bytes per launch in profiles/traffic.json")
    ap.add_argument("--pmc-kernel", default=None, help="kernel for --pmc-summary")
    ap.add_argument("--pmc-copy-mib", type=int, default=1024, help="copy size of the calibration runs")
    ap.add_argument("--pmc-workload", default=None, help="workload name of the record (default: --config's)")
    ap.add_argument("--front-end", action="store_true",
                    help="time the RMSNorm + 1x128 quantisation front end alone on --config's activations")
    ap.add_argument("--router-gemm", action="store_true",
                    help="time BF16 routing fused with the top-k alone on --config's activations")
    ap.add_argument("--mxfp4", action="store_true",
                    help="time the layer with MXFP4 expert weights (default shape: the wide-decode batch)")
    args = ap.parse_args()
    args.config_given = any(a == "--config" or a.startswith("--config=") for a in sys.argv[1:])
    return args


def weight_bytes_per_expert(cfg):
    w13 = 2 * cfg.i * cfg.h + (2 * cfg.i // 128) * (cfg.h // 128) * 4
    w2 = cfg.h * cfg.i + (cfg.h // 128) * (cfg.i // 128) * 4
    return w13, w2


# Sources whose text decides each measured kernel (traffic records are tied
# to their digest).
KERNEL_SOURCES = {
    "fused_decode_kernel": ["fp8_block_scaled_router_amd/csrc/fused_decode.hip",
                            "fp8_block_scaled_router_amd/csrc/fused_decode.h",
                            "fp8_block_scaled_router_amd/csrc/device.h"],
    "stream_gate_up_kernel": ["fp8_block_scaled_router_amd/csrc/stream_gemm.hip",
                              "fp8_block_scaled_router_amd/csrc/device.h"],
    "prefill_gate_up_kernel": ["fp8_block_scaled_router_amd/csrc/prefill_gemm.hip",
                               "fp8_block_scaled_router_amd/csrc/device.h",
                               "fp8_block_scaled_router_amd/csrc/launch.h"],
}
KERNEL_SOURCES["stream_down_kernel"] = KERNEL_SOURCES["stream_gate_up_kernel"]
KERNEL_SOURCES["stream_gate_up_mx_kernel"] = ["fp8_block_scaled_router_amd/csrc/mxfp4_gemm.hip",
                                              "fp8_block_scaled_router_amd/csrc/device.h"]
KERNEL_SOURCES["stream_down_mx_kernel"] = KERNEL_SOURCES["stream_gate_up_mx_kernel"]
KERNEL_SOURCES["prefill_down_kernel"] = KERNEL_SOURCES["prefill_gate_up_kernel"]


def copy_calibration(mib):
    """Three plain device-to-device copies of a known size: rocprofv3's
    FETCH_SIZE / WRITE_SIZE of these dispatches calibrate the counters."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}))


def pmc_mean_kb(folder, name_prefix, largest_grid=False):
    """Mean Counter_Value (KiB) over the dispatches of one kernel in a
    rocprofv3 --pmc CSV folder (largest grid only, if asked)."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Kernel_Name"].startswith(name_prefix):
                rows.append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no dispatch of {name_prefix} in {folder}")
    if largest_grid:
        g = max(r[0] for r in rows)
        rows = [r for r in rows if r[0] == g]
    return sum(v for _, v in rows) / len(rows), len(rows)


def pmc_summary(args):
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.pmc_summary
    kernel = args.pmc_kernel
    import synth
    cfg = synth.CONFIGS[args.config]
    copy_bytes = args.pmc_copy_mib << 20
    cf, ncf = pmc_mean_kb(cfetch_dir, "__amd_rocclr_copyBuffer", largest_grid=True)
    cw, ncw = pmc_mean_kb(cwrite_dir, "__amd_rocclr_copyBuffer", largest_grid=True)
    f_scale, w_scale = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    fk, nf = pmc_mean_kb(fetch_dir, f"moe::{kernel}(")
    wk, nw = pmc_mean_kb(write_dir, f"moe::{kernel}(")
    fetch, write = fk * 1024 * f_scale, wk * 1024 * w_scale
    path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    srcs = KERNEL_SOURCES[kernel]
    name = args.pmc_workload or cfg.name
    db[f"{name}:{kernel}"] = {
        "bytes_per_launch": int(round(fetch + write)),
        "fetch_bytes_per_launch": int(round(fetch)), "write_bytes_per_launch": int(round(write)),
        "raw_fetch_kib": round(fk, 1), "raw_write_kib": round(wk, 1), "dispatches": [nf, nw],
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                             "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "sources": srcs, "source_sha256_16": source_digest(srcs),
    }
    with open(path, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(db[f"{name}:{kernel}"]))


def stage_work(cfg, stage, U):
    """Algorithmic bytes (HBM-bound stages) and FLOPs of one launch of a stage."""
    M, h, i, k = cfg.M, cfg.h, cfg.i, cfg.k
    w13, w2 = weight_bytes_per_expert(cfg)
    act = M * h + M * (h // 128) * 4
    if stage.startswith("stream_gate_up"):
        return U * w13 + act, 4.0 * M * k * h * i
    if stage.startswith("stream_down"):
        return U * w2, 2.0 * M * k * h * i
    if stage.startswith("prefill_gate_up"):
        # weights once, activation rows per route in, E4M3 codes + scales out
        return U * w13 + M * k * (h + i + (h // 128 + i // 128) * 4), 4.0 * M * k * h * i
    if stage.startswith("prefill_down"):   # bf16 partials out
        return U * w2 + M * k * (i + (i // 128) * 4 + h * 2), 2.0 * M * k * h * i
    if stage.startswith("route_quant"):
        return M * h * 2 + M * cfg.E * 4 + act + M * k * 8, 0.0
    if stage.startswith("combine_bf16"):
        return M * k * h * 2 + M * h * 2 + M * k * 4, 0.0   # bf16 partials in, bf16 out
    if stage.startswith("combine"):
        return M * k * h * 4 + M * h * 2 + M * k * 4, 0.0   # fp32 partials in, bf16 out
    if stage.startswith("fused"):
        return U * (w13 + w2) + M * h * 2 * 2 + M * cfg.E * 4, 6.0 * M * k * h * i
    return 0, 0.0


def source_digest(paths):
    """Digest of the sources' code lines (lines that are whole // comments are
    left out, so editing a comment keeps a measurement valid)."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            for line in f:
                if not line.lstrip().startswith(b"//"):
                    h.update(line)
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))[f"{workload}:{kernel}"]
    except (KeyError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_digest(rec["sources"]):
        return None
    return rec["bytes_per_launch"]


def time_single_kernel(launch, C, args):
    """Mean duration of one launch: launch(c) for the C rotation copies
    captured in one HIP graph on a side stream, W warm-up launches, then
    K launches between HIP events on that stream, queued behind a GPU spin so
    that the GPU, not the host, sets the pace.  Returns (ms per launch,
    replays, warm-up replays)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for c in range(C):
            launch(c)
    reps_w = max(1, args.warmup // C)
    reps = max(1, args.steps // C)
    with torch.cuda.stream(side):
        for _ in range(reps_w):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)
        e0.record(side)
        for _ in range(reps):
            g.replay()
        e1.record(side)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * C), reps, reps_w


def router_gemm_bench(args):
    """BF16 routing fused with the top-k alone, on the activation rows of a
    layer shape and a bf16 router weight N(0, 1/sqrt(h)) [E, h]: x and the
    weight rotated over copies that together exceed 4x the Infinity Cache.
    HBM roofline from the algorithmic bytes: x (2h per row) and the router
    weight (2Eh) in, logits (4E per row), ids and weights (8k per row) out."""
    import numpy as np
    import torch

    import fp8_block_scaled_router_amd as moe
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    moe.lib()
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    seed = synth.default_seed(args.config) if args.seed is None else args.seed
    M, h, E, k = cfg.M, cfg.h, cfg.E, cfg.k
    copy_bytes = 2 * M * h + 2 * E * h + M * (4 * E + 8 * k)
    C = args.copies or max(2, math.ceil(4 * MALL_BYTES / copy_bytes) + 1)
    C = min(C, 4096)
    x0 = torch.from_numpy(synth.make_x(cfg, seed).view(np.int16)).view(torch.bfloat16).to(dev)
    w0 = torch.from_numpy(synth.make_wr(cfg, seed).view(np.int16)).view(torch.bfloat16).to(dev)
    X = [x0] + [x0.clone() for _ in range(C - 1)]
    W = [w0] + [w0.clone() for _ in range(C - 1)]
    OUT = [(torch.empty((M, E), dtype=torch.float32, device=dev),
            torch.empty((M, k), dtype=torch.int32, device=dev),
            torch.empty((M, k), dtype=torch.float32, device=dev)) for _ in range(C)]
    for c in range(C):
        moe.router_gemm_topk(X[c], W[c], k, out=OUT[c])
    torch.cuda.synchronize()
    ms, reps, reps_w = time_single_kernel(lambda c: moe.router_gemm_topk(X[c], W[c], k, out=OUT[c]), C, args)
    achieved = copy_bytes / (ms / 1e3) / 1e9
    flops = 2.0 * M * h * E
    line = {
        "metric": "BF16 routing tokens/s (router logits GEMM fused with top-k)",
        "value": round(M / (ms / 1e3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": reps * C, "warmup": reps_w * C, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, fp32 accumulate", "data": "synthetic",
        "config": {"workload": f"router_gemm_topk_m{M}_h{h}_e{E}_top{k}", "M": M, "h": h, "E": E, "k": k,
                   "rotation_copies": C, "timing": "HIP graph of C launches, events around the replays"},
        "roofline": {"bound": "hbm", "kernel": "router_gemm_topk_kernel", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": int(copy_bytes),
                     "algorithmic_flops_per_launch": flops,
                     "bf16_mfma_frac": round(flops / (ms / 1e3) / 2.5e15, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def mxfp4_bench(args):
    """The layer with MXFP4 expert weights (E2M1 codes, E8M0 scale per 32 K
    elements) on --config's shape (default: the wide-decode batch, the MXFP4
    kernel's h 6144 / i 768 / E 128 / top-4).  The codes are uniform random
    bytes and the scales random powers of two near 2^-8 (values do not change
    the streamed bytes; routing comes from the shape's own logits).  Weight
    copies, inputs and workspaces rotate over C copies that together exceed
    4x the Infinity Cache; stage durations from graph replays of forwards cut
    after each stage, as in the FP8 bench."""
    import numpy as np
    import torch

    import fp8_block_scaled_router_amd as moe
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    moe.lib()
    dev = torch.device("cuda:0")
    ci = args.config if args.config_given else 3
    cfg = synth.CONFIGS[ci]
    seed = synth.default_seed(ci) if args.seed is None else args.seed
    M, h, i, E, k = cfg.M, cfg.h, cfg.i, cfg.E, cfg.k
    w13b = 2 * i * (h // 2) + 2 * i * (h // 32)
    w2b = h * (i // 2) + h * (i // 32)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def weights():
        return (torch.randint(0, 256, (E, 2 * i, h // 2), dtype=torch.uint8, device=dev, generator=gen),
                torch.randint(117, 122, (E, 2 * i, h // 32), dtype=torch.uint8, device=dev, generator=gen),
                torch.randint(0, 256, (E, h, i // 2), dtype=torch.uint8, device=dev, generator=gen),
                torch.randint(117, 122, (E, h, i // 32), dtype=torch.uint8, device=dev, generator=gen))

    ids0, _ = moe.router_topk(torch.from_numpy(synth.make_logits(cfg, seed, copy=0)).to(dev), k)
    U0 = int(torch.unique(ids0).numel())
    C = args.copies or max(2, math.ceil(4 * MALL_BYTES / (U0 * (w13b + w2b))) + 1)
    C = max(1, min(C, int((48 << 30) // (E * (w13b + w2b)))))
    W = [weights() for _ in range(C)]
    X, Lg, WS, OUT = [], [], [], []
    for c in range(C):
        X.append(torch.from_numpy(synth.make_x(cfg, seed, copy=c).view(np.int16)).view(torch.bfloat16).to(dev))
        Lg.append(torch.from_numpy(synth.make_logits(cfg, seed, copy=c)).to(dev))
        WS.append(moe.alloc_mxfp4_workspace(M, h, i, E, k, device=dev))
        OUT.append(torch.empty((M, h), dtype=torch.bfloat16, device=dev))
    U = []
    for c in range(C):
        ids, _ = moe.router_topk(Lg[c], k)
        U.append(int(torch.unique(ids).numel()))
    torch.cuda.synchronize()

    def fwd(c, n=None):
        a = W[c]
        moe.moe_mxfp4_forward_ws(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], out=OUT[c], n_stages=n)

    for c in range(C):
        fwd(c)
    torch.cuda.synchronize()
    assert all(torch.isfinite(OUT[c].float()).all().item() for c in range(C))
    ms, reps, reps_w = time_single_kernel(lambda c: fwd(c), C, args)
    names = moe.moe_mxfp4_stage_names(M, k)
    T = [0.0]
    for j in range(1, len(names) + 1):
        tj, _, _ = time_single_kernel(lambda c, j=j: fwd(c, j), C, args)
        T.append(tj)
    stage_ms = np.maximum(np.diff(np.array(T)), 0.0)
    dom = int(np.argmax(stage_ms))
    Um = float(np.mean(U))
    work = {"stream_gate_up_mx_kernel": Um * w13b + M * h + 4 * M * h / 128,
            "stream_down_mx_kernel": Um * w2b,
            "combine_kernel": 4 * M * k * h + 2 * M * h + 4 * M * k}
    abytes = work.get(names[dom], 0.0)
    achieved = abytes / (stage_ms[dom] / 1e3) / 1e9
    fw_bytes = Um * (w13b + w2b) + M * h * 4 + M * E * 4
    workload = "mxfp4_" + cfg.name
    line = {
        "metric": "MXFP4 MoE-layer tokens/s",
        "value": round(M / (ms / 1e3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": reps * C, "warmup": reps_w * C, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e2m1 weights x e4m3 activations (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": workload,
                   "M": M, "h": h, "i": i, "E": E, "k": k, "rotation_copies": C, "distinct_experts_mean": Um,
                   "layer_bytes_per_step": int(fw_bytes),
                   "stage_us": {n: round(float(t) * 1e3, 3) for n, t in zip(names, stage_ms)},
                   "timing": "HIP graph of C forwards; stages from graphs of forwards cut after each stage"},
        "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(names[dom], workload),
                     "avg_launch_us": round(stage_ms[dom] * 1e3, 3), "algorithmic_bytes_per_launch": int(abytes),
                     "forward_hbm_frac": round(fw_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def front_end_bench(args):
    """The RMSNorm + 1x128 E4M3 quantisation front end alone, on the
    activation rows of a layer shape: inputs and outputs rotated over copies
    that together exceed 4x the Infinity Cache, C launches per HIP graph,
    events around K launches on the launch stream.  HBM roofline from the
    algorithmic bytes: x in (2h per row), codes, scales and the bf16
    normalised rows out (h + h/32 + 2h per row), the norm weight once."""
    import numpy as np
    import torch

    import fp8_block_scaled_router_amd as moe
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    moe.lib()
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    seed = synth.default_seed(args.config) if args.seed is None else args.seed
    M, h = cfg.M, cfg.h
    eps = 1e-6
    row_bytes = 2 * h + h + (h // 128) * 4 + 2 * h
    launch_bytes = M * row_bytes + 4 * h
    C = args.copies or max(2, math.ceil(4 * MALL_BYTES / (M * row_bytes)) + 1)
    C = min(C, 4096)
    x0 = torch.from_numpy(synth.make_x(cfg, seed).view(np.int16)).view(torch.bfloat16).to(dev)
    gamma = torch.from_numpy(np.random.default_rng(seed).uniform(0.5, 1.5, h).astype(np.float32)).to(dev)
    X = [x0] + [x0.clone() for _ in range(C - 1)]
    OUT = [(torch.empty((M, h), dtype=torch.bfloat16, device=dev),
            torch.empty((M, h), dtype=torch.uint8, device=dev),
            torch.empty((M, h // 128), dtype=torch.float32, device=dev)) for _ in range(C)]
    for c in range(C):
        moe.rmsnorm_act_quant(X[c], gamma, eps, out=OUT[c])
    torch.cuda.synchronize()
    ms, reps, reps_w = time_single_kernel(lambda c: moe.rmsnorm_act_quant(X[c], gamma, eps, out=OUT[c]), C, args)
    achieved = launch_bytes / (ms / 1e3) / 1e9
    line = {
        "metric": "front end rows/s (RMSNorm + 1x128 E4M3 quantisation)",
        "value": round(M / (ms / 1e3), 2), "unit": "rows/s", "n_gpus": 1,
        "steps": reps * C, "warmup": reps_w * C, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, f64 row sums, e4m3 out", "data": "synthetic",
        "config": {"workload": f"rmsnorm_quant_m{M}_h{h}", "M": M, "h": h, "rotation_copies": C,
                   "timing": "HIP graph of C launches, events around the replays"},
        "roofline": {"bound": "hbm", "kernel": "rmsnorm_quant_kernel", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": int(launch_bytes)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer is not sharded across GPUs", file=sys.stderr)
        sys.exit(2)
    if args.front_end:
        front_end_bench(args)
        return
    if args.router_gemm:
        router_gemm_bench(args)
        return
    if args.mxfp4:
        mxfp4_bench(args)
        return

    import numpy as np
    import torch

    import fp8_block_scaled_router_amd as moe
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    moe.lib()
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    seed = synth.default_seed(args.config) if args.seed is None else args.seed
    M, h, i, E, k = cfg.M, cfg.h, cfg.i, cfg.E, cfg.k
    w13b, w2b = weight_bytes_per_expert(cfg)
    wbytes = E * (w13b + w2b)

    # ---- inputs: weights drawn on the host, quantised on the GPU by the library
    t0 = time.time()
    w13_f = synth.make_w13_f32(cfg, seed)
    w2_f = synth.make_w2_f32(cfg, seed)
    q13, s13 = moe.quantize_weight_block128(torch.from_numpy(w13_f).to(dev))
    q2, s2 = moe.quantize_weight_block128(torch.from_numpy(w2_f).to(dev))
    torch.cuda.synchronize()
    # Rotation: enough weight copies that a copy's experts are touched again
    # only after >= 4x the Infinity Cache of other traffic (distinct experts
    # per step measured with the library's own router on copy 0).
    ids0, _ = moe.router_topk(torch.from_numpy(synth.make_logits(cfg, seed, copy=0)).to(dev), k)
    U0 = int(torch.unique(ids0).numel())
    step_bytes = U0 * (w13b + w2b)
    C = args.copies or max(2, math.ceil(4 * MALL_BYTES / step_bytes) + 1)
    C = max(1, min(C, int((48 << 30) // wbytes)))
    W = [(q13, s13, q2, s2)] + [(q13.clone(), s13.clone(), q2.clone(), s2.clone()) for _ in range(C - 1)]
    X, Lg, WS, OUT = [], [], [], []
    for c in range(C):
        xb = synth.make_x(cfg, seed, copy=c)
        X.append(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev))
        Lg.append(torch.from_numpy(synth.make_logits(cfg, seed, copy=c)).to(dev))
        WS.append(moe.alloc_workspace(M, h, i, E, k, device=dev))
        OUT.append(torch.empty((M, h), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def fwd(c):
        a = W[c]
        moe.moe_fp8_forward_ws(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], out=OUT[c])

    # eager warm-up of every copy, then distinct experts per copy
    for c in range(C):
        fwd(c)
    torch.cuda.synchronize()
    lay = moe.workspace_layout(M, h, i, E, k)
    U = [int(WS[c][lay.num_active:lay.num_active + 4].view(torch.int32).item()) for c in range(C)]
    assert all(torch.isfinite(OUT[c].float()).all().item() for c in range(C))

    # ---- graphs: all C forwards, and the first r forwards for a remainder
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for c in range(n):
                fwd(c)
        return g

    g_all = capture(C)
    rem = args.steps % C
    g_rem = capture(rem) if rem else None

    def run_steps(n):
        for _ in range(n // C):
            g_all.replay()
        r = n % C
        if r:
            if r == rem:
                g_rem.replay()
            else:
                for c in range(r):
                    fwd(c)

    run_steps(args.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    run_steps(args.steps)
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / args.steps
    tokens_per_s = M / (ms_per_step / 1e3)

    # ---- per-stage durations: HIP-graph replays of the C forwards cut after
    # their first j stages (j = 1..n), timed by HIP events on the launch
    # stream; stage j's duration is T(j) - T(j - 1) per forward.  No event
    # sits between stages, so a short stage is not charged the event's own
    # cost, and the stages run back to back as in the timed steps.  The
    # replays wait behind a GPU spin kernel while the host queues them.
    names = moe.forward_kernel_names(M, h, i, E, k)
    nst = len(names)

    def capture_prefix(j):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for c in range(C):
                a = W[c]
                moe.moe_fp8_forward_ws_prefix(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], j, out=OUT[c])
        return g

    reps = max(1, args.timing_replays)
    T = [0.0]
    for j in range(1, nst + 1):
        gj = g_all if j == nst else capture_prefix(j)
        gj.replay()
        torch.cuda.synchronize()
        # the replays are queued behind a GPU spin, so that a short prefix
        # is timed on the GPU, not at the host's launch rate
        torch.cuda._sleep(20_000_000)
        e0.record()
        for _ in range(reps):
            gj.replay()
        e1.record()
        torch.cuda.synchronize()
        T.append(e0.elapsed_time(e1) / (reps * C))
        if gj is not g_all:
            del gj
    stage_ms = np.maximum(np.diff(np.array(T)), 0.0)
    count = reps * C
    timing_mode = "HIP-graph replays of forwards cut after each stage, differences"
    # the full forwards leave every copy's output complete again
    run_steps(C)
    torch.cuda.synchronize()
    dom = int(np.argmax(stage_ms))
    U_mean = float(np.mean(U))
    abytes, aflops = stage_work(cfg, names[dom], U_mean)
    dom_s = stage_ms[dom] / 1e3
    # the forward's bound: its algorithmic bytes (selected weights, x, logits,
    # out) against its FLOPs, each over its peak
    fw_bytes = U_mean * sum(weight_bytes_per_expert(cfg)) + M * h * 4 + M * E * 4
    fw_flops = 6.0 * M * k * h * i
    bound = "hbm" if fw_bytes / (HBM_PEAK_GBS * 1e9) >= fw_flops / (FP8_PEAK_TFLOPS * 1e12) else "mfma"
    if bound == "hbm":
        achieved = abytes / dom_s / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = aflops / dom_s / 1e12
        peak, unit = FP8_PEAK_TFLOPS, "TFLOP/s"
    roofline = {"bound": bound, "kernel": names[dom], "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": load_traffic(names[dom], cfg.name),
                "avg_launch_us": round(stage_ms[dom] * 1e3, 3),
                "algorithmic_bytes_per_launch": int(abytes),
                "algorithmic_flops_per_launch": aflops,
                "timing": f"{timing_mode}, {count} forwards per cut"}

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        q13h, s13h = oracle.quant_weight_block128(w13_f)
        q2h, s2h = oracle.quant_weight_block128(w2_f)
        del w13_f, w2_f
        batch = max(1, min(M, 64))
        done, t_cpu, first = 0, 0.0, 0
        while t_cpu < args.cpu_seconds and done < 1 << 16:
            xb = synth.make_x(cfg, seed, copy=C + 1, M=batch, first_token=first)
            lb = synth.make_logits(cfg, seed, copy=C + 1, M=batch, first_token=first)
            t1 = time.perf_counter()
            oracle.moe_forward(xb, lb, q13h, s13h, q2h, s2h, k)
            t_cpu += time.perf_counter() - t1
            done += batch
            first += batch
        cpu = {"value": round(done / t_cpu, 3), "unit": "tokens/s", "cores": oracle.get_threads(),
               "kind": "oracle",
               "sample": f"{done} tokens of {cfg.name} in batches of {batch}, {t_cpu:.1f} s wall"}

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "h": h, "i": i, "E": E, "k": k,
                   "rotation_copies": C, "distinct_experts_mean": U_mean,
                   "layer_bytes_per_step": int(U_mean * (w13b + w2b) + M * h * 4 + M * E * 4),
                   "timing": "HIP graph of C forwards, events around K steps",
                   "stage_us": {n: round(v * 1e3, 3) for n, v in zip(names, stage_ms)},
                   "setup_s": round(setup_s, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
