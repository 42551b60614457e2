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
sides.  Each stage's mean duration comes from the GPU's own stamps of its
dispatches: the library's timed entry launches the stage's kernels with HIP
start / stop events (hipExtLaunchKernel) in eager forwards on the launch
stream, queued behind a GPU spin; the dominant stage is reported against its
roofline.  The differences of graph replays of the forwards cut after their
first j stages are recorded beside them (stage_us_cut_graphs).  The CPU
baseline is the oracle (plain C, all host threads) on a bounded sample of the
same workload.
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
    ap.add_argument("--cpu-seconds", type=float, default=9.0,
                    help="CPU time of the headline shape's oracle baseline (three runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cpu-configs", action="store_true", help="CPU baseline of the headline shape only")
    ap.add_argument("--no-other-configs", action="store_true", help="skip the records of the other layer shapes")
    ap.add_argument("--no-floors", action="store_true", help="skip the empty-launch and streaming-read frames")
    ap.add_argument("--other-steps", type=int, default=200,
                    help="timed forwards of each other layer shape (rounded up to whole rotations)")
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
    ap.add_argument("--tiled-paths", action="store_true",
                    help="time the five-launch tiled path and the producer with its reducer on the same inputs "
                         "(default shape: the 768-row verify batch)")
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
KERNEL_SOURCES["prefill_gate_up_mx_kernel"] = KERNEL_SOURCES["prefill_gate_up_kernel"]
KERNEL_SOURCES["prefill_producer_kernel"] = KERNEL_SOURCES["prefill_gate_up_kernel"] + [
    "fp8_block_scaled_router_amd/csrc/route_quant.h", "fp8_block_scaled_router_amd/csrc/group.h",
    "fp8_block_scaled_router_amd/csrc/fused_decode.h"]
KERNEL_SOURCES["prefill_producer_mx_kernel"] = KERNEL_SOURCES["prefill_producer_kernel"]
KERNEL_SOURCES["prefill_down_mx_kernel"] = KERNEL_SOURCES["prefill_gate_up_kernel"]


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
    # name_prefix ends in "(": also take template instances ("name<8, 1>(...)")
    # and names that carry a "void " return type
    stem = name_prefix[:-1] if name_prefix.endswith("(") else None
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            n = r["Kernel_Name"]
            n = n[5:] if n.startswith("void ") else n
            if n.startswith(name_prefix) or (stem is not None and n.startswith(stem + "<")):
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


def stage_work(cfg, stage, U, wbytes=None):
    """Algorithmic bytes (HBM-bound stages) and FLOPs of one launch of a stage;
    wbytes = (w13, w2) bytes per expert of another weight format."""
    M, h, i, k = cfg.M, cfg.h, cfg.i, cfg.k
    w13, w2 = weight_bytes_per_expert(cfg) if wbytes is None else wbytes
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
    if stage.startswith("prefill_producer"):
        # the layer's inputs and the weights once; ids, weights and the bf16
        # partials out (the activation codes and the requantised intermediate
        # stay on chip or in the caches between its phases)
        return M * h * 2 + M * cfg.E * 4 + U * (w13 + w2) + M * k * (8 + h * 2), 6.0 * M * k * h * i
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
    names = moe.moe_mxfp4_stage_names(M, h, i, E, k)
    T = [0.0]
    for j in range(1, len(names) + 1):
        tj, _, _ = time_single_kernel(lambda c, j=j: fwd(c, j), C, args)
        T.append(tj)
    cut_ms = np.maximum(np.diff(np.array(T)), 0.0)
    # stage durations from the GPU's stamps of each stage's dispatches
    nst = len(names)
    nf = max(max(1, args.timing_replays) * C, 64)   # after one unmeasured rotation
    evs = [moe.HipEvents(2 * nst) for _ in range(C + nf)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)
        for f, ev in enumerate(evs):
            c = f % C
            a = W[c]
            moe.moe_mxfp4_forward_ws_timed(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], ev, out=OUT[c])
    torch.cuda.synchronize()
    stage_ms = np.array([[ev.elapsed_ms(2 * j, 2 * j + 1) for j in range(nst)] for ev in evs[C:]]).mean(axis=0)
    for ev in evs:
        ev.close()
    dom = int(np.argmax(stage_ms))
    Um = float(np.mean(U))
    # The FP4 x FP8 form of the block-scaled MFMA issues at the FP8 rate (32
    # clocks per 16x16x128 on one SIMD, measured), so the tiled kernels are
    # priced against the dense FP8 peak; the streaming kernels against HBM.
    abytes, aflops = stage_work(cfg, names[dom], Um, (w13b, w2b))
    bound = "mfma" if names[dom].startswith("prefill_") else "hbm"
    achieved, peak, unit, frac = frac_of(bound, abytes, aflops, stage_ms[dom] / 1e3)
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
                   "stage_us_cut_graphs": {n: round(float(t) * 1e3, 3) for n, t in zip(names, cut_ms)},
                   "timing": "HIP graph of C forwards; stages from the GPU's stamps of their dispatches "
                             f"(hipExtLaunchKernel events, mean of {nf} eager forwards)"},
        "roofline": {"bound": bound, "kernel": names[dom], "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(frac, 4),
                     "traffic": load_traffic(names[dom], workload),
                     "avg_launch_us": round(stage_ms[dom] * 1e3, 3), "algorithmic_bytes_per_launch": int(abytes),
                     "algorithmic_flops_per_launch": aflops,
                     "forward_hbm_frac": round(fw_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "forward_mfma_frac": round(6.0 * M * k * h * i / (ms / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def tiled_paths_bench(args):
    """The two forms of the tiled path on one workload: five launches
    (routing and quantisation, grouping, gate/up, down, combine) and the
    producer (routing through the down partials in one launch) with its route
    reducer.  Both forced on the same inputs (moe_fp8_forward_ws_path), HIP
    graphs of the rotation copies' forwards, events around the replays; the
    two give the same bits (checked here on the first copy)."""
    import numpy as np
    import torch

    import fp8_block_scaled_router_amd as moe
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    moe.lib()
    dev = torch.device("cuda:0")
    ci = args.config if args.config_given else 5
    cfg = synth.CONFIGS[ci]
    seed = synth.default_seed(ci) if args.seed is None else args.seed
    M, h, i, E, k = cfg.M, cfg.h, cfg.i, cfg.E, cfg.k
    C = rotation_copies(cfg, min(E, M * k), args)
    W, X, Lg = [], [], []
    for c in range(C):
        W.append(make_device_weights(moe, cfg, seed, dev, c))
        X.append(torch.from_numpy(synth.make_x(cfg, seed, copy=c).view(np.int16)).view(torch.bfloat16).to(dev))
        Lg.append(torch.from_numpy(synth.make_logits(cfg, seed, copy=c)).to(dev))
    OUT = [torch.empty((M, h), dtype=torch.bfloat16, device=dev) for _ in range(C)]
    res, first = {}, {}
    for path in (moe.PATH_PREFILL, moe.PATH_PRODUCER):
        WS = [moe.alloc_workspace(M, h, i, E, k, device=dev, path=path) for _ in range(C)]

        def fwd(c, path=path, WS=WS):
            a = W[c]
            moe.moe_fp8_forward_ws_path(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], path, out=OUT[c])

        for c in range(C):
            fwd(c)
        torch.cuda.synchronize()
        first[path] = OUT[0].clone()
        ms, reps, _ = time_single_kernel(fwd, C, args)
        errs = [moe.workspace_error(w) for w in WS]
        if any(errs):
            print("bench.py: a wait of the producer timed out", file=sys.stderr)
            sys.exit(3)
        res[path] = (ms, reps * C)
        del WS
        torch.cuda.empty_cache()
    same = bool(torch.equal(first[moe.PATH_PREFILL].view(torch.int16), first[moe.PATH_PRODUCER].view(torch.int16)))
    five, prod = res[moe.PATH_PREFILL][0], res[moe.PATH_PRODUCER][0]
    line = {
        "metric": "MoE-layer tokens/s, producer + route reducer (two launches)",
        "value": round(M / (prod / 1e3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": res[moe.PATH_PRODUCER][1], "warmup": None, "ms_per_step": round(prod, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "h": h, "i": i, "E": E, "k": k, "rotation_copies": C,
                   "five_launch_us_per_forward": round(five * 1e3, 3),
                   "producer_us_per_forward": round(prod * 1e3, 3),
                   "producer_vs_five_launch": round(five / prod, 4), "same_bits": same,
                   "timing": "HIP graph of the rotation copies' forwards on each path, events around the replays"},
        "roofline": None, "cpu_baseline": None,
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


def forward_work(cfg, U_mean):
    """Algorithmic bytes (selected experts' weights and scales, x, logits,
    out) and FLOPs of one whole forward."""
    M, h, i, E, k = cfg.M, cfg.h, cfg.i, cfg.E, cfg.k
    return U_mean * sum(weight_bytes_per_expert(cfg)) + M * h * 4 + M * E * 4, 6.0 * M * k * h * i


def forward_bound(cfg, fw_bytes, fw_flops):
    return "hbm" if fw_bytes / (HBM_PEAK_GBS * 1e9) >= fw_flops / (FP8_PEAK_TFLOPS * 1e12) else "mfma"


def frac_of(bound, nbytes, flops, seconds):
    """(achieved, peak, unit, frac) of a piece of work done in `seconds`."""
    if bound == "hbm":
        a = nbytes / seconds / 1e9
        return a, HBM_PEAK_GBS, "GB/s", a / HBM_PEAK_GBS
    a = flops / seconds / 1e12
    return a, FP8_PEAK_TFLOPS, "TFLOP/s", a / FP8_PEAK_TFLOPS


def make_device_weights(moe, cfg, seed, dev, copy):
    """Expert weights drawn on the GPU (N(0, 1/sqrt(K)), torch's seeded
    generator) and block-quantised by the library: the timing runs of the
    other shapes need the distribution, not the oracle's bytes."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed * 1000 + copy)
    q13, s13 = moe.quantize_weight_block128(torch.randn((cfg.E, 2 * cfg.i, cfg.h), generator=g, device=dev)
                                            / math.sqrt(cfg.h))
    q2, s2 = moe.quantize_weight_block128(torch.randn((cfg.E, cfg.h, cfg.i), generator=g, device=dev)
                                          / math.sqrt(cfg.i))
    torch.cuda.synchronize()
    return q13, s13, q2, s2


def rotation_copies(cfg, U0, args):
    w13b, w2b = weight_bytes_per_expert(cfg)
    step_bytes = U0 * (w13b + w2b)
    C = args.copies or max(2, math.ceil(4 * MALL_BYTES / step_bytes) + 1)
    return max(1, min(C, int((48 << 30) // (cfg.E * (w13b + w2b)))))


def time_layer(moe, cfg, W, X, Lg, WS, OUT, steps, warmup, timing_replays):
    """Graph-replay timing of the C rotation copies' forwards: W warm-up and
    exactly `steps` timed forwards between a synchronisation and HIP events
    on both sides; then stage durations two ways: from graphs of the same
    forwards cut after their first j stages (differences), and from the GPU's
    stamps of each stage's dispatches in eager forwards.  Returns (ms per
    forward, stage names, cut-graph stage ms, forwards per measurement,
    stamped stage ms)."""
    import numpy as np
    import torch
    M, h, i, E, k = cfg.M, cfg.h, cfg.i, cfg.E, cfg.k
    C = len(W)

    def fwd(c, n=None):
        a = W[c]
        if n is None:
            moe.moe_fp8_forward_ws(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], out=OUT[c])
        else:
            moe.moe_fp8_forward_ws_prefix(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], n, out=OUT[c])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def capture(n, cut=None):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for c in range(n):
                fwd(c, cut)
        return g

    g_all = capture(C)
    rem = steps % C
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

    run_steps(warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    run_steps(steps)
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / steps

    # Stage j's duration is T(j) - T(j - 1) per forward, T(j) from replays of
    # the forwards cut after their first j stages, queued behind a GPU spin so
    # that short prefixes are timed on the GPU, not at the host's launch rate.
    names = moe.forward_kernel_names(M, h, i, E, k)
    nst = len(names)
    reps = max(1, timing_replays)
    T = [0.0]
    for j in range(1, nst + 1):
        gj = g_all if j == nst else capture(C, j)
        gj.replay()
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)
        e0.record()
        for _ in range(reps):
            gj.replay()
        e1.record()
        torch.cuda.synchronize()
        T.append(e0.elapsed_time(e1) / (reps * C))
        if gj is not g_all:
            del gj
    run_steps(C)   # the full forwards leave every copy's output complete again
    torch.cuda.synchronize()

    # The same stages timed directly: the library's timed entry launches each
    # stage's kernels with HIP events that the GPU stamps at the start of the
    # stage's first dispatch and the end of its last, in eager
    # forwards on the launch stream, queued behind a GPU spin.
    # At least 64 forwards are averaged, after one unmeasured rotation (the
    # first forwards after the spin run at lower clocks).
    nf = max(reps * C, 64)
    evs = [moe.HipEvents(2 * nst) for _ in range(C + nf)]
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)
        for f, ev in enumerate(evs):
            c = f % C
            a = W[c]
            moe.moe_fp8_forward_ws_timed(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], ev, out=OUT[c])
    torch.cuda.synchronize()
    ev_ms = np.array([[ev.elapsed_ms(2 * j, 2 * j + 1) for j in range(nst)] for ev in evs[C:]]).mean(axis=0)
    for ev in evs:
        ev.close()
    return ms_per_step, names, np.maximum(np.diff(np.array(T)), 0.0), nf, ev_ms


def layer_record(cfg, names, stage_ms, U_mean, ms_per_step, count, traffic_workload=None):
    """The roofline of the dominant stage (algorithmic work of one launch over
    its mean duration) and of the whole forward (its algorithmic work over the
    time per forward)."""
    import numpy as np
    fw_bytes, fw_flops = forward_work(cfg, U_mean)
    bound = forward_bound(cfg, fw_bytes, fw_flops)
    dom = int(np.argmax(stage_ms))
    abytes, aflops = stage_work(cfg, names[dom], U_mean)
    achieved, peak, unit, frac = frac_of(bound, abytes, aflops, stage_ms[dom] / 1e3)
    fa, _, _, ff = frac_of(bound, fw_bytes, fw_flops, ms_per_step / 1e3)
    roofline = {"bound": bound, "kernel": names[dom], "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(frac, 4),
                "traffic": load_traffic(names[dom], traffic_workload or cfg.name),
                "avg_launch_us": round(stage_ms[dom] * 1e3, 3),
                "algorithmic_bytes_per_launch": int(abytes),
                "algorithmic_flops_per_launch": aflops,
                "timing": f"start / end of the stage's dispatches as the GPU stamps them (HIP events passed to "
                          f"hipExtLaunchKernel by the library's timed entry), mean of {count} eager forwards on "
                          f"the launch stream"}
    forward = {"bound": bound, "achieved": round(fa, 2), "peak": peak, "unit": unit, "frac": round(ff, 4),
               "algorithmic_bytes": int(fw_bytes), "algorithmic_flops": fw_flops,
               "timing": "HIP graph of the rotation copies' forwards, events around the timed steps"}
    return roofline, forward


def launch_and_read_floors(moe, n_launch, fw_bytes, C, dev):
    """Two frames for a forward's time: (1) a graph of C * n_launch empty
    kernels, per forward (what the launches cost by themselves); (2) one
    streaming-read kernel over fw_bytes, rotated over C buffers (the best
    time one launch reaches on the forward's algorithmic bytes), swept over
    grids of 256..2048 workgroups."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=20):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            fn()
        g.replay()
        torch.cuda.synchronize()
        torch.cuda._sleep(20_000_000)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / reps

    empty_ms = timed(lambda: [moe.probe_empty(256) for _ in range(C * n_launch)]) / C
    nb = (int(fw_bytes) + 15) // 16 * 16
    bufs = [torch.full((nb,), 1, dtype=torch.uint8, device=dev) for _ in range(C)]
    sink = torch.empty(4 * 2048, dtype=torch.int32, device=dev)
    best = None
    for grid in (256, 512, 1024, 2048):
        ms = timed(lambda: [moe.probe_read(b, grid, sink) for b in bufs]) / C
        if best is None or ms < best[0]:
            best = (ms, grid)
    del bufs
    return {"empty_kernels_per_forward": n_launch, "empty_graph_us_per_forward": round(empty_ms * 1e3, 3),
            "read_bytes": nb, "read_us": round(best[0] * 1e3, 3), "read_grid": best[1],
            "read_GBps": round(nb / (best[0] / 1e3) / 1e9, 1),
            "timing": "HIP graphs of C launches per forward, events around 20 replays"}


def other_config_records(moe, args, skip, dev):
    """Per-shape records of every other configured layer shape: tokens/s,
    the dominant stage against its roofline and the whole forward against
    the forward's bound (weights drawn on the GPU; x and logits from the
    shape's own recipe)."""
    import numpy as np
    import torch
    import synth
    out = {}
    for ci, cfg in enumerate(synth.CONFIGS):
        if ci == skip:
            continue
        t0 = time.time()
        seed = synth.default_seed(ci)
        M, h, i, E, k = cfg.M, cfg.h, cfg.i, cfg.E, cfg.k
        ids0, _ = moe.router_topk(torch.from_numpy(synth.make_logits(cfg, seed, copy=0)).to(dev), k)
        C = rotation_copies(cfg, int(torch.unique(ids0).numel()), args)
        W = [make_device_weights(moe, cfg, seed, dev, c) for c in range(C)]
        X, Lg, WS, OUT = [], [], [], []
        for c in range(C):
            X.append(torch.from_numpy(synth.make_x(cfg, seed, copy=c).view(np.int16)).view(torch.bfloat16).to(dev))
            Lg.append(torch.from_numpy(synth.make_logits(cfg, seed, copy=c)).to(dev))
            WS.append(moe.alloc_workspace(M, h, i, E, k, device=dev))
            OUT.append(torch.empty((M, h), dtype=torch.bfloat16, device=dev))
        for c in range(C):
            a = W[c]
            moe.moe_fp8_forward_ws(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], out=OUT[c])
        torch.cuda.synchronize()
        lay = moe.workspace_layout(M, h, i, E, k)
        U = [int(WS[c][lay.num_active:lay.num_active + 4].view(torch.int32).item()) for c in range(C)]
        assert all(torch.isfinite(OUT[c].float()).all().item() for c in range(C))
        steps = C * max(1, math.ceil(args.other_steps / C))
        ms, names, cut_ms, count, stage_ms = time_layer(moe, cfg, W, X, Lg, WS, OUT, steps, C, args.timing_replays)
        errs = [moe.workspace_error(WS[c]) for c in range(C)]
        U_mean = float(np.mean(U))
        roofline, forward = layer_record(cfg, names, stage_ms, U_mean, ms, count)
        out[cfg.name] = {
            "tokens_per_s": round(M / (ms / 1e3), 2), "ms_per_step": round(ms, 6), "steps": steps,
            "path": moe.PATH_NAMES[lay.path],
            "rotation_copies": C, "distinct_experts_mean": U_mean,
            "stage_us": {n: round(v * 1e3, 3) for n, v in zip(names, stage_ms)},
            "stage_us_cut_graphs": {n: round(v * 1e3, 3) for n, v in zip(names, cut_ms)},
            "roofline": roofline, "forward": forward, "sync_errors": int(sum(e != 0 for e in errs)),
            "weights": "GPU-drawn N(0, 1/sqrt(K)), library block quantisation",
            "wall_s": round(time.time() - t0, 1)}
        print(f"bench: {cfg.name} {out[cfg.name]['tokens_per_s']} tok/s, {ms * 1e3:.1f} us/forward",
              file=sys.stderr, flush=True)
        del W, X, Lg, WS, OUT
        torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_rate(oracle, synth, cfg, seed, weights, batch, min_s, runs, threads, max_tokens=1 << 16, reuse=False):
    """Median over `runs` of the oracle's tokens/s on consecutive batches of
    `batch` fresh tokens of the shape (the same first batch again and again
    with `reuse`), at least `min_s` seconds or `max_tokens` tokens per run,
    with `threads` OpenMP threads.  Returns (median tokens/s, tokens per run)."""
    import statistics
    q13h, s13h, q2h, s2h = weights
    oracle.set_threads(threads)
    rates, first, done_total = [], 0, 0
    for _ in range(runs):
        done, t = 0, 0.0
        while t < min_s and done < max_tokens:
            xb = synth.make_x(cfg, seed, copy=97, M=batch, first_token=first)
            lb = synth.make_logits(cfg, seed, copy=97, M=batch, first_token=first)
            t1 = time.perf_counter()
            oracle.moe_forward(xb, lb, q13h, s13h, q2h, s2h, cfg.k)
            t += time.perf_counter() - t1
            done += batch
            first += 0 if reuse else batch
        rates.append(done / t)
        done_total = done
    return statistics.median(rates), done_total


def cpu_baselines(cfg_head, seed_head, host_weights, args):
    """The oracle (plain C, OpenMP over rows) on the host cores: the headline
    shape on all threads (median of 3 runs of about args.cpu_seconds / 3 s),
    then every shape on all threads and on one thread (median of 3 runs of
    about 1 s; the prefill shape once, on 512 tokens)."""
    import numpy as np
    import oracle
    import synth
    nthreads = os.cpu_count() or 1
    oracle.set_threads(nthreads)
    used = oracle.get_threads()
    batch = max(1, min(cfg_head.M, 64))
    head, n = cpu_rate(oracle, synth, cfg_head, seed_head, host_weights, batch, args.cpu_seconds / 3, 3, used)
    cpu = {"value": round(head, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"median of 3 runs of {n} tokens of {cfg_head.name} in batches of {batch}",
           "cpu_model": cpu_model()}
    if args.no_cpu_configs:
        return cpu
    per = {}
    for ci, cfg in enumerate(synth.CONFIGS):
        seed = synth.default_seed(ci)
        b = max(1, min(cfg.M, 64))
        reuse = False
        if (cfg.h, cfg.i, cfg.E) == (cfg_head.h, cfg_head.i, cfg_head.E):
            weights, wnote = host_weights, f"weights of {cfg_head.name} (same sizes)"
        else:
            # one batch of b tokens run again and again; only the experts it
            # selects are drawn (the oracle reads no other expert)
            b = max(1, min(cfg.M, 4 if cfg.h > 4096 else 64))
            reuse = True
            ids, _ = oracle.router(synth.make_logits(cfg, seed, copy=97, M=b), cfg.k)
            experts = sorted(set(int(e) for e in np.unique(ids)))
            w13 = np.zeros((cfg.E, 2 * cfg.i, cfg.h), np.float32)
            w2 = np.zeros((cfg.E, cfg.h, cfg.i), np.float32)
            w13[experts] = synth.make_w13_f32(cfg, seed, experts)
            w2[experts] = synth.make_w2_f32(cfg, seed, experts)
            q13, s13 = oracle.quant_weight_block128(w13)
            q2, s2 = oracle.quant_weight_block128(w2)
            del w13, w2
            weights, wnote = (q13, s13, q2, s2), f"the shape's own weights; one batch of {b} tokens repeated"
        rec = {"weights": wnote}
        if cfg.M >= 4096:
            r, n = cpu_rate(oracle, synth, cfg, seed, weights, 512, 1e-9, 1, used, max_tokens=512)
            rec.update(all_threads=round(r, 3), all_threads_sample=f"1 run of {n} tokens in one batch")
        else:
            r, n = cpu_rate(oracle, synth, cfg, seed, weights, b, 1.0, 3, used, reuse=reuse)
            rec.update(all_threads=round(r, 3), all_threads_sample=f"median of 3 runs of {n} tokens, batches of {b}")
            r1, n1 = cpu_rate(oracle, synth, cfg, seed, weights, b, 1.0, 3, 1, reuse=reuse)
            rec.update(one_thread=round(r1, 3), one_thread_sample=f"median of 3 runs of {n1} tokens, batches of {b}")
        oracle.set_threads(used)
        per[cfg.name] = rec
        print(f"bench: cpu {cfg.name} {rec}", file=sys.stderr, flush=True)
    cpu["per_config"] = per
    return cpu


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
    if args.tiled_paths:
        tiled_paths_bench(args)
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
    C = rotation_copies(cfg, int(torch.unique(ids0).numel()), args)
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

    # eager warm-up of every copy, then distinct experts per copy
    for c in range(C):
        a = W[c]
        moe.moe_fp8_forward_ws(X[c], Lg[c], a[0], a[1], a[2], a[3], k, WS[c], out=OUT[c])
    torch.cuda.synchronize()
    lay = moe.workspace_layout(M, h, i, E, k)
    U = [int(WS[c][lay.num_active:lay.num_active + 4].view(torch.int32).item()) for c in range(C)]
    assert all(torch.isfinite(OUT[c].float()).all().item() for c in range(C))

    ms_per_step, names, cut_ms, count, stage_ms = time_layer(moe, cfg, W, X, Lg, WS, OUT, args.steps,
                                                             args.warmup, args.timing_replays)
    errs = [moe.workspace_error(WS[c]) for c in range(C)]
    if any(errs):
        print(f"bench.py: a wait between workgroups timed out in {sum(e != 0 for e in errs)} workspaces",
              file=sys.stderr)
        sys.exit(3)
    tokens_per_s = M / (ms_per_step / 1e3)
    U_mean = float(np.mean(U))
    roofline, forward = layer_record(cfg, names, stage_ms, U_mean, ms_per_step, count)
    fw_bytes, _ = forward_work(cfg, U_mean)
    floors = None
    if not args.no_floors:
        floors = launch_and_read_floors(moe, len(names), fw_bytes, C, dev)
    del W, X, Lg, WS, OUT
    torch.cuda.empty_cache()

    others = None
    if not args.no_other_configs:
        others = other_config_records(moe, args, args.config, dev)

    # ---- CPU baseline: the oracle on bounded samples of the same workloads
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        q13h, s13h = oracle.quant_weight_block128(w13_f)
        q2h, s2h = oracle.quant_weight_block128(w2_f)
        del w13_f, w2_f
        cpu = cpu_baselines(cfg, seed, (q13h, s13h, q2h, s2h), args)

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
                   "path": moe.PATH_NAMES[lay.path],
                   "rotation_copies": C, "distinct_experts_mean": U_mean,
                   "layer_bytes_per_step": int(fw_bytes),
                   "timing": "HIP graph of C forwards, events around K steps",
                   "stage_us": {n: round(v * 1e3, 3) for n, v in zip(names, stage_ms)},
                   "stage_us_cut_graphs": {n: round(v * 1e3, 3) for n, v in zip(names, cut_ms)},
                   "setup_s": round(setup_s, 1)},
        "roofline": roofline,
        "forward": forward,
        "floors": floors,
        "configs": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
