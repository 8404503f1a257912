"""Benchmark of the FP8 MoE expert forward on one MI355X.

One step = one moe_forward (planner, L1 GEMM + SwiGLU/requant epilogue, L2
GEMM, combine) over one batch of seeded synthetic inputs already resident
in HBM.  Prints ONE JSON line.  The headline workload is the largest
single-GPU configuration, the DeepSeek "Pro"-shaped prefill layer: T=8192
tokens, hidden 7168, intermediate 3072, 384 experts all resident (25 GB of
e4m3 weights), top-6, uniform routing.  The same line carries one entry per
further workload ("workloads": flash_decode, flash_prefill, skewed), each
with its own timing, rooflines and CPU-oracle baseline, and the pages'
8xH100 EP8 per-layer figures as context ("pages_context"; another machine
and a multi-GPU layer with communication, so vs_baseline stays null).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--tokens T]
                  [--extra-workloads a,b,c | --no-extra] [--no-cpu-baseline]
                  [--flush MIB] [--no-peaks] [--launch auto|single|split]
                  [--weights packed|row_major] [--recipe fp8|mxfp4]

Beside the timed steps it measures, unless told not to, (a) the same call
with caches flushed before each call (3 observations of K calls; median of
the per-observation medians and the range), and (b) the ceilings this GPU
sustains: a streaming HBM read and a dense FP8 MFMA loop (libmoe_peaks.so),
best of a small sweep of launch shapes; the roofline is then stated against
both the published and the measured peak.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, published


def algorithmic_bytes(cfg, idx, mx=False):
    """Bytes each kernel must move at least once (weights of active experts
    read once, activations read/written once).  Returns dict per kernel.
    mx: the FP8 x MXFP4 recipe (e2m1 weights, one UE8M0 byte per 32 values
    of x, the weights and h)."""
    import torch
    E, H, I, K, T = cfg.E, cfg.H, cfg.I, cfg.K, cfg.T
    valid = (idx >= 0) & (idx < E)
    rows = int(valid.sum())
    active = int(torch.unique(idx[valid]).numel())
    if mx:
        w1 = active * (2 * I * H // 2 + 2 * I * H // 32)
        w2 = active * (H * I // 2 + H * I // 32)
        x = T * H + T * H // 32
        h = rows * I + rows * I // 32
    else:
        w1 = active * (2 * I * H + 4 * (2 * I // 128) * (H // 128))
        w2 = active * (H * I + 4 * (H // 128) * (I // 128))
        x = T * H + 4 * T * (H // 128)
        h = rows * I + 4 * rows * (I // 128)
    topk = 8 * T * K
    part = 2 * rows * H
    y = 2 * T * H
    return {
        "route": 4 * T * K * 2,
        "l1": w1 + x + topk + h,
        "l2": w2 + h + part,
        "combine": part + y + 4 * T * K,
        "rows": rows,
        "active_experts": active,
    }


def kernel_source_digest(paths):
    """Digest of the code in the given sources: comments and whitespace are
    dropped first, so a changed comment leaves the measured counters valid
    and any changed code does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in paths:
        text = open(os.path.join(ROOT, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()[:16]


def measured_traffic(cfg, weights, recipe, dom):
    """HBM bytes per launch of the dominant step from the committed rocprofv3
    counter summary profiles/<workload>_<step>_traffic.json (FETCH_SIZE /
    WRITE_SIZE scaled by a plain copy's readings), or None when no summary
    matches this workload, layout and recipe, or the kernel sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{cfg.name}_{dom}_traffic.json")
    if weights != "packed" or recipe != "fp8" or not os.path.exists(path):
        return None
    d = json.load(open(path))
    if kernel_source_digest(d["source_files"]) != d["source_code_digest"]:
        return None
    return d["step_traffic_bytes"]


def _counter_means(d, counter):
    """Mean value per kernel name of one counter over the dispatches in the
    rocprofv3 CSV output under directory d."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def write_traffic_summary(args):
    """profiles/<workload>_<step>_traffic.json from counter runs: per kernel
    of the step the mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch), scaled by
    what the same counters read for a plain 1 GiB device copy (bytes per
    KiB of counter), summed over the step's kernels."""
    fetch_dir, write_dir, cf_dir, cw_dir = args.traffic_summary
    match = [m for m in args.kernel_match.split(",") if m]
    cal_bytes = 1 << 30

    def copy_kib(d, counter):
        v = {k: x for k, x in _counter_means(d, counter).items() if "moe::" not in k}
        return max(v.values())  # the 1 GiB copy is the largest non-library dispatch

    ff = cal_bytes / (copy_kib(cf_dir, "FETCH_SIZE") * 1024)
    wf = cal_bytes / (copy_kib(cw_dir, "WRITE_SIZE") * 1024)
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    kernels = {k: {"fetch_size_kib": fetch[k], "write_size_kib": write.get(k, 0.0)}
               for k in fetch if any(m in k for m in match)}
    if not kernels:
        raise SystemExit(f"no kernel matching {match} in {fetch_dir}")
    total = sum((v["fetch_size_kib"] * ff + v["write_size_kib"] * wf) * 1024
                for v in kernels.values())
    sources = [x for x in args.sources.split(",") if x]
    out = {
        "what": f"HBM traffic per launch of the {args.workload} {args.step.upper()} step, "
                f"{args.weights} weights, {args.recipe}",
        "command_fetch": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE "
                         "--kernel-include-regex \"moe::\" --output-format csv -d OUT -o out -- "
                         "python3 $GRAFT_REPO_ROOT/bench.py "
                         f"--workload {args.workload} --steps 2 --warmup 1 --no-extra "
                         "--no-cpu-baseline --no-peaks --flush 0",
        "command_write": "the same with --pmc WRITE_SIZE",
        "command_calibration": "the same counters without the kernel filter over: python3 "
                               "$GRAFT_REPO_ROOT/bench.py --copy-calibration 1024",
        "command_summary": "python3 bench.py --traffic-summary FETCH_OUT WRITE_OUT COPY_FETCH_OUT "
                           f"COPY_WRITE_OUT --workload {args.workload} --step {args.step} "
                           f"--kernel-match '{args.kernel_match}' --sources {args.sources}",
        "copy_calibration": {"bytes_per_dispatch": cal_bytes, "fetch_factor": ff,
                             "write_factor": wf},
        "kernels": kernels,
        "source_files": sources,
        "source_code_digest": kernel_source_digest(sources),
        "step_traffic_bytes": total,
    }
    path = os.path.join(ROOT, "profiles", f"{args.workload}_{args.step}_traffic.json")
    json.dump(out, open(path, "w"), indent=1)
    print(json.dumps({"written": path, "step_traffic_bytes": total}), flush=True)


def time_oracle_sample(inp, cfg, n_tokens, seed, mx=False, threads=None):
    """CPU oracle on a bounded sample of tokens; returns (us per layer
    extrapolated to T tokens, threads, seconds, sample description).
    threads: worker threads (default: every core this process may run on)."""
    import numpy as np

    import oracle
    rng = np.random.default_rng(seed)
    toks = sorted(rng.choice(cfg.T, min(n_tokens, cfg.T), replace=False).tolist())
    idx = inp["topk_idx"].cpu().numpy()
    need = sorted({int(e) for e in idx[toks].reshape(-1) if 0 <= e < cfg.E})
    sel = lambda t: [t[e].cpu().numpy() if e in need else None for e in range(cfg.E)]
    args = (inp["x"].cpu().numpy(), inp["x_sf"].cpu().numpy(), idx, inp["topk_w"].cpu().numpy(),
            sel(inp["w1"]), sel(inp["w1_sf"]), sel(inp["w2"]), sel(inp["w2_sf"]))
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    (oracle.moe_forward_mx if mx else oracle.moe_forward)(*args, tokens=toks, nthreads=threads)
    dt = time.perf_counter() - t0
    per_layer_us = dt * 1e6 * cfg.T / len(toks)
    return per_layer_us, threads, dt, f"{len(toks)} of {cfg.T} tokens ({len(toks) * cfg.K} slots), extrapolated linearly in tokens"


def measure_peaks(torch, dev, stream, read_gib=4, reps=3):
    """Best streaming-read GB/s and FP8 MFMA TFLOP/s over a small sweep."""
    from fp8_grouped_gemm_amd import peaks
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def best_ms(launch):
        launch()
        ts = []
        for _ in range(reps):
            e0.record(stream)
            launch()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    nbytes = read_gib << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty(4 * 16 * cus, dtype=torch.int32, device=dev)
    read = {"gbs": 0.0}
    for mode in (peaks.MOE_PEAK_READ_PLAIN, peaks.MOE_PEAK_READ_NONTEMPORAL):
        for unroll in (4, 8):
            for per_cu in (2, 4, 8, 16):
                ms = best_ms(lambda: peaks.stream_read(buf, per_cu * cus, out, unroll=unroll,
                                                       mode=mode, stream=stream))
                gbs = nbytes / (ms * 1e-3) / 1e9
                if gbs > read["gbs"]:
                    read = {"gbs": gbs, "workgroups_per_cu": per_cu, "unroll": unroll,
                            "nontemporal": bool(mode)}
    del buf, out
    mf = {"tflops": 0.0}
    iters = 2048
    fout = torch.empty(256 * 8 * cus, dtype=torch.float32, device=dev)
    for per_cu in (1, 2, 4, 8):
        blocks = per_cu * cus
        ms = best_ms(lambda: peaks.mfma_fp8(blocks, iters, fout, stream=stream))
        tf = peaks.mfma_flop(blocks, iters) / (ms * 1e-3) / 1e12
        if tf > mf["tflops"]:
            mf = {"tflops": tf, "workgroups_per_cu": per_cu}
    del fout
    return {
        "hbm_read_gbs": round(read["gbs"], 1),
        "hbm_read_launch": {k: v for k, v in read.items() if k != "gbs"},
        "hbm_read_bytes": nbytes,
        "mfma_fp8_tflops": round(mf["tflops"], 1),
        "mfma_launch": {"workgroups_per_cu": mf["workgroups_per_cu"], "rounds": iters,
                        "instruction": "v_mfma_f32_16x16x128_f8f6f4, 8 independent per wave"},
        "method": f"best of {reps} timed launches per shape after one untimed; HIP events",
    }


# The pages' own per-layer figures (DeepGEMM PR #440 "Performance": fused
# MegaMoE vs the split #383 path, bench_kineto device time, 8xH100 under
# 8-way expert parallelism, per tokens/rank).  Another machine, and a layer
# that includes NVLink dispatch and combine: context, not a target.
PAGES_CONTEXT = {
    "source": "DeepGEMM PR #440 'Performance' tables: 8xH100 EP8, fused #440 / split #383, "
              "us per layer per rank, includes NVLink dispatch/combine",
    "flash_fused_us": {"64": 351, "128": 353, "256": 388, "512": 423, "2048": 757, "8192": 2556},
    "flash_split_us": {"64": 368, "128": 363, "256": 417, "512": 545, "2048": 1174, "8192": 3702},
    "pro_fused_us": {"64": 1123, "128": 1134, "256": 1182, "512": 1237, "2048": 1978,
                     "8192": 6477},
    "pro_split_us": {"64": 1184, "128": 1173, "256": 1237, "512": 1291, "2048": 2809,
                     "8192": 8601},
}

# Tokens of each workload the CPU oracle computes for its baseline: the
# whole workload where that is under ~15 s on the GPU machine's 16 host threads,
# else a seeded sample of ~10-15 s (pro prefill: 512 tokens took 4.8 s).
CPU_SAMPLE_TOKENS = {"tiny": 64, "flash_decode": 128, "flash_decode_ep8": 128,
                     "flash_prefill": 2048, "skewed": 2048, "pro_prefill": 1536}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="pro_prefill")
    ap.add_argument("--extra-workloads", default="flash_decode,flash_prefill,skewed",
                    help="comma-separated workloads timed after the headline one, each an "
                         "entry of the line's 'workloads' object")
    ap.add_argument("--no-extra", action="store_true", help="time the headline workload only")
    ap.add_argument("--extra-steps", type=int, default=10)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's token count (same shapes and routing recipe)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture one forward in a HIP graph after the warm-up and replay it on "
                         "the timed steps that carry no stage events (the launches a serving "
                         "loop would replay; the same kernels and work)")
    ap.add_argument("--event-every", type=int, default=4, metavar="N",
                    help="record the per-stage HIP events on every N-th timed step (1: all)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens in the oracle sample (0 = the workload's default)")
    ap.add_argument("--cpu-sample-tokens-1t", type=int, default=2,
                    help="tokens in the one-thread oracle sample (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times "
                         "(the reference kernel for scaling HBM byte counters) and exit")
    ap.add_argument("--flush", type=int, default=1024, metavar="MIB",
                    help="also time each step alone after writing a MIB MiB scratch buffer "
                         "(evicts the 256 MB MALL and the L2s), in 3 observations of K "
                         "steps; adds a 'cold' object with the median of the observation "
                         "medians and the range (0 = skip)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the streaming-read and FP8 MFMA ceilings")
    ap.add_argument("--traffic-summary", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="only summarise rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE output "
                         "directories (of this workload, and of --copy-calibration 1024) into "
                         "profiles/<workload>_<step>_traffic.json and exit; needs --step, "
                         "--kernel-match and --sources")
    ap.add_argument("--step", choices=("l1", "l2"), default="l1")
    ap.add_argument("--kernel-match", default="",
                    help="substrings (comma-separated) of the step's kernel names in the CSVs")
    ap.add_argument("--sources", default="",
                    help="comma-separated source files whose code the counters belong to")
    ap.add_argument("--peaks-only", action="store_true",
                    help="only measure the streaming-read and FP8 MFMA ceilings, print them "
                         "as one JSON line and exit")
    ap.add_argument("--launch", choices=("auto", "single", "ring", "split"), default="auto",
                    help="single: L1, L2 and combine in one cooperative launch (direct "
                         "tiles); ring: the same over the lag-ordered ring pool; split: "
                         "one launch per step; auto: the library's choice")
    ap.add_argument("--tile-m", type=int, default=0, choices=(0, 16, 32, 64, 128, 160),
                    help="rows per GEMM tile (0 = the library's choice per call)")
    ap.add_argument("--recipe", choices=("fp8", "mxfp4"), default="fp8",
                    help="fp8: e4m3 x e4m3 with f32 block scales (1x128, 128x128); mxfp4: "
                         "e4m3 activations x e2m1 weights with UE8M0 scales per 32 "
                         "(row-major weights)")
    ap.add_argument("--act-sf-gran", type=int, default=0, choices=(0, 64, 128, -1),
                    help="FP8 recipe: columns per intermediate scale (0/128: per-128, 64: "
                         "per-64 with the dual-half L2, -1: the per-shape rule)")
    ap.add_argument("--weights", choices=("packed", "row_major"), default="packed",
                    help="expert weight layout the plan expects (packed = one-time "
                         "moe_prepare_weights re-layout, done before timing)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this forward keeps all experts resident on "
              "a single MI355X; multi-GPU runs are not part of it.", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp8_grouped_gemm_amd as moe
    import workload as wl

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": n}), flush=True)
        return

    if args.traffic_summary:
        write_traffic_summary(args)
        return

    if args.peaks_only:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        print(json.dumps({"achievable": measure_peaks(torch, dev, torch.cuda.current_stream())}),
              flush=True)
        return

    cfg = wl.CONFIGS[args.workload]
    if args.tokens is not None:
        cfg = wl.custom_config(args.tokens, cfg.H, cfg.I, cfg.E, cfg.K, cfg.skew,
                               name=f"{cfg.name}_T{args.tokens}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seed = args.seed if args.seed is not None else wl.default_seed(wl.CONFIGS[args.workload])
    line = run_workload(args, cfg, seed, args.steps, args.warmup, args.flush, cpu_1t=True)
    if not args.no_peaks:
        print("[bench] measuring the read and MFMA ceilings", file=sys.stderr, flush=True)
        pk = measure_peaks(torch, dev, torch.cuda.current_stream())
        line["achievable"] = pk
        add_achievable(line, pk)
    extras = [] if args.no_extra else [w for w in args.extra_workloads.split(",") if w]
    if extras:
        line["workloads"] = {}
    for name in extras:
        e = run_workload(args, wl.CONFIGS[name], wl.default_seed(wl.CONFIGS[name]),
                         args.extra_steps, max(2, args.warmup // 2), 0, cpu_1t=False)
        if "achievable" in line:
            add_achievable(e, line["achievable"])
        keep = ("value", "unit", "steps", "config", "tflops", "hbm_gbs_algorithmic",
                "pct_hbm_roof", "pct_mfma_roof", "pct_binding_roof", "binding_roof", "roof_us",
                "kernel_us", "algorithmic_bytes", "active_experts", "routed_rows", "roofline",
                "pct_hbm_achievable", "pct_mfma_achievable", "cpu_baseline")
        line["workloads"][name] = {k: e[k] for k in keep if k in e}
    line["pages_context"] = PAGES_CONTEXT
    # (keys starting with "_" are internal: figures add_achievable needs)
    print(json.dumps({k: v for k, v in line.items() if not k.startswith("_")}), flush=True)


def add_achievable(line, pk):
    """Roofline fractions against the measured ceilings as well."""
    rl = line["roofline"]
    rl["achievable_peak"] = pk["hbm_read_gbs"]
    rl["frac_of_achievable"] = round(rl["achieved"] / pk["hbm_read_gbs"], 4)
    us = line["value"]
    line["pct_hbm_achievable"] = round(100 * line["_t_bytes"] / (pk["hbm_read_gbs"] * 1e3) / us, 2)
    line["pct_mfma_achievable"] = round(100 * line["_t_flops"] / (pk["mfma_fp8_tflops"] * 1e6) / us,
                                        2)
    del line["_t_bytes"], line["_t_flops"]


def run_workload(args, cfg, seed, steps, warmup, flush, cpu_1t):
    """Time `steps` forwards of workload cfg (after `warmup`), return its
    JSON object (headline fields, stage times, rooflines, cold-cache times
    when flush > 0, CPU-oracle baseline unless disabled)."""
    import torch

    import fp8_grouped_gemm_amd as moe
    import workload as wl
    dev = torch.device("cuda:0")
    print(f"[bench] drawing {cfg} seed {seed} on the GPU", file=sys.stderr, flush=True)
    mx = args.recipe == "mxfp4"
    if cfg.H % 256:
        args.weights = "row_major"  # the packed layouts need whole 256-row L2 tiles
    inp = (wl.make_inputs_mx if mx else wl.make_inputs)(cfg, seed, dev)
    torch.cuda.synchronize()
    layout = moe.MOE_WEIGHTS_PACKED if args.weights == "packed" else moe.MOE_WEIGHTS_ROW_MAJOR
    flags = {"auto": 0, "single": moe.MOE_FLAG_SINGLE_LAUNCH | moe.MOE_FLAG_DIRECT_TILES,
             "ring": moe.MOE_FLAG_RING_POOL,
             "split": moe.MOE_FLAG_SPLIT_LAUNCH}[args.launch]
    runner = moe.MoEForward(cfg.H, cfg.I, cfg.E, cfg.K, cfg.T, tile_m=args.tile_m, device=dev,
                            weight_layout=layout,
                            recipe=moe.MOE_RECIPE_MXFP4 if mx else moe.MOE_RECIPE_FP8_BLOCK128,
                            flags=flags, act_sf_gran=0 if mx else args.act_sf_gran)
    info = moe.moe_plan_info(runner.plan, cfg.T)
    y = torch.empty(cfg.T, cfg.H, dtype=torch.uint16, device=dev)
    stream = torch.cuda.current_stream()
    prep0 = time.perf_counter()
    if mx:
        w1, w1_sf, w2, w2_sf = runner.prepare_mx(inp["w1"], inp["w1_sf"], inp["w2"],
                                                 inp["w2_sf"], stream)
    else:
        w1, w2 = runner.prepare(inp["w1"], inp["w2"], stream)
        w1_sf, w2_sf = inp["w1_sf"], inp["w2_sf"]
    torch.cuda.synchronize()
    prepare_ms = (time.perf_counter() - prep0) * 1e3
    # (the row-major copies stay for the CPU-oracle baseline, which reads them)
    forward = moe.moe_forward_mx if mx else moe.moe_forward
    forward_timed = moe.moe_forward_mx_timed if mx else moe.moe_forward_timed
    fwd_args = (inp["x"], inp["x_sf"], inp["topk_idx"], inp["topk_w"], w1, w1_sf,
                w2, w2_sf, y, runner.workspace)

    for _ in range(warmup):
        forward(runner.plan, cfg.T, *fwd_args, stream=stream)
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {steps} steps", file=sys.stderr, flush=True)

    # Stage events go on every `--event-every`-th timed step only: each event
    # recorded between two launches costs the step ~3.7 us (measured: 924 vs
    # 943 us per flash-decode layer with events on no step / every step), so
    # the other steps run as a caller would run them.
    every_n = max(1, args.event_every)
    event_steps = [k for k in range(steps) if k % every_n == 0]
    evs = {k: [torch.cuda.Event(enable_timing=True) for _ in range(5)] for k in event_steps}
    # torch creates the HIP event on first record(); do that once so the
    # library can record the same events between its launches.
    for step_evs in evs.values():
        for e in step_evs:
            e.record(stream)
    graph = None
    if getattr(args, "graph", False):
        # one forward captured on the bench stream (the library allocates and
        # copies nothing inside a forward, so it records kernel launches only)
        # (captured on a side stream of default priority: torch does not
        # capture on the default stream)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            forward(runner.plan, cfg.T, *fwd_args, stream=cap)
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for k in range(steps):
        if k in evs:
            forward_timed(runner.plan, cfg.T, *fwd_args, stream, evs[k])
        elif graph is not None:
            with torch.cuda.stream(stream):
                graph.replay()
        else:
            forward(runner.plan, cfg.T, *fwd_args, stream=stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    names = ["route", "l1", "l2", "combine"]
    per = {n: [] for n in names}
    for k in event_steps:
        for i, n in enumerate(names):
            per[n].append(evs[k][i].elapsed_time(evs[k][i + 1]) * 1e3)
    avg = {n: sum(v) / len(v) for n, v in per.items()}
    us_per_layer = total_ms * 1e3 / steps

    alg = algorithmic_bytes(cfg, inp["topk_idx"], mx)
    flops = 2.0 * alg["rows"] * 3 * cfg.H * cfg.I
    bytes_total = alg["route"] + alg["l1"] + alg["l2"] + alg["combine"]
    single = bool(info["single_launch"])
    if single:
        # one cooperative launch runs L1, L2 and the combine: its event span
        # is "l1" and its algorithmic bytes are the three steps'
        dom = "l1"
        dom_bytes = alg["l1"] + alg["l2"] + alg["combine"]
        kernel_name = (f"single launch: L1 + L2 + combine (direct-load tiles, tile_m "
                       f"{info['tile_m']}" +
                       (f"; h in a ring of {info['ring_blocks']} row blocks, L2 "
                        f"{info['l2_lag_units']} units behind L1)" if info["ring_blocks"]
                        else ")"))
    else:
        dom = max(("l1", "l2"), key=lambda n: avg[n])
        dom_bytes = alg[dom]
        kernel_name = (("MXFP4 " if mx else "") + ("L1 step: GEMM gate+up, SwiGLU x topk_w, e4m3 requant "
                        f"({('direct-load', 'LDS-staged', 'shared-A', 'LDS-staged')[info['kernel']]} tiles, "
                        f"tile_m {info['tile_m']})") if dom == "l1" else
                       ("MXFP4 " if mx else "") + f"L2 step: GEMM down (tile_m {info['tile_m']})")
    achieved = dom_bytes / (avg[dom] * 1e-6) / 1e9
    t_hbm = bytes_total / (HBM_PEAK_GBS * 1e9) * 1e6
    t_mfma = flops / (FP8_PEAK_TFLOPS * 1e12) * 1e6

    line = {
        "metric": "us per MoE layer forward (1 GPU), with FP8 TFLOP/s and HBM GB/s as % of roofline",
        "value": round(us_per_layer, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(total_ms / steps, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e4m3 x e2m1 (UE8M0 per 32) -> f32 accumulate, bf16 out" if mx else
                  "e4m3 x e4m3 -> f32 accumulate, bf16 out"),
        "data": ("synthetic (seeded N(0,1) activations, N(0,1/sqrt(fan_in)) weights, "
                 + ("MX-quantised: e4m3 / e2m1 with UE8M0 scales per 32)" if mx else
                    "e4m3 block-quantised)")),
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H,
                   "intermediate": cfg.I, "experts": cfg.E, "top_k": cfg.K,
                   "routing": "zipf-skewed" if cfg.skew else "uniform", "seed": seed,
                   "recipe": args.recipe, "weights": args.weights, "tile": info},
        "prepare_weights_ms_once": round(prepare_ms, 2) if layout else 0.0,
        "tflops": round(flops / (us_per_layer * 1e-6) / 1e12, 2),
        "hbm_gbs_algorithmic": round(bytes_total / (us_per_layer * 1e-6) / 1e9, 1),
        "pct_hbm_roof": round(100 * t_hbm / us_per_layer, 2),
        "pct_mfma_roof": round(100 * t_mfma / us_per_layer, 2),
        "pct_binding_roof": round(100 * max(t_hbm, t_mfma) / us_per_layer, 2),
        "binding_roof": "hbm" if t_hbm >= t_mfma else "mfma",
        "roof_us": {"hbm": round(t_hbm, 1), "mfma": round(t_mfma, 1)},
        "kernel_us": {n: round(v, 2) for n, v in avg.items()},
        "event_steps": len(event_steps),
        "algorithmic_bytes": {n: alg[n] for n in names},
        "active_experts": alg["active_experts"],
        "routed_rows": alg["rows"],
        "wall_s_timed": round(wall, 3),
        "graph_replay": graph is not None,
        "roofline": {
            "kernel": kernel_name,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (None if single else
                        measured_traffic(cfg, args.weights, args.recipe, dom)),
            "algorithmic_bytes": dom_bytes,
        },
        "cpu_baseline": None,
    }
    if flush:
        print("[bench] cold-cache observations", file=sys.stderr, flush=True)
        scratch = torch.empty(flush << 20, dtype=torch.uint8, device=dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        medians, every = [], []
        for _ in range(3):
            obs = []
            for _ in range(steps):
                scratch.fill_(1)
                e0.record(stream)
                forward(runner.plan, cfg.T, *fwd_args, stream=stream)
                e1.record(stream)
                e1.synchronize()
                obs.append(e0.elapsed_time(e1) * 1e3)
            obs.sort()
            medians.append(obs[len(obs) // 2])
            every += obs
        medians.sort()
        line["cold"] = {"flush_mib": flush, "median_us": round(medians[1], 2),
                        "observation_medians_us": [round(m, 2) for m in medians],
                        "min_us": round(min(every), 2), "max_us": round(max(every), 2),
                        "steps_per_observation": steps}
        del scratch
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        n_cpu = args.cpu_sample_tokens or CPU_SAMPLE_TOKENS.get(cfg.name, 64)
        us, threads, secs, sample = time_oracle_sample(inp, cfg, n_cpu, seed, mx)
        line["cpu_baseline"] = {"value": round(us, 1), "unit": "us", "cores": threads,
                                "kind": "oracle", "sample": sample,
                                "seconds": round(secs, 2)}
        if cpu_1t and args.cpu_sample_tokens_1t > 0:  # one thread, smaller sample
            us1, _, secs1, sample1 = time_oracle_sample(inp, cfg, args.cpu_sample_tokens_1t,
                                                        seed, mx, threads=1)
            line["cpu_baseline"]["one_thread"] = {"value": round(us1, 1), "unit": "us",
                                                  "sample": sample1, "seconds": round(secs1, 2)}
    line["_t_bytes"] = bytes_total
    line["_t_flops"] = flops
    del inp, runner, w1, w2, w1_sf, w2_sf, fwd_args, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return line


if __name__ == "__main__":
    main()
