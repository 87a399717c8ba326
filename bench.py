"""Benchmark of prefix-reuse prefill attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 4] [--no-cpu-baseline]

One step is one bat_attn_prefill call over the whole batch (device work
decomposition + attention with the prefix gathered from the paged cache +
any split merge), inputs and the prefix pool already resident in HBM.  The
prefix build (bat_kv_build) is the once-per-prefix cost that reuse amortises;
it is timed separately and reported beside the step.  Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP64_TFLOPS = 78.6     # MI355X fp64 vector: the fp32 path's scores and sums are fp64 FMAs
PEAK_HBM_GBS = 8000.0
# committed HBM-traffic summaries (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE), one per
# configuration, each with the hash of the kernel source it was measured on
PMC_SUMMARIES = {
    "config2": os.path.join(ROOT, "profiles", "attn_bf16_d64_config2_traffic.json"),
    "config3": os.path.join(ROOT, "profiles", "attn_bf16_d64_config3_traffic.json"),
    "config4": os.path.join(ROOT, "profiles", "attn_bf16_d128_config4_traffic.json"),
    "config5": os.path.join(ROOT, "profiles", "attn_bf16_d128_config5_traffic.json"),
}
PMC_SUMMARY = PMC_SUMMARIES["config4"]


def kernel_source_hash():
    """Hash of the attention kernel's code (comments and blank lines left
    out, so that an edit of a comment keeps a traffic measurement valid)."""
    import re
    h = hashlib.sha256()
    for f in ("attn_bf16.hip", "common.h"):
        with open(os.path.join(ROOT, "prefix_reuse_attention_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines())
        h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()[:16]


def measured_traffic(config, per_launch_units):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or
    None when the kernel source changed since the counters were taken."""
    path = PMC_SUMMARIES.get(config)
    if path is None:
        return None
    try:
        with open(path) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_hash") != kernel_source_hash() or s.get("config") != config:
        return None
    return s.get("hbm_bytes_per_launch")


def _pmc_kib(run_dir, counter, name_part):
    """Mean per-dispatch value (KiB) of one counter over the dispatches of
    kernels whose name contains name_part, from a rocprofv3 --pmc CSV run."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                    per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} values for '{name_part}' under {run_dir}")
    return sum(per.values()) / len(per)


def bf16_kernel_label(wl):
    """The bf16 kernel the library launches for this workload, by the same
    rule as its planner: the eight-wave ping-pong kernel (up to 256 rows per item,
    64-key tiles) when suffixes average more than 128 rows, except at D=64
    over a pool whose blocks are smaller than a 64-key tile (gathered key
    by key, faster on four waves); else the four-wave kernel.  Buffer-load
    copies: the global-load form only serves per-key pools of 2 GiB or
    more, and none of these workloads has one."""
    from prefix_reuse_attention_amd import workloads as W
    has_user = bool((wl.mode == W.USER).any())
    has_item = bool((wl.mode == W.ITEM).any())
    per_key = (has_user and wl.user_block_size < 64) or (has_item and W.ITEM_TOKENS < 64)
    eight = wl.total_s > 128 * wl.B and not (wl.D == 64 and per_key)
    if eight:
        return f"attn_bf16_pp_kernel<{wl.D}, false>"
    return f"attn_bf16_kernel<{wl.D}, 4, false>"


def batch_from_spec(spec):
    """A seeded synthetic batch from a spec of comma-separated key=value
    pairs: B, H, D (bf16), n_p and n_s (an integer, or lo:hi for lengths
    drawn uniformly from [lo, hi]), mode (user, item or mixed: each request
    user or item with probability one half; item prefixes are rounded down
    to whole 4-token items) and seed.  Example: "B=128,H=8,D=128,n_p=8192,
    n_s=257:512".  The lengths come from numpy's default generator with that
    seed, the tensors from the workload generator with it."""
    import numpy as np
    from prefix_reuse_attention_amd import workloads as W
    items = [item for item in spec.split(",") if item]
    if any("=" not in item for item in items):
        raise SystemExit(f"--batch: expected key=value pairs, got {spec!r}")
    kv = dict(item.split("=", 1) for item in items)
    unknown = set(kv) - {"B", "H", "D", "n_p", "n_s", "mode", "seed"}
    if unknown:
        raise SystemExit(f"--batch: unknown keys {sorted(unknown)}")
    B, H, D = int(kv.get("B", 16)), int(kv.get("H", 8)), int(kv.get("D", 128))
    seed = int(kv.get("seed", 11))
    rng = np.random.default_rng(seed)

    def lengths(text):
        if ":" in text:
            lo, hi = (int(x) for x in text.split(":"))
            return rng.integers(lo, hi + 1, B)
        return np.full(B, int(text))
    n_p, n_s = lengths(kv.get("n_p", "8192")), lengths(kv.get("n_s", "512"))
    how = kv.get("mode", "user")
    if how == "user":
        mode = np.full(B, W.USER)
    elif how == "item":
        mode = np.full(B, W.ITEM)
    elif how == "mixed":
        mode = np.where(rng.random(B) < 0.5, W.ITEM, W.USER)
    else:
        raise SystemExit(f"--batch: mode must be user, item or mixed, not {how}")
    n_p = np.where(mode == W.ITEM, W.ITEM_TOKENS * (n_p // W.ITEM_TOKENS), n_p)
    wl = W.make_custom(dtype="bf16", H=H, D=D, n_s=n_s.tolist(), n_p=n_p.tolist(),
                       mode=mode.tolist(), seed=seed, user_block_size=64,
                       name="batch:" + spec)
    wl.notes["description"] = f"synthetic batch {spec}"
    return wl


def write_traffic_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, config):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, of the
    benchmark and of --copy-calibration) into the HBM-traffic summary that
    the roofline record quotes: counter KiB scaled by what the same counter
    reads for a plain copy of known size."""
    n_kib = (1 << 30) / 1024.0
    f_scale = n_kib / _pmc_kib(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    w_scale = n_kib / _pmc_kib(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    f = _pmc_kib(fetch_dir, "FETCH_SIZE", "attn_bf16")
    w = _pmc_kib(write_dir, "WRITE_SIZE", "attn_bf16")
    summary = {"kernel": "attn_bf16", "config": config,
               "kernel_source_hash": kernel_source_hash(),
               "fetch_kib": f, "write_kib": w, "fetch_scale": f_scale, "write_scale": w_scale,
               "hbm_bytes_per_launch": (f * f_scale + w * w_scale) * 1024.0}
    if config not in PMC_SUMMARIES:
        raise SystemExit(f"no traffic summary file is kept for {config}")
    with open(PMC_SUMMARIES[config], "w") as fh:
        json.dump(summary, fh, indent=1)
        fh.write("\n")
    print(json.dumps(summary), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the board runs this kernel at its power cap; its clock settles within
    # about 50 calls (25 ms), so the default warmup covers that
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--workload", choices=("prefill", "isolated", "gqa", "prefix-rows",
                                           "item-local", "schedule", "split", "fp8"),
                    default="prefill",
                    help="prefill: bat_attn_prefill on --config (the default line); "
                         "isolated: bat_attn_prefill_isolated on --config with single-token "
                         "candidates; gqa: bat_attn_prefill_gqa on the 8k-history shape with 4 "
                         "key/value heads for its 16 query heads; prefix-rows: bat_attn_prefix_rows over the 8k-history "
                         "prefixes; item-local: bat_attn_item_local over the 20000-item pool; "
                         "schedule: the prefix-mode choice (bat_sched_*) on Zipf traffic and "
                         "the attention work it implies for a window of queries; split: "
                         "bat_attn_prefill on 2 requests with 32768-token prefixes, which "
                         "the planner splits into chunks merged by log-sum-exp; fp8: "
                         "bat_attn_prefill_fp8 on --config with the prefix pool in fp8 "
                         "(bat_kv_build_fp8)")
    ap.add_argument("--batch", default=None,
                    help="with the default workload: time a synthetic batch given by its sizes "
                         "instead of --config (e.g. B=128,H=8,D=128,n_p=8192,n_s=257:512,"
                         "mode=user); see batch_from_spec")
    ap.add_argument("--host-sweep", action="store_true",
                    help="with --workload schedule: only the host accounting of both policies "
                         "over a grid of traffic shapes (no GPU needed)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (scales the "
                         "HBM byte counters of rocprofv3 --pmc)")
    ap.add_argument("--write-traffic-summary", nargs=4,
                    metavar=("FETCH_RUN", "WRITE_RUN", "COPY_FETCH_RUN", "COPY_WRITE_RUN"),
                    help="write the committed HBM-traffic summary from four rocprofv3 --pmc "
                         "output directories (no GPU needed)")
    args = ap.parse_args()
    if args.write_traffic_summary:
        write_traffic_summary(*args.write_traffic_summary, config=f"config{args.config}")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by request with no exchange; see the design notes)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "repeats": 3}), flush=True)
        return
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd import workloads as W
    from prefix_reuse_attention_amd.device import DeviceWorkload

    api.load()  # the HIP library must be there: no fallback
    if args.workload == "schedule" and args.host_sweep:
        schedule_host_sweep()  # host code only
        return
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.workload == "schedule":
        bench_schedule_workload(args)
        return
    if args.workload in ("prefix-rows", "item-local"):
        bench_prefix_workload(args)
        return
    if args.workload == "fp8":
        bench_fp8_workload(args)
        return
    isolated = args.workload == "isolated"
    gqa_heads = 0
    t0 = time.time()
    if args.workload == "gqa":
        # the 8k-history shape: 16 query heads over 4 key/value heads
        gqa_heads = 16
        wl = W.make_custom(dtype="bf16", H=4, D=128, n_s=[512] * 16, n_p=[8192] * 16,
                           mode=[W.USER] * 16, seed=104, user_block_size=64, name="config4_gqa")
        wl.notes["description"] = ("bf16, B=16, 16 query heads over 4 key/value heads, D=128, "
                                   "user prefix 8192 (64-token pages), suffix 512")
    elif args.workload == "split":
        # too few items to fill the GPU unsplit: prefix chunks + merge launch
        wl = W.make_custom(dtype="bf16", H=16, D=128, n_s=[512] * 2, n_p=[32768] * 2,
                           mode=[W.USER] * 2, seed=105, user_block_size=64, name="split_32k")
        wl.notes["description"] = ("bf16, B=2, H=16, D=128, user prefix 32768 (64-token pages), "
                                   "suffix 512; prefixes split into chunks")
    elif args.batch:
        wl = batch_from_spec(args.batch)
    else:
        wl = W.make_config(args.config)
    print(f"[bench] generated {wl.name} in {time.time() - t0:.1f}s: {wl.notes['description']}",
          file=sys.stderr, flush=True)

    dw = DeviceWorkload(wl, build=False)
    stream = torch.cuda.current_stream()
    # ---- prefix build (amortised over reuse), timed on its own
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dw.upload_prefix()
    dw.alloc_pools()
    dw.build_kv()          # first launch also loads the code object: untimed
    torch.cuda.synchronize()
    reps = 5
    ev0.record(stream)
    for _ in range(reps):  # rebuilding the same pool is idempotent
        dw.build_kv()
    ev1.record(stream)
    torch.cuda.synchronize()
    build_ms = ev0.elapsed_time(ev1) / reps
    build_bytes = dw.prefix_bytes()
    dw.drop_prefix_source()
    ws = dw.workspace()
    out = torch.empty_like(dw.q)
    lse = torch.empty((wl.H, wl.total_s), dtype=torch.float32, device="cuda")
    if gqa_heads:
        from prefix_reuse_attention_amd.device import to_device
        q_big = to_device(W._normal(np.random.default_rng(105), (wl.total_s, gqa_heads, wl.D),
                                    "bf16"), "bf16")
        out = torch.empty_like(q_big)
        lse = torch.empty((gqa_heads, wl.total_s), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, api.load().bat_attn_gqa_workspace_size(
            wl.B, gqa_heads, wl.H, wl.D, api.BAT_BF16, wl.total_s, dw.max_s, dw.max_p)),
            dtype=torch.uint8, device="cuda")

    if isolated:
        # single-token candidates: each suffix row sees the prefix and itself
        ws = torch.empty(max(1, api.load().bat_attn_isolated_workspace_size(
            wl.B, wl.H, wl.D, api.BAT_BF16 if wl.dtype == "bf16" else api.BAT_F32, wl.total_s,
            dw.max_s, dw.max_p)), dtype=torch.uint8, device="cuda")

        def step():
            api.attn_prefill_isolated(dw.q, dw.k, dw.v, dw.cu_s, dw.prefix_lens, dw.prefix_mode,
                                      dw.block_table, 1, dw.user_pool, dw.item_pool, wl.scale,
                                      dw.max_s, dw.max_p, out=out, lse=lse, workspace=ws)
    elif gqa_heads:
        def step():
            api.attn_prefill_gqa(q_big, dw.k, dw.v, dw.cu_s, dw.prefix_lens, dw.prefix_mode,
                                 dw.block_table, dw.user_pool, dw.item_pool, wl.scale, dw.max_s,
                                 dw.max_p, out=out, lse=lse, workspace=ws)
    else:
        step = dw.prepared(out, lse, ws)  # arguments marshalled once

    ms_per_step, kernel_ms = _timed_steps(step, args.steps, args.warmup, stream)
    per_call = _per_call_ms(step, args.steps, stream)
    flops = wl.flops()
    alg_bytes = wl.alg_bytes()
    if gqa_heads:  # the work of the query heads
        flops = flops * gqa_heads / wl.H
    if isolated:  # each suffix row: its prefix plus one key
        flops = float(4.0 * wl.D * wl.H * np.sum(wl.n_s.astype(np.float64) * (wl.n_p + 1)))
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    tok_s = wl.total_s / (ms_per_step * 1e-3)
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    bf16 = wl.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP64_TFLOPS
    traffic = None if (isolated or gqa_heads) else measured_traffic(wl.name, 1)
    props = torch.cuda.get_device_properties(0)
    print(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step by wall clock, "
          f"{kernel_ms:.4f} by events on the stream; {tflops:.1f} TFLOP/s",
          file=sys.stderr, flush=True)

    base = None
    if not args.no_cpu_baseline and not isolated and not gqa_heads and args.workload != "split":
        base = run_cpu_baseline(wl, args.cpu_seconds)

    line = {
        "metric": ("candidate-isolated prefill TFLOP/s, 1 GPU" if isolated else
                   "grouped-head prefill TFLOP/s, 1 GPU" if gqa_heads else
                   "prefill attention TFLOP/s (% bf16 MFMA peak) + suffix tokens/s, 1 GPU"),
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1) activations, shuffled paged prefix pool)",
        "config": {"workload": f"{wl.name}: {wl.notes['description']}"
                               + ("; single-token candidates, each isolated" if isolated else ""),
                   "B": wl.B, "H": gqa_heads or wl.H,
                   **({"H_kv": wl.H} if gqa_heads else {}),
                   "D": wl.D, "total_suffix": wl.total_s, "total_prefix": int(wl.n_p.sum()),
                   "user_block_size": wl.user_block_size, "seed": wl.seed},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2) if bf16 else None,
        "suffix_tokens_per_s": round(tok_s, 1),
        "alg_flops_per_step": flops,
        "alg_bytes_per_step": alg_bytes,
        "prefix_unique": unique_prefix(wl),
        "roofline": {"bound": "mfma" if bf16 else "alu", "achieved": round(achieved, 3),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel": (bf16_kernel_label(wl) if bf16 else f"attn_f32_kernel<{wl.D}>")
                               + ((" (own key folded in)" if bf16
                                   else " + item_local_kernel (merge)") if isolated else ""),
                     "kernel_ms_mean": round(kernel_ms, 5)},
        "per_call_ms": per_call,
        "kv_build": {"ms": round(build_ms, 4), "bytes_copied": build_bytes,
                     "GB_per_s_read_plus_write": round(2 * build_bytes / (build_ms * 1e-3) / 1e9, 1),
                     "note": "once per prefix; amortised over every query that reuses it"},
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)


def bench_fp8_workload(args):
    """bat_attn_prefill_fp8 on --config (default config 4) with the prefix
    pool held in fp8 (E4M3 codes, a power-of-two scale per block and head):
    the pool's bytes against a bfloat16 pool, the quantising build
    (bat_kv_build_fp8, once per prefix), and the prefill's TFLOP/s."""
    import numpy as np
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd import workloads as W
    from prefix_reuse_attention_amd.device import DeviceWorkload
    wl = W.make_config(args.config)
    dw = DeviceWorkload(wl, build=False)
    stream = torch.cuda.current_stream()
    dw.build_pools_fp8()                  # first launch loads the code object: untimed
    dw.upload_prefix()
    src = dw._src
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    ev0.record(stream)
    for _ in range(reps):                 # rebuilding the same pool is idempotent
        for name, pool in (("user", dw.user_pool8), ("item", dw.item_pool8)):
            if name in src:
                api.kv_build_fp8(*src[name], pool)
    ev1.record(stream)
    torch.cuda.synchronize()
    build_ms = ev0.elapsed_time(ev1) / reps
    src_bytes = dw.prefix_bytes()
    dw.drop_prefix_source()
    pools = [p for p in (dw.user_pool8, dw.item_pool8) if p is not None]
    fp8_bytes = sum(p.k.numel() + p.v.numel() + 4 * (p.k_scale.numel() + p.v_scale.numel())
                    for p in pools)
    bf16_bytes = sum(2 * (p.k.numel() + p.v.numel()) for p in pools)
    out = torch.empty_like(dw.q)
    lse = torch.empty((wl.H, wl.total_s), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, api.fp8_workspace_size(wl.B, wl.H, wl.D, wl.total_s, dw.max_s,
                                                   dw.max_p)), dtype=torch.uint8, device="cuda")
    step = lambda: dw.run_fp8(out=out, lse=lse, workspace=ws)
    wall_ms, kernel_ms = _timed_steps(step, args.steps, args.warmup, stream)
    flops = wl.flops()
    tflops = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    print(f"[bench] fp8 {wl.name}: {wall_ms:.4f} ms/step (events {kernel_ms:.4f}); "
          f"{tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)
    line = {"workload": "fp8", "metric": "prefill attention TFLOP/s over an fp8 prefix pool, 1 GPU",
            "value": round(tflops, 3), "unit": "TFLOP/s", "higher_is_better": True, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
            "dtype": "bf16 (fp8 e4m3 prefix pool)",
            "data": "synthetic (seeded N(0,1) activations, shuffled paged prefix pool)",
            "config": {"workload": f"{wl.name}: {wl.notes['description']}; prefix pool in fp8",
                       "B": wl.B, "H": wl.H, "D": wl.D, "seed": wl.seed},
            "vs_baseline": None, "alg_flops_per_step": flops,
            "pool_bytes": {"fp8_codes_and_scales": fp8_bytes, "bf16_equivalent": bf16_bytes,
                           "ratio": round(fp8_bytes / bf16_bytes, 4)},
            "kv_build_fp8": {"ms": round(build_ms, 4), "bytes_read": src_bytes,
                             "bytes_written": fp8_bytes,
                             "GB_per_s_read_plus_write": round(
                                 (src_bytes + fp8_bytes) / (build_ms * 1e-3) / 1e9, 1)},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                         "kernel": "attn_bf16_kernel<{}, {}, false, true>".format(
                             wl.D, 8 if wl.D == 64 and wl.total_s > 128 * wl.B else 4),
                         "kernel_ms_mean": round(kernel_ms, 5)}}
    print(json.dumps(line), flush=True)


def unique_prefix(wl):
    """The distinct prefix blocks a batch reads, beside the algorithmic bytes
    (which count every request's prefix once): item blocks listed by several
    requests, and user pages, each counted once.  The gap between the two is
    the reuse an item-as-prefix batch gets from the pool."""
    from prefix_reuse_attention_amd import workloads as W
    e = 2 if wl.dtype == "bf16" else 4
    items, user_tokens, listed = set(), 0, 0
    for r in range(wl.B):
        n = int(wl.n_p[r])
        if wl.mode[r] == W.ITEM:
            ids = wl.block_table[r, : n // W.ITEM_TOKENS]
            items.update(int(i) for i in ids)
            listed += len(ids)
        else:
            user_tokens += n
    tokens = len(items) * W.ITEM_TOKENS + user_tokens
    return {"item_blocks_listed": listed, "item_blocks_unique": len(items),
            "kv_bytes_unique": tokens * wl.H * wl.D * e * 2}


def run_cpu_baseline(wl, target_s):
    """The oracle (float64, OpenMP) on a bounded random sample of (suffix row,
    head) pairs of the same workload, scaled to TFLOP/s of algorithmic work."""
    import numpy as np
    import oracle
    from prefix_reuse_attention_amd import workloads as W

    rng = np.random.default_rng(12345)

    def sample(n):
        rows = rng.integers(0, wl.total_s, size=n).astype(np.int32)
        heads = rng.integers(0, wl.H, size=n).astype(np.int32)
        return rows, heads

    # each request's prefix as the oracle sees it (contiguous, block-table order)
    ks, vs, cu = [], [], [0]
    for r in range(wl.B):
        if wl.mode[r] == W.ITEM:
            ids = wl.block_table[r, : wl.n_p[r] // W.ITEM_TOKENS]
            ks.append(oracle.gather_item_prefix(wl.item_k, ids, W.ITEM_TOKENS))
            vs.append(oracle.gather_item_prefix(wl.item_v, ids, W.ITEM_TOKENS))
        else:
            ks.append(wl.user_k[wl.cu_user[r]:wl.cu_user[r + 1]])
            vs.append(wl.user_v[wl.cu_user[r]:wl.cu_user[r + 1]])
        cu.append(cu[-1] + len(ks[-1]))
    k_p, v_p = np.concatenate(ks), np.concatenate(vs)
    cu_p = np.array(cu, np.int32)
    del ks, vs

    def pair_flops(rows):
        req = np.searchsorted(wl.cu_s, rows, side="right") - 1
        return float(np.sum(4.0 * wl.D * (wl.n_p[req] + wl.n_s[req])))

    n = 64
    while True:
        rows, heads = sample(n)
        t = time.perf_counter()
        oracle.prefill_suffix(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p, wl.scale,
                              rows=rows, heads=heads)
        dt = time.perf_counter() - t
        if dt >= target_s / 4 or n >= wl.total_s * wl.H:
            break
        n = int(min(wl.total_s * wl.H, max(2 * n, n * (target_s / 2) / max(dt, 1e-3))))
    rows, heads = sample(max(1, int(n * target_s / max(dt, 1e-6))))
    t = time.perf_counter()
    oracle.prefill_suffix(wl.q, wl.k_s, wl.v_s, wl.cu_s, k_p, v_p, cu_p, wl.scale,
                          rows=rows, heads=heads)
    dt = time.perf_counter() - t
    fl = pair_flops(rows)
    print(f"[bench] oracle baseline: {len(rows)} (row, head) pairs in {dt:.1f}s",
          file=sys.stderr, flush=True)
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu": cpu_model(), "precision": "float64",
            "sample": f"{len(rows)} random (suffix row, head) pairs of {wl.name}, float64, "
                      f"{dt:.1f} s; rate = algorithmic flops of those pairs / time",
            "suffix_tokens_per_s_equiv": round(len(rows) / wl.H / dt, 3)}


def cpu_model():
    """The host CPU's model name and the processors the OS shows."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{name} ({os.cpu_count()} logical processors visible)"


def _timed_steps(step, steps, warmup, stream):
    """warmup untimed steps, then exactly `steps` steps between two
    synchronisations.  Returns (wall-clock ms per step, ms per step by two HIP
    events on the stream the kernels run on, recorded around the timed steps
    only: nothing else is enqueued between the steps)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return wall_ms, start.elapsed_time(end) / steps


def _per_call_ms(step, calls, stream):
    """Distribution of single calls, in a pass of its own after the timed
    steps: each call between its own pair of HIP events on the kernels'
    stream (events between calls would slow the timed region itself).
    Returns {median, min, p90, calls} in ms, or None for no calls."""
    import numpy as np
    import torch
    if calls <= 0:
        return None
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    return {"median": round(float(np.median(ms)), 5), "min": round(float(ms.min()), 5),
            "p90": round(float(np.percentile(ms, 90)), 5), "calls": calls,
            "note": "per-call HIP events, in an untimed pass of as many calls after the timed steps"}


def bench_prefix_workload(args):
    """The prefix-building rows: prefix rows over the 8k-history prefixes
    (16 requests x 8192 tokens, H=16, D=128, bf16; MFMA-bound) or per-item
    rows over the item pool of the item-prefix configuration (20000 items x 4
    tokens, H=8, D=64, bf16; HBM-bound).  Seeded N(0, 1) inputs; one JSON line
    in the same form as the default one."""
    import numpy as np
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd import workloads as W
    from prefix_reuse_attention_amd.device import to_device

    rng = np.random.default_rng(2024)
    stream = torch.cuda.current_stream()
    if args.workload == "prefix-rows":
        B, n_p, H, D = 16, 8192, 16, 128
        n = B * n_p
        desc = f"prefix rows of the 8k-history prefixes: B={B} x {n_p} tokens, H={H}, D={D}, bf16"
        flops = 4.0 * B * n_p * n_p * D * H
    else:
        n_items, T, H, D = 20000, W.ITEM_TOKENS, 8, 64
        n = n_items * T
        desc = f"per-item rows of the item pool: {n_items} items x {T} tokens, H={H}, D={D}, bf16"
        flops = 4.0 * n_items * T * T * D * H
    q, k, v = (W._normal(rng, (n, H, D), "bf16") for _ in range(3))
    dq, dk, dv = (to_device(a, "bf16") for a in (q, k, v))
    del q, k, v
    out = torch.empty_like(dq)
    lse = torch.empty((H, n), dtype=torch.float32, device="cuda")
    scale = float(np.float32(1.0 / np.sqrt(D)))
    if args.workload == "prefix-rows":
        cu = torch.arange(0, n + 1, n_p, dtype=torch.int32, device="cuda")
        ws = torch.empty(api.workspace_size(B, H, D, api.BAT_BF16, n, n_p, 0), dtype=torch.uint8,
                         device="cuda")
        step = lambda: api.attn_prefix_rows(dq, dk, dv, cu, softmax_scale=scale, max_prefix_len=n_p,
                                            out=out, lse=lse, workspace=ws)
    else:
        step = lambda: api.attn_item_local(dq, dk, dv, T, softmax_scale=scale, out=out, lse=lse)
    steps = args.steps if args.workload == "item-local" else max(1, min(args.steps, 20))
    warmup = args.warmup if args.workload == "item-local" else max(1, min(args.warmup, 5))
    wall_ms, kernel_ms = _timed_steps(step, steps, warmup, stream)
    alg_bytes = 4.0 * n * H * D * 2 + 4.0 * n * H  # q, k, v read, out written; lse
    line = {"workload": args.workload, "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(wall_ms, 5), "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) activations)",
            "config": {"workload": desc}, "alg_flops_per_step": flops,
            "alg_bytes_per_step": alg_bytes}
    if args.workload == "prefix-rows":
        line.update({"metric": "prefix-row attention TFLOP/s, 1 GPU",
                     "value": round(flops / (wall_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
                     "higher_is_better": True,
                     "roofline": {"bound": "mfma", "achieved": round(flops / (kernel_ms * 1e-3) / 1e12, 3),
                                  "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(flops / (kernel_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                  "traffic": None, "kernel_ms_mean": round(kernel_ms, 5)}})
    else:
        gbs = alg_bytes / (kernel_ms * 1e-3) / 1e9
        line.update({"metric": "per-item row attention GB/s, 1 GPU",
                     "value": round(alg_bytes / (wall_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                     "higher_is_better": True,
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                  "traffic": None, "kernel_ms_mean": round(kernel_ms, 5)}})
    print(f"[bench] {args.workload}: {wall_ms:.4f} ms/step (events {kernel_ms:.4f} ms)",
          file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _prefix_cpu_baseline(args.workload, rng, H, D, scale,
                                                    n_p if args.workload == "prefix-rows" else T,
                                                    args.cpu_seconds)
    print(json.dumps(line), flush=True)


SCHED = dict(n_requests=40000, num_users=20000, num_items=20000, items_per_request=128,
             user_len_range=(256, 4096), user_zipf_s=0.9, item_zipf_s=1.1, seed=7,
             budget_tokens=1 << 21, item_slots=8192, user_block=64, window=64, H=8, D=128)


def _window_work(tr, c, policy, ucap, icap, H, D, seed):
    """The serving step of the last `window` queries of the stream under one
    policy, on the device: the library's scheduler serves the earlier queries
    on the host (warm pools), then each query of the window in order, with
    every prefix it computes written into its pool place (bat_kv_build), its
    prefix rows computed (bat_attn_prefix_rows / bat_attn_item_local), and
    the prefill of its suffix over its prefix read from the pools
    (bat_attn_prefill), grouped into sub-batches (serving.Placement).  What
    the window reads from the warm pools is written there beforehand.
    Returns a step callable, the window's query-key pairs and its plan."""
    import numpy as np
    import torch
    from prefix_reuse_attention_amd import api
    from prefix_reuse_attention_amd import workloads as W
    from prefix_reuse_attention_amd.device import to_device
    from prefix_reuse_attention_amd.serving import DeviceWindow, Placement
    T, bs, B = tr.item_tokens, c["user_block"], c["window"]
    lo = tr.R - B
    sch = api.Scheduler(policy, T, bs, ucap, icap, tr.user_len, tr.num_items)
    sch.step(tr.user[:lo], tr.items[:lo])
    pl = Placement(sch, tr.user_len, T, bs, ucap, icap,
                   transient_user_blocks=2 * (-(-int(tr.user_len.max()) // bs)),
                   transient_item_slots=2 * tr.items.shape[1])
    init_u, init_i = dict(pl.blocks_of), pl.slot_item.copy()
    subs, outs = pl.plan(tr.user[lo:], tr.items[lo:], first_r=lo)
    # what the window reads from the warm pools before writing it itself
    written_u, written_i, pro_u, pro_i = set(), set(), {}, {}
    for sb in subs:
        for _, blocks in sb.user_writes:
            written_u.update(blocks)
        written_i.update(s for _, s in sb.item_writes)
        for q in sb.queries:
            if q.mode == W.USER and not written_u.intersection(q.prefix_places):
                pro_u[q.user] = init_u[q.user]
            elif q.mode == W.ITEM:
                for s in q.prefix_places:
                    if s not in written_i:
                        pro_i[s] = int(init_i[s])
    user_pool = api.new_pool(pl.user_pool_blocks, H, bs, D, torch.bfloat16)
    item_pool = api.new_pool(pl.item_pool_slots, H, T, D, torch.bfloat16)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    for u, blocks in pro_u.items():
        _, k, v = W.entity_tokens(seed, W.USER_STREAM, u, int(tr.user_len[u]), H, D)
        api.kv_build(to_device(k, "bf16"), to_device(v, "bf16"), i32([0, len(k)]),
                     i32([blocks]), user_pool)
    if pro_i:
        xs = [W.entity_tokens(seed, W.ITEM_STREAM, i, T, H, D) for i in pro_i.values()]
        api.kv_build(to_device(np.concatenate([x[1] for x in xs]), "bf16"),
                     to_device(np.concatenate([x[2] for x in xs]), "bf16"),
                     i32(np.arange(0, (len(xs) + 1) * T, T)), i32([[s] for s in pro_i]),
                     item_pool)
    win = DeviceWindow(pl, subs, user_pool, item_pool, seed, H, D, scale)
    pairs = int(sum(int(o["pairs"][0]) for o in outs))
    plan = {"sub_batches": len(subs), "item_mode_queries": int(sum(int(o["mode"][0]) for o in outs)),
            "user_writes": sum(len(sb.user_writes) for sb in subs),
            "item_writes": sum(len(sb.item_writes) for sb in subs)}
    return win.run, pairs, plan


def _policy_accounting(tr, c):
    """Both policies over the whole stream with the library's scheduler:
    per-policy results and summary."""
    from prefix_reuse_attention_amd import api
    T, m, bs, budget = tr.item_tokens, tr.items.shape[1], c["user_block"], c["budget_tokens"]
    pol = {"user_prefix": (api.BAT_POLICY_USER_PREFIX, budget // bs, 0),
           "hotness": (api.BAT_POLICY_HOTNESS, (budget - c["item_slots"] * T) // bs,
                       c["item_slots"])}
    res, host = {}, {}
    for name, (p, ucap, icap) in pol.items():
        sch = api.Scheduler(p, T, bs, ucap, icap, tr.user_len, tr.num_items)
        t = time.perf_counter()
        res[name] = sch.step(tr.user, tr.items)
        dt = time.perf_counter() - t
        r = res[name]
        host[name] = {
            "user_capacity_blocks": int(ucap), "item_slots": int(icap),
            "item_mode_frac": round(float(r["mode"].mean()), 4),
            "user_hit_frac": round(float(r["user_hit"][r["mode"] == 0].mean()), 4),
            "item_hit_frac": round(float(r["item_hits"][r["mode"] == 1].sum()
                                         / max(1, m * (r["mode"] == 1).sum())), 4),
            "computed_tokens": int(r["prefix_tokens"].sum() + r["suffix_tokens"].sum()),
            "pairs": int(r["pairs"].sum()),
            "scheduler_queries_per_s": round(tr.R / dt, 1)}
    b, h = host["user_prefix"], host["hotness"]
    accounting = {
        "computed_tokens_vs_user_prefix": round(h["computed_tokens"] / b["computed_tokens"], 4),
        "pairs_vs_user_prefix": round(h["pairs"] / b["pairs"], 4)}
    return pol, res, host, accounting


def _traffic(c):
    from prefix_reuse_attention_amd import workloads as W
    return W.make_traffic(c["seed"], c["n_requests"], c["num_users"], num_items=c["num_items"],
                          items_per_request=c["items_per_request"],
                          user_len_range=c["user_len_range"], user_zipf_s=c["user_zipf_s"],
                          item_zipf_s=c["item_zipf_s"])


def schedule_host_sweep():
    """Host accounting of both policies over traffic shapes around the
    measured one (20000 queries each): user history range, items per query,
    user popularity skew.  One JSON line per shape."""
    for lens in ((256, 1024), (256, 4096), (1024, 8192)):
        for m in (64, 128, 512):
            for uz in (0.6, 0.9, 1.2):
                c = dict(SCHED, n_requests=20000, user_len_range=lens, items_per_request=m,
                         user_zipf_s=uz)
                tr = _traffic(c)
                _, _, host, acc = _policy_accounting(tr, c)
                print(json.dumps({"user_len_range": list(lens), "items_per_request": m,
                                  "user_zipf_s": uz,
                                  "item_mode_frac": host["hotness"]["item_mode_frac"],
                                  "user_hit_frac_user_prefix": host["user_prefix"]["user_hit_frac"],
                                  **acc}), flush=True)


def bench_schedule_workload(args):
    """The prefix-mode choice on seeded Zipf traffic.

    Host: the library's scheduler (bat_sched_*) serves the whole stream under
    the user-as-prefix policy (every token of the cache budget for users) and
    the hotness-aware one (the same budget less `item_slots` items of T
    tokens for the item pool); the accounting of both.  Device: the serving
    step of a window of consecutive queries at the end of the stream (warm
    pools): per query the scheduler's choice, the cache writes of what it
    computes at the places its pools give, its prefix rows and its prefill
    over the pools, timed per window.  One JSON line; `value` is queries per
    second of the hotness-aware window's device work."""
    import torch
    c = SCHED
    t = time.perf_counter()
    tr = _traffic(c)
    T, m, bs = tr.item_tokens, tr.items.shape[1], c["user_block"]
    budget = c["budget_tokens"]
    print(f"[bench] traffic: {tr.R} queries, {tr.num_users} users, {tr.num_items} items, "
          f"generated in {time.perf_counter() - t:.1f}s", file=sys.stderr, flush=True)
    pol, res, host, accounting = _policy_accounting(tr, c)
    print(f"[bench] host: {json.dumps(host)} {json.dumps(accounting)}", file=sys.stderr,
          flush=True)

    H, D, B = c["H"], c["D"], c["window"]
    lo, hi = tr.R - B, tr.R
    stream = torch.cuda.current_stream()
    steps, warmup = max(1, min(args.steps, 50)), max(1, min(args.warmup, 10))
    dev = {}
    for name in pol:
        p, ucap, icap = pol[name]
        step, pairs, plan = _window_work(tr, c, p, ucap, icap, H, D, seed=c["seed"] + 10)
        wall_ms, kernel_ms = _timed_steps(step, steps, warmup, stream)
        dev[name] = {"ms_per_window": round(kernel_ms, 5), "wall_ms": round(wall_ms, 5),
                     "pairs": pairs, **plan}
        assert pairs == int(res[name]["pairs"][lo:hi].sum())  # the same choices as the stream run
        print(f"[bench] window {name}: {kernel_ms:.4f} ms (events), {wall_ms:.4f} ms wall, "
              f"{pairs} pairs", file=sys.stderr, flush=True)
        del step
        torch.cuda.empty_cache()
    hk = dev["hotness"]
    flops = 4.0 * D * H * hk["pairs"]
    achieved = flops / (hk["ms_per_window"] * 1e-3) / 1e12
    line = {"workload": "schedule", "metric": "queries/s of the attention work a window of "
            "queries needs under the hotness-aware prefix choice, 1 GPU",
            "value": round(B / (hk["wall_ms"] * 1e-3), 1), "unit": "queries/s",
            "higher_is_better": True, "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": hk["wall_ms"], "dtype": "bf16",
            "data": "synthetic (seeded Zipf traffic, N(0,1) activations)",
            "config": {"workload": f"prefix-mode choice: {tr.R} queries, {tr.num_users} users "
                       f"Zipf({c['user_zipf_s']}) with U{list(c['user_len_range'])} tokens, "
                       f"{m} of {tr.num_items} items Zipf({c['item_zipf_s']}) x {T} tokens, "
                       f"cache budget {budget} tokens; window of the last {B} queries, "
                       f"H={H}, D={D}, bf16", **{k: v for k, v in c.items()}},
            "vs_baseline": None,
            "speedup_vs_user_prefix": round(dev["user_prefix"]["ms_per_window"]
                                            / hk["ms_per_window"], 4),
            "host": host, "accounting": accounting, "device": dev,
            "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                         "kernel": "window: cache writes + prefix rows + per-item rows "
                                   "+ prefill, per sub-batch",
                         "kernel_ms_mean": hk["ms_per_window"]}}
    if not args.no_cpu_baseline:
        import oracle.schedule as OS
        n = 200
        while True:
            t = time.perf_counter()
            p, ucap, icap = pol["hotness"]
            OS.schedule(tr.user[:n], tr.user_len, tr.items[:n], T, bs, ucap, icap, p,
                        num_items=tr.num_items)
            dt = time.perf_counter() - t
            if dt >= args.cpu_seconds / 4 or n >= tr.R:
                break
            n = int(min(tr.R, max(2 * n, n * (args.cpu_seconds / 2) / max(dt, 1e-3))))
        line["cpu_baseline"] = {"value": round(n / dt, 1), "unit": "queries/s (scheduler)",
                                "cores": 1, "kind": "oracle", "cpu": cpu_model(),
                                "sample": f"the oracle's choice over the first {n} queries of "
                                          f"the stream (hotness-aware policy), {dt:.1f} s"}
    print(json.dumps(line), flush=True)


def _prefix_cpu_baseline(workload, rng, H, D, scale, span, target_s):
    """The oracle on a bounded sample of the same workload: whole requests of
    `span` prefix tokens (prefix rows, on sampled rows) or whole items."""
    import numpy as np
    import oracle
    from prefix_reuse_attention_amd import workloads as W
    if workload == "prefix-rows":
        q, k, v = (W._normal(rng, (span, H, D), "bf16") for _ in range(3))
        cu = np.array([0, span], np.int32)
        n = 64
        while True:
            rows = rng.integers(0, span, n).astype(np.int32)
            heads = rng.integers(0, H, n).astype(np.int32)
            t = time.perf_counter()
            oracle.prefix_rows(q, k, v, cu, scale, rows=rows, heads=heads)
            dt = time.perf_counter() - t
            if dt >= target_s / 4:
                break
            n = int(max(2 * n, n * (target_s / 2) / max(dt, 1e-3)))
        fl = 4.0 * len(rows) * span * D
        return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
                "kind": "oracle", "cpu": cpu_model(),
                "sample": f"{len(rows)} random (prefix row, head) pairs of one {span}-token prefix, "
                          f"float64, {dt:.1f} s"}
    n_items = 1024
    while True:
        q, k, v = (W._normal(rng, (n_items * span, H, D), "bf16") for _ in range(3))
        t = time.perf_counter()
        oracle.item_local(q, k, v, span, scale)
        dt = time.perf_counter() - t
        if dt >= target_s / 4 or n_items >= 20000:
            break
        n_items = int(min(20000, max(2 * n_items, n_items * (target_s / 2) / max(dt, 1e-3))))
    by = 4.0 * n_items * span * H * D * 2 + 4.0 * n_items * span * H
    return {"value": round(by / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{n_items} items x {span} tokens, all heads, float64, {dt:.1f} s"}


if __name__ == "__main__":
    main()
