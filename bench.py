"""Benchmark of the MLA split-KV decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long32k]
                    [--splits auto|N] [--layers 24] [--mode graph|eager]
                    [--no-cpu-baseline]

A step is one MLA layer-step: the partial-attention kernel plus the LSE merge kernel
for the whole batch of one layer, on one stream.  Consecutive steps rotate through
`--layers` distinct per-layer KV pools (the model has 24 MLA layers, Kimi K3 on
MI355X, "Inside Kimi K3"), so the KV stream comes from HBM and not from the 256 MB
memory-side cache.  Inputs are synthetic and already resident in HBM.

The single JSON line reports KV-read GB/s (algorithmic KV bytes / time per layer-step,
each cached latent read once) and the time per layer-step; `roofline` prices the
partial kernel (the dominant one) against the 8 TB/s HBM peak, with its average
duration measured here with HIP events on the stream it runs on; `cpu_baseline` times
the fp64 oracle on a bounded sample of the same workload on the host cores.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

METRIC = "MLA decode KV-read GB/s (% of 8 TB/s) and µs/layer-step at 32K ctx"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

# rocprofv3 FETCH_SIZE / WRITE_SIZE of the partial kernel (KiB per dispatch, median) and
# the copy-kernel calibration factors (profiles/<kernel>_<workload>.md), keyed by
# (workload, splits, partial storage, library version): a kernel change bumps the
# version, so `traffic` reads null until the counters are taken again.
TRAFFIC = {
    ("long32k", 0, "fp32", "mla_split_kv_decode_amd 0.6.7 (gfx950)"):
        {"fetch_kib": 18593.0, "write_kib": 8924.1875, "fetch_factor": 2.0, "write_factor": 1.0},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2400)
    ap.add_argument("--warmup", type=int, default=240)
    ap.add_argument("--workload", default="long32k")
    ap.add_argument("--splits", default="auto")
    ap.add_argument("--partial", default="fp32", choices=["bf16", "fp32"],
                    help="storage type of the partial answers between the two kernels")
    ap.add_argument("--layers", type=int, default=24)
    ap.add_argument("--mode", default="graph", choices=["graph", "eager"])
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--q-len", type=int, default=0,
                    help="query tokens per request (draft depth of a verification step): the "
                         "workload's history prefix is kept and the T new tokens added to it")
    ap.add_argument("--append", action="store_true",
                    help="time the cache append of the step's new tokens (mla_kv_append) instead "
                         "of the decode, alone and followed by the decode")
    ap.add_argument("--fp8-qk", action="store_true",
                    help="q.k on the FP8 matrix cores (FP8 pool, two or more 16-row blocks)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain copy kernel of known size: the FETCH_SIZE / WRITE_SIZE counters it reads
    calibrate the counters read for the decode kernels."""
    import torch

    n = mib * 1024 * 1024 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)


def describe(wl, splits):
    return (f"{wl.name}: batch {wl.batch}, {wl.num_heads} heads (padded to "
            f"{-(-wl.num_heads // 16) * 16} MFMA rows), {wl.q_len} query token(s), "
            f"context {int(wl.seq_lens.max())}, {wl.kv_format} latent 576 (K 576 / V 512), "
            f"paged 64, {'shuffled' if wl.name != 'tiny' else 'contiguous'} pages, "
            f"{'auto' if splits == 0 else splits} splits")


def cpu_baseline(wl, seconds):
    """The fp64 oracle, untuned, on the host: full layer-steps of the same workload
    (all requests and heads) repeated for about `seconds`."""
    import oracle
    from mla_split_kv_decode_amd import workloads as wk

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_paged(wl.q_bits, wl.pool, wl.kv_format, wl.kv_scale, wl.block_table,
                            wl.seq_lens, wl.page_size, wl.softmax_scale, causal=wl.causal)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    return {
        "value": round(wk.kv_bytes(wl.seq_lens, wl.kv_format) / per / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n} full layer-steps of {wl.name} (all requests and heads), "
                  f"{per * 1e3:.1f} ms each, {len(os.sched_getaffinity(0))} host cores visible",
        "ms_per_step": round(per * 1e3, 3),
    }


def bench_append(args, wl, mb, pools, scales, dev0, kv_dtype, decode_step, nl):
    """µs per mla_kv_append of the step's B x T new latents into one layer's pool, alone
    and followed by that layer's decode (graph replay over the rotated pools)."""
    import torch

    B, T = wl.batch, wl.q_len
    rng = np.random.default_rng(5)
    lat = torch.from_numpy(rng.standard_normal((B, T, 576)).astype(np.float32)).to(torch.bfloat16).cuda()
    stream = torch.cuda.current_stream()

    def timed(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nl):
                fn(i)
        reps = max(1, args.steps // nl)
        for _ in range(max(1, args.warmup // nl)):
            g.replay()
        torch.cuda.synchronize()
        res = []
        for _ in range(args.repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            e1.synchronize()
            res.append(e0.elapsed_time(e1) / (reps * nl) * 1e3)
        return float(np.median(res))

    def append(i):
        mb.kv_append(pools[i % nl], dev0["block_table"], dev0["seq_lens"], lat, kv_dtype, scales[i % nl])

    def append_then_decode(i):
        append(i)
        decode_step(i)

    us_app = timed(append)
    us_both = timed(append_then_decode)
    us_dec = timed(lambda i: decode_step(i))
    elem = wk_elem(wl.kv_format)
    moved = B * T * 576 * (2 + elem)
    print(json.dumps({
        "metric": "MLA cache append us per layer (the step's new latents, FP8 quantised or bf16)",
        "value": round(us_app, 3), "unit": "us", "higher_is_better": False, "n_gpus": 1,
        "data": "synthetic", "dtype": wl.kv_format,
        "config": {"workload": describe(wl, 0), "new_rows": B * T},
        "append_GBps": round(moved / (us_app * 1e-6) / 1e9, 3),
        "append_then_decode_us": round(us_both, 3), "decode_us": round(us_dec, 3),
        "bytes_per_append": moved,
    }))


def wk_elem(kv_format):
    return 2 if kv_format == "bf16" else 1


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              f"multi-GPU path: run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from mla_split_kv_decode_amd import binding as mb
    from mla_split_kv_decode_amd import workloads as wk

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    mb.load(build_if_missing=False)
    torch.cuda.set_device(0)
    over = {}
    if args.q_len:
        spec = wk.CONFIGS[args.workload]
        if "seq_len" not in spec:
            sys.exit("--q-len needs a workload with one history length")
        over = dict(q_len=args.q_len, seq_len=spec["seq_len"] - spec["q_len"] + args.q_len)
    wl = wk.make_workload(args.workload, **over)
    splits = 0 if args.splits == "auto" else int(args.splits)
    kv_dtype = mb.MLA_BF16 if wl.kv_format == "bf16" else mb.MLA_FP8_E4M3FN
    nl = max(1, args.layers)

    t_gen = time.perf_counter()
    dev0 = wk.to_device(wl)
    pools, scales = [dev0["pool"]], [dev0["kv_scale"]]
    for layer in range(1, nl):
        pool, sc = wk.layer_pool(wl, layer)
        t = torch.from_numpy(pool.view(np.int16) if wl.kv_format == "bf16" else pool).cuda()
        pools.append(t.view(torch.bfloat16) if wl.kv_format == "bf16" else t)
        scales.append(float(sc))
    t_gen = time.perf_counter() - t_gen

    t_plan = time.perf_counter()
    plan = mb.Plan(wl.batch, wl.q_len, wl.num_heads, wl.seq_lens, wl.softmax_scale,
                   causal=wl.causal, num_splits=splits, kv_dtype=kv_dtype,
                   partials_bf16=args.partial == "bf16", fp8_qk=args.fp8_qk)
    t_plan = time.perf_counter() - t_plan
    ws = mb.workspace(plan)
    B, T, H = wl.batch, wl.q_len, wl.num_heads
    out = torch.empty((B, T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
    kvs = [mb.paged_kv(p, dev0["block_table"], dev0["seq_lens"], kv_dtype, s)
           for p, s in zip(pools, scales)]
    q = dev0["q"]

    def step(i, full=True):
        mb.decode_splitkv(plan, q, kvs[i % nl], ws, out=out if full else None,
                          out_dtype=mb.MLA_BF16, out_lse=lse if full else None)

    if args.append:
        bench_append(args, wl, mb, pools, scales, dev0, kv_dtype, step, nl)
        return

    def timed(full, steps):
        """Average ms per call over `steps` calls (events on the launch stream)."""
        stream = torch.cuda.current_stream()
        if args.mode == "graph":
            # one graph of `nl` consecutive layer-steps, replayed
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(nl):
                    step(i, full)
            reps = max(1, steps // nl)
            for _ in range(max(1, args.warmup // nl)):
                g.replay()
            torch.cuda.synchronize()
            res = []
            for _ in range(args.repeats):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
                e1.synchronize()
                res.append(e0.elapsed_time(e1) / (reps * nl))
            return res, reps * nl
        for i in range(args.warmup):
            step(i, full)
        torch.cuda.synchronize()
        res = []
        for _ in range(args.repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                step(i, full)
            e1.record(stream)
            e1.synchronize()
            res.append(e0.elapsed_time(e1) / steps)
        return res, steps

    step(0)  # first call outside any capture (sets kernel attributes)
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    full_ms, n_full = timed(True, args.steps)
    part_ms, _ = timed(False, args.steps)
    ms = float(np.median(full_ms))
    ms_part = float(np.median(part_ms))

    kv_b = wk.kv_bytes(wl.seq_lens, wl.kv_format)
    gbs = kv_b / (ms * 1e-3) / 1e9
    part_gbs = kv_b / (ms_part * 1e-3) / 1e9
    flops = wk.attention_flops(wl.seq_lens, wl.q_len, wl.num_heads, wl.causal)
    traffic = None
    tr = None if args.fp8_qk else TRAFFIC.get((wl.name, splits, args.partial, mb.version()))
    if tr:
        traffic = int(1024 * (tr["fetch_kib"] * tr["fetch_factor"] + tr["write_kib"] * tr["write_factor"]))
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n_full,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": describe(wl, splits),
            "batch": B, "q_len": T, "num_heads": H, "seq_len": int(wl.seq_lens.max()),
            "kv_dtype": wl.kv_format, "splits": "auto" if splits == 0 else splits,
            "layers_rotated": nl, "launch": args.mode, "partials": args.partial,
            "qk": "fp8" if args.fp8_qk else "bf16",
        },
        "us_per_layer_step": round(ms * 1e3, 3),
        "pct_of_8TBs": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(part_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(part_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "mla_partial_kernel",
            "kernel_us": round(ms_part * 1e3, 3),
            "bytes_per_launch": kv_b,
        },
        "detail": {
            "full_ms_repeats": [round(x, 6) for x in full_ms],
            "partial_ms_repeats": [round(x, 6) for x in part_ms],
            "merge_and_gap_us": round((ms - ms_part) * 1e3, 3),
            "units": plan.num_units, "row_groups": plan.row_groups, "parts": plan.num_parts,
            "mfma_tflops": round(flops / (ms_part * 1e-3) / 1e12, 3),
            "mfma_frac_bf16": round(flops / (ms_part * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
            "io_bytes": wk.io_bytes(wl.seq_lens, wl.q_len, wl.num_heads, wl.kv_format),
            "plan_host_us": round(t_plan * 1e6, 1),
            "input_gen_s": round(t_gen, 2),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
