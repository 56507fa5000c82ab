"""Benchmark of the MLA split-KV decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long32k]
                    [--splits auto|N] [--layers 24] [--repeats R]
                    [--no-cpu-baseline] [--no-other-workloads]
    python bench.py --read-ceiling [--workload long32k]
    python bench.py --lds-reserve 0,65536,98304 [--workload ragged256]

A step is one MLA layer-step: the partial-attention kernel plus the LSE merge kernel
for the whole batch of one layer, on one stream.  Consecutive steps rotate through
`--layers` distinct per-layer KV pools (the model has 24 MLA layers, Kimi K3 on
MI355X, "Inside Kimi K3"), so the KV stream comes from HBM and not from the 256 MB
memory-side cache.  Inputs are synthetic and already resident in HBM.

Timing: W untimed warm-up layer-steps, then R repeats of exactly K layer-steps, each
repeat one replay of a graph holding the K steps, bracketed by HIP events on the launch
stream and queued right behind three untimed replays of the same graph (so the GPU is busy
and at its working clocks when the timed region starts, and the host's launch of the
replay is not in it).  The reported time is the median repeat / K.

The JSON line reports KV-read GB/s (algorithmic KV bytes / time per layer-step, each
cached latent read once) and the time per layer-step.  `roofline` prices the partial
kernel (the dominant one), timed the same way on partial-only steps, against the 8 TB/s
HBM peak, or against the 2.5 PFLOP/s dense bf16 matrix peak for a workload whose
arithmetic intensity is past the ridge (the 96-head DCP shard).  `cpu_baseline` times
the fp64 oracle on a bounded sample of the same workload on all host cores and on one
thread.  `detail.workloads` holds a compact line for each other named workload (pools
drawn on the device), and `--read-ceiling` times a plain read of the same rotated pools
(the floor of any single launch that streams them) and an empty launch.  `--lds-reserve`
runs the residency experiment: the same decode with unused LDS reserved by every merge
workgroup (the MLA_LDS_RESERVE knob read at plan creation), one timing per reserve.
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
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # 312.5

# rocprofv3 FETCH_SIZE / WRITE_SIZE of the partial kernel (KiB per dispatch, median) and
# the copy-kernel calibration factors (profiles/<kernel>_<workload>.md), keyed by
# (workload, splits, library version): a kernel change bumps the version, so `traffic`
# reads null until the counters are taken again.
_V077 = "mla_split_kv_decode_amd 0.7.7 (gfx950)"
_V078 = "mla_split_kv_decode_amd 0.7.8 (gfx950)"
TRAFFIC = {
    ("long32k", 0, _V077): {"fetch_kib": 18596.0, "fetch_factor": 2.000, "write_kib": 6240.0, "write_factor": 1.000},
    ("tiny", 0, _V077): {"fetch_kib": 742.0, "fetch_factor": 2.000, "write_kib": 520.0, "write_factor": 1.000},
    ("ragged", 0, _V077): {"fetch_kib": 566958.8, "fetch_factor": 2.000, "write_kib": 10314.4, "write_factor": 1.000},
    ("spec_verify", 0, _V077): {"fetch_kib": 592344.8, "fetch_factor": 2.000, "write_kib": 16650.2,
                                "write_factor": 1.000},
    ("dcp_fp8", 0, _V077): {"fetch_kib": 43588.8, "fetch_factor": 2.000, "write_kib": 15600.0, "write_factor": 1.000},
}
# 0.7.8 added the streamed two-row-block kernels (one-row-group plans only); the kernels
# of these five workloads are instruction-for-instruction those of 0.7.7 (compared in the
# gfx950 assembly), so the 0.7.7 counters hold for them
TRAFFIC.update({(n, s, _V078): tr for (n, s, v), tr in list(TRAFFIC.items()) if v == _V077})


def traffic_of(name, splits, version):
    """Calibrated HBM bytes per partial-kernel launch from the counters above, or None."""
    tr = TRAFFIC.get((name, splits, version))
    if not tr:
        return None
    return int(1024 * (tr["fetch_kib"] * tr["fetch_factor"] + tr["write_kib"] * tr["write_factor"]))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480, help="layer-steps timed per repeat")
    ap.add_argument("--warmup", type=int, default=48, help="untimed layer-steps first")
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--workload", default="long32k")
    ap.add_argument("--splits", default="auto")
    ap.add_argument("--layers", type=int, default=24)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="seconds of oracle work on all host cores (half that again on one thread)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the compact lines of the other named workloads")
    ap.add_argument("--q-len", type=int, default=0,
                    help="query tokens per request (draft depth of a verification step): the "
                         "workload's history prefix is kept and the T new tokens added to it")
    ap.add_argument("--append", action="store_true",
                    help="time the cache append of the step's new tokens (mla_kv_append) instead "
                         "of the decode, alone and followed by the decode")
    ap.add_argument("--fp8-qk", action="store_true",
                    help="q.k on the FP8 matrix cores (FP8 pool, two or more 16-row blocks)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="time a plain read of the workload's rotated pools (registers and LDS "
                         "copies) and an empty launch, instead of the decode")
    ap.add_argument("--lds-reserve", default="",
                    help="comma-separated byte counts: time the decode with each as unused LDS "
                         "per merge workgroup (same binary; the residency experiment), instead "
                         "of the default line")
    ap.add_argument("--timeline", action="store_true",
                    help="device timestamps of one layer-step from the stamping build "
                         "(libmla_decode_timeline.so, include/mla_timeline.h), instead of the "
                         "default line")
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


LEAD_REPLAYS = 3  # untimed replays queued ahead of each timed one


def time_steps(step, steps, warmup, repeats, nl):
    """Per-repeat ms per layer-step: `warmup` eager layer-steps, then `repeats` times
    LEAD_REPLAYS untimed replays of a graph of exactly `steps` layer-steps (layer i % nl)
    followed by a timed replay of the same graph.  The timed replay is queued behind the
    untimed ones, so the GPU is busy (and at its working clocks) when the timed region
    starts, and the host's launch of the replay is not in it (with one untimed replay
    ahead, 20-step graphs of long32k read 1% higher)."""
    import torch

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i % nl)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i % nl)
    torch.cuda.synchronize()
    res = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(LEAD_REPLAYS):
            g.replay()  # untimed
        e0.record(stream)
        g.replay()  # timed: exactly `steps` layer-steps
        e1.record(stream)
        e1.synchronize()
        res.append(e0.elapsed_time(e1) / steps)
    del g
    return res


def cpu_baseline(wl, seconds):
    """The fp64 oracle, untuned, on the host: full layer-steps of the same workload
    (all requests and heads) repeated for about `seconds` on all cores, then for about
    half that on one thread."""
    import oracle
    from mla_split_kv_decode_amd import workloads as wk

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover - threadpoolctl is installed in the image
        threadpool_info, threadpool_limits = None, None

    def run(limit_s):
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.decode_paged(wl.q_bits, wl.pool, wl.kv_format, wl.kv_scale, wl.block_table,
                                wl.seq_lens, wl.page_size, wl.softmax_scale, causal=wl.causal)
            n += 1
            el = time.perf_counter() - t0
            if el >= limit_s:
                return n, el / n

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1]) if threadpool_info else 0
    n, per = run(seconds)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            n1, per1 = run(seconds / 2)
        one = {"value": round(wk.kv_bytes(wl.seq_lens, wl.kv_format) / per1 / 1e9, 4), "unit": "GB/s",
               "cores": 1, "ms_per_step": round(per1 * 1e3, 3),
               "sample": f"{n1} full layer-steps of {wl.name} on one BLAS thread"}
    return {
        "value": round(wk.kv_bytes(wl.seq_lens, wl.kv_format) / per / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n} full layer-steps of {wl.name} (all requests and heads), "
                  f"{per * 1e3:.1f} ms each, {len(os.sched_getaffinity(0))} host cores visible",
        "ms_per_step": round(per * 1e3, 3),
        "one_thread": one,
    }


def roofline_of(kv_b, flops, part_ms, traffic):
    """The partial kernel against the roofline its arithmetic intensity puts it under."""
    if flops / kv_b > RIDGE_FLOP_PER_BYTE:
        achieved = flops / (part_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": "mla_partial_kernel",
                "kernel_us": round(part_ms * 1e3, 3), "flops_per_launch": int(flops),
                "bytes_per_launch": int(kv_b),
                "hbm_frac": round(kv_b / (part_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    achieved = kv_b / (part_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "mla_partial_kernel", "kernel_us": round(part_ms * 1e3, 3),
            "bytes_per_launch": int(kv_b)}


def setup(mb, wk, wl, splits, nl, fp8_qk=False, device_pools=False):
    """Plan, workspace, outputs and the rotated pools' descriptors of a workload."""
    import torch

    kv_dtype = mb.MLA_BF16 if wl.kv_format == "bf16" else mb.MLA_FP8_E4M3FN
    q = torch.from_numpy(wl.q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    bt = torch.from_numpy(np.ascontiguousarray(wl.block_table)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(wl.seq_lens)).cuda()
    if device_pools:
        pools = wk.device_pools(wl, nl, wl.seed)
    else:
        pools = []
        for layer in range(nl):
            pool, sc = (wl.pool, wl.kv_scale) if layer == 0 else wk.layer_pool(wl, layer)
            t = torch.from_numpy(pool.view(np.int16) if wl.kv_format == "bf16" else pool).cuda()
            pools.append((t.view(torch.bfloat16) if wl.kv_format == "bf16" else t, float(sc)))
    t0 = time.perf_counter()
    plan = mb.Plan(wl.batch, wl.q_len, wl.num_heads, wl.seq_lens, wl.softmax_scale,
                   causal=wl.causal, num_splits=splits, kv_dtype=kv_dtype, fp8_qk=fp8_qk)
    t_plan = time.perf_counter() - t0
    ws = mb.workspace(plan)
    B, T, H = wl.batch, wl.q_len, wl.num_heads
    out = torch.empty((B, T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
    kvs = [mb.paged_kv(p, bt, sl, kv_dtype, s) for p, s in pools]

    def step(i, full=True):
        mb.decode_splitkv(plan, q, kvs[i], ws, out=out if full else None,
                          out_dtype=mb.MLA_BF16, out_lse=lse if full else None)

    return dict(plan=plan, step=step, pools=pools, kvs=kvs, kv_dtype=kv_dtype, q=q, bt=bt, sl=sl,
                t_plan=t_plan)


def measure(args, mb, wk, wl, splits, nl, fp8_qk=False, device_pools=False, steps=None, warmup=None):
    """Layer-step and partial-only timings of one workload."""
    import torch

    st = setup(mb, wk, wl, splits, nl, fp8_qk, device_pools)
    step = st["step"]
    step(0)  # first call outside any capture
    torch.cuda.synchronize()
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    full = time_steps(lambda i: step(i, True), steps, warmup, args.repeats, nl)
    part = time_steps(lambda i: step(i, False), steps, warmup, args.repeats, nl)
    plan = st["plan"]
    res = dict(full=full, part=part, ms=float(np.median(full)), ms_part=float(np.median(part)),
               units=plan.num_units, row_groups=plan.row_groups, parts=plan.num_parts,
               t_plan=st["t_plan"], steps=steps, warmup=warmup)
    del st
    torch.cuda.synchronize()
    return res


def compact_line(wl, splits, m, version):
    kv_b = wk_kv_bytes(wl)
    flops = wk_flops(wl)
    return {
        "workload": describe(wl, splits),
        "us_per_layer_step": round(m["ms"] * 1e3, 3),
        "GBps": round(kv_b / (m["ms"] * 1e-3) / 1e9, 2),
        "pct_of_8TBs": round(100 * kv_b / (m["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "partial_us": round(m["ms_part"] * 1e3, 3),
        "roofline": roofline_of(kv_b, flops, m["ms_part"], traffic_of(wl.name, splits, version)),
        "steps": m["steps"], "warmup": m["warmup"], "repeats": len(m["full"]),
        "units": m["units"], "row_groups": m["row_groups"], "parts": m["parts"],
        "data": "synthetic (pools drawn on the device)",
    }


def wk_kv_bytes(wl):
    from mla_split_kv_decode_amd import workloads as wk

    return wk.kv_bytes(wl.seq_lens, wl.kv_format)


def wk_flops(wl):
    from mla_split_kv_decode_amd import workloads as wk

    return wk.attention_flops(wl.seq_lens, wl.q_len, wl.num_heads, wl.causal)


def read_ceiling(args, mb, wk, wl, nl, big=False):
    """A plain read of the workload's rotated pools: every byte once, into registers or
    into LDS as the partial stage copies them, one launch per pool; and an empty launch.
    The floor of any single launch per layer-step that streams the same bytes."""
    import torch

    st = setup(mb, wk, wl, 0, nl, device_pools=big)
    # the KV bytes of each pool (its first pages; the pool's spare pages are left out),
    # rounded down to whole KiB as the read kernels take them
    kv_b = wk.kv_bytes(wl.seq_lens, wl.kv_format) // 1024 * 1024
    pools = [p.view(torch.uint8).view(-1)[:kv_b] for p, _ in st["pools"]]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool_b = kv_b
    out = {}
    for mode, name in ((0, "registers"), (1, "lds_copies"), (2, "empty_launch")):
        res = time_steps(lambda i: mb.read_reference(pools[i], mode, sink), args.steps, args.warmup,
                         args.repeats, nl)
        us = float(np.median(res)) * 1e3
        out[name] = {"us_per_launch": round(us, 3)}
        if mode != 2:
            out[name]["GBps"] = round(pool_b / (us * 1e-6) / 1e9, 2)
            out[name]["pct_of_8TBs"] = round(100 * pool_b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)
    print(json.dumps({
        "metric": "plain read of the rotated KV pools (one launch per pool): µs and GB/s",
        "value": out["lds_copies"]["GBps"], "unit": "GB/s", "higher_is_better": True, "n_gpus": 1,
        "data": "synthetic", "config": {"workload": describe(wl, 0), "bytes_read_per_launch": pool_b,
                                        "layers_rotated": nl},
        "steps": args.steps, "warmup": args.warmup, "repeats": args.repeats,
        "reads": out,
        "target_us_at_70pct": round(kv_b / (0.7 * HBM_PEAK_GBS * 1e9) * 1e6, 3),
    }), flush=True)


TL_PARTIAL = {0: "entry", 1: "first page copies issued", 2: "queries read", 3: "page 0 landed",
              4: "page 1 landed", 5: "epilogue denominators", 6: "partial answers issued",
              7: "partial answers stored"}
TL_MERGE = {0: "entry", 1: "LSE maximum known", 2: "partial answers consumed", 3: "end"}


def timeline(args, mb, wk, wl, splits, nl, big):
    """Device timestamps of a layer-step (include/mla_timeline.h): a graph of `nl`
    layer-steps captured, the stamps cleared, the graph replayed back to back (at least 96
    layer-steps); the stamps are then those of the last layer-step.  µs from the first partial workgroup's entry: the median over
    workgroups and the latest, per slot; per XCD (block index mod 8) the median of page 1
    landing and of the stores done."""
    import ctypes

    import torch

    lib = mb.load(build_if_missing=False)
    lib.mla_timeline_read.restype = ctypes.c_int
    lib.mla_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_timeline_clear.restype = ctypes.c_int
    lib.mla_timeline_clear.argtypes = []
    st = setup(mb, wk, wl, splits, nl, args.fp8_qk, device_pools=big)
    step = st["step"]
    for i in range(max(args.warmup, nl)):
        step(i % nl)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(nl):
            step(i)
    torch.cuda.synchronize()
    if lib.mla_timeline_clear() != 0:  # no stamp of another launch shape survives
        sys.exit("mla_timeline_clear failed")
    for _ in range(max(3, 96 // nl)):  # back to back, so the last layer-step runs at working clocks
        g.replay()
    torch.cuda.synchronize()
    part = np.zeros(4096 * 8, dtype=np.uint64)
    merge = np.zeros(16384 * 4, dtype=np.uint64)
    if lib.mla_timeline_read(part.ctypes.data, merge.ctypes.data) != 0:
        sys.exit("mla_timeline_read failed")
    part = part.reshape(4096, 8).astype(np.int64)
    merge = merge.reshape(16384, 4).astype(np.int64)
    blocks = np.nonzero(part[:, 0])[0]
    t0 = part[blocks, 0].min()

    def table(stamps, rows, names):
        out = {}
        for k, name in names.items():
            v = stamps[rows, k]
            v = v[v > 0]
            if len(v):
                us = (v - t0) * 0.01  # 100 MHz clock
                out[name] = {"median_us": round(float(np.median(us)), 2), "max_us": round(float(us.max()), 2)}
        return out

    mrows = np.nonzero(merge[:, 0])[0]
    per_xcd = {}
    for x in range(8):
        sel = blocks[blocks % 8 == x]
        per_xcd[str(x)] = {name: round(float(np.median((part[sel, k][part[sel, k] > 0] - t0) * 0.01)), 2)
                           for k, name in ((4, "page 1 landed"), (7, "partial answers stored"))
                           if (part[sel, k] > 0).any()}
    print(json.dumps({
        "metric": "device timeline of one layer-step (µs from the first partial workgroup's entry)",
        "unit": "us", "n_gpus": 1, "data": "synthetic",
        "config": {"workload": describe(wl, splits), "layers_rotated": nl},
        "library": mb.version() + " (timeline build)",
        "partial_workgroups": int(len(blocks)), "merge_workgroups": int(len(mrows)),
        "partial": table(part, blocks, TL_PARTIAL), "merge": table(merge, mrows, TL_MERGE),
        "per_xcd": per_xcd,
    }), flush=True)
    del g, st
    torch.cuda.synchronize()


# Static LDS of the merge kernels (largest variant, from the kernel metadata), the LDS of
# one compute unit and the allocation granule.
MERGE_STATIC_LDS = 672
CU_LDS = 160 * 1024
LDS_GRANULE = 1280


def lds_residency(args, mb, wk, wl, splits, nl, big):
    """The residency experiment: the same decode with each reserve of unused LDS per merge
    workgroup.  A reserve that lowers the number of merge workgroups a compute unit can
    hold but leaves the time unchanged shows the extra resident workgroups do not matter
    for this workload."""
    import os

    runs = []
    for b in [int(x) for x in args.lds_reserve.split(",") if x.strip()]:
        os.environ["MLA_LDS_RESERVE"] = str(b)
        try:
            m = measure(args, mb, wk, wl, splits, nl, args.fp8_qk, device_pools=big)
        finally:
            del os.environ["MLA_LDS_RESERVE"]
        alloc = -(-(MERGE_STATIC_LDS + b) // LDS_GRANULE) * LDS_GRANULE
        runs.append({
            "lds_reserve_bytes": b,
            "merge_workgroups_per_cu_lds_limit": CU_LDS // alloc,
            "us_per_layer_step": round(m["ms"] * 1e3, 3),
            "partial_us": round(m["ms_part"] * 1e3, 3),
            "merge_and_gap_us": round((m["ms"] - m["ms_part"]) * 1e3, 3),
            "full_ms_repeats": [round(x, 6) for x in m["full"]],
        })
        print(f"[bench] lds reserve {b}: {runs[-1]['us_per_layer_step']} us/layer-step", file=sys.stderr,
              flush=True)
    print(json.dumps({
        "metric": "decode µs/layer-step with unused LDS reserved per merge workgroup (residency experiment)",
        "unit": "us", "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
        "config": {"workload": describe(wl, splits), "layers_rotated": nl},
        "steps": args.steps, "warmup": args.warmup, "repeats": args.repeats,
        "merge_static_lds_bytes": MERGE_STATIC_LDS, "runs": runs,
        "library": mb.version(),
    }), flush=True)


def bench_append(args, wl, mb, st, nl):
    """µs per mla_kv_append of the step's B x T new latents into one layer's pool, alone
    and followed by that layer's decode."""
    import torch

    B, T = wl.batch, wl.q_len
    rng = np.random.default_rng(5)
    lat = torch.from_numpy(rng.standard_normal((B, T, 576)).astype(np.float32)).to(torch.bfloat16).cuda()
    pools, step, kv_dtype = st["pools"], st["step"], st["kv_dtype"]

    def append(i):
        mb.kv_append(pools[i][0], st["bt"], st["sl"], lat, kv_dtype, pools[i][1])

    def both(i):
        append(i)
        step(i)

    med = lambda f: float(np.median(time_steps(f, args.steps, args.warmup, args.repeats, nl))) * 1e3
    us_app, us_both, us_dec = med(append), med(both), med(lambda i: step(i))
    moved = B * T * 576 * (2 + (2 if wl.kv_format == "bf16" else 1))
    print(json.dumps({
        "metric": "MLA cache append us per layer (the step's new latents, FP8 quantised or bf16)",
        "value": round(us_app, 3), "unit": "us", "higher_is_better": False, "n_gpus": 1,
        "data": "synthetic", "dtype": wl.kv_format,
        "config": {"workload": describe(wl, 0), "new_rows": B * T},
        "append_GBps": round(moved / (us_app * 1e-6) / 1e9, 3),
        "append_then_decode_us": round(us_both, 3), "decode_us": round(us_dec, 3),
        "bytes_per_append": moved, "steps": args.steps, "warmup": args.warmup,
    }))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this library has no "
              f"multi-GPU path; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.repeats < 1:
        sys.exit("--steps and --repeats must be >= 1, --warmup >= 0")
    import torch

    from mla_split_kv_decode_amd import binding as mb
    from mla_split_kv_decode_amd import workloads as wk

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.timeline:  # the same kernels with the stamps compiled in
        from mla_split_kv_decode_amd import build as mbuild

        mb.LIB_PATH = mbuild.LIB_TIMELINE
    mb.load(build_if_missing=False)
    torch.cuda.set_device(0)
    over = {}
    if args.q_len:
        spec = wk.CONFIGS[args.workload]
        if "seq_len" not in spec:
            sys.exit("--q-len needs a workload with one history length")
        over = dict(q_len=args.q_len, seq_len=spec["seq_len"] - spec["q_len"] + args.q_len)
    nl = max(1, args.layers)
    big = args.workload in ("ragged", "ragged256", "spec_verify")
    t_gen = time.perf_counter()
    # the two gigabyte-sized workloads get their timing pools on the device; the others
    # use the oracle's generator (also for the CPU baseline)
    wl = wk.timing_workload(args.workload, **over) if big else wk.make_workload(args.workload, **over)
    t_gen = time.perf_counter() - t_gen
    splits = 0 if args.splits == "auto" else int(args.splits)

    if args.read_ceiling:
        read_ceiling(args, mb, wk, wl, nl, big)
        return
    if args.timeline:
        timeline(args, mb, wk, wl, splits, nl, big)
        return
    if args.lds_reserve:
        lds_residency(args, mb, wk, wl, splits, nl, big)
        return
    if args.append:
        st = setup(mb, wk, wl, splits, nl, args.fp8_qk, device_pools=big)
        bench_append(args, wl, mb, st, nl)
        return

    m = measure(args, mb, wk, wl, splits, nl, args.fp8_qk, device_pools=big)
    kv_b = wk.kv_bytes(wl.seq_lens, wl.kv_format)
    flops = wk.attention_flops(wl.seq_lens, wl.q_len, wl.num_heads, wl.causal)
    ms, ms_part = m["ms"], m["ms_part"]
    gbs = kv_b / (ms * 1e-3) / 1e9
    traffic = None if args.fp8_qk or args.q_len else traffic_of(wl.name, splits, mb.version())
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": m["steps"],
        "warmup": m["warmup"],
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.kv_format == "bf16" else "fp8_e4m3fn KV, bf16 q and MFMA",
        "data": "synthetic",
        "config": {
            "workload": describe(wl, splits),
            "batch": wl.batch, "q_len": wl.q_len, "num_heads": wl.num_heads,
            "seq_len": int(wl.seq_lens.max()), "kv_dtype": wl.kv_format,
            "splits": "auto" if splits == 0 else splits, "layers_rotated": nl,
            "qk": "fp8" if args.fp8_qk else "bf16",
        },
        "us_per_layer_step": round(ms * 1e3, 3),
        "pct_of_8TBs": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": roofline_of(kv_b, flops, ms_part, traffic),
        "detail": {
            "timing": f"{m['warmup']} warm-up layer-steps, then {args.repeats} repeats of a timed graph "
                      f"replay of {m['steps']} layer-steps, each queued behind {LEAD_REPLAYS} untimed "
                      f"replays of the same graph; median",
            "repeats": args.repeats,
            "full_ms_repeats": [round(x, 6) for x in m["full"]],
            "partial_ms_repeats": [round(x, 6) for x in m["part"]],
            "merge_and_gap_us": round((ms - ms_part) * 1e3, 3),
            "units": m["units"], "row_groups": m["row_groups"], "parts": m["parts"],
            "mfma_tflops": round(flops / (ms_part * 1e-3) / 1e12, 3),
            "mfma_frac_bf16": round(flops / (ms_part * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
            "io_bytes": wk.io_bytes(wl.seq_lens, wl.q_len, wl.num_heads, wl.kv_format),
            "plan_host_us": round(m["t_plan"] * 1e6, 1),
            "input_gen_s": round(t_gen, 2),
            "library": mb.version(),
        },
        "cpu_baseline": None,
    }
    if not args.no_other_workloads and args.workload == "long32k" and not over:
        lines = {}
        for name in ("tiny", "ragged", "spec_verify", "dcp_fp8"):
            other = wk.timing_workload(name)
            nlo = 2 if name in ("ragged", "spec_verify") else nl
            st_o = max(4 * nlo, 48) if name in ("ragged", "spec_verify") else args.steps
            mo = measure(args, mb, wk, other, 0, nlo, device_pools=True, steps=st_o,
                         warmup=min(args.warmup, st_o))
            lines[name] = compact_line(other, 0, mo, mb.version())
            print(f"[bench] {name}: {lines[name]['us_per_layer_step']} us/layer-step", file=sys.stderr,
                  flush=True)
        res["detail"]["workloads"] = lines
    if not args.no_cpu_baseline and wl.pool is not None:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
