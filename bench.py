"""Benchmark: effective HBM bandwidth and tokens/s of the causal depthwise
short conv on one MI355X.

Headline step: one conv1d_fwd_varlen call on the long single-sequence
prefill -- dim 8192, T 14807, width 4, SiLU, bias, initial state, bf16 x
stored token-contiguous (dim, T) as the benchmark page draws it.  K steps run
back to back, rotating over 4 independent buffer sets (each 485 MB, together
larger than the 256 MB Infinity Cache) so every step streams from HBM.

Printed: ONE JSON line with the metric, the roofline of the kernel (its
algorithmic bytes over its HIP-event-timed average duration, against the
8 TB/s HBM peak), the single-threaded CPU oracle on the same workload, and
secondary measurements (other prefill sizes, the T=1 decode latency, the
varlen batch, the paged step, a same-size device copy).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-extra] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "effective HBM GB/s (% of peak) + tokens/s, bf16 causal conv1d dim 8192 width 4"
HEADLINE = dict(dim=8192, T=14807, width=4)
KERNEL_SOURCES = ["causal_depthwise_short_conv1d_amd/csrc/fwd_tokmajor.hip",
                  "causal_depthwise_short_conv1d_amd/csrc/sconv_device.h",
                  "causal_depthwise_short_conv1d_amd/csrc/sconv_params.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_tok_long_dim8192_T14807_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_bytes(dim, lengths, width, bias=True, n_init=None, n_state=None,
              cache_indices=False, has_init=True):
    """Algorithmic bytes of one varlen forward: x read and out written once per
    processed token, weights and bias once, the state read for sequences that
    continue from it and written for every processed sequence, and the index
    arrays (query_start_loc, cache_indices, has_initial_state)."""
    B = len(lengths)
    n_init = B if n_init is None else n_init
    n_state = B if n_state is None else n_state
    toks = sum(lengths)
    return (4 * toks * dim + 2 * dim * width + (2 * dim if bias else 0)
            + 2 * (width - 1) * dim * (n_init + n_state)
            + 4 * (B + 1) + (4 * B if cache_indices else 0) + (B if has_init else 0))


def paged_bytes(C, T, valid, R, width, n_streams=1):
    """Algorithmic bytes of one paged step: per stream x read, out written,
    the valid rows inserted into the cache, width-1 cached taps read per
    request and the taps; once for all streams the per-token positions and
    slots and query_start_loc (block-table reads are counted with the taps'
    rows they locate, not separately)."""
    per_stream = 2 * C * T * 2 + 2 * C * valid + 2 * C * (width - 1) * R + 2 * C * width
    return n_streams * per_stream + 16 * T + 4 * (R + 1)


def spec_bytes(dim, batch_live, seqlen, width, n_idx):
    """Algorithmic bytes of one speculative verify step that rolls the state:
    x read and out written, the width-1 history read and width-2+seqlen
    columns written per live entry, taps and bias, and the index arrays."""
    return (2 * 2 * batch_live * dim * seqlen + 2 * batch_live * dim * (width - 1)
            + 2 * batch_live * dim * (width - 2 + seqlen) + 2 * dim * width + 2 * dim
            + 4 * n_idx)


def graph_time_ms(fn, reps=100, replays=20):
    """Per-launch device time of `reps` back-to-back launches captured in one
    HIP graph: no host launch gap between them (the caches stay warm)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) / reps)
    del g
    return statistics.median(times)


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def event_time_ms(fn, reps, flush=None, stream=None):
    """Median per-launch time (HIP events on the launch stream); `flush` runs
    untimed before each launch."""
    import torch
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    return statistics.median(times)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="headline only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not part of it "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import causal_depthwise_short_conv1d_amd as S
    import workloads as W

    S.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dim, T, width = HEADLINE["dim"], HEADLINE["T"], HEADLINE["width"]
    nbytes = fwd_bytes(dim, [T], width)

    # ---- headline buffers: 4 sets rotated so each step misses the caches
    log(f"[bench] headline dim={dim} T={T} width={width}: {nbytes/1e6:.2f} MB per step")
    base = W.single_sequence(dim=dim, T=T, width=width, seed=W.seed_for(3, 0), device=dev)
    sets = []
    for i in range(4):
        sets.append(dict(x=base["x"].clone(), out=torch.empty_like(base["x"]),
                         st=base["conv_states"].clone()))
    qsl, hi = base["query_start_loc"], base["has_initial_state"]
    w, b = base["weight"], base["bias"]

    def step(i):
        s = sets[i % len(sets)]
        S.conv1d_fwd_varlen(s["x"], w, b, s["st"], qsl, has_initial_state=hi,
                            activation="silu", out=s["out"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = ev0.elapsed_time(ev1) / args.steps
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    log(f"[bench] {args.steps} steps: {ms_per_step*1e3:.1f} us/step wall, "
        f"{kern_ms*1e3:.1f} us/launch (events) -> {achieved:.0f} GB/s")

    # Calibration copy of a known byte count (256 MiB read + 256 MiB written),
    # present in every run so that counter passes can scale HBM counters.
    src = torch.empty(1 << 27, dtype=torch.bfloat16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("kernel_hash") == kernel_hash():
            traffic = tr.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic (randn*0.02 bf16, seeded, drawn on the GPU)",
        "config": {"workload": "long single-sequence prefill, dim 8192, T 14807, width 4, "
                               "SiLU, bias, initial state, x (dim,T) token-contiguous bf16",
                   "dim": dim, "T": T, "width": width, "layout": "(dim,T)",
                   "bytes_per_step": nbytes},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "fwd_tok_long_kernel<4,true,4>",
                     "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(kern_ms * 1e3, 2)},
    }
    del sets

    if not args.no_extra:
        result["extra"] = extras(torch, S, W, dev)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(torch, W, nbytes, base)
    print(json.dumps(result), flush=True)


def extras(torch, S, W, dev):
    """Secondary measurements, each launch timed alone after reading 1 GiB,
    which evicts the caches and leaves no dirty lines to drain during the
    timed launch (median of the repetitions)."""
    ex = {}
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    sink = torch.empty((), dtype=torch.float32, device=dev)
    flush = lambda: torch.sum(scratch, dim=0, out=sink)

    sweep = {}
    for dim, Ts in ((4096, (1, 128, 256, 514, 1024)), (8192, (4195, 11027, 14807))):
        for T in Ts:
            for layout in ("dim_tok", "tok_dim"):
                d = W.single_sequence(dim=dim, T=T, width=4, seed=W.seed_for(3, T % 97),
                                      device=dev, layout=layout)
                out = torch.empty_like(d["x"])
                fn = lambda: S.conv1d_fwd_varlen(d["x"], d["weight"], d["bias"],
                                                 d["conv_states"], d["query_start_loc"],
                                                 has_initial_state=d["has_initial_state"],
                                                 out=out)
                fn()
                ms = event_time_ms(fn, 15, flush)
                nb = fwd_bytes(dim, [T], 4)
                sweep[f"dim{dim}_T{T}_{layout}"] = {"us": round(ms * 1e3, 2),
                                                    "GB/s": round(nb / ms / 1e6, 1)}
                log(f"[bench] prefill dim{dim} T{T} {layout}: {ms*1e3:.2f} us {nb/ms/1e6:.0f} GB/s")
    ex["prefill_sweep"] = sweep

    # decode: T=1 at dim 4096 through the decode entry point
    d = W.decode_batch(batch=1, dim=4096, width=4, seed=W.seed_for(2, 1), device=dev)
    xo = d["x"].clone()
    fn = lambda: S.conv1d_update_decode(d["x"], d["conv_state"], d["weight"], d["bias"],
                                        activation="silu", cache_indices=d["cache_indices"],
                                        out=xo)
    fn()
    cold = event_time_ms(fn, 50, flush)
    warm = graph_time_ms(fn)
    lat = []
    for _ in range(1000):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        lat.append(time.perf_counter() - t0)
    dec_bytes = 4 * 4096 + 4 * 3 * 4096 + 2 * 4096 * 4 + 2 * 4096 + 4
    ex["decode_dim4096_T1"] = {"graph_us_per_launch": round(warm * 1e3, 2),
                               "cold_cache_us": round(cold * 1e3, 2),
                               "host_latency_us_median": round(statistics.median(lat) * 1e6, 2),
                               "bytes": dec_bytes}
    log(f"[bench] decode dim4096 T1: {warm*1e3:.2f} us/launch in a graph, {cold*1e3:.2f} us "
        f"cold, host latency {statistics.median(lat)*1e6:.1f} us")

    # decode at a serving batch: 64 entries x dim 8192, one token each
    d = W.decode_batch(batch=64, dim=8192, width=4, seed=W.seed_for(2, 2), num_lines=128,
                       device=dev)
    xo = d["x"].clone()
    fn = lambda: S.conv1d_update_decode(d["x"], d["conv_state"], d["weight"], d["bias"],
                                        activation="silu", cache_indices=d["cache_indices"],
                                        out=xo)
    fn()
    cold = event_time_ms(fn, 50, flush)
    warm = graph_time_ms(fn)
    nb = 64 * (4 * 8192 + 4 * 3 * 8192) + 2 * 8192 * 4 + 2 * 8192 + 4 * 64
    ex["decode_64x8192_T1"] = {"graph_us_per_launch": round(warm * 1e3, 2),
                               "cold_cache_us": round(cold * 1e3, 2), "bytes": nb,
                               "GB/s_graph": round(nb / warm / 1e6, 1)}
    log(f"[bench] decode 64x8192 T1: {warm*1e3:.2f} us/launch in a graph "
        f"({nb / warm / 1e6:.0f} GB/s), {cold*1e3:.2f} us cold")

    # speculative verify: 64 entries x dim 8192, 4 tokens each, state rolled
    cfg = W.SPEC_DECODE
    d = W.spec_decode_batch(batch=cfg["batch"], dim=cfg["dim"], width=cfg["width"],
                            seqlen=cfg["seqlen"], num_lines=cfg["num_lines"],
                            n_pad=cfg["n_pad"], seed=W.seed_for(6, 0), mode="roll",
                            device=dev)
    so = torch.empty_like(d["x"])
    fn = lambda: S.conv1d_update(d["x"], d["conv_state"], d["weight"], d["bias"],
                                 activation="silu", cache_indices=d["cache_indices"],
                                 num_accepted_tokens=d["num_accepted_tokens"], out=so)
    fn()
    cold = event_time_ms(fn, 30, flush)
    warm = graph_time_ms(fn)
    live = cfg["batch"] - cfg["n_pad"]
    nb = spec_bytes(cfg["dim"], live, cfg["seqlen"], cfg["width"], 2 * cfg["batch"])
    ex["spec_verify_64x8192_seqlen4"] = {"cold_cache_us": round(cold * 1e3, 2),
                                         "graph_us_per_launch": round(warm * 1e3, 2),
                                         "GB/s_cold": round(nb / cold / 1e6, 1), "bytes": nb}
    log(f"[bench] spec verify 64x8192x4: {cold*1e3:.2f} us cold ({nb/cold/1e6:.0f} GB/s), "
        f"{warm*1e3:.2f} us/launch in a graph")
    del d, so

    # varlen continuous batch, widths 2..5, channel-contiguous (T, dim) storage;
    # then width 4 token-contiguous (dim, T)
    vl = {}
    for width, layout in ((2, "tok_dim"), (3, "tok_dim"), (4, "tok_dim"), (5, "tok_dim"),
                          (4, "dim_tok")):
        d = W.varlen_batch(dim=8192, width=width, seed=W.seed_for(4, width), device=dev,
                           layout=layout)
        out = torch.empty_like(d["x"])
        lens = d["lengths"].tolist()
        lines = d["cache_indices"].tolist()
        init = d["has_initial_state"].tolist()
        kept = [l for l, c in zip(lens, lines) if c != -1]
        n_init = sum(1 for l, c, h in zip(lens, lines, init) if c != -1 and h and l > 0)
        n_state = sum(1 for l, c in zip(lens, lines) if c != -1 and l > 0)
        nb = fwd_bytes(8192, kept, width, n_init=n_init, n_state=n_state,
                       cache_indices=True) + 4 * (len(lens) - len(kept)) + (len(lens) - len(kept))
        cs = d["conv_states"]
        fn = lambda: S.conv1d_fwd_varlen(d["x"], d["weight"], d["bias"], cs,
                                         d["query_start_loc"], cache_indices=d["cache_indices"],
                                         has_initial_state=d["has_initial_state"], out=out)
        fn()
        ms = event_time_ms(fn, 10, flush)
        key = f"W{width}" if layout == "tok_dim" else f"W{width}_{layout}"
        vl[key] = {"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1),
                   "tokens": sum(kept), "tokens_per_s": round(sum(kept) / ms * 1e3, 1)}
        log(f"[bench] varlen {key}: {ms*1e3:.1f} us {nb/ms/1e6:.0f} GB/s")
        del d, out, cs
    ex["varlen_64seq_dim8192"] = vl

    # paged mixed step: one stream, then the four streams sharing the cache
    cfg = {k: v for k, v in W.PAGED_MIXED.items() if k != "off_s"}
    d = W.paged_multi_batch(seed=W.seed_for(5), device=dev, **cfg)
    Tp, C = d["x"].shape
    valid = int((d["slot_mapping"] >= 0).sum())
    R = d["query_start_loc"].numel() - 1
    outs = [torch.empty_like(x) for x in d["xs"]]
    fn = lambda: S.sconv_paged_fused(d["x"], d["weight"], d["cache"], d["positions"],
                                     d["slot_mapping"], d["query_start_loc"], d["block_table"],
                                     W.PAGED_MIXED["off_s"], d["ws"], activation="silu",
                                     use_residual=True, out=outs[0])
    fn()
    ms = event_time_ms(fn, 20, flush)
    nb = paged_bytes(C, Tp, valid, R, cfg["width"])
    ex["paged_mixed_T4128_C4096"] = {"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1),
                                     "bytes": nb}
    log(f"[bench] paged: {ms*1e3:.1f} us {nb/ms/1e6:.0f} GB/s")
    fn = lambda: S.sconv_paged_fused_multi(d["xs"], d["weights"], d["cache"], d["positions"],
                                           d["slot_mapping"], d["query_start_loc"],
                                           d["block_table"], d["offs"], d["ws"],
                                           activation="silu", use_residual=True, outs=outs)
    fn()
    ms = event_time_ms(fn, 20, flush)
    nb = paged_bytes(C, Tp, valid, R, cfg["width"], n_streams=len(d["xs"]))
    ex["paged_mixed_4streams_T4128_C4096"] = {"us": round(ms * 1e3, 2),
                                              "GB/s": round(nb / ms / 1e6, 1), "bytes": nb}
    log(f"[bench] paged 4 streams: {ms*1e3:.1f} us {nb/ms/1e6:.0f} GB/s")
    del d, outs

    # practical copy ceiling: a device copy moving the headline's byte count
    n = 8192 * 14807
    src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    fn = lambda: dst.copy_(src)
    fn()
    ms = event_time_ms(fn, 15, flush)
    ex["device_copy_same_bytes"] = {"us": round(ms * 1e3, 2), "GB/s": round(4 * n / ms / 1e6, 1),
                                    "bytes": 4 * n}
    log(f"[bench] copy: {ms*1e3:.1f} us {4*n/ms/1e6:.0f} GB/s")
    del scratch, src, dst
    torch.cuda.synchronize()
    return ex


def cpu_baseline(torch, W, nbytes, base):
    """The oracle (plain C, one thread) on the headline workload, repeated
    until at least 10 s of CPU time have been spent (at most 3 passes)."""
    import oracle
    x = base["x"].cpu()
    wgt, b = base["weight"].cpu(), base["bias"].cpu()
    qsl, hi = base["query_start_loc"].cpu(), base["has_initial_state"].cpu()
    out = torch.empty_like(x)
    times = []
    while sum(times) < 10.0 and len(times) < 3:
        st = base["conv_states"].cpu().clone()
        t0 = time.perf_counter()
        oracle.fwd_varlen(x, wgt, b, st, qsl, out, has_initial_state=hi, activation="silu")
        times.append(time.perf_counter() - t0)
    per = sum(times) / len(times)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    log(f"[bench] cpu oracle: {per:.2f} s per pass ({len(times)} passes)")
    return {"value": round(nbytes / per / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"the full headline workload (dim 8192 x T 14807, width 4), "
                      f"{len(times)} pass(es), {per:.2f} s each, single thread",
            "tokens_per_s": round(HEADLINE['T'] / per, 1),
            "host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model}


def summarize(argv):
    """Turn rocprofv3 CSV output of headline runs into the committed summary:

        python bench.py summarize TRACE_DIR FETCH_DIR WRITE_DIR OUT_PREFIX CMDLINE

    TRACE_DIR holds --kernel-trace --stats output, FETCH_DIR / WRITE_DIR the
    --pmc FETCH_SIZE / --pmc WRITE_SIZE passes of the same command.  The
    counters are scaled by what they read for the run's calibration copies
    (the last three 256 MiB device copies).  Writes OUT_PREFIX.txt and, for
    the headline kernel, the traffic JSON that the benchmark reports."""
    import csv
    import glob
    trace_dir, fetch_dir, write_dir, out_prefix, cmdline = argv[:5]
    calib = float(1 << 28)

    def one(d, pattern):
        f = glob.glob(os.path.join(d, "**", pattern), recursive=True)
        if not f:
            raise SystemExit(f"no {pattern} under {d}")
        return f[0]

    stats = list(csv.DictReader(open(one(trace_dir, "*kernel_stats.csv"))))
    trace = list(csv.DictReader(open(one(trace_dir, "*kernel_trace.csv"))))

    def counters(d, name):
        rows = [r for r in csv.DictReader(open(one(d, "*counter_collection.csv")))
                if r["Counter_Name"] == name]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        cal = [float(r["Counter_Value"]) * 1024 for r in rows
               if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) == 131072][-3:]
        factor = calib / statistics.mean(cal)
        ours = [float(r["Counter_Value"]) * 1024 for r in rows if "sconv::" in r["Kernel_Name"]]
        return factor, statistics.mean(ours), len(ours)

    fr, fetch, nf = counters(fetch_dir, "FETCH_SIZE")
    fw, write, nw = counters(write_dir, "WRITE_SIZE")
    headline = [r for r in stats if "sconv::" in r["Name"]]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in trace
            if "sconv::" in r["Kernel_Name"]]
    nbytes = fwd_bytes(HEADLINE["dim"], [HEADLINE["T"]], HEADLINE["width"])
    traffic = fetch * fr + write * fw
    lines = [
        f"# rocprofv3 summary: token-contiguous forward, dim {HEADLINE['dim']}, "
        f"T {HEADLINE['T']}, width {HEADLINE['width']}, SiLU, bias, initial state",
        f"# command: {cmdline}",
        f"# kernel source hash: {kernel_hash()}",
        "",
        "## kernel trace (--kernel-trace --stats), all kernels of the run",
        "name | calls | avg us | min us | max us",
    ]
    for r in stats:
        lines.append(f"{r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f}")
    if durs:
        med = statistics.median(durs) / 1e3
        lines += ["", f"headline kernel: {len(durs)} dispatches, median {med:.2f} us, "
                      f"mean {statistics.mean(durs)/1e3:.2f} us",
                  f"algorithmic bytes per launch: {nbytes} -> "
                  f"{nbytes / statistics.mean(durs):.1f} GB/s at the mean duration "
                  f"({100 * nbytes / statistics.mean(durs) / HBM_PEAK_GBS:.1f}% of 8 TB/s)"]
    lines += ["", "## HBM counters (--pmc FETCH_SIZE, --pmc WRITE_SIZE), per headline launch",
              f"FETCH_SIZE raw {fetch:.0f} B x calibration {fr:.4f} = {fetch*fr:.0f} B ({nf} dispatches)",
              f"WRITE_SIZE raw {write:.0f} B x calibration {fw:.4f} = {write*fw:.0f} B ({nw} dispatches)",
              f"calibration: each counter divided into 268435456 B for the run's 256 MiB device copies",
              f"HBM traffic {traffic:.0f} B vs algorithmic {nbytes} B "
              f"({100 * (traffic / nbytes - 1):+.2f}%)"]
    open(out_prefix + ".txt", "w").write("\n".join(lines) + "\n")
    json.dump({"kernel_hash": kernel_hash(), "bytes_per_launch": round(traffic),
               "fetch_bytes": round(fetch * fr), "write_bytes": round(write * fw),
               "fetch_calibration": round(fr, 4), "write_calibration": round(fw, 4),
               "algorithmic_bytes": nbytes, "command": cmdline},
              open(TRAFFIC_FILE, "w"), indent=1)
    print("\n".join(lines))


def summarize_trace(argv):
    """Kernel-only durations of every libsconv dispatch in a rocprofv3
    --kernel-trace run, grouped by (kernel, grid size) in first-launch order:

        python bench.py summarize-trace TRACE_DIR OUT_TXT TITLE CMDLINE

    Each group is one workload of the run (the benchmark launches its
    workloads one after another, each with its own grid)."""
    import csv
    import glob
    import re
    trace_dir, out_txt, title, cmdline = argv[:4]
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    rows = sorted(csv.DictReader(open(f[0])), key=lambda r: int(r["Start_Timestamp"]))
    groups = {}
    for r in rows:
        if "sconv::" not in r["Kernel_Name"]:
            continue
        name = re.sub(r"\(.*", "", r["Kernel_Name"].replace("(anonymous namespace)::", "")
                      .replace("void ", ""))
        key = (name, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# rocprofv3 kernel trace summary: {title}", f"# command: {cmdline}", "",
             "kernel | grid (threads) | workgroup | calls | median us | min us | max us"]
    for (name, grid, wg), d in groups.items():
        lines.append(f"{name} | {grid} | {wg} | {len(d)} | {statistics.median(d):.2f} | "
                     f"{min(d):.2f} | {max(d):.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "summarize":
        summarize(sys.argv[2:])
    elif len(sys.argv) > 1 and sys.argv[1] == "summarize-trace":
        summarize_trace(sys.argv[2:])
    else:
        main()
