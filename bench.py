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
CSRC = os.path.join(ROOT, "causal_depthwise_short_conv1d_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "workloads_traffic.json")
HEADLINE_WORKLOAD = "long_T14807_dim_tok"
PROFILE_REPS = 10          # timed launches per workload in a profile run (after one warm-up)


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
    """Hash of every kernel source: counter figures are reported only while
    the kernels are the ones they were taken on."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    """Per-workload HBM counter figures (profiles/workloads_traffic.json),
    or {} when they were taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    tr = json.load(open(TRAFFIC_FILE))
    return tr.get("workloads", {}) if tr.get("kernel_hash") == kernel_hash() else {}


def varlen_bytes(d, width):
    """Algorithmic bytes of a varlen batch: the processed sequences' tokens,
    histories read where a sequence continues from its state, states written
    for every processed non-empty sequence, and all index arrays."""
    lens = d["lengths"].tolist()
    lines = d["cache_indices"].tolist()
    init = d["has_initial_state"].tolist()
    kept = [l for l, c in zip(lens, lines) if c != -1]
    n_init = sum(1 for l, c, h in zip(lens, lines, init) if c != -1 and h and l > 0)
    n_state = sum(1 for l, c in zip(lens, lines) if c != -1 and l > 0)
    dim = d["weight"].shape[0]
    n_pad = len(lens) - len(kept)
    return (fwd_bytes(dim, kept, width, n_init=n_init, n_state=n_state, cache_indices=True)
            + 5 * n_pad), sum(kept)


def workload_builders():
    """Every benchmarked workload as (name, builder); builder(torch, S, W, dev)
    returns (launch, algorithmic bytes, tokens).  The order is the order of a
    profile run."""
    def single(dim, T, layout):
        def b(torch, S, W, dev):
            d = W.single_sequence(dim=dim, T=T, width=4, seed=W.seed_for(3, T % 97),
                                  device=dev, layout=layout)
            out = torch.empty_like(d["x"])
            fn = lambda: S.conv1d_fwd_varlen(d["x"], d["weight"], d["bias"], d["conv_states"],
                                             d["query_start_loc"],
                                             has_initial_state=d["has_initial_state"], out=out)
            return fn, fwd_bytes(dim, [T], 4), T
        return b

    def varlen(width, layout):
        def b(torch, S, W, dev):
            d = W.varlen_batch(dim=8192, width=width, seed=W.seed_for(4, width), device=dev,
                               layout=layout)
            out = torch.empty_like(d["x"])
            nb, toks = varlen_bytes(d, width)
            fn = lambda: S.conv1d_fwd_varlen(d["x"], d["weight"], d["bias"], d["conv_states"],
                                             d["query_start_loc"],
                                             cache_indices=d["cache_indices"],
                                             has_initial_state=d["has_initial_state"], out=out)
            return fn, nb, toks
        return b

    def paged(n_streams):
        def b(torch, S, W, dev):
            cfg = {k: v for k, v in W.PAGED_MIXED.items() if k != "off_s"}
            d = W.paged_multi_batch(seed=W.seed_for(5), device=dev, **cfg)
            Tp, C = d["x"].shape
            valid = int((d["slot_mapping"] >= 0).sum())
            R = d["query_start_loc"].numel() - 1
            outs = [torch.empty_like(x) for x in d["xs"]]
            if n_streams == 1:
                fn = lambda: S.sconv_paged_fused(d["x"], d["weight"], d["cache"], d["positions"],
                                                 d["slot_mapping"], d["query_start_loc"],
                                                 d["block_table"], W.PAGED_MIXED["off_s"],
                                                 d["ws"], activation="silu", use_residual=True,
                                                 out=outs[0])
            else:
                fn = lambda: S.sconv_paged_fused_multi(d["xs"], d["weights"], d["cache"],
                                                       d["positions"], d["slot_mapping"],
                                                       d["query_start_loc"], d["block_table"],
                                                       d["offs"], d["ws"], activation="silu",
                                                       use_residual=True, outs=outs)
            return fn, paged_bytes(C, Tp, valid, R, cfg["width"], n_streams=n_streams), valid
        return b

    def decode(batch, dim):
        def b(torch, S, W, dev):
            d = W.decode_batch(batch=batch, dim=dim, width=4, seed=W.seed_for(2, 1 + (batch > 1)),
                               num_lines=max(batch, 128 if batch > 1 else 1), device=dev)
            xo = d["x"].clone()
            fn = lambda: S.conv1d_update_decode(d["x"], d["conv_state"], d["weight"], d["bias"],
                                                activation="silu",
                                                cache_indices=d["cache_indices"], out=xo)
            return fn, decode_bytes(batch, dim, 4), batch
        return b

    def verify(torch, S, W, dev):
        cfg = W.SPEC_DECODE
        d = W.spec_decode_batch(batch=cfg["batch"], dim=cfg["dim"], width=cfg["width"],
                                seqlen=cfg["seqlen"], num_lines=cfg["num_lines"],
                                n_pad=cfg["n_pad"], seed=W.seed_for(6, 0), mode="roll",
                                device=dev)
        so = torch.empty_like(d["x"])
        fn = lambda: S.conv1d_update(d["x"], d["conv_state"], d["weight"], d["bias"],
                                     activation="silu", cache_indices=d["cache_indices"],
                                     num_accepted_tokens=d["num_accepted_tokens"], out=so)
        live = cfg["batch"] - cfg["n_pad"]
        return fn, spec_bytes(cfg["dim"], live, cfg["seqlen"], cfg["width"], 2 * cfg["batch"]), \
            live * cfg["seqlen"]

    out = [(HEADLINE_WORKLOAD, single(8192, 14807, "dim_tok")),
           ("long_T14807_tok_dim", single(8192, 14807, "tok_dim"))]
    for T in (4195, 11027):
        for layout in ("dim_tok", "tok_dim"):
            out.append((f"long_T{T}_{layout}", single(8192, T, layout)))
    for width in (2, 3, 4, 5):
        out.append((f"varlen_W{width}_tok_dim", varlen(width, "tok_dim")))
    out.append(("varlen_W4_dim_tok", varlen(4, "dim_tok")))
    out += [("paged_1stream", paged(1)), ("paged_4streams", paged(4)),
            ("decode_1x4096", decode(1, 4096)), ("decode_64x8192", decode(64, 8192)),
            ("verify_64x8192x4", verify)]
    return out


def decode_bytes(batch, dim, width):
    """Algorithmic bytes of a decode step: per entry x read, out written, the
    width-1 history read and rewritten, its line index; taps and bias once."""
    return batch * (4 * dim + 4 * (width - 1) * dim + 4) + 2 * dim * width + 2 * dim


def profile_set(reps, bytes_out=None):
    """Every workload, one after another: a warm-up launch, then `reps`
    launches each after a 1 GiB read (cold caches, as the benchmark times
    them); three 256 MiB device copies first calibrate the HBM counters.
    Run under rocprofv3 (kernel trace, or one counter pass) and turned into
    the committed summaries by `bench.py summarize-set`."""
    import torch
    import causal_depthwise_short_conv1d_amd as S
    import workloads as W
    S.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    src = torch.empty(1 << 27, dtype=torch.bfloat16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    sizes = {}
    for name, build in workload_builders():
        fn, nb, _ = build(torch, S, W, dev)
        sizes[name] = nb
        fn()
        for _ in range(reps):
            torch.sum(scratch, dim=0, out=sink)
            fn()
        torch.cuda.synchronize()
        log(f"[profile] {name}: {reps + 1} launches, {nb} algorithmic bytes each")
        del fn
        torch.cuda.empty_cache()
    if bytes_out:
        json.dump(sizes, open(bytes_out, "w"), indent=1)


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
    ap.add_argument("--profile-set", action="store_true",
                    help="run every workload PROFILE_REPS times for rocprofv3, print no JSON")
    ap.add_argument("--bytes-out", default=None,
                    help="with --profile-set: write each workload's algorithmic bytes here")
    args = ap.parse_args()
    if args.profile_set:
        profile_set(PROFILE_REPS, args.bytes_out)
        return

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

    counters = load_traffic()
    head_tr = counters.get(HEADLINE_WORKLOAD)
    traffic = head_tr["traffic_bytes"] if head_tr else None

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
    counters = load_traffic()

    def with_counters(entry, name, us):
        """Add the workload's HBM counter figures (profiles/workloads_traffic.json,
        taken on these kernel sources): counter bytes, their ratio to the
        algorithmic bytes, and counter bytes over this run's time and over
        the profile's kernel-only median."""
        c = counters.get(name)
        if c:
            entry["counter_bytes"] = c["traffic_bytes"]
            entry["counter_over_algorithmic"] = c["ratio"]
            entry["achieved_GB/s"] = round(c["traffic_bytes"] / us / 1e3, 1)
            entry["kernel_only_us"] = c["median_us"]
            entry["achieved_GB/s_kernel_only"] = c["achieved_GBps"]
        return entry
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
                sweep[f"dim{dim}_T{T}_{layout}"] = with_counters(
                    {"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1)},
                    f"long_T{T}_{layout}", ms * 1e3)
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
    # Enqueue-to-completion latency seen by a host caller, three ways: the
    # Python binding with torch's synchronize; the binding with the HIP
    # runtime's stream synchronize; and the library itself, called through
    # a pre-bound launcher (arguments marshalled once) with the HIP stream
    # synchronize -- the C call and the wait, without the binding.
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")               # the runtime torch has loaded
    hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    bound = S.bind_update_decode(d["x"], d["conv_state"], d["weight"], d["bias"],
                                 activation="silu", cache_indices=d["cache_indices"], out=xo)

    def latency(call, sync):
        ts = []
        for _ in range(1000):
            t0 = time.perf_counter()
            call()
            sync()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts) * 1e6
    lat = latency(fn, torch.cuda.synchronize)
    lat_hip = latency(fn, lambda: hip.hipStreamSynchronize(stream))
    lat_lib = latency(bound, lambda: hip.hipStreamSynchronize(stream))
    dec_bytes = decode_bytes(1, 4096, 4)
    ex["decode_dim4096_T1"] = with_counters(
        {"graph_us_per_launch": round(warm * 1e3, 2), "cold_cache_us": round(cold * 1e3, 2),
         "host_latency_us_median": round(lat, 2),
         "host_latency_us_median_hip_sync": round(lat_hip, 2),
         "library_latency_us_median": round(lat_lib, 2), "bytes": dec_bytes},
        "decode_1x4096", cold * 1e3)
    log(f"[bench] decode dim4096 T1: {warm*1e3:.2f} us/launch in a graph, {cold*1e3:.2f} us "
        f"cold; host latency {lat:.1f} us (binding + torch sync), {lat_hip:.1f} us (binding + "
        f"HIP sync), {lat_lib:.1f} us (pre-bound C call + HIP sync)")

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
    nb = decode_bytes(64, 8192, 4)
    ex["decode_64x8192_T1"] = with_counters(
        {"graph_us_per_launch": round(warm * 1e3, 2), "cold_cache_us": round(cold * 1e3, 2),
         "bytes": nb, "GB/s_graph": round(nb / warm / 1e6, 1)}, "decode_64x8192", cold * 1e3)
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
    ex["spec_verify_64x8192_seqlen4"] = with_counters(
        {"cold_cache_us": round(cold * 1e3, 2), "graph_us_per_launch": round(warm * 1e3, 2),
         "GB/s_cold": round(nb / cold / 1e6, 1), "bytes": nb}, "verify_64x8192x4", cold * 1e3)
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
        nb, toks = varlen_bytes(d, width)
        cs = d["conv_states"]
        fn = lambda: S.conv1d_fwd_varlen(d["x"], d["weight"], d["bias"], cs,
                                         d["query_start_loc"], cache_indices=d["cache_indices"],
                                         has_initial_state=d["has_initial_state"], out=out)
        fn()
        ms = event_time_ms(fn, 10, flush)
        key = f"W{width}" if layout == "tok_dim" else f"W{width}_{layout}"
        vl[key] = with_counters({"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1),
                                 "tokens": toks, "tokens_per_s": round(toks / ms * 1e3, 1)},
                                f"varlen_W{width}_{layout}", ms * 1e3)
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
    ex["paged_mixed_T4128_C4096"] = with_counters(
        {"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1), "bytes": nb},
        "paged_1stream", ms * 1e3)
    log(f"[bench] paged: {ms*1e3:.1f} us {nb/ms/1e6:.0f} GB/s")
    fn = lambda: S.sconv_paged_fused_multi(d["xs"], d["weights"], d["cache"], d["positions"],
                                           d["slot_mapping"], d["query_start_loc"],
                                           d["block_table"], d["offs"], d["ws"],
                                           activation="silu", use_residual=True, outs=outs)
    fn()
    ms = event_time_ms(fn, 20, flush)
    nb = paged_bytes(C, Tp, valid, R, cfg["width"], n_streams=len(d["xs"]))
    ex["paged_mixed_4streams_T4128_C4096"] = with_counters(
        {"us": round(ms * 1e3, 2), "GB/s": round(nb / ms / 1e6, 1), "bytes": nb},
        "paged_4streams", ms * 1e3)
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
    until at least 10 s of CPU time have been spent (at most 5 passes)."""
    import oracle
    x = base["x"].cpu()
    wgt, b = base["weight"].cpu(), base["bias"].cpu()
    qsl, hi = base["query_start_loc"].cpu(), base["has_initial_state"].cpu()
    out = torch.empty_like(x)
    times = []
    while sum(times) < 10.0 and len(times) < 5:
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
    (the last three 256 MiB device copies).  Writes OUT_PREFIX.txt (the
    traffic figures the benchmark reports come from `summarize-set`)."""
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


def _profile_dispatches(d, counter=None):
    """The libsconv calls of a profile run in launch order, assigned to the
    workloads (each called PROFILE_REPS + 1 times, in the order of
    workload_builders), and the run's calibration copies.  With `counter`,
    d holds one --pmc pass and each call carries that counter's value in
    bytes summed over its dispatches (the CSV gives KiB); else d holds a
    kernel trace and each call the summed kernel-only time of its
    dispatches in us."""
    import csv
    import glob
    name = "*counter_collection.csv" if counter else "*kernel_trace.csv"
    f = glob.glob(os.path.join(d, "**", name), recursive=True)
    if not f:
        raise SystemExit(f"no {name} under {d}")
    rows = list(csv.DictReader(open(f[0])))
    if counter:
        rows = [r for r in rows if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        val = lambda r: float(r["Counter_Value"]) * 1024
        grid = lambda r: int(r["Grid_Size"])
    else:
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        val = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        grid = lambda r: int(r["Grid_Size_X"]) if "Grid_Size_X" in r else int(r["Grid_Size"])
    calib = [val(r) for r in rows if "copyBuffer" in r["Kernel_Name"] and grid(r) == 131072][:3]
    # One call is a run of consecutive libsconv dispatches (a token-contiguous
    # varlen batch is two: the stream kernel, then the head kernel); calls are
    # separated by the flush reads and by the input set-up of each workload.
    ours, prev = [], False
    for r in rows:
        mine = "sconv::" in r["Kernel_Name"]
        if mine and prev:
            k, v = ours[-1]
            ours[-1] = (k + " + " + r["Kernel_Name"], v + val(r))
        elif mine:
            ours.append((r["Kernel_Name"], val(r)))
        prev = mine
    names = [n for n, _ in workload_builders()]
    per = PROFILE_REPS + 1
    if len(ours) != per * len(names):
        raise SystemExit(f"{d}: {len(ours)} libsconv calls, expected {per * len(names)}")
    out = {}
    for i, n in enumerate(names):
        grp = ours[i * per:(i + 1) * per]
        kern = {k for k, _ in grp}
        if len(kern) != 1:
            raise SystemExit(f"{d}: workload {n} ran several kernels: {kern}")
        out[n] = (kern.pop(), [v for _, v in grp[1:]])      # the warm-up launch dropped
    return out, calib


def summarize_set(argv):
    """Per-workload kernel time and HBM traffic from three rocprofv3 runs of
    `bench.py --profile-set` (a kernel trace, a FETCH_SIZE pass and a
    WRITE_SIZE pass), and optionally one pass of SQ counters:

        python bench.py summarize-set BYTES_JSON TRACE_DIR FETCH_DIR WRITE_DIR SQ_DIR|- CMDLINE

    The counters are scaled by what they read for the run's three 256 MiB
    device copies (each reads and writes 268435456 bytes); BYTES_JSON is the
    algorithmic byte count of every workload that the profile run wrote.
    Writes profiles/workloads_counters.txt and profiles/workloads_traffic.json."""
    import re
    bytes_json, trace_dir, fetch_dir, write_dir, sq_dir, cmdline = argv[:6]
    calib = float(1 << 28)
    trace, _ = _profile_dispatches(trace_dir)
    fetch, fcal = _profile_dispatches(fetch_dir, "FETCH_SIZE")
    write, wcal = _profile_dispatches(write_dir, "WRITE_SIZE")
    ff = calib / statistics.mean(fcal)
    fw = calib / statistics.mean(wcal)
    sq = {}
    if sq_dir != "-":
        import csv
        import glob
        f = glob.glob(os.path.join(sq_dir, "**", "*counter_collection.csv"), recursive=True)
        rows = list(csv.DictReader(open(f[0])))
        for cname in sorted({r["Counter_Name"] for r in rows}):
            got, _ = _profile_dispatches(sq_dir, cname)
            for n, (_, vals) in got.items():
                sq.setdefault(n, {})[cname] = statistics.mean(vals) / 1024   # raw counts
    alg = json.load(open(bytes_json))
    lines = [f"# rocprofv3 per-workload summary: kernel-only time and HBM traffic of every "
             f"benchmarked workload ({PROFILE_REPS} cold-cache launches each)",
             f"# command: {cmdline}",
             f"# kernel source hash: {kernel_hash()}",
             f"# counters scaled by the run's 256 MiB device copies: FETCH_SIZE x {ff:.4f}, "
             f"WRITE_SIZE x {fw:.4f}",
             "",
             "workload | kernel | median us | algorithmic MB | counter MB (fetch + write) | "
             "counter / algorithmic | effective GB/s | achieved GB/s (counters) | % of 8 TB/s"]
    result = {}
    for n, (kern, durs) in trace.items():
        med = statistics.median(durs)
        fb = statistics.mean(fetch[n][1]) * ff
        wb = statistics.mean(write[n][1]) * fw
        nb = alg[n]
        k = " + ".join(re.sub(r"\(.*", "", part.replace("(anonymous namespace)::", "")
                              .replace("void ", "")) for part in kern.split(" + "))
        result[n] = {"kernel": k, "median_us": round(med, 2), "algorithmic_bytes": nb,
                     "fetch_bytes": round(fb), "write_bytes": round(wb),
                     "traffic_bytes": round(fb + wb), "ratio": round((fb + wb) / nb, 4),
                     "effective_GBps": round(nb / med / 1e3, 1),
                     "achieved_GBps": round((fb + wb) / med / 1e3, 1)}
        if n in sq:
            result[n]["sq"] = {c: round(v, 1) for c, v in sq[n].items()}
        lines.append(f"{n} | {k} | {med:.2f} | {nb / 1e6:.2f} | {fb / 1e6:.2f} + {wb / 1e6:.2f} | "
                     f"{(fb + wb) / nb:.3f} | {nb / med / 1e3:.0f} | {(fb + wb) / med / 1e3:.0f} | "
                     f"{100 * nb / med / 1e3 / HBM_PEAK_GBS:.1f}")
    if sq:
        cols = sorted({c for v in sq.values() for c in v})
        lines += ["", "## SQ counters, mean per launch (raw counts)", "workload | " + " | ".join(cols)]
        for n in trace:
            lines.append(f"{n} | " + " | ".join(f"{sq.get(n, {}).get(c, float('nan')):.0f}"
                                               for c in cols))
    txt = os.path.join(ROOT, "profiles", "workloads_counters.txt")
    open(txt, "w").write("\n".join(lines) + "\n")
    json.dump({"kernel_hash": kernel_hash(), "command": cmdline,
               "fetch_calibration": round(ff, 4), "write_calibration": round(fw, 4),
               "workloads": result}, open(TRAFFIC_FILE, "w"), indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "summarize":
        summarize(sys.argv[2:])
    elif len(sys.argv) > 1 and sys.argv[1] == "summarize-trace":
        summarize_trace(sys.argv[2:])
    elif len(sys.argv) > 1 and sys.argv[1] == "summarize-set":
        summarize_set(sys.argv[2:])
    else:
        main()
