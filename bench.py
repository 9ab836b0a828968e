#!/usr/bin/env python3
"""Long-context fp8 latent-KV MLA decode benchmark on one MI355X.

Workload (the long-context split-T decode of colibri PR #300, "KV8
long-context CUDA", second commit): H=64 heads, kv_lora Lc=512, rope Rc=64,
T=262144 e4m3 rows + f32 scales resident in HBM, batch 1.  One layer-token =
quantize and append one fresh row at row T-1 (the shadow holds T-1 rows before
it) and attend all T rows: one split-T partial launch, whose workgroups that
own row T-1 quantize it in their prologue, then the log-sum-exp merge.

A step is one decode token through `--layers` independent layers (default 8,
1.22 GB of shadows, so the 256 MB Infinity Cache cannot hold the stream).  The
step is captured once as a HIP graph and replayed: 0.25 s of untimed replays
while the GPU clocks ramp up from idle, W untimed warm-up steps, then K timed
steps between synchronisations.  Inputs are seeded synthetic
N(0,1) rows and queries.

Prints one JSON line: value = ms per layer-token (lower is better), plus the
effective HBM rate of the fp8 KV stream, the roofline of the split-T partial
kernel (its own duration from HIP events recorded on its launch stream around
every launch in a separate eager pass), and the CPU oracle timed on a bounded
sample on this host.
"""
from __future__ import annotations

import argparse
import atexit
import json
import os
import re
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms/layer-token + achieved HBM GB/s (fp8 KV stream), MLA decode at T=262144"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 MFMA
SETTLE_S = 0.25  # untimed replays before the warm-up steps (GPU clock ramp)



def kernel_code_sha256(path: str) -> str:
    """SHA-256 of a kernel source's code: comments removed and whitespace runs
    collapsed, so that an edit to comments alone does not count as a change of
    the kernel the traffic counters were taken on."""
    import hashlib
    import re
    s = open(path).read()
    s = re.sub(r"/\*.*?\*/", "", s, flags=re.S)
    s = re.sub(r"//[^\n]*", "", s)
    return hashlib.sha256(" ".join(s.split()).encode()).hexdigest()

def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=None,
                    help="layers per step (default 8 for the decode, 16 for the indexer: "
                         "more bytes than the 256 MB Infinity Cache holds)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="heads of the CPU-oracle sample on all threads (full T, scaled to 64 "
                         "heads; also the heads of layer 0 checked against the oracle)")
    ap.add_argument("--cpu-heads-one-core", type=int, default=2,
                    help="heads of the one-thread CPU-oracle sample (full T, scaled)")
    ap.add_argument("--traffic", type=str,
                    default=os.path.join(ROOT, "profiles", "k_partial32_long_t262144_traffic.txt"),
                    help="calibrated rocprofv3 FETCH_SIZE + WRITE_SIZE bytes per partial launch "
                         "(JSON); used only while the kernel source still matches its hash")
    ap.add_argument("--workload", default="long_t262144",
                    choices=["long_t262144", "dsv3_t4096", "dsa_index_t131072_k2048",
                             "kvfile_t262144",
                             "mixed_t262144", "dsa_t131072_ns2048", "batch_s64_t32768"],
                    help="long_t262144: the fused append + split-T decode step (default); "
                         "dsv3_t4096: the same step at the DeepSeek-V3 shape (H=128, T=4096); "
                         "dsa_index_t131072_k2048: the fp8 indexer score + top-k; "
                         "kvfile_t262144: resume a persisted shadow file into device shadows; "
                         "mixed_t262144: the decode step over mixed rows (noPE e4m3 448 + RoPE "
                         "bf16 64); dsa_t131072_ns2048: the selected-row decode over 2048 "
                         "rows; batch_s64_t32768: the causal batch of 64 queries")
    ap.add_argument("--splits", type=int, default=0,
                    help="dsa_t131072_ns2048 and dsv3_t4096: force this many row chunks "
                         "(mla8_opts.n_splits) instead of the library's plan")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="long-context and causal-batch workloads: also sample the board's socket "
                         "power and GFX clocks (amd-smi) while the step replays (long context: and "
                         "while the stream-read kernel replays), each for SECONDS of wall time, "
                         "and at idle")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    return ap.parse_args()


def host_info():
    """What the CPU baseline ran on: logical CPUs, the ones this process may
    use, and the CPU model."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": model}


def cpu_baseline(w, heads, heads_one_core, runs=3):
    """The oracle (as it stands) on bounded samples of the same step: quantize
    the fresh row into row T-1, then dense fp64 attention over all T rows for
    `heads` heads with every OpenMP thread, and for `heads_one_core` heads on
    one thread; `runs` runs of each, the median scaled to the full 64-head
    layer-token.  The inputs are layer 0's (the same seeds as the GPU's layer
    0), so the all-threads run's outputs also check the GPU's layer-0 result.
    Returns (record, (out, lse) of heads 0 .. heads-1)."""
    import numpy as np

    import oracle
    from fp8_mla_latent_amd import workloads as W

    x = W.rows(w, w.t_rows, seed_offset=0)
    codes, scales = oracle.quantize_rows(x[:-1])
    codes = np.concatenate([codes, np.zeros((1, w.d), np.uint8)])
    scales = np.concatenate([scales, np.zeros(1, np.float32)])
    ql, qr = W.queries(w, seed_offset=0)

    def one(nh):
        t0 = time.perf_counter()
        c1, s1 = oracle.quantize_rows(x[-1:])
        codes[-1], scales[-1] = c1[0], s1[0]
        res = oracle.decode(codes, scales, w.t_rows, w.lc, w.rc, ql[:nh], qr[:nh], w.sm_scale)
        return time.perf_counter() - t0, res

    oracle.set_threads(0)
    threads = oracle.threads()
    t_all, res = [], None
    for _ in range(runs):
        dt, res = one(heads)
        t_all.append(dt)
    oracle.set_threads(1)
    try:
        t_one = [one(heads_one_core)[0] for _ in range(runs)]
    finally:
        oracle.set_threads(0)
    ms_all = float(np.median(t_all)) * 1e3 * (w.n_heads / heads)
    ms_one = float(np.median(t_one)) * 1e3 * (w.n_heads / heads_one_core)
    info = host_info()
    rec = {"value": round(ms_all, 3), "unit": "ms/layer-token", "cores": threads,
           "kind": "oracle",
           "sample": f"append 1 row + fp64 attention of {heads} of {w.n_heads} heads over "
                     f"T={w.t_rows} rows on {threads} OpenMP threads, median of {runs} runs "
                     f"({', '.join(f'{t:.2f}' for t in t_all)} s), scaled "
                     f"x{w.n_heads / heads:g} to all heads",
           "one_core": {"value": round(ms_one, 3), "unit": "ms/layer-token", "cores": 1,
                        "sample": f"{heads_one_core} of {w.n_heads} heads on 1 thread, median "
                                  f"of {runs} runs ({', '.join(f'{t:.2f}' for t in t_one)} s), "
                                  f"scaled x{w.n_heads / heads_one_core:g}"},
           **info}
    return rec, res


def settle(run, log_name):
    """Untimed replays for SETTLE_S of wall time (GPU clock ramp after idle)."""
    import torch
    t_set = time.perf_counter()
    n = 0
    while time.perf_counter() - t_set < SETTLE_S:
        for _ in range(10):
            run()
        torch.cuda.synchronize()
        n += 10
    log(f"clock settle: {n} untimed {log_name} in {time.perf_counter() - t_set:.3f} s")
    return n


def cpu_baseline_index(w, rows):
    """The oracle's indexer score + top-k on the first `rows` rows of one
    layer's keys, scaled to all T rows."""
    import numpy as np

    import oracle
    from fp8_mla_latent_amd import workloads as W

    keys = W.rows(w, rows)
    kc, ks = oracle.quantize_rows(keys)
    q = W.queries(w)[0]
    wt = W.index_weights(w)
    t0 = time.perf_counter()
    sc = oracle.index_scores(kc, ks, q, wt)
    oracle.index_topk(sc, w.n_sel)
    dt = time.perf_counter() - t0
    ms = dt * 1e3 * (w.t_rows / rows)
    return {"value": round(ms, 3), "unit": "ms/layer-token", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"fp64 indexer scores of {rows} of {w.t_rows} rows x {w.n_heads} heads "
                      f"+ top-{w.n_sel} ({dt:.2f} s), scaled x{w.t_rows / rows:g}"}


def bench_index(args):
    """fp8 indexer score + top-k (k_index_score dominant): one token through
    --layers layers, each with its own T=131072 x 128 e4m3 key cache."""
    import numpy as np
    import torch

    from fp8_mla_latent_amd import mla8 as m
    from fp8_mla_latent_amd import workloads as W

    w = W.DSA_INDEX
    L, K, WU = args.layers or 16, args.steps, args.warmup
    T = w.t_rows
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = []
    for l in range(L):
        x = torch.from_numpy(W.rows(w, T, seed_offset=l)).to(dev)
        kc, ks = m.mla8_quantize_rows(x, w.lc, 0)
        del x
        layers.append(dict(kc=kc, ks=ks,
                           q=torch.from_numpy(W.queries(w, seed_offset=l)[0]).to(dev),
                           w=torch.from_numpy(W.index_weights(w, seed_offset=l)).to(dev),
                           sel=torch.empty((w.n_sel,), dtype=torch.int32, device=dev)))
    ws = torch.empty(m.mla8_workspace_bytes(m.MLA8_OP_INDEX, T, w.n_heads, 1, w.lc),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"{L} layers of {T} e4m3 key rows quantized")

    def call(ly, events=None):
        m.mla8_index_topk(ly["kc"], ly["ks"], ly["q"], ly["w"], w.n_sel, sel=ly["sel"],
                          workspace=ws, events=events)

    def step():
        for ly in layers:
            call(ly)

    run, ms_step, n_settle, graph = _timed_steps(step, args)
    ms_lt = ms_step / L
    log(f"step {ms_step:.4f} ms ({L} layers), {ms_lt * 1e3:.2f} us/layer-token")
    durs = _event_pass(run, K, layers, call)
    k_us = float(np.mean(durs))
    key_bytes = T * (w.lc + 4)
    alg_bytes = key_bytes + w.n_heads * w.lc * 4 + w.n_heads * 4  # keys + scales, q, w
    achieved = alg_bytes / (k_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "k_index_score<4>", "kernel_us": round(k_us, 3),
                "kernel_us_p10_p90": [round(float(np.percentile(durs, 10)), 3),
                                      round(float(np.percentile(durs, 90)), 3)],
                "algorithmic_bytes": alg_bytes}
    log(f"score kernel {k_us:.2f} us mean -> {achieved:.0f} GB/s "
        f"({100 * achieved / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f})")
    for ly in layers:
        s = ly["sel"]
        assert bool(((s[1:] - s[:-1]) > 0).all()) and int(s.min()) >= 0 and int(s.max()) < T
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_index(w, 16384)
        log(f"cpu oracle: {cpu}")
    rec = {
        "metric": "ms/layer-token + achieved HBM GB/s (fp8 indexer keys), fp8 indexer score + "
                  "top-k at T=131072",
        "value": round(ms_lt, 6),
        "unit": "ms/layer-token",
        "n_gpus": 1,
        "steps": K,
        "warmup": WU,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 keys x e4m3 query (fp8 mfma), f32 scores; u32 radix top-k",
        "data": "synthetic: seeded N(0,1) keys and queries, N(0,1/64) head weights",
        "config": {"workload": w.name, "indexer_heads": w.n_heads, "index_dim": w.lc,
                   "t_rows": T, "top_k": w.n_sel, "batch": 1, "layers_per_step": L,
                   "launch": "hip graph" if graph is not None else "eager"},
        "key_stream_gb_per_s": round(key_bytes / (ms_lt * 1e-3) / 1e9, 1),
        "clock_settle": {"seconds": SETTLE_S, "untimed_steps": n_settle},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def _event_pass(run, K, layers, call):
    """Library-side HIP events around every partial-kernel launch of K eager
    steps (30 graph steps queued ahead so launches never wait for the GPU);
    returns the durations in us."""
    import numpy as np
    import torch

    from fp8_mla_latent_amd import mla8 as m

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K * len(layers))]
    for a_, b_ in evs:
        a_.record()
        b_.record()
    torch.cuda.synchronize()
    for _ in range(30):
        run()
    i = 0
    for _ in range(K):
        for ly in layers:
            call(ly, events=evs[i])
            i += 1
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs]) * 1e3


def _timed_steps(step, args):
    """Capture step as a HIP graph (unless --no-graph), settle the clocks, run
    the warm-up, then time K steps; returns (run, ms per step, settle count,
    graph or None)."""
    import torch

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    else:
        run = step
    n_settle = settle(run, "steps")
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return run, e0.elapsed_time(e1) / args.steps, n_settle, graph


def bench_dsa(args):
    """Selected-row (DSA gather) decode: per layer, mla8_decode_sel over 2048
    sorted unique rows of its own T=131072 shadow, H=64.  Latency-bound: the
    gathered rows are 1.19 MB."""
    import numpy as np
    import torch

    from fp8_mla_latent_amd import mla8 as m
    from fp8_mla_latent_amd import workloads as W

    w = W.DSA
    L, K = args.layers or 8, args.steps
    T, NS = w.t_rows, w.n_sel
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = []
    for l in range(L):
        x = torch.from_numpy(W.rows(w, T, seed_offset=l)).to(dev)
        codes, scales = m.mla8_quantize_rows(x, w.lc, w.rc)
        del x
        ql, qr = W.queries(w, seed_offset=l)
        layers.append(dict(codes=codes, scales=scales,
                           sel=torch.from_numpy(W.selection(w, seed_offset=l)).to(dev),
                           ql=torch.from_numpy(ql).to(dev), qr=torch.from_numpy(qr).to(dev),
                           out=torch.empty((w.n_heads, w.lc), dtype=torch.float32, device=dev),
                           lse=torch.empty((w.n_heads,), dtype=torch.float32, device=dev)))
    ws = torch.empty(m.mla8_workspace_bytes(m.MLA8_OP_DECODE_SEL, NS, w.n_heads, 1, w.lc,
                                            args.splits),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"{L} layers of {T} rows quantized, {NS} selected per layer")

    def call(ly, events=None):
        m.mla8_decode_sel(ly["codes"], ly["scales"], T, w.lc, w.rc, ly["sel"], ly["ql"], ly["qr"],
                          w.sm_scale, out=ly["out"], lse=ly["lse"], workspace=ws, events=events,
                          n_splits=args.splits)

    def step():
        for ly in layers:
            call(ly)

    run, ms_step, n_settle, graph = _timed_steps(step, args)
    ms_lt = ms_step / L
    log(f"step {ms_step:.4f} ms ({L} layers), {ms_lt * 1e3:.2f} us/layer-token")
    durs = _event_pass(run, K, layers, call)
    part_us = float(np.mean(durs))
    alg_bytes = NS * (w.d + 4) + NS * 4 + w.n_heads * w.d * 4  # gathered rows + scales, indices, q
    achieved = alg_bytes / (part_us * 1e-6) / 1e9
    log(f"partial kernel {part_us:.2f} us mean -> {achieved:.0f} GB/s")
    for ly in layers:
        assert torch.isfinite(ly["out"]).all() and torch.isfinite(ly["lse"]).all()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        x = W.rows(w, T, seed_offset=0)
        oc, os_ = oracle.quantize_rows(x)
        ql, qr = W.queries(w, seed_offset=0)
        sel = W.selection(w, seed_offset=0)
        t0 = time.perf_counter()
        oracle.decode_sel(oc, os_, T, w.lc, w.rc, sel, ql, qr, w.sm_scale)
        dt = time.perf_counter() - t0
        cpu = {"value": round(dt * 1e3, 3), "unit": "ms/layer-token", "cores": oracle.threads(),
               "kind": "oracle",
               "sample": f"fp64 attention of all {w.n_heads} heads over the {NS} selected rows "
                         f"of one layer ({dt:.3f} s)"}
        log(f"cpu oracle: {cpu}")
    rec = {
        "metric": "ms/layer-token, DSA selected-row decode (2048 of T=131072 rows)",
        "value": round(ms_lt, 6),
        "unit": "ms/layer-token",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 kv; scores e4m3->f16 rows x f16 hi q (f16 mfma) + e4m3 rows x e4m3 lo q "
                 "(scaled e4m3 mfma), context f16 weights x e4m3->f16 rows (f16 mfma); "
                 "f32 accumulate",
        "data": "synthetic: seeded N(0,1) rows and queries, sorted unique uniform selections",
        "config": {"workload": w.name, "heads": w.n_heads, "kv_lora": w.lc, "rope": w.rc,
                   "t_rows": T, "selected": NS, "batch": 1, "layers_per_step": L,
                   "launch": "hip graph" if graph is not None else "eager",
                   "splits": m.mla8_plan_splits(m.MLA8_OP_DECODE_SEL, NS, w.n_heads, 1,
                                                args.splits)},
        "clock_settle": {"seconds": SETTLE_S, "untimed_steps": n_settle},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_partial32<true, true, false>", "kernel_us": round(part_us, 3),
                     "algorithmic_bytes": alg_bytes,
                     "note": "latency-bound: 1.19 MB of gathered rows per launch"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def bench_dsv3(args):
    """DeepSeek-V3-shaped decode step: per layer, one mla8_append_decode call
    that quantizes the fresh row into row T-1 of its own shadow (T = 4096, 1 %
    of rows scaled x50) and attends all 4096 rows with H = 128 heads.  A 2.4 MB
    shadow per layer: MFMA- and launch-bound, not HBM-bound."""
    import numpy as np
    import torch

    from fp8_mla_latent_amd import mla8 as m
    from fp8_mla_latent_amd import workloads as W

    w = W.DSV3
    L, K = args.layers or 8, args.steps
    T = w.t_rows
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = []
    for l in range(L):
        x = torch.from_numpy(W.rows(w, T, seed_offset=l)).to(dev)
        codes = torch.empty((T, w.d), dtype=torch.uint8, device=dev)
        scales = torch.empty((T,), dtype=torch.float32, device=dev)
        assert m.mla8_append(codes, scales, 0, x[:T - 1], w.lc, w.rc) == T - 1
        fresh = x[T - 1:].clone()
        del x
        ql, qr = W.queries(w, seed_offset=l)
        layers.append(dict(codes=codes, scales=scales, fresh=fresh,
                           ql=torch.from_numpy(ql).to(dev), qr=torch.from_numpy(qr).to(dev),
                           out=torch.empty((w.n_heads, w.lc), dtype=torch.float32, device=dev),
                           lse=torch.empty((w.n_heads,), dtype=torch.float32, device=dev)))
    ws = torch.empty(m.mla8_workspace_bytes(m.MLA8_OP_DECODE, T, w.n_heads, 1, w.lc, args.splits),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"{L} layers of {T - 1} rows quantized")

    def call(ly, events=None):
        m.mla8_append_decode(ly["codes"], ly["scales"], T - 1, ly["fresh"], w.lc, w.rc,
                             ly["ql"], ly["qr"], w.sm_scale, out=ly["out"], lse=ly["lse"],
                             workspace=ws, events=events, n_splits=args.splits)

    def step():
        for ly in layers:
            call(ly)

    run, ms_step, n_settle, graph = _timed_steps(step, args)
    ms_lt = ms_step / L
    log(f"step {ms_step:.4f} ms ({L} layers), {ms_lt * 1e3:.2f} us/layer-token")
    durs = _event_pass(run, K, layers, call)
    part_us = float(np.mean(durs))
    # the method's flops, one pass per product: scores over D, context over Lc
    flops = 2.0 * w.n_heads * T * (w.d + w.lc)
    tflops = flops / (part_us * 1e-6) / 1e12
    log(f"partial kernel {part_us:.2f} us mean -> {tflops:.0f} TFLOP/s")
    for ly in layers:
        assert torch.isfinite(ly["out"]).all() and torch.isfinite(ly["lse"]).all()
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        import oracle
        x = W.rows(w, T, seed_offset=0)
        oc, os_ = oracle.quantize_rows(x)
        ql, qr = W.queries(w, seed_offset=0)
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            ro, rl = oracle.decode(oc, os_, T, w.lc, w.rc, ql, qr, w.sm_scale)
            times.append(time.perf_counter() - t0)
        dt = float(np.median(times))
        cpu = {"value": round(dt * 1e3, 3), "unit": "ms/layer-token", "cores": oracle.threads(),
               "kind": "oracle",
               "sample": f"fp64 attention of all {w.n_heads} heads over the {T} rows of one "
                         f"layer, median of 3 runs", **host_info()}
        log(f"cpu oracle: {cpu}")
        # layer 0 against the oracle (outlier rows: the per-vector reading)
        g = layers[0]["out"].double().cpu().numpy()
        err = np.abs(g - ro).max(1)
        bar = 1e-4 + 2e-3 * np.abs(ro).max(1)
        parity = {"layer": 0, "heads_checked": w.n_heads,
                  "worst_err_over_bar": round(float((err / bar).max()), 4),
                  "form": "per (head) output vector", "ok": bool(np.all(err <= bar))}
        log(f"layer-0 parity vs oracle: {parity}")
        if not parity["ok"]:
            raise SystemExit(f"bench.py: layer-0 output differs from the oracle: {parity}")
    rec = {
        "metric": "ms/layer-token, DeepSeek-V3-shaped decode (H=128, T=4096)",
        "value": round(ms_lt, 6),
        "unit": "ms/layer-token",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 kv; scores e4m3->f16 rows x f16 hi q (f16 mfma) + e4m3 rows x e4m3 lo q "
                 "(scaled e4m3 mfma), context f16 weights x e4m3->f16 rows (f16 mfma); f32 accumulate",
        "data": "synthetic: seeded N(0,1) rows (1 % of rows x50) and queries",
        "config": {"workload": w.name, "heads": w.n_heads, "kv_lora": w.lc, "rope": w.rc,
                   "t_rows": T, "batch": 1, "layers_per_step": L,
                   "launch": "hip graph" if graph is not None else "eager",
                   "splits": m.mla8_plan_splits(m.MLA8_OP_DECODE, T, w.n_heads, 1, args.splits)},
        "clock_settle": {"seconds": SETTLE_S, "untimed_steps": n_settle},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "k_partial32<true, false, false>", "kernel_us": round(part_us, 3),
                     "algorithmic_flops": flops},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(rec), flush=True)


def bench_batch(args, sampler=None):
    """Causal batch (prefill / streaming): per layer, append 64 fresh rows at
    pos0 = 32704 of its own shadow (T = 32768), then mla8_batch with S = 64
    queries, query s attending rows [0, pos0 + s], H = 64.  MFMA-bound."""
    import numpy as np
    import torch

    from fp8_mla_latent_amd import mla8 as m
    from fp8_mla_latent_amd import workloads as W

    w = W.BATCH
    L, K = args.layers or 8, args.steps
    T, S = w.t_rows, w.n_q
    pos0 = T - w.n_append
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = []
    for l in range(L):
        x = torch.from_numpy(W.rows(w, T, seed_offset=l)).to(dev)
        codes = torch.empty((T, w.d), dtype=torch.uint8, device=dev)
        scales = torch.empty((T,), dtype=torch.float32, device=dev)
        assert m.mla8_append(codes, scales, 0, x[:pos0], w.lc, w.rc) == pos0
        fresh = x[pos0:].clone()
        del x
        ql, qr = W.queries(w, seed_offset=l)
        layers.append(dict(codes=codes, scales=scales, fresh=fresh,
                           ql=torch.from_numpy(ql).to(dev), qr=torch.from_numpy(qr).to(dev),
                           out=torch.empty((S, w.n_heads, w.lc), dtype=torch.float32, device=dev),
                           lse=torch.empty((S, w.n_heads), dtype=torch.float32, device=dev)))
    ws = torch.empty(m.mla8_workspace_bytes(m.MLA8_OP_BATCH, T, w.n_heads, S, w.lc),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"{L} layers of {pos0} rows quantized; {S} fresh rows appended per step")

    def attend(ly, events=None):
        m.mla8_batch(ly["codes"], ly["scales"], T, w.lc, w.rc, ly["ql"], ly["qr"], pos0,
                     w.sm_scale, out=ly["out"], lse=ly["lse"], workspace=ws, events=events)

    def step():
        for ly in layers:
            m.mla8_append(ly["codes"], ly["scales"], pos0, ly["fresh"], w.lc, w.rc)
            attend(ly)

    run, ms_step, n_settle, graph = _timed_steps(step, args)
    ms_layer = ms_step / L
    log(f"step {ms_step:.4f} ms ({L} layers), {ms_layer * 1e3:.1f} us/layer, "
        f"{ms_layer * 1e3 / S:.2f} us/layer-token")
    durs = _event_pass(run, K, layers, attend)
    part_us = float(np.mean(durs))
    # algorithmic flops of the method (one pass per product): every query-head
    # scores its rows (2 D flops each) and accumulates them (2 Lc flops each)
    rows_attended = sum(pos0 + s + 1 for s in range(S))
    alg_flops = w.n_heads * rows_attended * (2 * w.d + 2 * w.lc)
    achieved = alg_flops / (part_us * 1e-6) / 1e12
    log(f"partial kernel {part_us:.1f} us mean -> {achieved:.0f} TFLOP/s "
        f"({100 * achieved / MFMA_F16_PEAK_TFLOPS:.1f}% of {MFMA_F16_PEAK_TFLOPS:.0f})")
    for ly in layers:
        assert torch.isfinite(ly["out"]).all() and torch.isfinite(ly["lse"]).all()
    power = None
    if sampler is not None:
        # board power and clocks: idle, then the step's graph replayed
        torch.cuda.synchronize()
        t_idle = time.time()
        time.sleep(3.0)
        idle_win = (t_idle + 1.0, time.time())
        step_win, n_steps = power_run(run, args.power)
        samples = sampler.stop()
        step_s = step_win[1] - step_win[0] + 1.0
        power = {"sampler": PowerSampler.CMD,
                 "idle": power_window(samples, *idle_win),
                 "step": dict(power_window(samples, *step_win), replays=n_steps,
                              us_per_layer_token=round(step_s / (n_steps * L * S) * 1e6, 3))}
        log(f"power: {power}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nq = 4
        x = W.rows(w, T, seed_offset=0)
        oc, os_ = oracle.quantize_rows(x)
        ql, qr = W.queries(w, seed_offset=0)
        t0 = time.perf_counter()
        oracle.batch(oc, os_, T, w.lc, w.rc, np.ascontiguousarray(ql[:nq]),
                     np.ascontiguousarray(qr[:nq]), pos0, w.sm_scale)
        dt = time.perf_counter() - t0
        cpu = {"value": round(dt * 1e3 / nq, 3), "unit": "ms/layer-token",
               "cores": oracle.threads(), "kind": "oracle",
               "sample": f"fp64 causal attention of {nq} of the {S} queries (all {w.n_heads} "
                         f"heads, about {pos0} rows each; {dt:.2f} s), per query-token"}
        log(f"cpu oracle: {cpu}")
    rec = {
        "metric": "ms/layer-token, causal batch (S=64 queries at T=32768) incl. the 64-row append",
        "value": round(ms_layer / S, 6),
        "unit": "ms/layer-token",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 kv; scores e4m3->f16 rows x f16 hi q (f16 mfma) + e4m3 rows x e4m3 lo q "
                 "(scaled e4m3 mfma), context f16 weights x e4m3->f16 rows (f16 mfma); "
                 "f32 accumulate",
        "data": "synthetic: seeded N(0,1) rows and queries",
        "config": {"workload": w.name, "heads": w.n_heads, "kv_lora": w.lc, "rope": w.rc,
                   "t_rows": T, "queries": S, "pos0": pos0, "layers_per_step": L,
                   "launch": "hip graph" if graph is not None else "eager"},
        "ms_per_layer_batch": round(ms_layer, 6),
        "clock_settle": {"seconds": SETTLE_S, "untimed_steps": n_settle},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "k_partial32<true, false, false>", "kernel_us": round(part_us, 3),
                     "algorithmic_flops": alg_flops,
                     "note": "flops of one pass per product; the hi and lo query terms take "
                             "1.5x the matrix-pipe time of one fp16 pass over the scores"},
        "cpu_baseline": cpu,
    }
    if power is not None:
        rec["power"] = power
    print(json.dumps(rec), flush=True)


def cpu_baseline_mixed(w, lc, rc, heads):
    """The oracle on mixed rows: quantize one fresh row, then fp64 attention of
    `heads` heads over all T rows, scaled to every head."""
    import numpy as np

    import oracle
    from fp8_mla_latent_amd import workloads as W

    x = np.ascontiguousarray(W.rows(w, w.t_rows, seed_offset=0)[:, :lc + rc])
    rows, scales = oracle.quantize_rows_mx(x, lc, rc)
    ql, qr = W.queries(w, seed_offset=0)
    ql = np.ascontiguousarray(ql[:heads, :lc])
    t0 = time.perf_counter()
    r1, s1 = oracle.quantize_rows_mx(x[-1:], lc, rc)
    rows[-1], scales[-1] = r1[0], s1[0]
    oracle.decode_mx(rows, scales, w.t_rows, lc, rc, ql, qr[:heads], w.sm_scale)
    dt = time.perf_counter() - t0
    ms = dt * 1e3 * (w.n_heads / heads)
    return {"value": round(ms, 3), "unit": "ms/layer-token", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"append 1 mixed row + fp64 attention of {heads} of {w.n_heads} heads over "
                      f"T={w.t_rows} rows ({dt:.2f} s), scaled x{w.n_heads / heads:g} to all heads"}


def bench_mixed(args):
    """Decode step over mixed rows (448 noPE values e4m3 + 64 RoPE values bf16,
    576 bytes + scale per row), H=64, T=262144: append one row, attend all."""
    import numpy as np
    import torch

    from fp8_mla_latent_amd import mla8 as m
    from fp8_mla_latent_amd import workloads as W

    w = W.LONG
    LC, RC = 448, 64
    L, K, WU = args.layers or 8, args.steps, args.warmup
    T = w.t_rows
    RB = LC + 2 * RC
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = []
    for l in range(L):
        x = torch.from_numpy(np.ascontiguousarray(W.rows(w, T, seed_offset=l)[:, :LC + RC])).to(dev)
        rows = torch.empty((T, RB), dtype=torch.uint8, device=dev)
        scales = torch.empty((T,), dtype=torch.float32, device=dev)
        assert m.mla8_append_mx(rows, scales, 0, x[:T - 1], LC, RC) == T - 1
        fresh = x[T - 1:].clone()
        del x
        ql, qr = W.queries(w, seed_offset=l)
        layers.append(dict(rows=rows, scales=scales, fresh=fresh,
                           ql=torch.from_numpy(np.ascontiguousarray(ql[:, :LC])).to(dev),
                           qr=torch.from_numpy(qr).to(dev),
                           out=torch.empty((w.n_heads, LC), dtype=torch.float32, device=dev),
                           lse=torch.empty((w.n_heads,), dtype=torch.float32, device=dev)))
    ws = torch.empty(m.mla8_workspace_bytes(m.MLA8_OP_DECODE, T, w.n_heads, 1, LC),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"{L} layers of {T - 1} mixed rows quantized")

    def call(ly, events=None):
        m.mla8_append_decode_mx(ly["rows"], ly["scales"], T - 1, ly["fresh"], LC, RC, ly["ql"],
                                ly["qr"], w.sm_scale, out=ly["out"], lse=ly["lse"],
                                workspace=ws, events=events)

    def step():
        for ly in layers:
            call(ly)

    run, ms_step, n_settle, graph = _timed_steps(step, args)
    ms_lt = ms_step / L
    log(f"step {ms_step:.4f} ms ({L} layers), {ms_lt * 1e3:.2f} us/layer-token")
    durs = _event_pass(run, K, layers, call)
    part_us = float(np.mean(durs))
    row_bytes = T * (RB + 4)
    alg_bytes = row_bytes + w.n_heads * (LC + RC) * 4
    achieved = alg_bytes / (part_us * 1e-6) / 1e9
    for ly in layers:
        assert torch.isfinite(ly["out"]).all() and torch.isfinite(ly["lse"]).all()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_mixed(w, LC, RC, args.cpu_heads)
        log(f"cpu oracle: {cpu}")
    rec = {
        "metric": "ms/layer-token + achieved HBM GB/s (mixed fp8/bf16 rows), MLA decode at "
                  "T=262144",
        "value": round(ms_lt, 6),
        "unit": "ms/layer-token",
        "n_gpus": 1,
        "steps": K,
        "warmup": WU,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 noPE + bf16 RoPE rows; scores e4m3->f16 x f16 hi q (f16 mfma) + e4m3 x "
                 "e4m3 lo q (scaled e4m3 mfma) + bf16 x 2-term bf16 q (bf16 mfma), context f16 "
                 "weights x e4m3->f16 (f16 mfma); f32 accumulate",
        "data": "synthetic: seeded N(0,1) rows and queries",
        "config": {"workload": "mixed_t262144", "heads": w.n_heads, "nope": LC, "rope": RC,
                   "t_rows": T, "batch": 1, "layers_per_step": L,
                   "launch": "hip graph" if graph is not None else "eager"},
        "kv_stream_gb_per_s": round(row_bytes / (ms_lt * 1e-3) / 1e9, 1),
        "clock_settle": {"seconds": SETTLE_S, "untimed_steps": n_settle},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_partial32<true, false, true>", "kernel_us": round(part_us, 3),
                     "algorithmic_bytes": alg_bytes},
        "cpu_baseline": cpu,
    }
    log(f"partial kernel {part_us:.2f} us mean -> {achieved:.0f} GB/s")
    print(json.dumps(rec), flush=True)


def bench_kvfile(args):
    """Persistent shadow file: append one token per layer (latency) and resume
    a T=262144 file into device shadows (throughput).  Host file I/O through
    the page cache plus pageable host-to-device copies; no GPU kernel."""
    import tempfile

    import numpy as np
    import torch

    from fp8_mla_latent_amd import mla8 as m
    from fp8_mla_latent_amd import workloads as W

    w = W.LONG
    L, T, D = args.layers or 4, w.t_rows, w.d
    dev = torch.device("cuda:0")
    codes, scales = [], []
    for l in range(L):
        x = torch.from_numpy(W.rows(w, T, seed_offset=l)).to(dev)
        c, sc = m.mla8_quantize_rows(x, w.lc, w.rc)
        del x
        codes.append(c)
        scales.append(sc)
    torch.cuda.synchronize()
    tmpdir = tempfile.mkdtemp(prefix="mla8kv_", dir=os.environ.get("TMPDIR", "/tmp"))
    path = os.path.join(tmpdir, "shadow.mla8kv")
    try:
        m.mla8_kvfile_create(path, L, w.lc, w.rc)
        t0 = time.perf_counter()
        m.mla8_kvfile_append(path, codes, scales, 0, T - 64, w.lc, w.rc)
        t_bulk = time.perf_counter() - t0
        lat = []
        for t in range(T - 64, T):  # one token (all layers) per call, as a decode loop would
            t1 = time.perf_counter()
            m.mla8_kvfile_append(path, codes, scales, t, 1, w.lc, w.rc)
            lat.append(time.perf_counter() - t1)
        file_bytes = os.path.getsize(path)
        c2 = [torch.empty_like(c) for c in codes]
        s2 = [torch.empty_like(sc) for sc in scales]
        loads = []
        for _ in range(max(args.steps // 10, 3)):
            t1 = time.perf_counter()
            assert m.mla8_kvfile_load(path, c2, s2, w.lc, w.rc) == T
            loads.append(time.perf_counter() - t1)
        for l in range(L):
            assert torch.equal(c2[l], codes[l]) and torch.equal(s2[l], scales[l])
    finally:
        for f in os.listdir(tmpdir):
            os.unlink(os.path.join(tmpdir, f))
        os.rmdir(tmpdir)
    body = L * T * (D + 4)
    load_s = float(np.median(loads))
    rec = {
        "metric": "GB/s shadow-file resume into device shadows (T=262144), us per appended token",
        "value": round(body / load_s / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": len(loads),
        "warmup": 0,
        "ms_per_step": round(load_s * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 rows + f32 scales (bytes copied as stored)",
        "data": "synthetic: seeded N(0,1) rows quantized on the GPU",
        "config": {"workload": "kvfile_t262144", "layers": L, "t_rows": T, "row_bytes": D + 4,
                   "file_bytes": file_bytes},
        "append_us_per_token": {"median": round(float(np.median(lat)) * 1e6, 1),
                                "p90": round(float(np.percentile(lat, 90)) * 1e6, 1)},
        "bulk_append_gb_per_s": round(L * (T - 64) * (D + 4) / t_bulk / 1e9, 3),
        "roofline": None,
        "cpu_baseline": None,
        "note": "host I/O path (page cache, fdatasync per commit, pageable copies); "
                "no device kernel, so no roofline",
    }
    log(f"resume {load_s * 1e3:.1f} ms for {body / 1e6:.0f} MB; append median "
        f"{rec['append_us_per_token']['median']} us/token")
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the split-T path would shard rows across GPUs with one all-gather of partials; "
              "that exchange is not built)", file=sys.stderr)
        sys.exit(2)

    sampler = (PowerSampler() if args.power > 0
               and args.workload in ("long_t262144", "batch_s64_t32768") else None)

    import numpy as np
    import torch

    if args.calibrate_copy:
        # A plain copy kernel of known size: 1 GiB read + 1 GiB written per
        # launch (an elementwise kernel, so the counter collection sees it; a
        # same-dtype copy_ would go to the DMA engines).  rocprofv3
        # FETCH_SIZE / WRITE_SIZE of this kernel calibrate the same counters
        # taken on the attention kernels.
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": max(args.steps, 1)}))
        return

    if args.workload == "dsa_index_t131072_k2048":
        bench_index(args)
        return
    if args.workload == "kvfile_t262144":
        bench_kvfile(args)
        return
    if args.workload == "dsa_t131072_ns2048":
        bench_dsa(args)
        return
    if args.workload == "dsv3_t4096":
        bench_dsv3(args)
        return
    if args.workload == "batch_s64_t32768":
        bench_batch(args, sampler)
        return
    if args.workload == "mixed_t262144":
        bench_mixed(args)
        return

    from fp8_mla_latent_amd import mla8 as m
    from fp8_mla_latent_amd import workloads as W

    w = W.LONG
    L, K, WU = args.layers or 8, args.steps, args.warmup
    T, D = w.t_rows, w.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- setup (untimed): L layer shadows of T-1 rows, quantized on the GPU
    layers = []
    for l in range(L):
        x = torch.from_numpy(W.rows(w, T, seed_offset=l)).to(dev)
        codes = torch.empty((T, D), dtype=torch.uint8, device=dev)
        scales = torch.empty((T,), dtype=torch.float32, device=dev)
        t = m.mla8_append(codes, scales, 0, x[:T - 1], w.lc, w.rc)
        assert t == T - 1
        fresh = x[T - 1:].clone()
        del x
        ql, qr = W.queries(w, seed_offset=l)
        layers.append(dict(codes=codes, scales=scales, fresh=fresh,
                           ql=torch.from_numpy(ql).to(dev), qr=torch.from_numpy(qr).to(dev),
                           out=torch.empty((w.n_heads, w.lc), dtype=torch.float32, device=dev),
                           lse=torch.empty((w.n_heads,), dtype=torch.float32, device=dev)))
        log(f"layer {l}: {T - 1} rows quantized")
    ws_bytes = m.mla8_workspace_bytes(m.MLA8_OP_DECODE, T, w.n_heads, 1, w.lc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        for ly in layers:
            m.mla8_append_decode(ly["codes"], ly["scales"], T - 1, ly["fresh"], w.lc, w.rc,
                                 ly["ql"], ly["qr"], w.sm_scale, out=ly["out"],
                                 lse=ly["lse"], workspace=ws)

    # ---- main measurement: K steps (graph replay unless --no-graph)
    for _ in range(max(WU, 1)):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    else:
        run = step
    # Clock settle (untimed): after an idle period the GPU needs tens of
    # milliseconds of load before its clocks reach their steady state (measured
    # here: the first 40 ms of replays run ~20% slower), so the step is
    # replayed for SETTLE_S of wall time before the W warm-up steps.
    n_settle = settle(run, "steps")
    for _ in range(WU):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(K):
        run()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / K
    ms_lt = ms_step / L
    kv_bytes = T * (D + 4)
    log(f"step {ms_step:.4f} ms ({L} layers), {ms_lt * 1e3:.2f} us/layer-token, "
        f"wall {t_wall:.3f} s")

    # ---- partial-kernel duration: HIP events recorded by the library around
    # every split-T partial launch, on the launch stream, eager pass of K steps
    # queued behind graph replays
    n_ev = K * L
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_ev)]
    for a_, b_ in evs:  # torch creates the hipEvent on first record
        a_.record()
        b_.record()
    torch.cuda.synchronize()
    # Queue 30 graph steps (~17 ms of GPU work) ahead of the eager pass, so that
    # the host's launches stay ahead of the GPU and each event pair brackets
    # the kernel, not the wait for the host's next launch.
    for _ in range(30):
        run()
    i = 0
    for _ in range(K):
        for ly in layers:
            m.mla8_append_decode(ly["codes"], ly["scales"], T - 1, ly["fresh"], w.lc,
                                 w.rc, ly["ql"], ly["qr"], w.sm_scale, out=ly["out"],
                                 lse=ly["lse"], workspace=ws, events=evs[i])
            i += 1
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3  # us
    part_us = float(np.mean(durs))
    # fp8 rows + scales, f32 query, the fresh f32 row read and its code + scale written
    alg_bytes = kv_bytes + w.n_heads * D * 4 + D * 4 + (D + 4)
    achieved = alg_bytes / (part_us * 1e-6) / 1e9
    traffic = None
    if args.traffic and os.path.exists(args.traffic):
        rec = json.load(open(args.traffic))
        src = os.path.join(ROOT, "fp8_mla_latent_amd", "csrc", "mla8_partial32.hip")
        if rec.get("kernel_code_sha256") == kernel_code_sha256(src):
            traffic = rec.get("bytes_per_launch")
        else:
            log("traffic counters were taken on other kernel code: reporting null")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_partial32<true, false, false>", "kernel_us": round(part_us, 3),
                "kernel_us_p10_p90": [round(float(np.percentile(durs, 10)), 3),
                                      round(float(np.percentile(durs, 90)), 3)],
                "algorithmic_bytes": alg_bytes}
    log(f"partial kernel {part_us:.2f} us mean -> {achieved:.0f} GB/s "
        f"({100 * achieved / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f})")

    # every layer's output finite; layer 0 against the oracle below
    for ly in layers:
        assert torch.isfinite(ly["out"]).all() and torch.isfinite(ly["lse"]).all()

    f32s = time_f32_scores(m, w, layers, ws, T, K, WU, args.no_graph)
    log(f"f32_scores path: {f32s}")

    ceiling = stream_ceiling([ly["codes"] for ly in layers])
    log(f"stream-read ceiling {ceiling['gb_per_s']:.0f} GB/s; the partial kernel reaches "
        f"{100 * achieved / ceiling['gb_per_s']:.1f}% of it")

    power = None
    if sampler is not None:
        # board power and clocks: idle, then the step's graph replayed, then
        # the stream-read kernel over the same shadows replayed
        torch.cuda.synchronize()
        t_idle = time.time()
        time.sleep(3.0)
        idle_win = (t_idle + 1.0, time.time())
        step_win, n_steps = power_run(run, args.power)
        out_sr = torch.empty((m.MLA8_STREAM_WORDS,), dtype=torch.int32, device=dev)

        def sread():
            for ly in layers:
                m.mla8_stream_read(ly["codes"], out_sr)

        sr_win, n_sr = power_run(sread, args.power)
        samples = sampler.stop()
        sampler = None
        step_s = step_win[1] - step_win[0] + 1.0
        sr_s = sr_win[1] - sr_win[0] + 1.0
        power = {"sampler": PowerSampler.CMD,
                 "idle": power_window(samples, *idle_win),
                 "step": dict(power_window(samples, *step_win), replays=n_steps,
                              us_per_layer_token=round(step_s / (n_steps * L) * 1e6, 2)),
                 "stream_read": dict(power_window(samples, *sr_win), passes=n_sr,
                                     gb_per_s=round(n_sr * L * T * D / sr_s / 1e9, 1))}
        log(f"power: {power}")

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, (ro, rl) = cpu_baseline(w, args.cpu_heads, args.cpu_heads_one_core)
        log(f"cpu oracle: {cpu}")
        # layer 0's last step against the oracle on the same inputs, elementwise
        # (|gpu - ref| <= 1e-4 + 2e-3 |ref|), for the heads the oracle ran
        g = layers[0]["out"][:args.cpu_heads].double().cpu().numpy()
        gl = layers[0]["lse"][:args.cpu_heads].double().cpu().numpy()
        ratio = float((np.abs(g - ro) / (1e-4 + 2e-3 * np.abs(ro))).max())
        lratio = float((np.abs(gl - rl) / (1e-4 + 2e-3 * np.abs(rl))).max())
        parity = {"layer": 0, "heads_checked": args.cpu_heads,
                  "worst_err_over_bar": round(ratio, 4), "lse_worst_err_over_bar":
                  round(lratio, 4), "ok": ratio <= 1.0 and lratio <= 1.0}
        log(f"layer-0 parity vs oracle: {parity}")
        if not parity["ok"]:
            raise SystemExit(f"bench.py: layer-0 output differs from the oracle: {parity}")

    rec = {
        "metric": METRIC,
        "value": round(ms_lt, 6),
        "unit": "ms/layer-token",
        "n_gpus": 1,
        "steps": K,
        "warmup": WU,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 kv; scores e4m3->f16 rows x f16 hi q (f16 mfma) + e4m3 rows x e4m3 lo q (scaled e4m3 mfma), context f16 weights x e4m3->f16 rows (f16 mfma); f32 accumulate",
        "data": "synthetic: seeded N(0,1) rows and queries",
        "config": {"workload": w.name, "heads": w.n_heads, "kv_lora": w.lc, "rope": w.rc,
                   "t_rows": T, "batch": 1, "layers_per_step": L,
                   "launch": "hip graph" if graph is not None else "eager",
                   "splits": m.mla8_plan_splits(m.MLA8_OP_DECODE, T, w.n_heads)},
        "kv_stream_gb_per_s": round(kv_bytes / (ms_lt * 1e-3) / 1e9, 1),
        "clock_settle": {"seconds": SETTLE_S, "untimed_steps": n_settle},
        "roofline": roofline,
        "stream_ceiling": dict(ceiling, kernel_frac=round(achieved / ceiling["gb_per_s"], 4)),
        "cpu_baseline": cpu,
        "parity": parity,
        "f32_scores": f32s,
    }
    if power is not None:
        rec["power"] = power
    print(json.dumps(rec), flush=True)


def time_f32_scores(m, w, layers, ws, T, K, WU, no_graph):
    """The same step with mla8_opts.f32_scores (the query's lo term as fp16 on
    the fp16 MFMA instead of e4m3 on the e4m3 MFMA: scores of f32 grade):
    step time per layer-token and the partial kernel's mean duration (library
    events, eager pass).  Reported beside the headline value (the default)."""
    import numpy as np
    import torch

    def step():
        for ly in layers:
            m.mla8_append_decode(ly["codes"], ly["scales"], T - 1, ly["fresh"], w.lc, w.rc,
                                 ly["ql"], ly["qr"], w.sm_scale, out=ly["out"],
                                 lse=ly["lse"], workspace=ws, f32_scores=True)

    for _ in range(max(WU, 1)):
        step()
    torch.cuda.synchronize()
    run = step
    if not no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    settle(run, "f32_scores steps")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms_lt = e0.elapsed_time(e1) / K / len(layers)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K * len(layers))]
    for a_, b_ in evs:
        a_.record()
        b_.record()
    torch.cuda.synchronize()
    for _ in range(30):
        run()
    i = 0
    for _ in range(K):
        for ly in layers:
            m.mla8_append_decode(ly["codes"], ly["scales"], T - 1, ly["fresh"], w.lc, w.rc,
                                 ly["ql"], ly["qr"], w.sm_scale, out=ly["out"],
                                 lse=ly["lse"], workspace=ws, events=evs[i], f32_scores=True)
            i += 1
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    for ly in layers:
        assert torch.isfinite(ly["out"]).all() and torch.isfinite(ly["lse"]).all()
    return {"ms_per_layer_token": round(ms_lt, 6), "kernel": "k_partial32<false, false, false>",
            "kernel_us": round(float(np.mean(durs)), 3),
            "note": "mla8_opts.f32_scores: the query's lo term as fp16 on the fp16 MFMA "
                    "(scores of f32 grade); not the headline"}


class PowerSampler:
    """A child shell, started before this process touches the GPU, that runs
    `amd-smi metric -p -c` (socket power, per-XCD GFX clocks) back to back,
    each sample stamped with the wall time it was taken at, until stop()."""

    CMD = "amd-smi metric -p -c"

    def __init__(self):
        fd, self.path = tempfile.mkstemp(prefix="mla8_power_", suffix=".txt")
        os.close(fd)
        self.flag = self.path + ".run"
        open(self.flag, "w").close()
        # the loop also ends when this process has gone
        loop = (f'while [ -e "{self.flag}" ] && kill -0 $PPID 2>/dev/null; do '
                f'echo "SAMPLE $(date +%s.%N)"; {self.CMD} 2>&1; sleep 0.2; done')
        self.out = open(self.path, "w")
        self.proc = subprocess.Popen(["bash", "-c", loop], stdout=self.out,
                                     stderr=subprocess.STDOUT)
        atexit.register(self._end)

    def _end(self):
        if os.path.exists(self.flag):
            os.remove(self.flag)

    def stop(self):
        self._end()
        try:
            self.proc.wait(timeout=30)
        except subprocess.TimeoutExpired:
            self.proc.kill()
            self.proc.wait()
        self.out.close()
        text = open(self.path).read()
        os.remove(self.path)
        return parse_power_samples(text)


def parse_power_samples(text):
    """(wall time, socket W, mean GFX MHz or None) per sample of the
    sampler's output: blocks that open with 'SAMPLE <unix time>'; a block
    without a socket power reading is dropped."""
    samples = []
    for blk in text.split("SAMPLE ")[1:]:
        head, _, body = blk.partition("\n")
        pw = re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", body)
        clk = [float(c) for c in re.findall(r"GFX_\d+:\s*CLK:\s*([0-9.]+)\s*MHz", body)]
        try:
            t = float(head.strip())
        except ValueError:
            continue
        if pw:
            samples.append((t, float(pw[0]), sum(clk) / len(clk) if clk else None))
    return samples


def power_window(samples, t0, t1):
    """Median socket power and mean GFX clock of the samples taken in [t0, t1]."""
    import numpy as np
    sel = [s for s in samples if t0 <= s[0] <= t1]
    if not sel:
        return {"samples": 0}
    clk = [s[2] for s in sel if s[2] is not None]
    return {"samples": len(sel), "socket_w_median": float(np.median([s[1] for s in sel])),
            "socket_w_max": max(s[1] for s in sel),
            "gfx_mhz_mean": round(float(np.mean(clk)), 1) if clk else None}


def power_run(fn, seconds):
    """Run fn() back to back for `seconds` of wall time; return the window
    (start + 1 s, so that the clocks have settled, to the end) and the calls."""
    import torch
    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        n += 20
    return (t0 + 1.0, time.time()), n


def stream_ceiling(bufs, passes=10):
    """The achievable-HBM line: mla8_stream_read over the same layer shadows
    (every 16-byte word loaded once per pass, coalesced), timed with events
    over `passes` passes after one untimed pass."""
    import torch

    from fp8_mla_latent_amd import mla8 as m

    out = torch.empty((m.MLA8_STREAM_WORDS,), dtype=torch.int32, device=bufs[0].device)
    for b in bufs:
        m.mla8_stream_read(b, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(passes):
        for b in bufs:
            m.mla8_stream_read(b, out)
    e1.record()
    torch.cuda.synchronize()
    nbytes = sum(b.numel() * b.element_size() for b in bufs)
    gbs = passes * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    return {"gb_per_s": round(gbs, 1), "bytes_per_pass": nbytes, "passes": passes,
            "kernel": "k_stream_read (mla8_stream_read): 16-byte coalesced loads, XOR-folded per wave"}


if __name__ == "__main__":
    main()
