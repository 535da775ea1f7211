"""Benchmark of the MoE-VQ routed-expert step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config b1|b32|b8mx|p4096]
                    [--no-b32] [--no-cpu-baseline]
    python bench.py --copy-probe                 # plain device copy of known size (counter scale)
    python bench.py --traffic-from DIR [--config C]   # counter CSVs -> profiles/traffic_fc1_C.json

One step = route (router product, softmax/top-k/renormalise, worklist) -> FC1 with
SiLU*up -> FC2 with the weighted combine, for one batch of synthetic tokens whose
activations already sit in HBM, through the single-call entry point moe_vq_forward.  The
kernel-timing pass runs the same step as its three calls (route_topk, fc1_silu,
fc2_combine: the same kernels) so that FC1 and FC2 can be timed one by one.  The default workload is decode batch 1 of a
DeepSeek-style layer (H=7168, I=2048, 256 experts, top-8, VQ2 experts at 2.125
bits/weight, all resident in one HBM slot pool).  Tokens are cycled from a pool of
256 distinct pre-drawn tokens so consecutive steps touch different experts (the
256 MB Infinity Cache holds about two steps' experts, not the pool).  The metric
names batch 1 and batch 32: the default run measures batch 32 (Zipf(1.1) expert
popularity) the same way and reports it as the "b32" block of the same line.

Prints one JSON line.  `value` is tokens/s of K steps timed on the host between two
device synchronisations, with nothing else on the stream.  The same K steps then run
again, each preceded by a 512 MiB read that evicts the memory-side cache, with FC1 and
FC2 launched through hipExtLaunchKernel with HIP events that record each kernel's own
start and end (moe_vq_time_next_kernel; events cost the device a few microseconds, so
they stay out of the throughput region).  `roofline` rates the dominant kernel (FC1) by
its algorithmic code+scale bytes per launch over the mean duration those events measure
(median, p10 and p90 beside it): the same run time a rocprofv3 kernel trace reports,
without the dispatch that events recorded on the stream around the launch would add.
Prefill is timed by events on the stream around the whole call.

`read_probe` is the rate of a plain streaming read of 1 GiB on the same device
(moe_vq_read_probe, timed like the FC kernels); `code_stream.frac_of_read_probe` sets
the code stream against it, beside the fraction of the published 8 TB/s.

`roofline.traffic` is the FC1 kernel's HBM traffic per launch as the hardware
counters saw it: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one rocprofv3 --pmc
run each) scaled by what the same counters read for a plain device copy of known
size (--copy-probe).  --traffic-from turns the four runs' CSV files into
profiles/traffic_fc1_<config>.json, tagged with a hash of the kernel sources; the
figure is reported only while the sources still match it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
WORKLOADS = {
    "b1": "decode batch 1: H=7168 I=2048 E=256 top-8, VQ2 2.125 b/w, bf16 x ~N(0,1), 256 experts resident",
    "b32": "decode batch 32: H=7168 I=2048 E=256 top-8, VQ2, router logits with Zipf(1.1) expert popularity",
    "b8mx": "decode batch 8: 52 most-routed experts MXFP4, 204 VQ2, Zipf(1.1) routing",
    "p4096": "prefill chunk of 4096 tokens: H=7168 I=2048 E=256 top-8, VQ2, grouped fp16 MFMA GEMMs",
    "b1d": "decode batch 1 as b1, with an FP4 (MXFP4) copy of every expert in the delta cache and the "
           "confidence gate at 0.60",
    "b32d": "decode batch 32 as b32, with an FP4 (MXFP4) copy of every expert in the delta cache and the "
            "confidence gate at 0.60",
}
PREFILL = {"p4096"}
DELTA = {"b1d": "b1", "b32d": "b32"}  # workload -> the preset it adds the FP4 delta cache to
GATE_TAU = 0.60


def preset(config):
    import synth
    return synth.PRESETS[DELTA.get(config, config)]
MFMA_F16_PEAK_TFLOPS = 2500.0


def listed_format(dev, e):
    """Format of a listed expert: e < E the expert itself, E + e its FP4 copy."""
    return int(dev.formats[e]) if e < dev.n_experts else int(dev.copy_formats[e - dev.n_experts])


def expert_stream_bytes(dev, experts):
    """Exact code+scale bytes of whole experts (gate, up, down), without alignment padding."""
    H, I = dev.hidden, dev.inter
    tot = 0
    for e in experts:
        f = listed_format(dev, e)
        if f == 1:
            tot += 3 * H * I // 4 + 3 * (H * I // 128) * 2
        else:
            tot += 3 * H * I // 2 + 3 * (H * I // 32)
    return tot


def fc1_exact_bytes(dev, experts):
    H, I = dev.hidden, dev.inter
    tot = 0
    for e in experts:
        f = listed_format(dev, e)
        tot += (2 * I * H // 4 + 2 * (I * H // 128) * 2) if f == 1 else (2 * I * H // 2 + 2 * (I * H // 32))
    return tot


def source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "bit_vector_quantised_amd", "csrc"))):
        with open(os.path.join(ROOT, "bit_vector_quantised_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


COPY_PROBE_BYTES = 256 << 20


def copy_probe():
    """A plain device-to-device copy of COPY_PROBE_BYTES, five times: under a counter run
    its FETCH_SIZE / WRITE_SIZE per dispatch give the scale of those counters."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "launches": 5}), flush=True)


def _counter_rows(d, counter):
    """(kernel name, value) of every dispatch in rocprofv3 counter CSVs under d."""
    import csv
    rows = []
    for root, _, files in os.walk(d):
        for fn in files:
            if not fn.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(root, fn)) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def traffic_from(d, config):
    """Combine four counter runs (d/fc1_fetch, d/fc1_write, d/copy_fetch, d/copy_write)
    into the FC1 traffic record read by the benchmark."""
    import statistics

    def fc1(rows):
        v = [x for n, x in rows if "fc_" in n and "true>" in n]
        return statistics.median(v), len(v), sorted({n for n, x in rows if "fc_" in n and "true>" in n})

    def copy(rows):
        # the largest dispatch of the copy run is the copy of COPY_PROBE_BYTES
        return max(x for n, x in rows)

    fetch, nf, names = fc1(_counter_rows(os.path.join(d, "fc1_fetch"), "FETCH_SIZE"))
    write, nw, _ = fc1(_counter_rows(os.path.join(d, "fc1_write"), "WRITE_SIZE"))
    c_fetch = copy(_counter_rows(os.path.join(d, "copy_fetch"), "FETCH_SIZE"))
    c_write = copy(_counter_rows(os.path.join(d, "copy_write"), "WRITE_SIZE"))
    f_scale = COPY_PROBE_BYTES / c_fetch   # bytes per counter unit, from the copy
    w_scale = COPY_PROBE_BYTES / c_write
    rec = {"source_hash": source_hash(), "config": config, "kernels": names,
           "fetch_counter_per_launch": fetch, "write_counter_per_launch": write,
           "copy_fetch_counter": c_fetch, "copy_write_counter": c_write,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "bytes_per_launch": fetch * f_scale + write * w_scale,
           "dispatches": [nf, nw]}
    out = os.path.join(ROOT, "profiles", f"traffic_fc1_{config}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(syn, x_pool_np, top_k, budget_s=15.0, tokens_per_call=None):
    """The fp64 oracle (as it is) on consecutive tokens of the same pool, until about
    budget_s seconds of work; returns tokens/s and the sample description."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    t0 = time.perf_counter()
    n = 0
    T = tokens_per_call or syn.cfg.n_tokens
    while True:
        x = x_pool_np[(n * T) % x_pool_np.shape[0]:][:T]
        oracle.forward(syn, oracle.x_value(x, "bf16"), top_k)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": n * T / dt, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{n} step(s) of {T} token(s) of the same workload in {dt:.1f} s; fp64 numpy oracle, "
                      f"decode single-threaded, products on {blas_threads} BLAS thread(s); "
                      f"host has {len(os.sched_getaffinity(0))} usable cores"}


def bench_tier(args, cfg, syn, x_pool, n_batches):
    """Decode steps with every expert in a pinned host pool and args.tier_slots device
    slots: route, copy the missing experts over PCIe (least recently used out), route
    again, FC1, FC2.  Prints one JSON line; the copies are inside the timed region."""
    import torch
    from bit_vector_quantised_amd import _lib
    from bit_vector_quantised_amd.layer import Step, TieredLayer, cpu_miss_forward, tiered_forward

    T = cfg.n_tokens
    print(f"[bench] tier: {args.tier_slots} device slots of {cfg.n_experts} experts", file=sys.stderr, flush=True)
    tl = TieredLayer.from_synth(syn, n_dev_slots=args.tier_slots)
    st = Step(tl, T)
    fmts = [int(f) for f in syn.formats]
    start = 0
    if args.cpu_miss or args.tier_slots >= cfg.n_experts:
        # fill the device slots once from the first batches.  With the CPU miss path the
        # timed steps then take the batches after them (whose experts the fill did not
        # choose); with a slot for every expert they measure the tier's own cost on
        # steps that never miss.
        for i in range(4 * n_batches):
            tiered_forward(st, tl, x_pool[(i % n_batches) * T:(i % n_batches + 1) * T])
            start = i + 1
            if all(e >= 0 for e in tl.tier.held()):
                break

    def one(i):
        i += start
        xb = x_pool[(i % n_batches) * T:(i % n_batches + 1) * T]
        if args.cpu_miss:
            _, miss = cpu_miss_forward(st, tl, xb)
            return len(miss), sum(_lib.expert_bytes(fmts[e], cfg.hidden, cfg.inter) for e in miss)
        _, n = tiered_forward(st, tl, xb)
        if not n:
            return 0, 0
        now = set(tl.tier.held())
        new = now - held[0]
        held[0] = now
        return n, sum(_lib.expert_bytes(fmts[e], cfg.hidden, cfg.inter) for e in new if e >= 0)

    held = [set(tl.tier.held())]

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    copied = nbytes = 0
    t0 = time.perf_counter()
    for i in range(args.steps):
        n, b = one(args.warmup + i)
        copied += n
        nbytes += b
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    status, info = st.check()
    if status != _lib.OK and not (args.cpu_miss and status == _lib.ENOTRESIDENT):
        raise RuntimeError(f"tier step status {status} ({_lib.strerror(status)}), expert {info}")
    ms = dt / args.steps * 1e3
    what = ("experts without a device slot computed on the host cores" if args.cpu_miss
            else "experts copied into device slots over PCIe")
    print(json.dumps({
        "metric": f"MoE-VQ layer tokens/s, experts in host RAM behind a device-slot tier ({what})",
        "value": T * args.steps / dt, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16/fp32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} with a host-RAM tier", "tokens_per_step": T,
                   "n_experts": cfg.n_experts, "device_slots": args.tier_slots,
                   "tier_mode": "cpu-miss" if args.cpu_miss else "copy"},
        "tier": ({"experts_on_host_per_step": copied / args.steps, "host_expert_bytes_per_step": nbytes / args.steps,
                  "host_GBps": nbytes / dt / 1e9, "host_threads": max(1, min(64, len(os.sched_getaffinity(0))))}
                 if args.cpu_miss else
                 {"experts_copied_per_step": copied / args.steps, "h2d_bytes_per_step": nbytes / args.steps,
                  "h2d_GBps": nbytes / dt / 1e9}),
    }))


SCRUB_BYTES = 512 << 20
READ_PROBE_BYTES = 1 << 30


def read_peak(reps=10):
    """The HBM read rate of a plain streaming read (moe_vq_read_probe) of 1 GiB, four
    times the memory-side cache: median over reps runs, each timed by events its own
    launch records.  GB/s."""
    import torch
    from bit_vector_quantised_amd import _lib
    buf = torch.zeros(READ_PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:  # (a torch event holds a HIP event only once it has been recorded)
        a.record(stream)
        b.record(stream)
    for _ in range(3):
        _lib.read_probe(buf.data_ptr(), READ_PROBE_BYTES, sink.data_ptr(), stream.cuda_stream)
    for a, b in evs:
        _lib.time_next_kernel(a.cuda_event, b.cuda_event)
        _lib.read_probe(buf.data_ptr(), READ_PROBE_BYTES, sink.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    del buf
    return READ_PROBE_BYTES / (ms[len(ms) // 2] * 1e-3) / 1e9


def measure(args, config, with_events=True):
    """Build one configuration's layer, run warmup, the throughput region (K steps back
    to back) and, with_events, the kernel-timing pass.  Returns the per-config block of
    the JSON line (value, ms_per_step, roofline, code_stream or prefill)."""
    import numpy as np
    import torch

    import synth
    from bit_vector_quantised_amd import _lib
    from bit_vector_quantised_amd.layer import DeviceLayer, Step

    cfg = preset(config)
    T, k = cfg.n_tokens, cfg.top_k
    delta = config in DELTA
    print(f"[bench] building {config} layer ({cfg.n_experts} experts)", file=sys.stderr, flush=True)
    syn_dev = synth.SynthLayer(cfg, cache=False)
    if delta:  # every expert also stored as MXFP4 in the delta cache
        dev = DeviceLayer.from_synth(syn_dev, fp4_copies=range(cfg.n_experts), gate_tau=GATE_TAU)
    else:
        dev = DeviceLayer.from_synth(syn_dev)
    prefill = config in PREFILL
    n_pool = 256 if T == 1 else (max(8, 256 // T) * T if T <= 256 else 2 * T)
    x_pool_np = synth.SynthLayer(cfg, cache=False).x(n=n_pool, stream=7)
    x_pool = torch.from_numpy(x_pool_np.view(np.int16)).cuda().view(torch.bfloat16)
    n_batches = n_pool // T
    step = Step(dev, T)
    stream = torch.cuda.current_stream()
    if args.tier_slots:
        return bench_tier(args, cfg, syn_dev, x_pool, n_batches)

    def run_step(i, ev=None):
        xb = x_pool[(i % n_batches) * T:(i % n_batches + 1) * T]
        if ev is None and not prefill:
            step.step(xb)  # the whole step in one call (moe_vq_forward)
            return
        step.route(xb)
        if prefill:
            if ev is not None:
                ev[0].record(stream)
            step.prefill(xb)
            if ev is not None:
                ev[1].record(stream)
            return
        if ev is not None:  # FC1's kernel records ev[0] at its start and ev[1] at its end
            _lib.time_next_kernel(ev[0].cuda_event, ev[1].cuda_event)
        step.fc1(xb)
        if ev is not None:
            _lib.time_next_kernel(ev[2].cuda_event, ev[3].cuda_event)
        step.fc2(T)

    print(f"[bench] {config}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    st, info = step.check()
    if st != _lib.OK:
        raise RuntimeError(f"step status {st} ({_lib.strerror(st)}), expert {info}")

    # distinct experts per step (for the algorithmic bytes), read outside the timed region
    uniq, fc1_bytes, step_bytes, gated, copies = [], [], [], [], []
    for i in range(n_batches):
        run_step(i)
        inf = step.info(T)
        uniq.append(inf["n_active"])
        fc1_bytes.append(fc1_exact_bytes(dev, inf["experts"]))
        step_bytes.append(expert_stream_bytes(dev, inf["experts"]))
        if delta:  # (every expert has a copy: a pair is gated when its weight reaches the gate)
            gated.append(int((step.w[:T] >= GATE_TAU).sum().item()))
            copies.append(sum(1 for e in inf["experts"] if e >= cfg.n_experts))
    torch.cuda.synchronize()

    # throughput: K steps, nothing but the step on the stream
    print(f"[bench] {config}: timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(args.warmup + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    bidx = [(args.warmup + i) % n_batches for i in range(args.steps)]
    fc1_b = float(np.mean([fc1_bytes[b] for b in bidx]))
    step_b = float(np.mean([step_bytes[b] for b in bidx]))
    out = {"value": args.steps * T / dt, "unit": "tokens/s", "ms_per_step": dt * 1e3 / args.steps,
           "workload": WORKLOADS[config], "tokens_per_step": T,
           "unique_experts_per_step": float(np.mean([uniq[b] for b in bidx]))}
    if delta:
        out["delta"] = {"gate_tau": GATE_TAU, "fp4_copies": cfg.n_experts,
                        "gated_pairs_per_step": float(np.mean([gated[b] for b in bidx])),
                        "copies_listed_per_step": float(np.mean([copies[b] for b in bidx]))}
    if not with_events:
        return out, dev, syn_dev, x_pool_np

    # kernel durations: the same K steps again, each after a 512 MiB read that evicts the
    # 256 MB memory-side cache (so the experts come from HBM: the cold case).  The scrub
    # only reads: a read-modify-write would leave dirty lines whose write-back competes
    # with FC1.  The FC kernels are launched with HIP events that record their own start
    # and end (moe_vq_time_next_kernel), so a duration is the kernel's run alone, as in a
    # rocprofv3 kernel trace; prefill is timed by events on the stream around the call.
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device="cuda")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for ev in events:  # (a torch event holds a HIP event only once it has been recorded)
        for e in ev:
            e.record(stream)
    print(f"[bench] {config}: kernel timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    for i in range(args.steps):
        scrub.sum()
        run_step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    del scrub
    fc1_ms = np.array([events[i][0].elapsed_time(events[i][1]) for i in range(args.steps)])
    fc2_ms = np.array([events[i][2].elapsed_time(events[i][3]) for i in range(args.steps)]) if not prefill else None
    fc1_avg = float(np.mean(fc1_ms)) * 1e-3

    def spread(ms):
        return {"median_us": float(np.median(ms)) * 1e3, "mean_us": float(np.mean(ms)) * 1e3,
                "p10_us": float(np.percentile(ms, 10)) * 1e3, "p90_us": float(np.percentile(ms, 90)) * 1e3}

    if prefill:
        # FC1 + FC2 as grouped MFMA GEMMs: 2 * 3 * H * I flops per routed pair
        flops = 2.0 * 3 * cfg.hidden * cfg.inter * T * k
        tflops = flops / fc1_avg / 1e12  # the events bracket the whole prefill call
        out["dtype"] = "fp16 MFMA (decoded weights x fp16-staged activations), fp32 accumulate"
        out["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": tflops / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                           "kernel": "moe_vq_prefill_gemm (prefill_fc_kernel FC1 + FC2, grouped fp16 MFMA)",
                           "flops_per_launch": flops, "launch_us": spread(fc1_ms)}
        out["prefill"] = {"code_bytes_per_step": step_b}
        return out, dev, syn_dev, x_pool_np

    fc2_avg = float(np.mean(fc2_ms)) * 1e-3
    achieved = fc1_b / fc1_avg / 1e9
    code_stream = step_b / (fc1_avg + fc2_avg) / 1e9
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_fc1_{config}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash():
            traffic = tr.get("bytes_per_launch")
    out["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                       "kernel": ("fc_stream_kernel" if T <= 1 else "fc_mfma_kernel")
                       + " FC1 (gate/up code decode + SiLU*up)",
                       "bytes_per_launch": fc1_b, "launch_us": spread(fc1_ms),
                       "timing": "HIP events recorded by the kernel's own launch (hipExtLaunchKernel) at its "
                                 "start and end, mean over the timed steps, memory-side cache evicted by a "
                                 "512 MiB read before each step"}
    out["code_stream"] = {"GBps": code_stream, "frac": code_stream / HBM_PEAK_GBPS, "bytes_per_step": step_b,
                          "fc1": spread(fc1_ms), "fc2": spread(fc2_ms)}
    return out, dev, syn_dev, x_pool_np


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="b1", choices=sorted(WORKLOADS))
    ap.add_argument("--no-b32", action="store_true", help="with the default config, skip the batch-32 block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--traffic-from", default=None)
    ap.add_argument("--tier-slots", type=int, default=0,
                    help="experts in pinned host RAM, this many device slots (host-RAM tier; "
                         "PCIe-inclusive, not the headline)")
    ap.add_argument("--cpu-miss", action="store_true",
                    help="with --tier-slots: compute the experts without a device slot on the host cores "
                         "(no copies) instead of copying them in")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from, args.config)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the routed-expert step is measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return

    import torch

    import synth

    torch.cuda.set_device(0)
    peak_read = read_peak() if not args.tier_slots and args.config not in PREFILL else None
    res = measure(args, args.config)
    if res is None:  # (the host-RAM tier mode printed its own line)
        return
    main_block, dev, syn_dev, x_pool_np = res
    cfg = preset(args.config)
    out = {
        "metric": "MoE-VQ layer tokens/s and code-stream HBM GB/s (% peak), batch 1 & 32",
        "value": main_block["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_block["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_block.get("dtype", "fp16xfp16->fp32 (decoded VQ2 weights x fp16-staged activations, "
                                         "fp32 accumulate)"),
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "tokens_per_step": cfg.n_tokens, "hidden": cfg.hidden,
                   "inter": cfg.inter, "n_experts": cfg.n_experts, "top_k": cfg.top_k,
                   "unique_experts_per_step": main_block["unique_experts_per_step"],
                   "parallelism": "single GPU"},
        "roofline": main_block["roofline"],
    }
    for key in ("code_stream", "prefill", "delta"):
        if key in main_block:
            out[key] = main_block[key]
    if peak_read:
        # the code stream against a plain read of the same device (beside the published peak)
        out["read_probe"] = {"GBps": peak_read, "bytes": READ_PROBE_BYTES, "kernel": "moe_vq_read_probe",
                             "frac_of_peak": peak_read / HBM_PEAK_GBPS}
        out["code_stream"]["frac_of_read_probe"] = out["code_stream"]["GBps"] / peak_read
    if not args.no_cpu_baseline and args.config not in DELTA:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        syn_or = synth.SynthLayer(cfg)
        out["cpu_baseline"] = cpu_baseline(syn_or, x_pool_np, cfg.top_k, args.cpu_budget,
                                           tokens_per_call=8 if args.config in PREFILL else None)
    else:
        out["cpu_baseline"] = None
    del dev
    torch.cuda.empty_cache()
    # the metric's second batch size, in the same line
    if args.config == "b1" and not args.no_b32:
        b32, dev32, _, _ = measure(args, "b32")
        out["b32"] = {k: b32[k] for k in ("value", "unit", "ms_per_step", "workload", "tokens_per_step",
                                           "unique_experts_per_step", "roofline", "code_stream")}
        if peak_read:
            out["b32"]["code_stream"]["frac_of_read_probe"] = b32["code_stream"]["GBps"] / peak_read
        del dev32
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
