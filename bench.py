"""Decode-attention benchmark of the hybrid layer-reuse policy on one MI355X.

A step is one hybrid decode step of every layer of the workload (reset layers:
full attention + block scores + top-k; reuse layers: attention over the
carried blocks) for the whole batch, inputs resident in HBM, launched in layer
order on one stream.  `value` times the step replayed as one HIP graph (the
form a decode loop with static shapes runs); the eager step rate is reported
beside it.  Also timed: the plain full-attention step (every layer full
attention, no scores) and the all-reset step (every layer full attention +
scores + top-k).

Options beyond the timed default: --jump N (a static reset-every-N policy),
--ctx T (context sweep), --profiled (policy from the DP on a similarity
matrix measured on the GPU from an all-reset step's logged top-k sets).

Prints one JSON line.  `value` is hybrid decode steps/s.  `roofline` covers
the dominant kernel (full split attention of the reset layers): algorithmic
bytes per launch = 4*B*Hkv*T*d (bf16 K and V, each read once), divided by its
average launch time from HIP events that each launch stamps itself on its
stream (hipExtLaunchKernel) during the timed eager hybrid steps; `traffic` is
the HBM bytes per launch from the committed rocprofv3 counter summary, null
once the kernel source differs from the one profiled.  `cpu_baseline` times
the CPU oracle on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attn steps/s @32K-128K ctx; achieved HBM GB/s vs peak; hybrid/full speedup"
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama3_8b_32k")
    p.add_argument("--topk", type=int, default=None)
    p.add_argument("--theta", type=float, default=None)
    p.add_argument("--layers", type=int, default=None, help="use only the first N layers")
    p.add_argument("--ctx", type=int, default=None,
                   help="override the context length of every sequence (context sweeps)")
    p.add_argument("--jump", type=int, default=None, metavar="N",
                   help="static policy: reset every N layers (a Jump-N baseline)")
    p.add_argument("--e2e", action="store_true",
                   help="time a whole random-weight Llama-3-8B-shaped decode step (projections, "
                        "RoPE, KV append, attention, MLP) for the hybrid and the full policy "
                        "instead of attention alone")
    p.add_argument("--batch", type=int, default=0,
                   help="override the workload's batch size (sequences per step)")
    p.add_argument("--shard-heads", type=int, default=0, metavar="P",
                   help="one GPU's share under P-way KV-head (tensor-parallel) sharding: "
                        "Hkv/P KV heads and Hq/P query heads, the group size unchanged")
    p.add_argument("--offload", action="store_true",
                   help="index-guided offloading: the reuse layers' KV caches in pinned host "
                        "memory, their selected blocks gathered on a copy stream (with --e2e: "
                        "the end-to-end step as well)")
    p.add_argument("--profiled", action="store_true",
                   help="policy from the DP on a similarity matrix profiled on the GPU "
                        "(all-reset step, logged top-k overlaps) instead of the synthetic one")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="budget of the CPU oracle baseline (0 disables it)")
    p.add_argument("--skip-baselines", action="store_true",
                   help="time only the hybrid step (for short profiler runs)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only copy a MIB-sized buffer 4 times (calibrates HBM byte counters)")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the 64K-128K workloads of the `configs` object (headline only)")
    p.add_argument("--config-steps", type=int, default=10,
                   help="timed steps per policy of the `configs` workloads")
    return p.parse_args()


def copy_probe(mib):
    """Four device-to-device copies of `mib` MiB: a kernel of known traffic
    (mib MiB read + mib MiB written each) for scaling profiler byte counters."""
    import torch
    x = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(4):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": mib << 20, "copies": 4}), flush=True)


def measured_traffic(workload, scored):
    """HBM bytes per full-attention launch (with fused block scores and
    top-k when `scored`) from the committed rocprofv3 PMC summary of this
    workload (FETCH_SIZE and WRITE_SIZE, scaled by a copy kernel of known
    size), or None when there is none or when the kernel source has changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_traffic_%s.json" % workload)
    src = os.path.join(ROOT, "sparse_layer_reuse_amd", "csrc", "hylra_kernels.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if rec.get("kernel_source_sha256") != digest or rec.get("workload") != workload:
        return None
    return rec.get("scored_layer_traffic_bytes" if scored else "full_layer_traffic_bytes")


def policy_for(wl, hylra, theta, L, jump=None, profiled_layers=None, k=None):
    from sparse_layer_reuse_amd import synth, workloads as W
    if jump:
        resets = tuple(range(0, wl.layers, jump))
        return W.src_from_resets(wl.layers, resets)[:L], "jump %d" % jump, None
    if profiled_layers is not None:
        if theta is None:
            theta = wl.dp_theta[0] if wl.dp_theta else 0.8
        force = [j in wl.dp_force for j in range(L)] if wl.policy == "dp" else None
        src, nres, _, _ = hylra.profile_policy([profiled_layers], k, theta, force)
        return src, "dp on a profiled overlap matrix, theta=%g" % theta, theta
    if wl.policy == "fixed":
        src = W.src_from_resets(wl.layers, wl.resets)
        desc = "fixed resets %s" % (list(wl.resets),)
        theta = None
    else:
        theta = wl.dp_theta[0] if theta is None else theta
        M = synth.workload_similarity(wl)
        force = [j in wl.dp_force for j in range(wl.layers)]
        src, _, _ = hylra.policy_dp(M, theta, force)
        desc = "dp theta=%g decay=%g force=%s" % (theta, wl.dp_decay, list(wl.dp_force))
    src = src[:L]
    return src, desc, theta


def timed(fn, steps, warmup, torch, timers, hylra):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    for kind in timers:
        hylra.timer_start(kind, capacity=max(64, steps * 128))
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    kern = {}
    for kind in timers:
        tot, n = hylra.timer_stop(kind)
        kern[kind] = (tot / n if n else None, n)
    return ms, kern


def graph_timed(fn, steps, warmup, torch):
    """Capture one call of fn (all its launches) in a HIP graph and time
    `steps` replays.  Returns (ms per step, graph)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps, graph


def step_percentiles(graph, steps, torch):
    """Per-step times of `steps` graph replays, each bracketed by its own
    events: (p10, p50, p90) in ms."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    pick = lambda q: t[min(len(t) - 1, int(q * (len(t) - 1) + 0.5))]
    return pick(0.1), pick(0.5), pick(0.9)


def stream_ceiling(torch, hylra, mib=512, buffers=4, reps=3):
    """Practical HBM read ceiling: the library's read probe (the attention
    kernels' K/V load pattern, no arithmetic) over `buffers` distinct
    `mib`-MiB buffers in turn, so no launch finds its data in a cache."""
    bufs = [torch.ones(mib << 20, dtype=torch.uint8, device="cuda") for _ in range(buffers)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b in bufs:
        hylra.read_probe(b, sink)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        for b in bufs:
            hylra.read_probe(b, sink)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop)
    launches = reps * buffers
    del bufs
    return {"gbs": launches * (mib << 20) / (ms * 1e-3) / 1e9, "bytes_per_launch": mib << 20,
            "launches": launches, "kernel": "read_probe (hylra_read_probe)"}


def settle(torch, hylra, max_s=30.0):
    """Waits until nothing else takes HBM bandwidth: device memory released
    by an earlier process (or an earlier workload of this run) is cleared by
    the driver in the background for several seconds, and a run started
    meanwhile streams ~5% slower.  Reads a 512 MiB buffer with the read
    probe until its rate reaches 97% of a 7.0 TB/s idle ceiling, or stops
    rising for 5 s after at least 10 s, or max_s pass.  Returns the seconds
    waited and the last rate (GB/s)."""
    buf = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    best, best_t, rate = 0.0, t0, 0.0
    while True:
        start.record()
        for _ in range(8):
            hylra.read_probe(buf, sink)
        stop.record()
        torch.cuda.synchronize()
        rate = 8 * (512 << 20) / (start.elapsed_time(stop) * 1e-3) / 1e9
        now = time.time()
        if rate > best * 1.01:
            best, best_t = rate, now
        if rate >= 0.97 * 7000.0 or now - t0 >= max_s or \
                (now - t0 >= 10.0 and now - best_t >= 5.0):
            break
        time.sleep(0.25)
    del buf
    return time.time() - t0, rate


def cpu_baseline(wl, layers, src, k, budget_s):
    """Oracle timed on the host: passes over the step's layers in order (the
    carried indices flow from each reset layer to its reuse layers) until the
    time budget is spent; the step time is the mean reset-layer time times
    the number of reset layers plus the mean reuse-layer time times the
    number of reuse layers."""
    import oracle
    from sparse_layer_reuse_amd import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    t_reset, t_reuse = [], []
    carried = None
    passes, measured = 0, 0
    t_start = time.time()
    done = False
    while not done:
        for j, lay in enumerate(layers):
            o = synth.layer_to_oracle(lay)
            t0 = time.perf_counter()
            if src[j] == j:
                _, _, score = oracle.decode_full(o["q"], o["k_pool"], o["v_pool"], o["table"],
                                                 o["ctx"], num_kv_heads=wl.num_kv_heads)
                carried, _ = oracle.topk(score, o["ctx"], k)
                t_reset.append(time.perf_counter() - t0)
            else:
                oracle.attend(o["q"], o["k_pool"], o["v_pool"], o["table"], o["ctx"],
                              num_kv_heads=wl.num_kv_heads, sel=carried, k=k)
                t_reuse.append(time.perf_counter() - t0)
            del o
            measured += 1
            if time.time() - t_start > budget_s and t_reset and (t_reuse or j + 1 == len(layers)):
                done = True
                break
        else:
            passes += 1
    n_reset = sum(1 for j, s in enumerate(src) if s == j)
    n_reuse = len(src) - n_reset
    mean = lambda v: sum(v) / len(v) if v else 0.0
    step_s = n_reset * mean(t_reset) + n_reuse * mean(t_reuse)
    # one host thread: layer 0 (a reset layer) and the first reuse layer, twice each
    single = None
    reuse_j = next((j for j, s in enumerate(src) if s != j), None)
    oracle.set_threads(1)
    try:
        s_reset, s_reuse = [], []
        for _ in range(2):
            o = synth.layer_to_oracle(layers[0])
            t0 = time.perf_counter()
            _, _, score = oracle.decode_full(o["q"], o["k_pool"], o["v_pool"], o["table"],
                                             o["ctx"], num_kv_heads=wl.num_kv_heads)
            sel, _ = oracle.topk(score, o["ctx"], k)
            s_reset.append(time.perf_counter() - t0)
            if reuse_j is not None:
                o = synth.layer_to_oracle(layers[reuse_j])
                t0 = time.perf_counter()
                oracle.attend(o["q"], o["k_pool"], o["v_pool"], o["table"], o["ctx"],
                              num_kv_heads=wl.num_kv_heads, sel=sel, k=k)
                s_reuse.append(time.perf_counter() - t0)
            del o
        s_step = n_reset * mean(s_reset) + n_reuse * mean(s_reuse)
        single = {"value": 1.0 / s_step, "unit": "steps/s", "cores": 1,
                  "reset_layer_s": mean(s_reset), "reuse_layer_s": mean(s_reuse),
                  "sample": "layer 0 (reset) and layer %s (reuse) timed twice each on one "
                            "thread; same step formula" % reuse_j}
    finally:
        oracle.set_threads(threads)
    return {
        "value": 1.0 / step_s if step_s > 0 else None,
        "unit": "steps/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d layer calls timed (%d full passes over the %d-layer hybrid step, then "
                  "layers 0-%d): %d reset, %d reuse; step time = %d x mean reset-layer time "
                  "+ %d x mean reuse-layer time; float64 C oracle, OpenMP, %.1f s"
                  % (measured, passes, len(layers), (measured - 1) % len(layers),
                     len(t_reset), len(t_reuse), n_reset, n_reuse, time.time() - t_start),
        "reset_layer_s": mean(t_reset),
        "reuse_layer_s": mean(t_reuse),
        "single_core": single,
    }


def host_cpu():
    """Model name and socket count of the host CPU (from /proc/cpuinfo)."""
    model, sockets = None, set()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "model name" and model is None:
                    model = val.strip()
                elif key == "physical id":
                    sockets.add(val.strip())
    except OSError:
        pass
    return {"cpu_model": model, "sockets": len(sockets) or None,
            "logical_cpus": os.cpu_count()}


def oracle_layer_times(wl, layers, src, k):
    """Oracle (all host threads) on one reset layer and one reuse layer of the
    workload (the reuse layer attends the reset layer's top-k set): seconds
    per reset layer and per reuse layer."""
    import oracle
    from sparse_layer_reuse_amd import synth
    reset_j = 0
    reuse_j = next((j for j, s_ in enumerate(src) if s_ != j), None)
    o = synth.layer_to_oracle(layers[reset_j])
    t0 = time.perf_counter()
    _, _, score = oracle.decode_full(o["q"], o["k_pool"], o["v_pool"], o["table"], o["ctx"],
                                     num_kv_heads=wl.num_kv_heads)
    sel, _ = oracle.topk(score, o["ctx"], k)
    t_reset = time.perf_counter() - t0
    del o, score
    t_reuse = None
    if reuse_j is not None:
        o = synth.layer_to_oracle(layers[reuse_j])
        t0 = time.perf_counter()
        oracle.attend(o["q"], o["k_pool"], o["v_pool"], o["table"], o["ctx"],
                      num_kv_heads=wl.num_kv_heads, sel=sel, k=k)
        t_reuse = time.perf_counter() - t0
        del o
    return t_reset, t_reuse


def reuse_similarity(M, src):
    """Fidelity of a policy on the similarity matrix the DP runs on (row =
    target layer, column = source): the similarity of every reuse layer to
    the reset layer whose index set it attends -- the quantity the DP keeps
    above its threshold and a static Jump-N schedule does not look at."""
    sims = [float(M[j][s_]) for j, s_ in enumerate(src) if s_ != j]
    if not sims:
        return {"reuse_similarity_min": None, "reuse_similarity_mean": None,
                "reuse_layers_below_0.8": 0}
    return {"reuse_similarity_min": min(sims), "reuse_similarity_mean": sum(sims) / len(sims),
            "reuse_layers_below_0.8": sum(1 for x in sims if x <= 0.8)}


def measure_policy(layers, src, k, steps, warmup, torch, hylra, full_bytes, sparse_bytes):
    """One policy on resident layers: graph-replayed steps/s and the average
    launch time of each kernel kind (events stamped by the launches) with its
    fraction of the HBM peak."""
    plan = hylra.PolicyPlan(layers, src, k)
    kinds = (hylra.KERNEL_FULL_SCORED, hylra.KERNEL_FULL_ATTN, hylra.KERNEL_SPARSE_ATTN)
    _, kern = timed(plan.run, steps, warmup, torch, kinds, hylra)
    ms, g = graph_timed(plan.run, steps, warmup, torch)
    del g, plan
    us = lambda kind: kern[kind][0] * 1e3 if kern[kind][0] is not None else None
    frac = lambda b, t: b / (t * 1e-6) / 1e9 / HBM_PEAK_GBS if t else None
    resets = sum(1 for j, s_ in enumerate(src) if s_ == j)
    return {
        "resets": resets, "reuses": len(src) - resets,
        "steps_per_s": 1000.0 / ms, "ms_per_step": ms,
        "reset_with_topk_us": us(hylra.KERNEL_FULL_SCORED),
        "reset_without_topk_us": us(hylra.KERNEL_FULL_ATTN),
        "reuse_us": us(hylra.KERNEL_SPARSE_ATTN),
        "frac_reset_with_topk": frac(full_bytes, us(hylra.KERNEL_FULL_SCORED)),
        "frac_reset_without_topk": frac(full_bytes, us(hylra.KERNEL_FULL_ATTN)),
        "frac_reuse": frac(sparse_bytes, us(hylra.KERNEL_SPARSE_ATTN)),
    }


def measure_configs(args, torch, hylra):
    """The 64K-128K workloads of the metric beside the headline: for each,
    the full-attention step and every policy it is quoted with (the DP
    thresholds or the top-k sweep, and static Jump-3 / Jump-4 policies for
    the DP workloads), each as graph-replayed steps/s with per-kernel launch
    times and fractions of the HBM peak; plus the oracle on one reset and
    one reuse layer of the workload, scaled to the policy's layer counts
    (labelled extrapolated)."""
    from sparse_layer_reuse_amd import synth, workloads as W
    plans = [
        ("llama3_70b_128k_dp", [("dp", 0.7, 32), ("dp", 0.8, 32), ("dp", 0.9, 32),
                                ("jump", 3, 32), ("jump", 4, 32)]),
        ("llama3_8b_b8_64k_dp", [("dp", 0.8, 32), ("jump", 3, 32), ("jump", 4, 32)]),
        ("llama3_8b_paged_128k", [("fixed", None, 8), ("fixed", None, 32), ("fixed", None, 64)]),
    ]
    steps, warmup = args.config_steps, 3
    out = {}
    for name, policies in plans:
        wl = W.get(name)
        t0 = time.time()
        layers = synth.workload_layers(wl, device="cuda")
        torch.cuda.synchronize()
        gen_s = time.time() - t0
        settle_s, settle_gbs = settle(torch, hylra)
        full_bytes = wl.kv_bytes_per_layer()
        full = hylra.FullPlan(layers)
        _, kf = timed(full.run, steps, warmup, torch, (hylra.KERNEL_FULL_ATTN,), hylra)
        ms_full, g = graph_timed(full.run, steps, warmup, torch)
        del g, full
        full_us = kf[hylra.KERNEL_FULL_ATTN][0] * 1e3
        entry = {
            "batch": wl.batch, "layers": wl.layers, "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads, "ctx": wl.ctx, "paged": wl.paged,
            "kv_bytes_per_layer": full_bytes, "input_generation_s": gen_s,
            "settle": {"seconds": settle_s, "read_gbs": settle_gbs},
            "full_steps_per_s": 1000.0 / ms_full, "full_layer_us": full_us,
            "frac_full_layer": full_bytes / (full_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "policies": {},
        }
        oracle_t = None
        for kind, param, k in policies:
            if kind == "jump":
                src = W.src_from_resets(wl.layers, range(0, wl.layers, param))
                label = "jump%d_k%d" % (param, k)
            elif kind == "dp":
                M = synth.workload_similarity(wl)
                force = [j in wl.dp_force for j in range(wl.layers)]
                src, _, _ = hylra.policy_dp(M, param, force)
                label = "dp_theta%g_k%d" % (param, k)
            else:
                src = W.src_from_resets(wl.layers, wl.resets)
                label = "fixed_k%d" % k
            sparse_bytes = full_bytes * min(k, wl.blocks) // wl.blocks
            r = measure_policy(layers, src, k, steps, warmup, torch, hylra, full_bytes,
                               sparse_bytes)
            r["hybrid_over_full"] = r["steps_per_s"] / entry["full_steps_per_s"]
            if wl.policy == "dp":
                r.update(reuse_similarity(synth.workload_similarity(wl), src))
            if args.cpu_seconds > 0:
                if oracle_t is None or oracle_t[2] != k:
                    tr, tu = oracle_layer_times(wl, layers, src, k)
                    oracle_t = (tr, tu, k)
                tr, tu = oracle_t[0], oracle_t[1]
                step_s = r["resets"] * tr + r["reuses"] * (tu or 0.0)
                r["cpu_oracle_extrapolated"] = {
                    "steps_per_s": 1.0 / step_s, "reset_layer_s": tr, "reuse_layer_s": tu,
                    "note": "extrapolated: one reset and one reuse layer timed, scaled by "
                            "the policy's layer counts"}
            entry["policies"][label] = r
        out[name] = entry
        del layers
        torch.cuda.empty_cache()
    return out


def e2e(args, wl, k, src, policy_desc):
    """End-to-end decode step of a random-weight decoder of the workload's
    batch, context, heads and layer count, hybrid vs full attention."""
    import torch
    from sparse_layer_reuse_amd import decode_step as DS
    import dataclasses
    base = DS.shape_for(wl.num_q_heads, wl.num_kv_heads, wl.head_dim)
    if base is None:
        sys.exit("--e2e needs a Llama-3-8B or -70B head shape (workload %s)" % wl.name)
    shape = dataclasses.replace(base, layers=len(src))
    dec = DS.RandomDecoder(shape, wl.batch, wl.ctx, seed=wl.seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 99)
    x = torch.randn(wl.batch, shape.hidden, generator=g, device="cuda").to(torch.bfloat16)
    ms_h, _ = graph_timed(lambda: dec.step(x, "hybrid", src, k), args.steps, args.warmup, torch)
    ms_f, _ = graph_timed(lambda: dec.step(x, "full", src, k), args.steps, args.warmup, torch)
    extra = {}
    if args.offload:
        reuse = [j for j, s in enumerate(src) if s != j]
        dec.offload(reuse)
        ms_o, _ = graph_timed(lambda: dec.step(x, "hybrid", src, k), args.steps, args.warmup, torch)
        elt = 2
        kv_layer = 2 * wl.batch * wl.num_kv_heads * wl.blocks * 128 * wl.head_dim * elt
        extra = {"offload": {
            "offloaded_layers": len(reuse),
            "hybrid_offload_ms_per_step": ms_o,
            "hybrid_offload_steps_per_s": 1000.0 / ms_o,
            "offload_over_device": ms_o / ms_h,
            "kv_bytes_in_host_memory": kv_layer * len(reuse),
            "kv_bytes_on_device": kv_layer * (len(src) - len(reuse)),
            "host_link_bytes_per_step": len(reuse) * 2 * wl.batch * wl.num_kv_heads
                                        * min(k, wl.blocks) * 128 * wl.head_dim * elt,
        }}
    return {
        "metric": "end-to-end decode steps/s, random-weight Llama-3-shaped model, hybrid vs full",
        "value": 1000.0 / ms_h, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_h, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random weights, seeded KV history)",
        "config": {"workload": wl.name, "batch": wl.batch, "ctx": wl.ctx, "layers": len(src),
                   "hidden": shape.hidden, "ffn": shape.ffn, "topk": k, "policy": policy_desc},
        "full_steps_per_s": 1000.0 / ms_f, "full_ms_per_step": ms_f,
        "hybrid_over_full": ms_f / ms_h,
        "pages_context": {"speedup_vs_full_attention": 1.45, "scope": "end-to-end LLM decode",
                          "sequence_length": 60000, "hardware": "not stated"},
        **extra,
    }


def link_ceiling(torch, mib=1024, reps=3):
    """Pinned host -> device copy rate (copy engine) of `mib` MiB: the
    practical ceiling of the host link, in GB/s."""
    src = torch.empty(mib << 20, dtype=torch.uint8).pin_memory()
    dst = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        best = max(best, (mib << 20) / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    return best


def offload_bench(args, wl, k, src, policy_desc, layers, torch, hylra):
    """Attention-only step with the reuse layers' caches in pinned host
    memory, against the same step with every cache on the device."""
    L = len(src)
    reuse = [j for j, s in enumerate(src) if s != j]
    offloaded = [s != j for j, s in enumerate(src)]
    device_plan = hylra.PolicyPlan(layers, src, k)
    ms_dev, g = graph_timed(device_plan.run, args.steps, args.warmup, torch)
    del g, device_plan
    host_layers = []
    for j, lay in enumerate(layers):
        if offloaded[j]:
            lay = dict(lay, k_pool=lay["k_pool"].cpu().pin_memory(),
                       v_pool=lay["v_pool"].cpu().pin_memory())
        host_layers.append(lay)
    del layers
    torch.cuda.empty_cache()
    copy = torch.cuda.Stream()
    plan = hylra.OffloadPlan(host_layers, src, k, offloaded)
    # eager steps with the gather and attention kernels timed
    kinds = (hylra.KERNEL_GATHER, hylra.KERNEL_SPARSE_ATTN, hylra.KERNEL_FULL_ATTN,
             hylra.KERNEL_FULL_SCORED)
    ms_eager, kern = timed(lambda: plan.run(copy_stream=copy), args.steps, args.warmup, torch,
                           kinds, hylra)
    ms_off, g = graph_timed(lambda: plan.run(copy_stream=copy), args.steps, args.warmup, torch)
    del g
    B, Hkv, d = wl.batch, wl.num_kv_heads, wl.head_dim
    elt = 4 if wl.dtype == "f32" else 2
    per_gather = 2 * B * Hkv * min(k, wl.blocks) * 128 * d * elt  # every selected slot valid
    gather_us = kern[hylra.KERNEL_GATHER][0] * 1e3 if kern[hylra.KERNEL_GATHER][0] else None
    ceiling = link_ceiling(torch)
    kv_layer = 2 * B * Hkv * wl.blocks * 128 * d * elt
    achieved = per_gather / (gather_us * 1e-6) / 1e9 if gather_us else None
    return {
        "metric": "offloaded hybrid decode attention steps/s (reuse layers' KV in host memory)",
        "value": 1000.0 / ms_off, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_off, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V with planted hot blocks; no trained weights)",
        "config": {"workload": wl.name, "batch": B, "layers": L, "ctx": wl.ctx, "topk": k,
                   "policy": policy_desc, "offloaded_layers": len(reuse)},
        "device_hybrid_ms_per_step": ms_dev,
        "offload_over_device": ms_off / ms_dev,
        "eager_ms_per_step": ms_eager,
        "gather": {"avg_launch_us": gather_us, "bytes_per_launch": per_gather,
                   "achieved_GBps": achieved, "link_peak_GBps": 64.0,
                   "link_peak_note": "PCIe 5.0 x16, one direction",
                   "copy_engine_ceiling_GBps": ceiling,
                   "frac_of_copy_ceiling": achieved / ceiling if achieved else None},
        "kv_bytes_in_host_memory": kv_layer * len(reuse),
        "kv_bytes_on_device": kv_layer * (L - len(reuse)),
        "host_link_bytes_per_step": per_gather * len(reuse),
        "dense_host_link_bytes_per_step": kv_layer * len(reuse),
    }


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_layer_reuse_amd import hylra, synth, workloads as W

    wl = W.get(args.workload)
    if args.ctx:
        import dataclasses
        wl = dataclasses.replace(wl, name="%s_ctx%d" % (wl.name, args.ctx), ctx=args.ctx,
                                 hot_blocks=min(wl.hot_blocks, (args.ctx + 127) // 128))
    if args.batch:
        import dataclasses
        wl = dataclasses.replace(wl, name="%s_b%d" % (wl.name, args.batch), batch=args.batch)
    if args.shard_heads:
        import dataclasses
        P = args.shard_heads
        if P < 1 or wl.num_kv_heads % P:
            print("--shard-heads %d does not divide the %d KV heads" % (P, wl.num_kv_heads),
                  file=sys.stderr)
            sys.exit(2)
        wl = dataclasses.replace(wl, name="%s_tp%d" % (wl.name, P),
                                 num_kv_heads=wl.num_kv_heads // P,
                                 num_q_heads=wl.num_q_heads // P)
    k = args.topk or wl.topk[0]
    L = min(wl.layers, args.layers or wl.layers)
    t0 = time.time()
    layers = None
    if args.profiled or not args.e2e:
        layers = synth.workload_layers(wl, device="cuda", layers=range(L))
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    src, policy_desc, theta = policy_for(wl, hylra, args.theta, L, jump=args.jump,
                                         profiled_layers=layers if args.profiled else None, k=k)
    if args.e2e:
        del layers
        torch.cuda.empty_cache()
        print(json.dumps(e2e(args, wl, k, src, policy_desc)), flush=True)
        return
    if args.offload:
        print(json.dumps(offload_bench(args, wl, k, src, policy_desc, layers, torch, hylra)),
              flush=True)
        return
    n_reset = sum(1 for j, s in enumerate(src) if s == j)

    hybrid = hylra.PolicyPlan(layers, src, k)
    ALL = (hylra.KERNEL_FULL_SCORED, hylra.KERNEL_FULL_ATTN, hylra.KERNEL_SPARSE_ATTN)
    settle_s, settle_gbs = settle(torch, hylra)
    # eager steps with per-kernel HIP events (per-layer latency, roofline)
    ms_eager, kern = timed(hybrid.run, args.steps, args.warmup, torch, ALL, hylra)
    # the step as one HIP graph (how a decode loop replays a static step): value
    ms_h, graph_h = graph_timed(hybrid.run, args.steps, args.warmup, torch)
    p10, p50, p90 = step_percentiles(graph_h, args.steps, torch)
    del graph_h
    result_extra = {"eager_steps_per_s": 1000.0 / ms_eager, "eager_ms_per_step": ms_eager,
                    "settle": {"seconds": settle_s, "read_gbs": settle_gbs},
                    "step_ms_p10_p50_p90": [p10, p50, p90]}
    if not args.skip_baselines:
        full = hylra.FullPlan(layers)
        _, kern_f = timed(full.run, args.steps, args.warmup, torch,
                          (hylra.KERNEL_FULL_ATTN,), hylra)
        ms_f, _ = graph_timed(full.run, args.steps, args.warmup, torch)
        # every layer resets and computes its top-k (the index log makes the
        # library keep scores and selection on layers no one reuses)
        allreset = hylra.PolicyPlan(
            layers, list(range(L)), k,
            idx_log=torch.empty(L, wl.batch, wl.num_kv_heads, k, dtype=torch.int32, device="cuda"))
        ms_a, _ = graph_timed(allreset.run, args.steps, args.warmup, torch)
        result_extra.update({
            "full_steps_per_s": 1000.0 / ms_f,
            "full_ms_per_step": ms_f,
            "all_reset_steps_per_s": 1000.0 / ms_a,
            "hybrid_over_full": ms_f / ms_h,
            "full_attn_no_scores_us": kern_f[hylra.KERNEL_FULL_ATTN][0] * 1e3,
        })

    B, Hkv, T, d = wl.batch, wl.num_kv_heads, wl.ctx, wl.head_dim
    elt = 4 if wl.dtype == "f32" else 2
    full_bytes = 2 * B * Hkv * T * d * elt          # K and V of every token, once
    sparse_bytes = 2 * B * Hkv * min(k, wl.blocks) * 128 * d * elt
    us = lambda kind: (kern[kind][0] * 1e3) if kern[kind][0] is not None else None
    scored_us, plain_us = us(hylra.KERNEL_FULL_SCORED), us(hylra.KERNEL_FULL_ATTN)
    sparse_us = us(hylra.KERNEL_SPARSE_ATTN)
    # the roofline kernel: the reset layer whose index set is used (full
    # attention + fused block scores + top-k); a policy without one falls back
    # to the plain full-attention launch
    full_us = scored_us if scored_us is not None else plain_us
    roof_kind = "full mode with fused block scores and top-k" if scored_us is not None \
        else "full mode without block scores"
    achieved = full_bytes / (full_us * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": 1000.0 / ms_h,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_h,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V with planted hot blocks; no trained weights)",
        "config": {
            "workload": wl.name, "batch": B, "layers": L, "num_q_heads": wl.num_q_heads,
            "num_kv_heads": Hkv, "head_dim": d, "ctx": T, "block": 128, "topk": k,
            "paged": wl.paged, "policy": policy_desc, "resets": n_reset, "reuses": L - n_reset,
        },
        "per_layer_us": {
            "reset_layer_with_topk": scored_us,
            "reset_layer_without_topk": plain_us,
            "reuse_layer": sparse_us,
            "wall_avg": ms_h * 1e3 / L,
        },
        "kernels_us": {hylra.KERNEL_NAMES[kk]: us(kk) for kk in ALL},
        "kernel_launches": {hylra.KERNEL_NAMES[kk]: kern[kk][1] for kk in ALL},
        "sparse_attn_gbs": (sparse_bytes / (sparse_us * 1e-6) / 1e9) if sparse_us else None,
        "roofline": {
            "kernel": ("attn_split_bf16 (d=%d)" if wl.dtype == "bf16" else "attn_split_f32 (d=%d)")
                      % d + ", " + roof_kind,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(wl.name, scored_us is not None),
            "bytes_per_launch": full_bytes,
            "avg_launch_us": full_us,
        },
        "input_generation_s": gen_s,
        # the only speed figure the pages give: end-to-end (projections, MLP and
        # attention), model and hardware not stated -- context, not this metric
        "pages_context": {"speedup_vs_full_attention": 1.45, "scope": "end-to-end LLM decode",
                          "sequence_length": 60000, "hardware": "not stated"},
    }
    out.update(result_extra)
    if not args.skip_baselines:
        ceil = stream_ceiling(torch, hylra)
        out["stream_ceiling"] = ceil
        out["roofline"]["frac_of_stream_ceiling"] = achieved / ceil["gbs"]
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(wl, layers, src, k, args.cpu_seconds)
        out["cpu_baseline"].update(host_cpu())
    else:
        out["cpu_baseline"] = None
    if not args.no_configs and wl.name == "llama3_8b_32k" and L == wl.layers:
        del hybrid, layers
        torch.cuda.empty_cache()
        out["configs"] = measure_configs(args, torch, hylra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
