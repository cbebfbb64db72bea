"""Decoder-layer step throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4|c2|c3|c5]

One step = one nf_layer_step of the whole layer (norm, QKV, RoPE + paged KV
append, decode/prefill attention, O-proj, norm, FFN or experts) over one batch
of seeded synthetic inputs that are resident in HBM before timing starts.  The
default workload is c4 (the Llama-2-70B 1/8 tensor-parallel shard, 1536
decode requests + a 512-token prefill chunk, 2048 tokens); the plan is chosen
by the library's plan search.  Prints one JSON line:
  - value: tokens/s over K steps with cold caches (a 512 MiB scratch read
    before each step, outside the step's events); warm_cache: the same K
    steps back to back;
  - the fraction of the compute-bound optimum (peaks measured in this run);
  - roofline of the dominant kernel (its duration measured with HIP events on
    its own stream during K cold steps; HBM traffic from the committed
    counter summary when its sources are unchanged);
  - comparisons: unsplit, two nano-batches in sequence, two on two streams,
    and the searched plan; search: what the search predicted and measured;
  - a stack of --stack layers (eager and as a HIP graph; unsplit, split in
    sequence, split pipelined across layers) and the single-layer graph;
  - the emulated tensor-parallel all-reduce (copy engines, third stream),
    with and without, unsplit and overlapped;
  - the serving loop, synchronous vs asynchronous control flow, with the
    host's share of each iteration;
  - the KV offload to pinned host memory alone and beside steps, the host
    time to enqueue one step, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
PEAK_BF16_TFLOPS = 2500.0       # MI355X published dense bf16 MFMA
DEFAULT_WORKLOAD = "c4"         # the Llama-2-70B 1/8 shard, 2048 tokens: the largest batch


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ algorithmic work
def kernel_work(kind, wl, batch, plan_sizes, logits=None):
    """(bytes, flops) the method must move/compute in ONE launch of `kind`,
    averaged over the launches of one step (one per nano-batch)."""
    s = wl.shape
    H, F, d = s.hidden, s.ffn, s.head_dim
    nq, nkv = s.n_q_heads, s.n_kv_heads
    Nqkv = (nq + 2 * nkv) * d
    eb = 2 if s.dtype == "bf16" else 4
    T = batch.n_tokens
    n = max(1, len(plan_sizes))
    if kind == "attention":
        # each cached K and V element of every request read once per KV head,
        # q read once, output written once
        keys = 0
        for r in range(batch.n_requests):
            keys += int(batch.req_pos0[r]) + int(batch.req_q_len[r])
        kv = keys * nkv * d * 2 * eb
        qo = 2 * T * nq * d * eb
        flops = 0
        for r in range(batch.n_requests):
            for i in range(int(batch.req_q_len[r])):
                flops += 4 * nq * d * (int(batch.req_pos0[r]) + i + 1)
        return (kv + qo) / n, flops / n
    if kind in ("moe_gemm_gate_up_swiglu", "moe_gemm_down"):
        # every expert that receives a token has its weights read once
        k, E = s.top_k, s.n_experts
        touched = E if logits is None else len(np.unique(np.argsort(-logits, axis=1, kind="stable")[:, :k]))
        A = T * k / n
        if kind == "moe_gemm_gate_up_swiglu":
            byts = touched * 2 * F * H * eb + A * H * eb + A * F * eb
            return byts, 2.0 * A * 2 * F * H
        byts = touched * H * F * eb + A * F * eb + A * H * 4
        return byts, 2.0 * A * H * F
    gemms = {
        "gemm_qkv": (Nqkv, H, False),
        "gemm_o_residual": (H, nq * d, True),
        "gemm_gate_up_swiglu": (2 * F, H, False),
        "gemm_down_residual": (H, F, True),
    }
    if kind in gemms:
        N, K, res = gemms[kind]
        M = T / n
        out_cols = F if kind == "gemm_gate_up_swiglu" else N
        byts = N * K * eb + M * K * eb + M * out_cols * eb + (M * N * eb if res else 0)
        return byts, 2.0 * M * N * K
    return None, None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--plan", default="auto",
                    help="auto (workload default / search), k1 (unsplit), overlap2 (two nano-batches on two "
                         "streams), overlap2:G:A (the same with G GEMM and A attention CUs per XCD), lanes2 (two "
                         "nano-batches, each on a lane of its own) or lanes2:G:A")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the KV-offload measurement (nf_kv_offload alone and beside steps)")
    ap.add_argument("--stack", type=int, default=4,
                    help="also time a stack of this many layers of the workload's shape (nf_stack_step, eager "
                         "and as a HIP graph; unsplit and two nano-batches pipelined across layers); 0: skip")
    ap.add_argument("--traffic", default=None, help="text file with the rocprofv3 FETCH/WRITE bytes per launch")
    ap.add_argument("--no-allreduce", action="store_true",
                    help="skip the emulated tensor-parallel all-reduce measurement")
    ap.add_argument("--no-loop", action="store_true", help="skip the serving-loop measurement (sync vs async)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 5 times (counter calibration) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would run its own "
              "replica of the step); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from intra_operation_overlap_amd import binding as B
    from intra_operation_overlap_amd import workload as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    wl = W.WORKLOADS[args.workload]
    s = wl.shape
    log(f"workload {wl.name}: {wl.description}")
    batch = W.make_batch(wl)
    weights = W.make_weights(wl, "cuda")
    acts = W.make_activations(wl, batch, "cuda")
    k_plain, v_plain = W.make_pool(wl, batch.n_pages, "cuda")
    out = torch.empty_like(acts["x"])
    T = batch.n_tokens
    layer = B.Layer(s, weights, T, int(batch.pos.max()) + 1)
    # a stream of the bench's own: the null stream would synchronise
    # implicitly with the library's CU-masked (blocking) streams
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    sp = stream.cuda_stream
    pool = B.KVPool.from_plain(layer, k_plain, v_plain, sp)
    hb = B.HostBatch(batch, acts["x"].data_ptr(), out.data_ptr(),
                     acts["router_logits"].data_ptr() if "router_logits" in acts else None)

    log("probing peaks")
    peak_tflops = B.probe_mfma_bf16_tflops()
    peak_gbps = B.probe_hbm_read_gbps(4 << 30)
    log(f"measured peaks: bf16 MFMA {peak_tflops:.0f} TFLOP/s, HBM read {peak_gbps:.0f} GB/s")

    host_us = []
    flush_buf = torch.ones(128 << 20, dtype=torch.int32, device="cuda")     # 512 MiB

    def time_steps(n):
        """Warm caches: K back-to-back steps bracketed by two events."""
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        h0 = time.perf_counter()
        for _ in range(n):
            layer.step(pool, hb, sp)
        host_us.append((time.perf_counter() - h0) / n * 1e6)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def time_cold(n):
        """Cold caches: before each step a 512 MiB read of a scratch buffer
        evicts the weights and the KV pool from L2 and the Infinity Cache, so
        the step reads them from HBM (a read rather than a write: a write
        would leave dirty lines for the step to write back).  Each step is
        bracketed by its own events, the flush outside them.  Returns the
        mean and the median ms per step."""
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            torch.sum(flush_buf)
            a.record(stream)
            layer.step(pool, hb, sp)
            b.record(stream)
        torch.cuda.synchronize()
        times = sorted(a.elapsed_time(b) for a, b in evs)
        return sum(times) / n, times[n // 2]

    comparisons, comparisons_warm = {}, {}
    search = None
    half = [T - T // 2, T // 2]
    baselines = (("sequential_unsplit_ms", B.make_plan(1, [T])),
                 ("sequential_split2_ms", B.make_plan(2, half, order=B.NF_ORDER_SEQUENTIAL)),
                 ("overlapped_split2_two_streams_ms", B.make_plan(2, half, n_streams=2)),
                 ("overlapped_split2_lanes_ms", B.make_plan(2, half, order=B.NF_ORDER_LANES, n_streams=2)))
    if args.plan.startswith("overlap2") or args.plan.startswith("lanes2"):
        parts = args.plan.split(":")
        g, a = (int(parts[1]), int(parts[2])) if len(parts) == 3 else (0, 0)
        order = B.NF_ORDER_LANES if parts[0] == "lanes2" else B.NF_ORDER_PIPELINED
        plan = B.make_plan(2, half, order=order, n_streams=2, gemm_cus_per_xcd=g, attn_cus_per_xcd=a)
        layer.set_plan(plan)
    elif args.plan == "k1" or wl.plan_sizes == (T,):
        plan = B.make_plan(1, [T])
        layer.set_plan(plan)
    elif wl.plan_sizes is not None:
        plan = B.make_plan(len(wl.plan_sizes), list(wl.plan_sizes), n_streams=2)
        layer.set_plan(plan)
    else:
        log("plan search")
        t_search = time.perf_counter()
        plan, (best_ms, n_cands) = layer.search(pool, hb, max_count=4, warmup=2, reps=5, stream=sp)
        t_search = time.perf_counter() - t_search
        log(f"searched plan {B.plan_dict(plan)} ({best_ms:.3f} ms, {int(n_cands)} candidates predicted, "
            f"{t_search:.2f} s)")
        rep = layer.search_report()
        search = {"candidates_predicted": int(n_cands), "seconds": round(t_search, 3),
                  "calibration": [{"plan": d, "measured_ms": round(me, 4)} for d, pr, me, cal in rep if cal],
                  "timed": [{"plan": d, "predicted_ms": round(pr, 4), "measured_ms": round(me, 4)}
                            for d, pr, me, cal in rep if not cal]}
        # over the candidates the model ranked (the calibration runs are fitted)
        errs = [abs(pr - me) / me for _, pr, me, cal in rep if me > 0 and not cal]
        search["median_abs_rel_error"] = round(sorted(errs)[len(errs) // 2], 4) if errs else None
        # the baselines the searched plan is compared with: the unsplit step,
        # two nano-batches one after the other on one stream, and the same two
        # nano-batches overlapped on two streams without CU masks; cold
        # caches as for the headline, warm as well
        for key, p in baselines:
            layer.set_plan(p)
            for _ in range(3):
                layer.step(pool, hb, sp)
            comparisons[key] = time_cold(20)[0]
            comparisons_warm[key] = time_steps(20)
            log(f"  {key}: cold {comparisons[key] * 1e3:.1f} us, warm {comparisons_warm[key] * 1e3:.1f} us")
        layer.set_plan(plan)
    plan_sizes = list(plan.sizes)[:plan.count]

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        layer.step(pool, hb, sp)
    torch.cuda.synchronize()

    # dominant kernel: the kind with the largest summed time over a short pass
    layer.profile_enable(True)
    for _ in range(5):
        layer.step(pool, hb, sp)
    prof = layer.profile_read()
    layer.profile_enable(False)
    dominant = max(prof, key=lambda k: prof[k][1])
    log("per-kernel (5 steps): " + ", ".join(f"{k} {v[1] / v[0] * 1e3:.1f}us x{v[0] // 5}" for k, v in prof.items()))

    # timed region: K steps with cold caches, each bracketed by events on
    # the caller stream (the headline); then the same K steps warm, back to
    # back
    log(f"timing {args.steps} steps, cold caches")
    ms, ms_median = time_cold(args.steps)
    log(f"{ms * 1e3:.1f} us per step on the GPU (median {ms_median * 1e3:.1f})")
    ms_warm = time_steps(args.steps)
    log(f"warm caches: {ms_warm * 1e3:.1f} us per step, {host_us[-1]:.1f} us per step to enqueue on the host")
    # the same K cold steps again, with the dominant kernel's own start/end
    # timestamps recorded into HIP events on the stream it runs on (kept out
    # of the throughput pass: the event packets add a few microseconds of
    # queue time around that kernel in every step)
    layer.profile_enable(True, dominant)
    ms_events = time_cold(args.steps)[0]
    dprof = layer.profile_read()
    layer.profile_enable(False)
    launches, dom_ms = dprof[dominant]
    dom_avg_ms = dom_ms / launches
    value = T / (ms * 1e-3)
    cold = {"ms_per_step": round(ms, 5), "median_ms_per_step": round(ms_median, 5), "steps": args.steps,
            "flush": "512 MiB read of a scratch buffer before each step, outside the step's events"}
    warm = {"ms_per_step": round(ms_warm, 5), "steps": args.steps, "tokens_per_s": round(T / (ms_warm * 1e-3), 1),
            "timing": "events around K back-to-back steps"}
    if comparisons:
        comparisons["searched_plan_ms"] = ms
        comparisons_warm["searched_plan_ms"] = ms_warm

    # roofline of the dominant kernel
    logits = acts["router_logits"].float().cpu().numpy() if "router_logits" in acts else None
    byts, flops = kernel_work(dominant, wl, batch, plan_sizes, logits)
    roofline = None
    if byts is not None:
        intensity = flops / byts
        ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
        if intensity < ridge:
            ach = byts / (dom_avg_ms * 1e-3) / 1e9
            roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": round(ach / PEAK_HBM_GBPS, 4)}
        else:
            ach = flops / (dom_avg_ms * 1e-3) / 1e12
            roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        roofline["traffic"] = None
        roofline["kernel"] = dominant
        roofline["avg_launch_us"] = round(dom_avg_ms * 1e3, 2)
        roofline["launches"] = int(launches)
        roofline["ms_per_step_with_kernel_events"] = round(ms_events, 5)
        roofline["algorithmic_bytes_per_launch"] = int(byts)
        roofline["traffic"] = measured_traffic(args.traffic or os.path.join(
            ROOT, "profiles", f"traffic_{dominant}_{wl.name}.txt"), dominant)

    # fraction of the compute-bound optimum: tokens/s / (peak / FLOPs per token)
    fpt = W.layer_flops_per_token(s)
    optimum = peak_tflops * 1e12 / fpt
    frac_opt = value / optimum

    # host cost of one step: the enqueue of a single nf_layer_step with the
    # device idle (in the timed loop the host also waits for the staging
    # buffer of the step two back, so that figure includes device time)
    host_idle = []
    for _ in range(10):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        layer.step(pool, hb, sp)
        host_idle.append((time.perf_counter() - h0) * 1e6)
    torch.cuda.synchronize()
    host = {"step_enqueue_us": round(sorted(host_idle)[5], 1),
            "step_enqueue_frac_of_step": round(sorted(host_idle)[5] / (ms_warm * 1e3), 4)}
    log(f"host enqueue of one step with the device idle: {host['step_enqueue_us']} us "
        f"({100 * host['step_enqueue_frac_of_step']:.1f}% of the step)")

    offload = None
    if not args.no_offload:
        offload = offload_measure(batch, layer, pool, pool.k, hb, sp, ms_warm)

    stack = None
    if args.stack > 0:
        stack = stack_measure(args.stack, wl, batch, layer, pool, acts, plan, sp)
        layer.set_plan(plan)

    single_graph = graph_single_layer(layer, pool, hb, plan, sp, ms_warm)

    allreduce = None
    if not args.no_allreduce and s.n_experts == 1:
        allreduce = allreduce_measure(layer, pool, hb, T, sp)
        layer.set_plan(plan)

    loop = None
    if not args.no_loop and s.n_experts == 1:
        loop = loop_measure(wl, layer, sp)
        layer.set_plan(plan)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, batch, weights, acts, k_plain, v_plain)

    line = {
        "metric": "decoder-layer tokens/s on 1 MI355X + fraction of compute-bound optimal",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "tokens": T,
                   "requests": batch.n_requests, "hidden": s.hidden, "q_heads": s.n_q_heads,
                   "kv_heads": s.n_kv_heads, "head_dim": s.head_dim, "ffn": s.ffn, "experts": s.n_experts,
                   "plan": B.plan_dict(plan)},
        "frac_compute_optimal": round(frac_opt, 4),
        "peaks_measured": {"bf16_mfma_tflops": round(peak_tflops, 1), "hbm_read_gbps": round(peak_gbps, 1)},
        "flops_per_token": fpt,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cold_cache": cold,
        "warm_cache": warm,
    }
    if comparisons:
        line["comparisons"] = {k: round(v, 5) for k, v in comparisons.items()}
        line["comparisons"]["caches"] = "cold"
        line["comparisons_warm"] = {k: round(v, 5) for k, v in comparisons_warm.items()}
    line["host"] = host
    if single_graph is not None:
        line["single_layer_graph"] = single_graph
    if search is not None:
        line["search"] = search
    if allreduce is not None:
        line["allreduce_emulation"] = allreduce
    if loop is not None:
        line["serving_loop"] = loop
    if offload is not None:
        line["kv_offload"] = offload
    if stack is not None:
        line["stack"] = stack
    print(json.dumps(line), flush=True)


def graph_single_layer(layer, pool, hb, plan, sp, step_ms, steps=20):
    """The single-layer step recorded as a HIP graph (a one-layer stack):
    time per replay and host time to launch one replay."""
    import torch
    from intra_operation_overlap_amd import binding as B
    if plan.n_streams == 2 and (plan.gemm_cus_per_xcd or plan.attn_cus_per_xcd):
        return None
    g = B.StackGraph([layer], [pool], hb, sp)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        g.launch(sp)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    h0 = time.perf_counter()
    for _ in range(steps):
        g.launch(sp)
    host = (time.perf_counter() - h0) / steps * 1e6
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    hs = []
    for _ in range(10):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        g.launch(sp)
        hs.append((time.perf_counter() - h0) * 1e6)
    torch.cuda.synchronize()
    g.close()
    res = {"ms_per_step": round(ms, 5), "eager_ms_per_step": round(step_ms, 5),
           "host_launch_us_idle": round(sorted(hs)[5], 1), "host_us_per_step_in_loop": round(host, 1)}
    log(f"single-layer graph: {ms * 1e3:.1f} us per step (eager {step_ms * 1e3:.1f}), launch {res['host_launch_us_idle']} us")
    return res


def allreduce_measure(layer, pool, hb, T, sp, steps=20):
    """The network-bound third resource, emulated on one GPU: after the
    O-projection and the down projection of every nano-batch, its rows make a
    send and a receive leg (2 x T_j x H elements) on a third stream, on the
    copy engines (nf_layer_set_allreduce_emulation mode 1).  Times the
    unsplit step with and without it, and overlapped plans with it (warm
    caches, events around `steps` steps)."""
    import torch
    from intra_operation_overlap_amd import binding as B
    stream = torch.cuda.current_stream()

    def timed():
        for _ in range(3):
            layer.step(pool, hb, sp)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            layer.step(pool, hb, sp)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    half = [T - T // 2, T // 2]
    plans = {"unsplit": B.make_plan(1, [T]),
             "split2_sequential": B.make_plan(2, half, order=B.NF_ORDER_SEQUENTIAL),
             "split2_pipelined_two_streams": B.make_plan(2, half, n_streams=2),
             "split2_deep_two_streams": B.make_plan(2, half, order=B.NF_ORDER_DEEP, n_streams=2),
             "split2_deep_one_stream": B.make_plan(2, half, order=B.NF_ORDER_DEEP),
             "split2_lanes": B.make_plan(2, half, order=B.NF_ORDER_LANES, n_streams=2),
             "split3_lanes": B.make_plan(3, [T // 3, T // 3, T - 2 * (T // 3)], order=B.NF_ORDER_LANES,
                                         n_streams=2)}
    res = {"mode": "copy engines", "bytes_per_step": None, "ms_per_step": {}}
    layer.set_allreduce_emulation(0)
    layer.set_plan(plans["unsplit"])
    res["ms_per_step"]["unsplit_without_allreduce"] = round(timed(), 5)
    layer.set_allreduce_emulation(1)
    for name, p in plans.items():
        layer.set_plan(p)
        res["ms_per_step"][name] = round(timed(), 5)
    layer.set_allreduce_emulation(0)
    H = layer.shape.hidden
    res["bytes_per_step"] = 2 * 2 * 2 * T * H * (2 if layer.shape.dtype == B.NF_BF16 else 4)
    log("all-reduce emulation: " + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in res["ms_per_step"].items()))
    return res


def loop_measure(wl, layer, sp, n_requests=96):
    """The serving loop (nf_loop_*) on the bench's layer and a pool of its
    own: requests with prompts of 64-512 tokens and 16-64 generated
    positions, a third of them ended early by an end marker in an input row,
    2048 tokens and 512 prompt tokens per iteration; synchronous control flow
    (flags read after every iteration) against asynchronous (iteration i + 1
    launched before i's flags are read).  Each variant runs twice; the second
    run is reported."""
    import torch
    from intra_operation_overlap_amd import binding as B
    s = wl.shape
    rng = np.random.Generator(np.random.PCG64(17))
    reqs = []
    top = min(512, int(layer.shape.max_pos) - 65)
    for i in range(n_requests):
        prompt = int(rng.integers(min(64, top), top + 1))
        max_len = prompt + int(rng.integers(16, 65))
        g = torch.Generator(device="cuda")
        g.manual_seed(17000 + i)
        rows = torch.randn(max_len, s.hidden, generator=g, device="cuda").to(torch.bfloat16)
        if i % 3 == 0:
            rows[int(rng.integers(prompt, max_len - 1)), 0] = 200.0
        reqs.append((prompt, rows))
    need = sum(-(-r.shape[0] // 16) for _, r in reqs)
    n_pages = need // 2                                   # about half the requests fit at once
    kp = torch.zeros(n_pages, s.n_kv_heads, 16, s.head_dim, dtype=torch.bfloat16, device="cuda")
    pool = B.KVPool.from_plain(layer, kp, kp, sp)
    del kp
    max_tokens = min(2048, int(layer.shape.max_tokens))
    layer.set_plan(B.make_plan(1, [0]))
    out = {}
    for name, async_ in (("sync", False), ("async", True)):
        for rep in range(2):
            loop = B.Loop(layer, pool, max_tokens, 512, async_, 100.0)
            outs = [torch.empty_like(r) for _, r in reqs]
            for (prompt, rows), o in zip(reqs, outs):
                loop.add(prompt, rows, o)
            st = loop.run(sp)
            torch.cuda.synchronize()
            loop.close()
        it = max(1, st["iterations"])
        out[name] = {"iterations": st["iterations"], "tokens": st["tokens"], "wasted_tokens": st["wasted_tokens"],
                     "wall_ms": round(st["wall_us"] / 1e3, 3), "wall_us_per_iteration": round(st["wall_us"] / it, 1),
                     "host_us_per_iteration": round(st["host_us"] / it, 1),
                     "host_share_of_wall": round(st["host_us"] / st["wall_us"], 4),
                     "tokens_per_s": round(st["tokens"] / (st["wall_us"] * 1e-6), 1)}
        log(f"serving loop {name}: {st['iterations']} iterations, {st['wall_us'] / 1e3:.1f} ms, host "
            f"{st['host_us'] / it:.1f} us per iteration ({100 * st['host_us'] / st['wall_us']:.1f}% of wall), "
            f"{st['wasted_tokens']} wasted tokens")
    pool.close()
    out["requests"] = n_requests
    out["pool_pages"] = n_pages
    return out


def offload_measure(batch, layer, pool, k_pool, hb, sp, step_ms, reps=10):
    """nf_kv_offload of the KV pages of the batch's first eighth of requests
    (the pages the step only reads), to pinned host memory on a stream of its
    own: alone, and beside as many back-to-back steps on the main stream as
    span it (medians)."""
    import torch
    from intra_operation_overlap_amd import binding as B
    R = batch.n_requests
    written = set()
    for r in range(R):
        p0, ql, st = int(batch.req_pos0[r]), int(batch.req_q_len[r]), int(batch.page_indptr[r])
        for p in range(p0, p0 + ql):
            written.add(int(batch.page_indices[st + p // 16]))
    pages = [int(p) for r in range(max(1, R // 8))
             for p in batch.page_indices[batch.page_indptr[r]:batch.page_indptr[r + 1]] if int(p) not in written]
    if not pages:
        return None
    pages = np.array(pages, np.int32)
    n = len(pages)
    hk = torch.empty((n,) + tuple(k_pool.shape[1:]), dtype=k_pool.dtype, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    nbytes = 2 * hk.numel() * hk.element_size()
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    log(f"KV offload: {n} pages, {nbytes / 2**20:.0f} MiB")

    def ev():
        return torch.cuda.Event(enable_timing=True)
    alone = []
    for _ in range(reps):
        a0, a1 = ev(), ev()
        a0.record(side)
        B.kv_offload(pool, pages, hk, hv, side.cuda_stream)
        a1.record(side)
        torch.cuda.synchronize()
        alone.append(a0.elapsed_time(a1))
    med = lambda v: sorted(v)[len(v) // 2]
    # beside steps: enough back-to-back steps on the main stream to span the
    # whole offload, so their mean is the offload's amortised cost per step
    m = int(med(alone) / step_ms) + 2
    beside, steps = [], []
    for _ in range(max(3, reps // 2)):
        torch.cuda.synchronize()
        a0, a1, s0, s1 = ev(), ev(), ev(), ev()
        a0.record(side)
        s0.record(main)
        B.kv_offload(pool, pages, hk, hv, side.cuda_stream)
        for _ in range(m):
            layer.step(pool, hb, sp)
        a1.record(side)
        s1.record(main)
        torch.cuda.synchronize()
        beside.append(a0.elapsed_time(a1))
        steps.append(s0.elapsed_time(s1) / m)
    res = {"pages": n, "bytes": int(nbytes), "alone_ms": round(med(alone), 4),
           "alone_gbps": round(nbytes / (med(alone) * 1e-3) / 1e9, 1),
           "beside_steps_ms": round(med(beside), 4),
           "beside_steps_gbps": round(nbytes / (med(beside) * 1e-3) / 1e9, 1),
           "steps_beside": m, "step_ms_alone": round(step_ms, 5),
           "step_ms_beside_offload": round(med(steps), 5),
           "requests": max(1, R // 8), "host_memory": "pinned"}
    log(f"  alone {res['alone_gbps']} GB/s; beside {m} steps {res['beside_steps_gbps']} GB/s, step "
        f"{res['step_ms_beside_offload'] * 1e3:.1f} us (alone {step_ms * 1e3:.1f})")
    return res


def stack_measure(n, wl, batch, layer0, pool0, acts, main_plan, sp, steps=10):
    """A stack of n layers of the workload's shape: layer 0 is the bench's
    layer, layers 1.. have their own seeded weights and KV pools.  Times
    nf_stack_step eagerly and as a replayed HIP graph, with the unsplit plan
    and with two nano-batches on two streams pipelined across layers; returns
    milliseconds per layer (events around `steps` stack steps).  The same
    two nano-batches run one after the other on one stream are the baseline
    the pipelined overlap is compared with."""
    import torch
    from intra_operation_overlap_amd import binding as B
    from intra_operation_overlap_amd import workload as W
    s = wl.shape
    T = batch.n_tokens
    log(f"stack of {n} layers")
    layers, pools, keep = [layer0], [pool0], []
    for l in range(1, n):
        seed = wl.seed + 1000 * l
        w = W.make_weights(wl, "cuda", seed=seed)
        k, v = W.make_pool(wl, batch.n_pages, "cuda", seed=seed)
        L = B.Layer(s, w, T, int(batch.pos.max()) + 1)
        layers.append(L)
        pools.append(B.KVPool.from_plain(L, k, v, sp))
        torch.cuda.synchronize()
        del k, v
        keep.append(w)
    out = torch.empty_like(acts["x"])
    hb = B.HostBatch(batch, acts["x"].data_ptr(), out.data_ptr(),
                     acts["router_logits"].data_ptr() if "router_logits" in acts else None)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps / n

    res = {}
    half = [T - T // 2, T // 2]
    for name, plan in (("unsplit", B.make_plan(1, [T])),
                       ("split2_sequential", B.make_plan(2, half, order=B.NF_ORDER_SEQUENTIAL)),
                       ("overlap2_pipelined", B.make_plan(2, half, n_streams=2)),
                       ("lanes2", B.make_plan(2, half, order=B.NF_ORDER_LANES, n_streams=2))):
        for L in layers:
            L.set_plan(plan)
        res[f"{name}_eager"] = timed(lambda: B.stack_step(layers, pools, hb, sp))
        g = B.StackGraph(layers, pools, hb, sp)
        res[f"{name}_graph"] = timed(lambda: g.launch(sp))
        if name == "unsplit":
            hs = []
            for _ in range(10):
                torch.cuda.synchronize()
                h0 = time.perf_counter()
                g.launch(sp)
                hs.append((time.perf_counter() - h0) * 1e6)
            torch.cuda.synchronize()
            graph_launch_us = sorted(hs)[5]
        g.close()
        log(f"  {name}: eager {res[name + '_eager'] * 1e3:.1f} us/layer, graph {res[name + '_graph'] * 1e3:.1f} us/layer")
    for L in layers:
        L.set_plan(main_plan)
    for L in layers[1:]:
        L.close()
    return {"layers": n, "ms_per_layer": {k: round(v, 5) for k, v in res.items()},
            "tokens_per_s_per_layer": {k: round(T / (v * 1e-3), 1) for k, v in res.items()},
            "graph_launch_host_us": round(graph_launch_us, 1), "steps": steps}


# Sources that decide the HBM traffic of each kernel kind; a counter summary
# records their hash and is ignored once any of them changes.
_CSRC = os.path.join(ROOT, "intra_operation_overlap_amd", "csrc")
_COMMON = ["nf_device.h"]
KERNEL_SOURCES = {
    "attention": ["attention.hip"] + _COMMON,
    "gemm_qkv": ["gemm.hip"] + _COMMON,
    "gemm_o_residual": ["gemm.hip"] + _COMMON,
    "gemm_gate_up_swiglu": ["gemm.hip"] + _COMMON,
    "gemm_down_residual": ["gemm.hip"] + _COMMON,
    # the streaming kernel's configuration is chosen in gemm.hip
    "moe_gemm_gate_up_swiglu": ["gemm_stream.hip", "gemm.hip"] + _COMMON,
    "moe_gemm_down": ["gemm_stream.hip", "gemm.hip"] + _COMMON,
}


def source_hash(kind):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kind, []):
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path, kind):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by the copy-kernel calibration factor), or None
    when there is none or the kernel's sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    fields = {}
    for ln in open(path):
        if ":" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split(":", 1)
            fields[k.strip()] = v.strip()
    if kind not in KERNEL_SOURCES or fields.get("source_sha256") != source_hash(kind) or "bytes_per_launch" not in fields:
        return None
    return int(float(fields["bytes_per_launch"]))


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)


def cpu_baseline(wl, batch, weights, acts, k_pool, v_pool, budget_s=20.0):
    """The CPU oracle, as it stands, on a bounded sample of this workload's
    requests (rows are independent, so a subset is a fair per-token rate).
    k_pool / v_pool: the generator's plain paged caches [P][nkv][16][d]."""
    import torch
    import oracle
    from intra_operation_overlap_amd import workload as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    wn = {k: v.detach().to("cpu", torch.float32).numpy() for k, v in weights.items()}
    rng = np.random.Generator(np.random.PCG64(1))
    reqs = list(range(batch.n_requests))
    rng.shuffle(reqs)
    done_tokens, elapsed, used = 0, 0.0, []
    chunk = 8
    while reqs and elapsed < budget_s:
        pick = sorted(reqs[:chunk])
        reqs = reqs[chunk:]
        sub, rows = W.sub_batch(batch, pick)
        pages = torch.as_tensor(np.asarray(sub.page_indices, np.int64), device=k_pool.device)
        kp, vp = W.to_f64(k_pool[pages]), W.to_f64(v_pool[pages])
        ridx = torch.as_tensor(rows, device="cuda")
        bd = dict(x=W.to_f64(acts["x"][ridx]), req_q_start=sub.req_q_start, req_q_len=sub.req_q_len,
                  req_pos0=sub.req_pos0, pos=sub.pos, page_indptr=sub.page_indptr,
                  page_indices=np.arange(len(sub.page_indices)))
        if "router_logits" in acts:
            bd["router_logits"] = W.to_f64(acts["router_logits"][ridx])
        t0 = time.perf_counter()
        oracle.layer_step(wl.shape.as_dict(), wn, bd, kp, vp)
        elapsed += time.perf_counter() - t0
        done_tokens += sub.n_tokens
        used += pick
    return {"value": round(done_tokens / elapsed, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(used)} of {batch.n_requests} requests ({done_tokens} tokens) of workload {wl.name}, "
                      f"{elapsed:.1f} s of fp64 numpy work"}


if __name__ == "__main__":
    main()
