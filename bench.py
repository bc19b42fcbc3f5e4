"""Benchmark of the AWQ int4 MoE expert stage for small-batch decode on one MI355X.

Headline workload: the 512-expert rank-share layer (hidden 2560, local
intermediate 160, top-k 10, int4 group 32, 4-byte records), M = 1 token,
the same 10 hot experts on every call, 48 calls per HIP-graph replay with a
fresh fp16 x ~ N(0,1) and softmax router weights per call (PR #522,
Operator results: 48 calls per graph replay). One *step* is one replay: 48
awq_moe_decode calls (W13+SwiGLU, then W2+reduction; two launches each).

Printed: one JSON line with the layer's achieved weight bandwidth (touched
weight + record bytes / layer time), per-kernel times from graphs of one
kernel, the roofline of the dominant (longer) kernel from HIP events on its
stream, side measurements (cold M=1 with 3-byte records over 480 rotating
experts; M=8 with a shared expert pool and with 80 distinct experts), two
live references (a 1 GiB streaming read and the per-launch floor of a
graph of empty launches), and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from awq_int4_mixture_amd import inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0
CALLS = 48
SEED = 2026
E, K_TOP, H, I = 512, 10, 2560, 160


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--only", default="", help="comma list of workloads: m1_hot,m1_cold,m8_pool,m8_distinct,p128,p256,p512,p1024,p4096,stack48,stack48_gemv")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return p.parse_args()


class Workload:
    """48 calls of one configuration, all inputs resident on the device."""

    def __init__(self, name, abi, torch, dims, bank, ids_calls, M, rng, per_expert):
        self.name, self.dims, self.bank, self.M = name, dims, bank, M
        dev = bank.device
        self.x = [torch.from_numpy(inputs.activations(rng, M, H)).to(dev) for _ in range(CALLS)]
        self.ids = [torch.from_numpy(np.ascontiguousarray(ids_calls[c])).to(dev) for c in range(CALLS)]
        self.w = [torch.from_numpy(inputs.router_weights(rng, M, K_TOP)).to(dev) for _ in range(CALLS)]
        self.out = torch.empty((M, H), dtype=torch.float16, device=dev)
        self.ws = [abi.alloc_workspace(dims, M, K_TOP, dev) for _ in range(CALLS)]
        self.dec = abi.Decoder(dims, bank, K_TOP, max_tokens=M)
        self.routes = [abi.alloc_route(M * K_TOP, dev) for _ in range(CALLS)]
        self.ids_np = [np.asarray(ids_calls[c]) for c in range(CALLS)]
        distinct = [len(np.unique(a)) for a in self.ids_np]
        self.distinct_mean = float(np.mean(distinct))
        self.w13_bytes = [d * per_expert["w13"] for d in distinct]
        self.w2_bytes = [d * per_expert["w2"] for d in distinct]


def measure_stack(abi, torch, steps, warmup, layers=48, M=8, router="given"):
    """One decode step of a stack of 512-expert layers (3-byte records, banks
    drawn on the device). Per layer, with router="given": residual update +
    RMS norm and router top-k over fp32 N(0,1) logits (one launch), then the
    stage (two launches). With router="gemv": residual update + RMS norm +
    logits = x . Wr^T from fp16 router weights N(0,1)/sqrt(H) (one launch),
    router top-k (one launch), then the stage. One graph replay = one step."""
    dims = abi.make_dims(E, H, I, 3)
    Lq = abi.awq_moe_bank_layout_query(dims)
    sections = [(int(Lq.w13_meta_off), (H // 32) * 2 * I), (int(Lq.w2_meta_off), (I // 32) * H)]
    banks = [inputs.device_bank(SEED + 9000 + l, E, sections, int(Lq.expert_bytes), 3) for l in range(layers)]
    rng = inputs.call_rng(SEED, 900)
    if router == "gemv":
        wr = [inputs.device_router_weights(SEED + 9500 + l, E, H) for l in range(layers)]
        logits = [torch.empty((M, E), dtype=torch.float32, device="cuda") for _ in range(layers)]
    else:
        logits = [torch.from_numpy(inputs.router_logits(rng, M, E)).to("cuda") for _ in range(layers)]
    r0 = torch.from_numpy(inputs.activations(rng, M, H)).to("cuda")
    rbuf = [torch.empty_like(r0) for _ in range(2)]
    xbuf = torch.empty_like(r0)
    outs = [torch.empty_like(r0) for _ in range(layers)]
    ids = [torch.empty((M, K_TOP), dtype=torch.int32, device="cuda") for _ in range(layers)]
    wts = [torch.empty((M, K_TOP), dtype=torch.float32, device="cuda") for _ in range(layers)]
    ws = abi.alloc_workspace(dims, M, K_TOP, "cuda")

    def step():
        r = r0
        for l in range(layers):
            rn = rbuf[l % 2]
            delta = None if l == 0 else outs[l - 1]
            if router == "gemv":
                abi.awq_moe_router_gemv(r, wr[l], delta, r_next=rn, x=xbuf, logits=logits[l])
                abi.awq_moe_router_topk(logits[l], K_TOP, ids=ids[l], w=wts[l])
            else:
                abi.awq_moe_router_residual(logits[l], K_TOP, r, delta, ids=ids[l], w=wts[l], r_next=rn, x=xbuf)
            abi.awq_moe_decode(dims, banks[l], xbuf, ids[l], wts[l], out=outs[l], workspace=ws)
            r = rn

    step()
    torch.cuda.synchronize()
    distinct = [len(np.unique(t.cpu().numpy())) for t in ids]
    g = capture(torch, step)
    ms = time_graph(torch, g, steps, warmup)
    del g
    touched = float(sum(distinct)) * float(Lq.expert_bytes)
    out = {"layers": layers, "M": M, "step_us": ms * 1e3, "layer_us": ms * 1e3 / layers,
           "distinct_experts_per_layer": float(np.mean(distinct)), "touched_bytes_per_step": touched,
           "gbs": touched / (ms * 1e6), "pct_peak": 100.0 * touched / (ms * 1e6) / HBM_PEAK_GBS,
           "resident_bank_bytes": int(Lq.total_bytes) * layers, "launches_per_layer": 4 if router == "gemv" else 3,
           "router": router}
    if router == "gemv":
        out["router_weight_bytes_per_step"] = layers * E * H * 2
        del wr
    del banks
    torch.cuda.empty_cache()
    return out


def per_expert_bytes(abi, dims):
    L = abi.awq_moe_bank_layout_query(dims)
    return {"w13": int(L.w2_off - L.w13_off), "w2": int(L.expert_bytes - L.w2_off)}


def capture(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps, warmup):
    """Mean ms per replay, from HIP events recorded on the replay stream."""
    s = torch.cuda.current_stream()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(s)
    for _ in range(reps):
        g.replay()
    t1.record(s)
    t1.synchronize()
    return t0.elapsed_time(t1) / reps


def measure(abi, torch, wl: Workload, steps, warmup):
    def full():
        for c in range(CALLS):
            wl.dec(wl.x[c], wl.ids[c], wl.w[c], out=wl.out)

    def route():
        for c in range(CALLS):
            abi.awq_moe_route_compact(wl.ids[c], E, out=wl.routes[c])

    def w13():
        for c in range(CALLS):
            abi.awq_moe_w13_swiglu(wl.dims, wl.bank, wl.x[c], wl.ids[c], workspace=wl.ws[c])

    def w2():
        for c in range(CALLS):
            abi.awq_moe_w2_reduce(wl.dims, wl.bank, wl.ids[c], wl.w[c], wl.ws[c], out=wl.out)

    route()
    torch.cuda.synchronize()
    res = {}
    # "layer" = awq_moe_decode (two launches, one workgroup per slot and tile);
    # "route" = the standalone awq_moe_route_compact kernel, not part of the layer.
    graphs = {name: capture(torch, fn) for name, fn in (("layer", full), ("route", route), ("w13", w13), ("w2", w2))}
    for name, g in graphs.items():
        ms = time_graph(torch, g, steps, warmup)
        res[name + "_us"] = ms * 1e3 / CALLS
        if name == "layer":
            res["step_ms"] = ms
    # 7 further samples per graph, in alternating (ABBA) order, for the median and the minimum
    per_sample = max(steps // 7, 10)
    samples = {name: [] for name in graphs}
    names = list(graphs)
    for r in range(7):
        for name in (names if r % 2 == 0 else names[::-1]):
            samples[name].append(time_graph(torch, graphs[name], per_sample, 2) * 1e3 / CALLS)
    for name, v in samples.items():
        res[name + "_us_median7"] = float(np.median(v))
        res[name + "_us_min7"] = float(np.min(v))
    del graphs
    w13b = float(np.mean(wl.w13_bytes))
    w2b = float(np.mean(wl.w2_bytes))
    res.update(
        M=wl.M, distinct_experts_per_call=wl.distinct_mean,
        w13_bytes_per_call=w13b, w2_bytes_per_call=w2b,
        w13_gbs=w13b / (res["w13_us"] * 1e3), w2_gbs=w2b / (res["w2_us"] * 1e3),
        layer_gbs=(w13b + w2b) / (res["layer_us"] * 1e3),
    )
    for k in ("w13", "w2", "layer"):
        res[k + "_pct_peak"] = 100.0 * res[k + "_gbs"] / HBM_PEAK_GBS
    return res


def measure_prefill(abi, torch, dims, bank, M, steps, warmup, per_expert, calls=8):
    """Indexed prefill of M tokens (awq_moe_prefill, four launches) on the
    512-expert rank layer: each token picks 10 distinct experts uniformly.
    One graph replays `calls` calls with different inputs; reported per call."""
    dev = bank.device
    xs, idss, ws_, distinct = [], [], [], []
    for c in range(calls):
        rng = inputs.call_rng(SEED, 700 + 16 * M + c)
        xs.append(torch.from_numpy(inputs.activations(rng, M, H)).to(dev))
        ids = inputs.ids_distinct(rng, M, K_TOP, E)
        distinct.append(len(np.unique(ids)))
        idss.append(torch.from_numpy(ids).to(dev))
        ws_.append(torch.from_numpy(inputs.router_weights(rng, M, K_TOP)).to(dev))
    out = torch.empty((M, H), dtype=torch.float16, device=dev)
    work = abi.alloc_prefill_workspace(dims, M, K_TOP, dev)

    def run():
        for c in range(calls):
            abi.awq_moe_prefill(dims, bank, xs[c], idss[c], ws_[c], out=out, workspace=work)

    g = capture(torch, run)
    ms = time_graph(torch, g, steps, warmup)
    samples = [time_graph(torch, g, max(steps // 7, 5), 2) for _ in range(7)]
    del g
    n = M * K_TOP
    wbytes = float(np.mean(distinct)) * (per_expert["w13"] + per_expert["w2"])
    flops = 6.0 * n * H * I
    us = ms * 1e3 / calls
    res = {"M": M, "call_us": us, "call_us_median7": float(np.median(samples)) * 1e3 / calls,
           "call_us_min7": float(np.min(samples)) * 1e3 / calls,
           "distinct_experts_per_call": float(np.mean(distinct)), "weight_bytes_per_call": wbytes,
           "weight_gbs": wbytes / (us * 1e3), "weight_pct_peak": 100.0 * wbytes / (us * 1e3) / HBM_PEAK_GBS,
           "row_result_bytes_per_call": float(n * H * 4 * 2 + n * I * 2 * 2),
           "tflops": flops / (us * 1e-6) / 1e12, "tokens_per_s": M / (us * 1e-6)}
    del work
    return res


def stage_source_hash() -> str:
    """sha256[:16] over the stage kernels' device sources (kernels.hip, then device_util.h)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("kernels.hip", "device_util.h"):
        h.update(open(os.path.join(ROOT, "awq_int4_mixture_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, summary: str = "pmc_traffic_m1_hot.txt"):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a 1 GiB copy in the same run), or None
    when the summary is missing or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    h = stage_source_hash()
    for line in open(path):
        parts = [p.strip() for p in line.split("|")]
        if len(parts) == 4 and parts[0] == "TRAFFIC" and kernel in parts[1] and parts[3] == f"source {h}":
            return float(parts[2].split()[0])
    return None


def copy_ceiling(torch, nbytes=1 << 30, reps=20):
    """Device-to-device copy of a known size: a reference read+write rate."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    t1.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del a, b
    return {"bytes_moved": 2 * nbytes, "us": ms * 1e3, "gbs": 2 * nbytes / (ms * 1e6)}


def read_ceiling(torch, nbytes=1 << 30, reps=20):
    """1 GiB streaming reads (row sums of float32 tiles of 1, 4 and 16 KiB, and
    a full sum): the best rate is reported as a reference read rate."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    best = None
    for cols in (256, 1024, 4096, None):
        fn = (lambda: a.sum()) if cols is None else (lambda c=cols: a.view(-1, c).sum(dim=1))
        r = fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            r = fn()
        t1.record()
        t1.synchronize()
        ms = t0.elapsed_time(t1) / reps
        gbs = nbytes / (ms * 1e6)
        if best is None or gbs > best["gbs"]:
            best = {"bytes_read": nbytes, "us": ms * 1e3, "gbs": gbs,
                    "op": "sum" if cols is None else f"row sums of {cols} float32"}
        del r
    del a
    return best


def launch_floor(torch, steps=50, warmup=5):
    """Per-launch time of a HIP graph of 48 launches that do (almost) nothing:
    the floor under any one-launch kernel timed the same way."""
    t = torch.zeros(64, dtype=torch.float32, device="cuda")
    g = capture(torch, lambda: [t.add_(1.0) for _ in range(CALLS)])
    ms = time_graph(torch, g, steps, warmup)
    del g
    return {"us_per_launch": ms * 1e3 / CALLS}


def cpu_baseline(bi, ids_calls, rng_seed, budget_s=12.0):
    """The float64 oracle on the headline workload's calls (cycling through the
    48 expert sets with fresh inputs) for about budget_s seconds."""
    from threadpoolctl import threadpool_limits

    from oracle import ref as R
    rng = inputs.call_rng(rng_seed, 77)
    per_call = K_TOP * (409_600 + 102_400 + 204_800 + 51_200)
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            x = inputs.activations(rng, 1, H)
            w = inputs.router_weights(rng, 1, K_TOP)
            R.moe_stage(x, ids_calls[done % CALLS], w, E, bi.expert)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": round(per_call * done / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} M=1 calls on the hot-expert sets (4-byte records), float64 NumPy on one "
                      f"thread, dequantisation of the touched experts included, {dt:.1f} s",
            "layer_us": round(dt / done * 1e6, 1)}


def stage_kernel_names(M, H=H, I=I, topk=K_TOP, rb=4):
    """Names of the W13 and W2 kernels the library launches for a shape (the
    launchers' rules: lane pairs for W13 when every workgroup has a CU of its
    own, W2 slot segments of I/8 lanes at inter <= 256)."""
    pair = 2 * (H // 8) <= 1024 and (2 * I // 16) * M * topk <= 256
    w13 = f"w13_swiglu_pair_kernel<{rb}>" if pair else f"w13_swiglu_kernel<{rb}>"
    if I <= 256:
        spw = 64 // (I // 8)
        spw = max(v for v in (2, 3, 4, 5, 8, 16) if v <= spw)
        w2 = f"w2_reduce_seg_kernel<{rb}, {spw}>"
    else:
        w2 = f"w2_reduce_kernel<{rb}, 1>"
    return w13, w2


def roofline(head):
    """HBM roofline of the longer of the two stage kernels at the headline workload."""
    k = "w2" if head["w2_us"] >= head["w13_us"] else "w13"
    w13_name, w2_name = stage_kernel_names(head["M"])
    name = {"w13": w13_name, "w2": w2_name}[k]
    gbs = head[k + "_gbs"]
    return {
        "bound": "hbm",
        "kernel": name,
        "achieved": round(gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "traffic": recorded_traffic(name),
        "algorithmic_bytes_per_launch": head[k + "_bytes_per_call"],
        "avg_launch_us": round(head[k + "_us"], 3),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    from awq_int4_mixture_amd import abi
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    prefill_wls = {"p128": 128, "p256": 256, "p512": 512, "p1024": 1024, "p4096": 4096}
    only = set(filter(None, args.only.split(","))) or {"m1_hot", "m1_cold", "m8_pool", "m8_distinct", "stack48",
                                                       "stack48_gemv", *prefill_wls}

    t_gen = time.perf_counter()
    bi = inputs.bank_inputs(SEED, E, H, I)
    banks = {}
    for rb in (4, 3):
        if rb == 4 and "m1_hot" not in only:
            continue
        if rb == 3 and not ({"m1_cold", "m8_pool", "m8_distinct", *prefill_wls} & only):
            continue
        dims = abi.make_dims(E, H, I, rb)
        banks[rb] = (dims, torch.from_numpy(abi.prepare_from_inputs(dims, bi)).to("cuda"))
    t_gen = time.perf_counter() - t_gen

    rng = inputs.call_rng(SEED, 1)
    hot = inputs.hot_experts(SEED, K_TOP, E)
    hot_calls = [hot[None, :].copy() for _ in range(CALLS)]
    results = {}
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        if "m1_hot" in only:
            dims, bank = banks[4]
            wl = Workload("m1_hot", abi, torch, dims, bank, hot_calls, 1, rng, per_expert_bytes(abi, dims))
            results["m1_hot"] = measure(abi, torch, wl, args.steps, args.warmup)
        if "m1_cold" in only:
            dims, bank = banks[3]
            rot = inputs.rotating_ids(SEED, CALLS, K_TOP, E)
            wl = Workload("m1_cold", abi, torch, dims, bank, [rot[c] for c in range(CALLS)], 1, rng,
                          per_expert_bytes(abi, dims))
            results["m1_cold"] = measure(abi, torch, wl, args.steps, args.warmup)
        if "m8_pool" in only:
            dims, bank = banks[3]
            ids = [inputs.ids_shared_pool(inputs.call_rng(SEED, 300 + c), 8, K_TOP, E) for c in range(CALLS)]
            wl = Workload("m8_pool", abi, torch, dims, bank, ids, 8, rng, per_expert_bytes(abi, dims))
            results["m8_pool"] = measure(abi, torch, wl, args.steps, args.warmup)
        if "m8_distinct" in only:
            dims, bank = banks[3]
            ids = [inputs.ids_all_distinct(inputs.call_rng(SEED, 400 + c), 8, K_TOP, E) for c in range(CALLS)]
            wl = Workload("m8_distinct", abi, torch, dims, bank, ids, 8, rng, per_expert_bytes(abi, dims))
            results["m8_distinct"] = measure(abi, torch, wl, args.steps, args.warmup)
        for name, Mp in prefill_wls.items():
            if name in only:
                dims, bank = banks[3]
                results[name] = measure_prefill(abi, torch, dims, bank, Mp, max(args.steps // 4, 10),
                                                max(args.warmup // 4, 2), per_expert_bytes(abi, dims))
        stack = stack_gemv = None
        if {"stack48", "stack48_gemv"} & only:
            del banks
            torch.cuda.empty_cache()
        if "stack48" in only:
            stack = measure_stack(abi, torch, max(args.steps // 4, 10), max(args.warmup // 4, 2))
        if "stack48_gemv" in only:
            stack_gemv = measure_stack(abi, torch, max(args.steps // 4, 10), max(args.warmup // 4, 2), router="gemv")
        ceiling = copy_ceiling(torch)
        read_ref = read_ceiling(torch)
        floor = launch_floor(torch)

    decode_results = {k: v for k, v in results.items() if k not in prefill_wls}
    if not decode_results:
        print(json.dumps({"per_config": results, "stack48": stack, "stack48_gemv": stack_gemv}), flush=True)
        return
    head = decode_results.get("m1_hot") or next(iter(decode_results.values()))
    line = {
        "metric": "MoE layer decode µs and achieved weight HBM GB/s (% of peak) at M=1 and M=8",
        "value": round(head["layer_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 x int4 -> fp32 accumulate",
        "data": "synthetic (seeded int4 weights, fp16 scales |N(0,1)|*0.02, zeros U{0..15}, x ~ N(0,1))",
        "config": {
            "workload": "AWQ int4 MoE expert stage, 512 experts, hidden 2560, inter 160, top-k 10, group 32, "
                        "M=1, 4-byte records, same 10 hot experts on all 48 calls of a graph replay",
            "layer_us": round(head["layer_us"], 3),
            "calls_per_step": CALLS,
        },
        "roofline": roofline(head),
        "per_config": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                       for k, v in results.items()},
        "stack48": stack,
        "stack48_gemv": stack_gemv,
        "copy_reference": ceiling,
        "read_reference": read_ref,
        "launch_floor": floor,
        "setup_s": round(t_gen, 1),
    }
    if not args.no_cpu and "m1_hot" in results:
        line["cpu_baseline"] = cpu_baseline(bi, hot_calls, SEED)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
