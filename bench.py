"""Benchmark of the AWQ int4 MoE expert stage for small-batch decode on one MI355X.

Headline workload: the 512-expert rank-share layer (hidden 2560, local
intermediate 160, top-k 10, int4 group 32) with compact 3-byte records, M = 1
token, cold weights: every call takes 10 experts that no call has touched
within the last ~1.4 GB of weight traffic. Calls go round robin over four
device copies of the layer bank (4 x 373.6 MB), each call taking the next
window of its bank's own expert permutation, and the replays cycle through
four graphs of 48 calls (PR #522 "Coalesce AWQ QPN W13 compact metadata
loads...", Operator results: 48 calls per graph replay, hot and rotating
experts), so nothing a call reads can still sit in the 256 MB MALL or the
4 MB L2s. One *step* is one replay: 48 awq_moe_decode calls (W13+SwiGLU,
then W2+reduction; two launches each).

Printed: one JSON line with the layer's achieved weight bandwidth (touched
weight + record bytes / layer time), per-kernel times from graphs of one
kernel, the roofline of the dominant (longer) kernel with its duration on
two clocks (HIP events on its stream, which ``frac`` uses, and the
committed rocprofv3 kernel trace), M = 8 with a shared expert pool and with
80 distinct experts (also cold), the same 10 hot experts on every call
(4-byte records: cache-resident by construction, reported as effective
bandwidth), the indexed prefill and the 48-layer stack, live references (a
1 GiB copy, a 1 GiB streaming read, the per-launch floor), and the float64
CPU oracle timed on the host (three configurations, all cores and one
thread, median of 5).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME,...] [--no-cpu]
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
COLD_BANKS = 4       # device copies of the 3-byte layer bank that cold calls rotate over
COLD_GRAPHS = 4      # graphs of CALLS calls each; replays cycle through them
SEED = 2026
E, K_TOP, H, I = 512, 10, 2560, 160


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--only", default="", help="comma list of workloads: m1_cold,m1_hot,m8_pool,m8_distinct "
                   "(any mN_pool / mN_distinct, N = 1..8),p9,p16,p32,p48,p64,p96,p128,p256,p512,p1024,p4096,stack48,stack48_gemv")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--tactics", action="store_true",
                   help="time every kernel form of both stages for M = 1..8 and both record sizes (cold weights) "
                        "and print that table instead of the benchmark line")
    return p.parse_args()


class Workload:
    """``graphs`` graphs of CALLS decode calls of one configuration, all inputs
    resident on the device. ``calls[j] = (bank index, ids [M][k])`` for call
    j = g * CALLS + c of graph g."""

    def __init__(self, name, abi, torch, dims, banks, calls, M, rng, per_expert, graphs=1):
        self.name, self.dims, self.banks, self.M, self.graphs = name, dims, banks, M, graphs
        dev = banks[0].device
        n = graphs * CALLS
        assert len(calls) == n
        self.bank_of = [banks[b] for b, _ in calls]
        self.x = [torch.from_numpy(inputs.activations(rng, M, H)).to(dev) for _ in range(n)]
        self.ids = [torch.from_numpy(np.ascontiguousarray(ids)).to(dev) for _, ids in calls]
        self.w = [torch.from_numpy(inputs.router_weights(rng, M, K_TOP)).to(dev) for _ in range(n)]
        self.out = torch.empty((M, H), dtype=torch.float16, device=dev)
        self.ws = [abi.alloc_workspace(dims, M, K_TOP, dev) for _ in range(n)]
        self.routes = [abi.alloc_route(M * K_TOP, dev) for _ in range(n)]
        distinct = [len(np.unique(ids)) for _, ids in calls]
        self.distinct_mean = float(np.mean(distinct))
        self.w13_bytes = [d * per_expert["w13"] for d in distinct]
        self.w2_bytes = [d * per_expert["w2"] for d in distinct]
        self.bank_copies = len(banks)


def measure_stack(abi, torch, steps, warmup, layers=48, M=8, router="given"):
    """One decode step of a stack of 512-expert pre-norm layers (3-byte
    records, banks drawn on the device): per layer r_{l+1} = fp16(r_l +
    stage(fp16(rms_norm(r_l)))), one awq_moe_decode_rmsnorm_residual call
    (two launches: the norm inside W13, the residual inside W2).
    router="given": the fp32 N(0,1) logits of every layer are inputs of the
    step, so the top-k of all layers is one launch at its start.
    router="gemv": each layer's logits are x_l . Wr^T from fp16 router
    weights N(0,1)/sqrt(H) (one launch, which also normalises r_l), then
    top-k (one launch), then the layer: four launches per layer.
    One graph replay = one step."""
    dims = abi.make_dims(E, H, I, 3)
    Lq = abi.awq_moe_bank_layout_query(dims)
    sections = [(int(Lq.w13_meta_off), (H // 32) * 2 * I), (int(Lq.w2_meta_off), (I // 32) * H)]
    banks = [inputs.device_bank(SEED + 9000 + l, E, sections, int(Lq.expert_bytes), 3) for l in range(layers)]
    rng = inputs.call_rng(SEED, 900)
    ids_all = torch.empty((layers * M, K_TOP), dtype=torch.int32, device="cuda")
    wts_all = torch.empty((layers * M, K_TOP), dtype=torch.float32, device="cuda")
    ids = [ids_all[l * M:(l + 1) * M] for l in range(layers)]
    wts = [wts_all[l * M:(l + 1) * M] for l in range(layers)]
    if router == "gemv":
        wr = [inputs.device_router_weights(SEED + 9500 + l, E, H) for l in range(layers)]
        logits = [torch.empty((M, E), dtype=torch.float32, device="cuda") for _ in range(layers)]
        rcopy = torch.empty((M, H), dtype=torch.float16, device="cuda")
    else:
        logits_all = torch.from_numpy(inputs.router_logits(rng, layers * M, E)).to("cuda")
    r0 = torch.from_numpy(inputs.activations(rng, M, H)).to("cuda")
    rbuf = [torch.empty_like(r0) for _ in range(2)]
    xbuf = torch.empty_like(r0)
    ws = abi.alloc_workspace(dims, M, K_TOP, "cuda")

    def step():
        if router != "gemv":
            abi.awq_moe_router_topk(logits_all, K_TOP, ids=ids_all, w=wts_all)
        r = r0
        for l in range(layers):
            rn = rbuf[l % 2]
            if router == "gemv":
                abi.awq_moe_router_gemv(r, wr[l], None, r_next=rcopy, x=xbuf, logits=logits[l])
                abi.awq_moe_router_topk(logits[l], K_TOP, ids=ids[l], w=wts[l])
            abi.awq_moe_decode_rmsnorm_residual(dims, banks[l], r, ids[l], wts[l], r_next=rn, workspace=ws)
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
           "resident_bank_bytes": int(Lq.total_bytes) * layers,
           "launches_per_layer": 4 if router == "gemv" else 2 + 1.0 / layers, "router": router}
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
    """Mean ms per replay of one graph, from HIP events recorded on the replay stream."""
    return time_graphs(torch, [g], reps, warmup)


def time_graphs(torch, gs, reps, warmup):
    """Mean ms per replay when the graphs ``gs`` are replayed round robin
    (reps rounded up to a multiple of len(gs)), from HIP events recorded on
    the replay stream."""
    s = torch.cuda.current_stream()
    n = len(gs)
    reps = -(-reps // n) * n
    for i in range(max(warmup, n)):
        gs[i % n].replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(s)
    for i in range(reps):
        gs[i % n].replay()
    t1.record(s)
    t1.synchronize()
    return t0.elapsed_time(t1) / reps


def measure(abi, torch, wl: Workload, steps, warmup):
    def calls_of(g):
        return range(g * CALLS, (g + 1) * CALLS)

    def full(g):
        for c in calls_of(g):
            abi.awq_moe_decode(wl.dims, wl.bank_of[c], wl.x[c], wl.ids[c], wl.w[c], out=wl.out, workspace=wl.ws[c])

    def route(g):
        for c in calls_of(g):
            abi.awq_moe_route_compact(wl.ids[c], E, out=wl.routes[c])

    def w13(g):
        for c in calls_of(g):
            abi.awq_moe_w13_swiglu(wl.dims, wl.bank_of[c], wl.x[c], wl.ids[c], workspace=wl.ws[c])

    def w2(g):
        for c in calls_of(g):
            abi.awq_moe_w2_reduce(wl.dims, wl.bank_of[c], wl.ids[c], wl.w[c], wl.ws[c], out=wl.out)

    for g in range(wl.graphs):
        route(g)
        w13(g)
    torch.cuda.synchronize()
    res = {}
    # "layer" = awq_moe_decode (two launches, one workgroup per slot and tile);
    # "route" = the standalone awq_moe_route_compact kernel, not part of the layer.
    graphs = {name: [capture(torch, lambda g=g, f=fn: f(g)) for g in range(wl.graphs)]
              for name, fn in (("layer", full), ("route", route), ("w13", w13), ("w2", w2))}
    for name, gs in graphs.items():
        ms = time_graphs(torch, gs, steps, warmup)
        res[name + "_us"] = ms * 1e3 / CALLS
        if name == "layer":
            res["step_ms"] = ms
    # 7 further samples per graph set, in alternating (ABBA) order, for the median and the minimum
    per_sample = max(steps // 7, 2 * wl.graphs)
    samples = {name: [] for name in graphs}
    names = list(graphs)
    for r in range(7):
        for name in (names if r % 2 == 0 else names[::-1]):
            samples[name].append(time_graphs(torch, graphs[name], per_sample, wl.graphs) * 1e3 / CALLS)
    for name, v in samples.items():
        res[name + "_us_median7"] = float(np.median(v))
        res[name + "_us_min7"] = float(np.min(v))
    del graphs
    w13b = float(np.mean(wl.w13_bytes))
    w2b = float(np.mean(wl.w2_bytes))
    res.update(
        M=wl.M, distinct_experts_per_call=wl.distinct_mean, bank_copies=wl.bank_copies,
        graphs=wl.graphs, w13_bytes_per_call=w13b, w2_bytes_per_call=w2b,
        w13_gbs=w13b / (res["w13_us"] * 1e3), w2_gbs=w2b / (res["w2_us"] * 1e3),
        layer_gbs=(w13b + w2b) / (res["layer_us"] * 1e3),
    )
    for k in ("w13", "w2", "layer"):
        res[k + "_pct_peak"] = 100.0 * res[k + "_gbs"] / HBM_PEAK_GBS
    return res


def measure_prefill(abi, torch, dims, bank, M, steps, warmup, per_expert, calls=8):
    """Indexed prefill of M tokens (awq_moe_prefill, two to five launches) on the
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


def recorded_traffic(kernel: str, summary: str = "pmc_traffic_m1_cold.txt"):
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


def recorded_trace(kernel: str, summary: str = "kernel_stats_m1_cold.txt"):
    """(average ns, median ns) of ``kernel`` in the committed rocprofv3 kernel-trace
    summary, or None when it is missing or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if f"sha256[:16] at collection: {stage_source_hash()}" not in text:
        return None
    for line in text.splitlines():
        parts = [p.strip() for p in line.split("|")]
        if len(parts) == 7 and parts[0].split("awq_moe::")[-1] == kernel:
            return float(parts[2]), float(parts[3])
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


def cpu_baseline(bi, cold_calls, pool_calls, per_sample_s=0.6, samples=5):
    """The float64 oracle (oracle.ref.moe_stage: dequantisation of the touched
    experts, W13 + SwiGLU, W2, weighted sum; input generation excluded) on the
    host, for the tiny layer (16 experts, hidden 256, inter 32, top-k 2,
    4-byte records, M = 1), the cold M = 1 calls and the M = 8 shared-pool
    calls of the rank layer. Each sample repeats calls for about
    ``per_sample_s`` seconds; the median of ``samples`` samples is reported,
    once with the BLAS thread pool at every core this process may use and
    once at one thread (NumPy's elementwise dequantisation runs on one
    thread either way)."""
    from threadpoolctl import threadpool_limits

    from oracle import ref as R
    cores = len(os.sched_getaffinity(0))
    tiny = inputs.bank_inputs(1, 16, 256, 32)
    rng = inputs.call_rng(SEED, 77)
    tiny_calls = [inputs.ids_distinct(rng, 1, 2, 16) for _ in range(64)]
    cfgs = {
        # name: (bank, experts, hidden, list of ids, bytes per distinct expert)
        # tiny expert (4-byte records): W13 8,192 + 512 * 4 B, W2 4,096 + 256 * 4 B
        "tiny_m1": (tiny, 16, 256, tiny_calls, (8192 + 512 * 4) + (4096 + 256 * 4)),
        "m1_cold": (bi, E, H, [ids for _, ids in cold_calls], 729_600),
        "m8_pool": (bi, E, H, [ids for _, ids in pool_calls], 729_600),
    }
    out = {"cores_all": cores}
    for name, (bank, En, Hn, id_list, per_expert) in cfgs.items():
        entry = {}
        done = 0
        for threads in (cores, 1):
            per_sample = []
            with threadpool_limits(limits=threads):
                for _ in range(samples):
                    n, byts, busy = 0, 0, 0.0
                    while busy < per_sample_s:
                        ids = id_list[done % len(id_list)]
                        M = ids.shape[0]
                        x = inputs.activations(rng, M, Hn)
                        w = inputs.router_weights(rng, M, ids.shape[1])
                        t0 = time.perf_counter()
                        R.moe_stage(x, ids, w, En, bank.expert)
                        busy += time.perf_counter() - t0
                        n += 1
                        done += 1
                        byts += len(np.unique(ids)) * per_expert
                    per_sample.append((busy / n, byts / n))
            us = float(np.median([a for a, _ in per_sample])) * 1e6
            byts = float(np.mean([b for _, b in per_sample]))
            entry["threads_1" if threads == 1 else "threads_all"] = {
                "threads": threads, "us_per_layer_median5": round(us, 1), "gbs": round(byts / (us * 1e3), 4)}
        out[name] = entry
    head = out["m1_cold"]["threads_all"]
    return {"value": head["gbs"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": (f"float64 NumPy oracle on the host: the cold M=1 rank-layer calls (3-byte records, "
                       f"10 experts per call), median of {samples} samples of ~{per_sample_s} s, BLAS threads = "
                       f"{cores} (all cores this process may use); dequantisation of the touched experts "
                       f"included, input generation excluded; also tiny M=1 and M=8 shared pool, and one thread"),
            "layer_us": head["us_per_layer_median5"], "per_config": out}


def stage_kernel_names(abi, M, rb, H=H, I=I, topk=K_TOP, E_=E):
    """Names (as the kernel trace prints them) of the W13 and W2 kernels the
    library's tactic table picks for a shape (awq_moe_decode_table)."""
    f13, f2 = abi.awq_moe_decode_table(abi.make_dims(E_, H, I, rb), M, topk)
    # single lanes read their weights non-temporally when the grid's waves
    # fit the chip at once (256 CUs x 4 SIMDs x 8)
    nt = "true" if (2 * I // 16) * M * topk * ((4 * (H // 32) + 63) // 64) <= 256 * 32 else "false"
    w13 = {abi.W13_PAIR: f"w13_swiglu_pair_kernel<{rb}, false>",
           abi.W13_SINGLE: f"w13_swiglu_kernel<{rb}, false, 1, {nt}>",
           abi.W13_SINGLE_TWO_TILES: f"w13_swiglu_kernel<{rb}, false, 2, {nt}>"}[f13]
    choices = [v for v in (16, 8, 5, 4, 3, 2, 1) if v <= 64 // (I // 8)]  # slots per wave that fit
    pick = 0 if f2 == abi.W2_SEG_MOST else 1
    spw = choices[pick] if pick < len(choices) else 0
    if spw and (topk + spw - 1) // spw <= 16:
        w2 = f"w2_reduce_seg_kernel<{rb}, {spw}, false>"
    elif f2 == abi.W2_SEG_MOST and 512 < I <= 1024 and topk <= 16:
        w2 = f"w2_reduce_seg2_kernel<{rb}, false>"
    else:
        w2 = f"w2_reduce_kernel<{rb}, 1, false>"
    return w13, w2


def roofline(abi, head, rb):
    """HBM roofline of the longer of the two stage kernels at the headline
    workload. ``achieved`` and ``frac`` use the HIP-event clock (per-launch
    period of a graph of 48 launches of that kernel alone); the committed
    kernel-trace duration of the same kernel is carried next to it."""
    k = "w2" if head["w2_us"] >= head["w13_us"] else "w13"
    w13_name, w2_name = stage_kernel_names(abi, head["M"], rb)
    name = {"w13": w13_name, "w2": w2_name}[k]
    gbs = head[k + "_gbs"]
    algo = head[k + "_bytes_per_call"]
    out = {
        "bound": "hbm",
        "kernel": name,
        "achieved": round(gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "traffic": recorded_traffic(name),
        "algorithmic_bytes_per_launch": algo,
        "clock": "hip_events",
        "avg_launch_us": round(head[k + "_us"], 3),
    }
    tr = recorded_trace(name)
    if tr is not None:
        out["trace_avg_us"] = round(tr[0] / 1e3, 3)
        out["trace_median_us"] = round(tr[1] / 1e3, 3)
        out["frac_trace_avg"] = round(algo / (tr[0] / 1e3) / 1e3 / HBM_PEAK_GBS, 4)
    return out


def tactic_sweep(abi, torch, steps, rounds=3):
    """Per record size and M = 1..8: every W13 form alone and every W2 form
    alone, timed as graphs of 48 calls on cold weights (the headline's bank
    rotation; M = 1 distinct experts, M >= 2 shared pools), in alternating
    order over `rounds` rounds (minimum and median per form), next to the
    forms the library's table picks."""
    bi = inputs.bank_inputs(SEED, E, H, I)
    out = {}
    for rb in (3, 4):
        dims = abi.make_dims(E, H, I, rb)
        host = torch.from_numpy(abi.prepare_from_inputs(dims, bi))
        banks = [host.to("cuda") for _ in range(COLD_BANKS)]
        del host
        per_expert = per_expert_bytes(abi, dims)
        rng = inputs.call_rng(SEED, 5)
        table = {}
        for M in range(1, 9):
            calls = inputs.rotating_calls(SEED + M, COLD_GRAPHS * CALLS, M, K_TOP, E, COLD_BANKS,
                                          "distinct" if M == 1 else "pool")
            wl = Workload(f"m{M}", abi, torch, dims, banks, calls, M, rng, per_expert, graphs=COLD_GRAPHS)
            forms = {}
            for f13 in (abi.W13_PAIR, abi.W13_SINGLE, abi.W13_SINGLE_TWO_TILES):
                forms[("w13", f13)] = (f13, 0, 1)
            for f2 in (abi.W2_SEG_MOST, abi.W2_SEG_FEWER):
                forms[("w2", f2)] = (0, f2, 2)
            graphs = {}
            for key, (f13, f2, st) in forms.items():
                def run(g, f13=f13, f2=f2, st=st):
                    for c in range(g * CALLS, (g + 1) * CALLS):
                        abi.awq_moe_decode_forms(wl.dims, wl.bank_of[c], wl.x[c], wl.ids[c], wl.w[c], f13, f2,
                                                 stages=st, out=wl.out, workspace=wl.ws[c])
                for g in range(COLD_GRAPHS):
                    run(g)
                graphs[key] = [capture(torch, lambda g=g, f=run: f(g)) for g in range(COLD_GRAPHS)]
            samples = {key: [] for key in graphs}
            keys = list(graphs)
            for r in range(rounds):
                for key in (keys if r % 2 == 0 else keys[::-1]):
                    samples[key].append(time_graphs(torch, graphs[key], steps, COLD_GRAPHS) * 1e3 / CALLS)
            del graphs
            f13_t, f2_t = abi.awq_moe_decode_table(dims, M, K_TOP)
            table[f"M{M}"] = {
                "w13_us": {str(k[1]): round(float(np.min(v)), 3) for k, v in samples.items() if k[0] == "w13"},
                "w13_us_median": {str(k[1]): round(float(np.median(v)), 3) for k, v in samples.items()
                                  if k[0] == "w13"},
                "w2_us": {str(k[1]): round(float(np.min(v)), 3) for k, v in samples.items() if k[0] == "w2"},
                "w2_us_median": {str(k[1]): round(float(np.median(v)), 3) for k, v in samples.items()
                                 if k[0] == "w2"},
                "table": [f13_t, f2_t], "distinct_experts_per_call": wl.distinct_mean,
            }
            del wl
            print(f"tactics rb={rb} M={M} {table[f'M{M}']}", flush=True)
        out[f"rb{rb}"] = table
        del banks
        torch.cuda.empty_cache()
    return out


def decode_workloads(only):
    """Names of the decode workloads asked for, in run order: (name, M, mode)."""
    out = []
    for name in sorted(only, key=lambda n: (n != "m1_cold", n)):
        if name == "m1_hot":
            out.append((name, 1, "hot"))
            continue
        if not name.startswith("m") or "_" not in name:
            continue
        m, mode = name[1:].split("_", 1)
        if m.isdigit() and 1 <= int(m) <= 8 and mode in ("cold", "pool", "distinct"):
            out.append((name, int(m), "distinct" if mode == "cold" else mode))
    return out


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
    if args.tactics:
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            print(json.dumps({"tactics": tactic_sweep(abi, torch, max(args.steps // 4, 8))}), flush=True)
        return
    prefill_wls = {"p9": 9, "p16": 16, "p32": 32, "p48": 48, "p64": 64, "p96": 96, "p128": 128, "p256": 256, "p512": 512, "p1024": 1024, "p4096": 4096}
    only = set(filter(None, args.only.split(","))) or {"m1_cold", "m1_hot", "m8_pool", "m8_distinct", "stack48",
                                                       "stack48_gemv", *prefill_wls}
    decode_wls = decode_workloads(only)
    cold_needed = any(mode != "hot" for _, _, mode in decode_wls) or bool(set(prefill_wls) & only)

    t_gen = time.perf_counter()
    bi = inputs.bank_inputs(SEED, E, H, I)
    dims3 = abi.make_dims(E, H, I, 3)
    dims4 = abi.make_dims(E, H, I, 4)
    banks3, bank4 = [], None
    if cold_needed:
        host3 = torch.from_numpy(abi.prepare_from_inputs(dims3, bi))
        banks3 = [host3.to("cuda") for _ in range(COLD_BANKS)]   # physically distinct copies of one layer
        del host3
    if "m1_hot" in only:
        bank4 = torch.from_numpy(abi.prepare_from_inputs(dims4, bi)).to("cuda")
    t_gen = time.perf_counter() - t_gen

    rng = inputs.call_rng(SEED, 1)
    hot = inputs.hot_experts(SEED, K_TOP, E)
    results, cold_calls = {}, {}
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for name, M, mode in decode_wls:
            if mode == "hot":
                calls = [(0, hot[None, :].copy()) for _ in range(CALLS)]
                wl = Workload(name, abi, torch, dims4, [bank4], calls, 1, rng, per_expert_bytes(abi, dims4))
            else:
                calls = inputs.rotating_calls(SEED + M, COLD_GRAPHS * CALLS, M, K_TOP, E, COLD_BANKS, mode)
                cold_calls[name] = calls
                wl = Workload(name, abi, torch, dims3, banks3, calls, M, rng, per_expert_bytes(abi, dims3),
                              graphs=COLD_GRAPHS)
            results[name] = measure(abi, torch, wl, args.steps, args.warmup)
            del wl
        for name, Mp in prefill_wls.items():
            if name in only:
                results[name] = measure_prefill(abi, torch, dims3, banks3[0], Mp, max(args.steps // 4, 10),
                                                max(args.warmup // 4, 2), per_expert_bytes(abi, dims3))
        stack = stack_gemv = None
        if {"stack48", "stack48_gemv"} & only:
            del banks3, bank4
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
    head_name = "m1_cold" if "m1_cold" in decode_results else next(iter(decode_results))
    head = decode_results[head_name]
    head_rb = 4 if head_name == "m1_hot" else 3

    def brief(r):
        return {k: round(r[k], 3) for k in ("layer_us", "w13_us", "w2_us", "layer_gbs", "layer_pct_peak",
                                            "w13_pct_peak", "w2_pct_peak", "distinct_experts_per_call")}

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
            "workload": ("AWQ int4 MoE expert stage, 512 experts, hidden 2560, inter 160, top-k 10, group 32, "
                         "M=1, 3-byte records, cold weights: calls rotate over 4 device copies of the layer "
                         "bank and 4 graphs of 48 calls, every expert read at least 1.39 GB of weight traffic "
                         "after its previous read") if head_name == "m1_cold" else head_name,
            "layer_us": round(head["layer_us"], 3),
            "calls_per_step": CALLS,
        },
        "roofline": roofline(abi, head, head_rb),
        "m8_distinct": brief(results["m8_distinct"]) if "m8_distinct" in results else None,
        "m8_pool": brief(results["m8_pool"]) if "m8_pool" in results else None,
        "m1_hot_effective": (dict(brief(results["m1_hot"]), note="the same 10 experts on every call: "
                                  "cache-resident, effective (not HBM) bandwidth")
                             if "m1_hot" in results else None),
        "per_config": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                       for k, v in results.items()},
        "stack48": stack,
        "stack48_gemv": stack_gemv,
        "copy_reference": ceiling,
        "read_reference": read_ref,
        "launch_floor": floor,
        "setup_s": round(t_gen, 1),
    }
    if not args.no_cpu and "m1_cold" in cold_calls and "m8_pool" in cold_calls:
        line["cpu_baseline"] = cpu_baseline(bi, cold_calls["m1_cold"], cold_calls["m8_pool"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
