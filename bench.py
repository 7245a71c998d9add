"""Benchmark of the W4 g128 sparse-MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode_stack]

A step is one forward of the workload (per layer: route + permute -> grouped
W4 FFN -> combine) over one batch of synthetic tokens already resident in
HBM: one moe_layer_forward call for a single layer, one
moe_decode_stack_forward call for the stacked decode step (layer i's combine
and layer i+1's routing in one launch; --per-layer makes it one
moe_layer_forward call per layer).  Steps are timed as HIP-graph replays
(each step's launches captured once after the warm-up, as the pages run the
grouped expert GEMM in a fixed captured graph; --eager times the same calls
launched one by one).  By default the largest configuration, the decode step
through 42 stacked layers (288 experts + 1 shared, hidden 4096, ffn 1536,
top-8, 16 tokens, RMS norm between layers, 119 GB of weights).  The
single-layer workloads rotate several independently drawn weight sets so
that no expert byte is served from the 256 MB Infinity Cache across steps.
Prints ONE JSON line.

`roofline` is for the dominant stage, the grouped FFN (one
moe_w4_grouped_ffn call: two launches, gate/up then down): decode: algorithmic
bytes = distinct experts with tokens in the step x bytes per expert (packed
int4 + fp16 scales) + the fp16 shared expert; prefill: algorithmic FLOPs =
6*H*F per (token, chosen expert) pair; divided by the stage's average
duration: the FFN calls of the steps' layers (weight sets, layer inputs and
routing recorded in one untimed pass), K per layer of a step, run back to
back on the launch stream between one pair of HIP events (so no
event-processing gaps land on the kernels).  `layer_achieved` / `layer_frac`
put the whole step on the same roofline: the algorithmic bytes of every
layer of the step (each counted from its own offsets) over the mean step
time of the timed region.  `traffic` is the HBM bytes per
call measured by rocprofv3 counters
(profiles/traffic_<workload>.json, taken with --copy-calibration-mib and
turned into bytes with --summarize-traffic), or null when the FFN sources
have changed since.

`step_ms_p10_p50_p90`: percentiles of single steps timed one by one with an
event pair each, after the timed region (the events add their own cost).

`cpu_baseline` times the float64 oracle (test infrastructure, run only in
this leg) on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import get_config  # noqa: E402
from workloads import gen as G  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 matrix peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode_stack",
                    choices=["decode_fine", "decode_coarse", "prefill", "decode_stack",
                             "decode_fine512", "tiny"])
    ap.add_argument("--group-size", type=int, default=128, choices=[64, 128, 256],
                    help="int4 quantization group size of the experts")
    ap.add_argument("--shared-bits", type=int, default=16, choices=[16, 8],
                    help="shared expert weights: fp16, or 8-bit g128")
    ap.add_argument("--weight-sets", type=int, default=0, help="0 = workload default")
    ap.add_argument("--batches", type=int, default=4, help="distinct token batches rotated")
    ap.add_argument("--tokens", type=int, default=0, help="tokens per step (0 = the workload's)")
    ap.add_argument("--per-layer", action="store_true",
                    help="stacked workloads: one moe_layer_forward call per layer instead of "
                         "one moe_decode_stack_forward call per step")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps as eager launches (one C call per layer) instead of "
                         "HIP-graph replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, copy this many MiB 3 times (a plain copy "
                         "kernel of known size, the reference for PMC byte counters)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, "
                         "WRITE_SIZE) of a run with --copy-calibration-mib into "
                         "profiles/traffic_<workload>[_g<group size>].json")
    return ap.parse_args()


# ---------------------------------------------------------------- HBM traffic
# Measured HBM bytes of the FFN come from rocprofv3 counter runs; they are
# valid only for the kernel sources they were taken with.
FFN_SOURCES = ("w4_group_quantized_amd/csrc/ffn.hip", "w4_group_quantized_amd/csrc/ffn_split.hip",
               "w4_group_quantized_amd/csrc/ffn_decode.h", "w4_group_quantized_amd/csrc/ffn_prefill.hip",
               "w4_group_quantized_amd/csrc/tiles.h", "w4_group_quantized_amd/csrc/common.h",
               "w4_group_quantized_amd/csrc/split_plan.h")
FFN_KERNELS = ("ffn_decode_kernel", "ffn_prefill_kernel")


def ffn_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _pmc_rows(path, counter):
    """(kernel name, grid size, value) per dispatch of one counter in a
    rocprofv3 CSV."""
    import csv
    out = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def traffic_from_csv(fetch_csv, write_csv, copy_mib):
    """FFN HBM bytes per moe_w4_grouped_ffn call from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by bytes/counter of the plain copy."""
    res = {"copy_mib": copy_mib}
    known = copy_mib * 1024 * 1024
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _pmc_rows(path, counter)
        # the calibration copies are the HIP runtime's device-to-device copy
        # kernel (torch copies contiguous same-dtype tensors with it); they are
        # the three largest dispatches of that kernel in the run
        copies = sorted(v for n, _, v in rows if "copybuffer" in n.lower())
        if len(copies) < 3:
            raise SystemExit(f"{path}: calibration copy dispatches not found")
        copy_kib = float(np.median(copies[-3:]))
        factor = known / (copy_kib * 1024.0)
        per_kernel = {}
        for n, _, v in rows:
            if any(k in n for k in FFN_KERNELS):
                per_kernel.setdefault(n, []).append(v)
        if not per_kernel:
            raise SystemExit(f"{path}: no FFN dispatch found")
        call_kib = sum(float(np.mean(v)) for v in per_kernel.values())
        res[key] = {"counter": counter, "copy_counter_kib": copy_kib, "bytes_per_counter_byte": factor,
                    "ffn_kib_per_call": call_kib, "ffn_bytes_per_call": call_kib * 1024.0 * factor,
                    "dispatches": {n: len(v) for n, v in per_kernel.items()}}
    res["traffic_bytes_per_call"] = res["fetch"]["ffn_bytes_per_call"] + res["write"]["ffn_bytes_per_call"]
    return res


def traffic_path(workload, group_size, shared_bits=16):
    tag = ("" if group_size == 128 else f"_g{group_size}") + ("" if shared_bits == 16 else "_s8")
    return os.path.join(ROOT, "profiles", f"traffic_{workload}{tag}.json")


def summarize_traffic(workload, group_size, shared_bits, fetch_csv, write_csv, copy_mib):
    """Write the traffic summary of a workload for the current FFN sources."""
    res = {"workload": workload, "group_size": group_size, "shared_bits": shared_bits,
           "source_sha256": ffn_source_hash()}
    res.update(traffic_from_csv(fetch_csv, write_csv, copy_mib))
    out = traffic_path(workload, group_size, shared_bits)
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res))


def measured_traffic(workload, group_size=128, shared_bits=16):
    """HBM bytes per FFN call measured for the current kernel sources, else None."""
    path = traffic_path(workload, group_size, shared_bits)
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != ffn_source_hash():
        return None
    return float(t["traffic_bytes_per_call"])


# ---------------------------------------------------------------- device weights
def gpu_normal16(shape, std, seed, dev):
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(
        torch.float16)


def build_layer(cfg, wset, layer_idx, dev):
    """fp16 masters N(0, weight_std) drawn on the device, quantized by the HIP
    quantizer; router and bias from the numpy generators; fp16 shared expert."""
    import torch
    from w4_group_quantized_amd import W4MoELayer, _native as NAT
    E, H, F = cfg.num_experts, cfg.hidden, cfg.ffn
    mats = {}
    for m, name in ((G.GATE, "gate"), (G.UP, "up"), (G.DOWN, "down")):
        out_dim, in_dim = G.matrix_shape(cfg, m)
        q = torch.empty((E, out_dim, in_dim // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((E, out_dim, in_dim // cfg.group_size), dtype=torch.float16, device=dev)
        # a few experts per draw keeps the fp32 temporaries small
        per = max(1, min(E, (1 << 28) // (out_dim * in_dim)))
        for e0 in range(0, E, per):
            e1 = min(E, e0 + per)
            seed = G.torch_seed(cfg, G.T_EXPERT, layer=layer_idx, expert=e0, matrix=m, batch=wset)
            w = gpu_normal16(((e1 - e0) * out_dim, in_dim), cfg.weight_std, seed, dev)
            NAT.moe_w4_quantize(w, (e1 - e0) * out_dim, in_dim, cfg.group_size, q[e0:e1],
                                s[e0:e1])
            del w
        mats[name] = (q, s)
    wr, b = G.router(cfg, layer_idx + 1000 * wset)
    shared = None
    if cfg.shared_ffn:
        Fs = cfg.shared_ffn
        shared = tuple(
            gpu_normal16(shp, cfg.shared_std,
                         G.torch_seed(cfg, G.T_SHARED, layer=layer_idx, matrix=m, batch=wset), dev)
            for m, shp in ((G.GATE, (Fs, H)), (G.UP, (Fs, H)), (G.DOWN, (H, Fs))))
    shared_w8 = None
    if shared is not None and cfg.shared_bits == 8:   # quantized by the HIP 8-bit quantizer
        shared_w8 = []
        for w in shared:
            q = torch.empty(w.shape, dtype=torch.uint8, device=dev)
            s = torch.empty((w.shape[0], w.shape[1] // 128), dtype=torch.float16, device=dev)
            NAT.moe_w8_quantize(w, w.shape[0], w.shape[1], q, s)
            shared_w8.append((q, s))
        shared_w8, shared = tuple(shared_w8), None
    t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    return W4MoELayer(cfg.top_k, t(wr), t(b) if b is not None else None,
                      mats["gate"][0], mats["gate"][1], mats["up"][0], mats["up"][1],
                      mats["down"][0], mats["down"][1], shared=shared, shared_w8=shared_w8)


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(cfg, budget_s):
    """The float64 oracle on a bounded sample of the workload, on host cores.

    The sample is one layer forward of `cfg` at its full shape (all layers'
    shapes are equal in the stacked workload, so one layer stands for one of
    its 42).  Expert weights are drawn directly as packed codes (the forward's
    cost does not depend on their values) and only for the experts the oracle's
    own routing selects; drawing them is not timed.  Repeats the forward until
    `budget_s` is spent (at least once)."""
    import functools
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    wr, b = G.router(cfg, 0)
    x = G.activations(cfg, batch=0)
    shared = G.shared_expert(cfg, 0)
    if shared is not None and cfg.shared_bits == 8:   # the 8-bit weights, dequantized
        shared = tuple(O.dequant_w8(O.pack_w8(q), O.pack_scales(s)) for q, s in
                       (O.group_quantize(w, 128, bits=8) for w in shared))
    idx, _, _ = O.route(x, wr, b, cfg.top_k)
    cache = {}

    class Lazy:
        def __getitem__(self, e):
            if e not in cache:
                tup = []
                for m in (G.GATE, G.UP, G.DOWN):
                    tup += list(G.expert_codes(cfg, 0, int(e), m))
                cache[e] = tuple(tup)
            return cache[e]

    lazy = Lazy()
    for e in np.unique(idx):
        lazy[int(e)]
    runs, t_total = 0, 0.0
    while runs == 0 or t_total < budget_s:
        t0 = time.perf_counter()
        O.moe_layer(x, wr, b, lazy, cfg.top_k, shared=shared,
                    expert_ffn=functools.partial(O.expert_ffn_w4, group=cfg.group_size))
        t_total += time.perf_counter() - t0
        runs += 1
        if t_total > budget_s * 0.5 and runs >= 1 and t_total / runs > budget_s * 0.5:
            break
    per_call = t_total / runs
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": cfg.tokens / per_call, "unit": "tokens/s", "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"{runs} float64 oracle layer forward(s) of {cfg.name} at full shape "
                   f"(T={cfg.tokens}, {len(np.unique(idx))} distinct experts), "
                   f"{per_call * 1e3:.1f} ms each; host {cpu_model or platform.processor()}, "
                   f"{len(os.sched_getaffinity(0))} cpus visible"),
    }


# ---------------------------------------------------------------- main
def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args.workload, args.group_size, args.shared_bits,
                          args.summarize_traffic[0], args.summarize_traffic[1],
                          args.copy_calibration_mib)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    import w4_group_quantized_amd  # noqa: F401  (fails loudly without the HIP library)

    over = {"tokens": args.tokens} if args.tokens else {}
    cfg = get_config(args.workload, group_size=args.group_size, shared_bits=args.shared_bits,
                     **over)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    layers_per_step = cfg.layers
    n_sets = args.weight_sets or (1 if layers_per_step > 1 or cfg.name == "decode_coarse" else 4)
    if cfg.name == "prefill":
        n_sets = args.weight_sets or 2

    # weights: n_sets independent sets (each `layers_per_step` layers)
    sets = []
    for s in range(n_sets):
        sets.append([build_layer(cfg, s, l, dev) for l in range(layers_per_step)])
    T = cfg.tokens
    xs = [torch.from_numpy(G.activations(cfg, batch=bt)).to(dev) for bt in range(args.batches)]
    bufs = sets[0][0].alloc(T)
    act = [torch.empty((T, cfg.hidden), dtype=torch.float16, device=dev) for _ in range(2)]
    torch.cuda.synchronize()

    n_combo = n_sets * args.batches
    # a stacked step is one moe_decode_stack_forward call (layer i's combine
    # and layer i+1's routing share a launch), unless --per-layer
    use_stack = layers_per_step > 1 and not args.per_layer
    stacks = [w4_group_quantized_amd.W4MoEStack(layers) for layers in sets] if use_stack else None
    acts = (torch.empty((layers_per_step, T, cfg.hidden), dtype=torch.float16, device=dev)
            if use_stack else None)

    def step(i):
        x = xs[(i // n_sets) % args.batches]
        if use_stack:
            stacks[i % n_sets].forward(x, bufs, acts=acts, T=T, rmsnorm=True, eps=cfg.rms_eps)
            return
        layers = sets[i % n_sets]
        for li, layer in enumerate(layers):
            if li == len(layers) - 1:
                layer.forward(x, bufs, T, rmsnorm=layers_per_step > 1, eps=cfg.rms_eps)
            else:
                nxt = act[li % 2]
                layer.forward(x, bufs, T, rmsnorm=True, eps=cfg.rms_eps, out=nxt)
                x = nxt

    # One untimed pass per (weight set, batch) combination that keeps every
    # layer's input and routing: the algorithmic expert bytes of each layer
    # are counted from that layer's own offsets, and the FFN-only loop below
    # replays the FFN calls of exactly these layers.
    def routing_buffers():
        return dataclasses.replace(bufs, topk_idx=torch.empty_like(bufs.topk_idx),
                                   topk_w=torch.empty_like(bufs.topk_w),
                                   offsets=torch.empty_like(bufs.offsets),
                                   perm_src=torch.empty_like(bufs.perm_src),
                                   inv_pos=torch.empty_like(bufs.inv_pos))

    plans = []          # per combination: [(layer, layer input, routing buffers)]
    layer_bytes = []    # per combination: expert bytes of each layer
    layer_u = []        # per combination: distinct routed experts of each layer
    for c in range(n_combo):
        x = xs[(c // n_sets) % args.batches]
        plan, lb, lu = [], [], []
        if use_stack:
            # the stack's own layer inputs; a call over the first n layers
            # leaves layer n-1's routing (as the full call computes it)
            full = stacks[c % n_sets].forward(x, bufs, T=T, rmsnorm=True, eps=cfg.rms_eps)
        for li, layer in enumerate(sets[c % n_sets]):
            b = routing_buffers()
            if use_stack:
                x_in = x.clone() if li == 0 else full[li - 1].clone()
                stacks[c % n_sets].forward(x, b, T=T, rmsnorm=True, eps=cfg.rms_eps,
                                           n_layers=li + 1)
                nxt = x            # every prefix call starts from the step's input
            else:
                x_in = x.clone()
                nxt = torch.empty_like(x_in)
                layer.forward(x_in, b, T, rmsnorm=layers_per_step > 1, eps=cfg.rms_eps, out=nxt)
            torch.cuda.synchronize()
            U = int((np.diff(b.offsets.cpu().numpy()) > 0).sum())
            plan.append((layer, x_in, b))
            lu.append(U)
            lb.append(U * cfg.expert_bytes() + cfg.shared_bytes())
            x = nxt
        plans.append(plan)
        layer_bytes.append(lb)
        layer_u.append(lu)
    step_bytes = [float(sum(lb)) for lb in layer_bytes]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if not args.eager:
        # every library call is asynchronous with no host reads, so a whole
        # step (all its layers) is captured as launched; nothing allocates
        graphs = []
        for c in range(n_combo):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        torch.cuda.synchronize()

        def step(i):            # noqa: F811 (the timed step is a replay)
            graphs[i % n_combo].replay()

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()

    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / K

    # The FFN stage alone: the FFN calls of the steps' layers (their weight
    # sets, inputs and routing, every layer of the stack in turn), back to
    # back between one pair of events, so that the per-call figure carries no
    # event-processing gaps.  K * layers_per_step calls.
    calls = [(pl, lb) for plan, lbs in zip(plans, layer_bytes) for pl, lb in zip(plan, lbs)]
    n_ffn = K * layers_per_step
    for i in range(min(args.warmup * layers_per_step, len(calls))):
        (layer, x_in, b), _ = calls[i % len(calls)]
        layer.ffn(x_in, b, T)
    f_start = torch.cuda.Event(enable_timing=True)
    f_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f_start.record(stream)
    for i in range(n_ffn):
        (layer, x_in, b), _ = calls[i % len(calls)]
        layer.ffn(x_in, b, T)
    f_end.record(stream)
    torch.cuda.synchronize()
    ffn_ms_mean = f_start.elapsed_time(f_end) / n_ffn
    ffn_bytes = np.array([calls[i % len(calls)][1] for i in range(n_ffn)], dtype=np.float64)

    # Spread of single steps: a third loop with an event pair around each
    # step (event processing adds to each figure; the headline is the
    # timed region above, which has no events inside)
    n_single = min(K, 200)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_single)]
    torch.cuda.synchronize()
    for i in range(n_single):
        pairs[i][0].record(stream)
        step(i)
        pairs[i][1].record(stream)
    torch.cuda.synchronize()
    single_ms = np.array([a.elapsed_time(b) for a, b in pairs])
    achieved_gbs = float(ffn_bytes.mean() / (ffn_ms_mean * 1e-3) / 1e9)
    tokens_per_s = T * K / (ms_total * 1e-3)
    # algorithmic FFN FLOPs: every (token, chosen expert) pair costs 6*H*F
    # (gate, up, down), the shared expert 6*H*Fs per token
    ffn_flops = T * (cfg.top_k * 6.0 * cfg.hidden * cfg.ffn + 6.0 * cfg.hidden * cfg.shared_ffn)
    achieved_tflops = float(ffn_flops / (ffn_ms_mean * 1e-3) / 1e12)
    traffic = measured_traffic(cfg.name, cfg.group_size, cfg.shared_bits)
    if cfg.name == "prefill":
        roofline = {"bound": "mfma", "achieved": achieved_tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved_tflops / MFMA_F16_PEAK_TFLOPS,
                    "traffic": traffic}
    else:
        roofline = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic}
    # the whole step against the same roofline: every layer's algorithmic
    # expert bytes (decode) or FLOPs (prefill) over the mean step time of the
    # timed region, route, permutation and combine included
    mean_step_bytes = float(np.mean([step_bytes[i % n_combo] for i in range(K)]))
    layer_gbs = mean_step_bytes / (ms_step * 1e-3) / 1e9
    layer_tflops = ffn_flops * layers_per_step / (ms_step * 1e-3) / 1e12
    if cfg.name == "prefill":
        roofline.update({"layer_achieved": layer_tflops,
                         "layer_frac": layer_tflops / MFMA_F16_PEAK_TFLOPS})
    else:
        roofline.update({"layer_achieved": layer_gbs, "layer_frac": layer_gbs / HBM_PEAK_GBS})
    roofline.update({"layer_scope": (f"whole step ({layers_per_step} layer(s): route, permute, "
                                     "FFN, combine) in the timed region"),
                     "step_expert_bytes_mean": mean_step_bytes,
                     "kernel": "moe_w4_grouped_ffn (gate/up launch + down launch)",
                     "ffn_us_mean": float(ffn_ms_mean * 1e3),
                     "ffn_bytes_mean": float(ffn_bytes.mean()), "ffn_flops": ffn_flops,
                     "ffn_tflops": achieved_tflops, "ffn_gbs": achieved_gbs})

    if args.copy_calibration_mib:
        # a plain copy of known size for the PMC byte counters (not timed)
        n = args.copy_calibration_mib * 1024 * 1024 // 2
        src = torch.empty(n, dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        layer_cfg = cfg if cfg.layers == 1 else get_config(cfg.name, layers=1,
                                                           group_size=cfg.group_size,
                                                           shared_bits=cfg.shared_bits,
                                                           tokens=cfg.tokens)
        cpu = cpu_baseline(layer_cfg, args.cpu_budget_s)
        if cfg.layers > 1:       # one oracle layer of the 42: scale to a whole step
            cpu["value"] /= cfg.layers
            cpu["sample"] += f"; value scaled to a {cfg.layers}-layer step"

    res = {
        "metric": "MoE-layer tokens/s",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "experts": cfg.num_experts, "shared_ffn": cfg.shared_ffn,
            "hidden": cfg.hidden, "ffn": cfg.ffn, "top_k": cfg.top_k, "tokens": T,
            "layers_per_step": layers_per_step, "weight_sets": n_sets, "batches": args.batches,
            "group_size": cfg.group_size, "shared_bits": cfg.shared_bits,
            "launch": "eager" if args.eager else "HIP graph replay",
            "call": ("moe_decode_stack_forward per step" if use_stack else
                     "moe_layer_forward per layer"),
            "weights": (f"int4 g{cfg.group_size} (fp16 scales), router fp16, shared expert "
                        + ("fp16" if cfg.shared_bits == 16 else "8-bit g128")),
            "distinct_experts_per_layer_mean": float(np.mean(layer_u)),
        },
        "roofline": roofline,
        "wall_s_timed": wall,
        "step_ms_p10_p50_p90": [float(np.percentile(single_ms, q)) for q in (10, 50, 90)],
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
