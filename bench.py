"""Benchmark of the routed int4 MoE layer on one MI355X.

A step is one pass of the whole layer (router, bucketing, routed + shared expert FFN,
combine) through every layer of a synthetic stack resident in HBM, for one batch of fresh
tokens.  Default workload: Gemma-4-26B-A4B-shaped decode -- hidden 2816, 128 experts, top-8,
expert width 704, shared width 2112, int4 groups of 64 with bf16 scale and bias, int8
router, 30 stacked layers with distinct seeds, 1 token per step.  Each step is one HIP graph
replay (one kernel per layer for a single token).

Every layer of the stack receives its own N(0,1) bf16 hidden states (the layer-input
distribution of the workload).  The synthetic weights come without the model's
normalisation layers, so feeding one layer's raw output into the next grows the residual
stream quadratically (inf after about ten layers); the layers still run back to back, each
writing its own output.

Prints one JSON line with the throughput, the roofline of the dominant kernel (for one token
the single layer kernel; for more tokens the routed gate/up kernel), timed with HIP events on
the stream it runs on inside the timed region, and the CPU oracle timed on a bounded sample
on the host.

python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-layer tokens/s + routed int4 expert GB/s (% HBM peak), decode/prefill"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="gemma4_26b_a4b_decode")
    p.add_argument("--layers", type=int, default=0, help="0 = the workload's full stack")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the post-norm stack and the other workload shapes")
    p.add_argument("--cpu-sample", type=int, default=8, help="token-layers timed on the oracle")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (reads MIB, writes MIB) a few "
                        "times and exit: the reference kernel for scaling rocprof byte counters")
    return p.parse_args()


def sources_digest():
    """sha256 over the HIP sources of the library (kernels and their launch code)."""
    import hashlib
    csrc = os.path.join(ROOT, "quantized_moe_router_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".h", ".hip")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def stored_traffic(name):
    """HBM bytes per launch of a kernel from the counter summary profiles/<name>.md, if that
    summary was taken on the current sources (else None: the kernel may have changed)."""
    path = os.path.join(ROOT, "profiles", name + ".md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        item = line.strip().lstrip("-").strip().strip("`")
        if "=" in item and item.startswith(("traffic_bytes_per_launch", "sources_sha256")):
            k, v = item.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("sources_sha256") != sources_digest() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def copy_calibration(mib):
    """A plain copy kernel of known size (torch copy_), run 5 times."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB 5 times")


def build_stack(cfg, n_layers):
    import stacks
    layers = []
    for l in range(n_layers):
        pl, li = stacks.build_layer(cfg, l, "cuda")
        layers.append((pl, li))
        if (l + 1) % 10 == 0 or l + 1 == n_layers:
            log(f"  built layer {l + 1}/{n_layers}")
    return layers


def capture_step(ops, layers, xin, outs, ws, events=None, timed_layer=-1):
    """One HIP graph: every layer of the stack, xin[l] -> outs[l].  With `events` (start,
    stop): for one token, graph event nodes right before the first layer's kernel and right
    after the last one's (the step is nothing but those kernels); for more tokens, around the
    routed gate/up kernel of layer `timed_layer`."""
    import torch
    g = torch.cuda.CUDAGraph()
    L = len(layers)
    with torch.cuda.graph(g):
        for l, (pl, _) in enumerate(layers):
            if events is not None:
                if xin.shape[1] == 1:
                    ops.set_profile_events(events[0] if l == 0 else None,
                                           events[1] if l == L - 1 else None)
                elif l == timed_layer:
                    ops.set_profile_events(*events)
            ops.layer_forward(pl.weights, xin[l], ws, out=outs[l])
            ops.set_profile_events(None, None)
    return g


def layer_inputs(cfg, step, n_layers, T):
    """bf16 device tensor [n_layers, T, H]: the hidden states of every layer at `step`."""
    import torch
    import stacks
    return torch.stack([stacks.hidden(cfg, step * 1000 + l, T)[1] for l in range(n_layers)]
                       ).view(torch.bfloat16)


def eager_kernel_times(ops, layers, xs, outs, ws, steps):
    """Routed gate/up kernel durations from events recorded around it in eager layer calls.
    A large copy queued first keeps the GPU busy while the host enqueues the step, so the
    kernels then run back to back and the events bracket only the kernel."""
    import torch
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    big2 = torch.empty_like(big)
    L = len(layers)
    evs = [[(ops.Event(), ops.Event()) for _ in range(L)] for _ in range(steps)]
    for s in range(steps):
        big2.copy_(big)
        for l, (pl, _) in enumerate(layers):
            ops.set_profile_events(*evs[s][l])
            ops.layer_forward(pl.weights, xs[s + 1][l], ws, out=outs[l])
            ops.set_profile_events(None, None)
    torch.cuda.synchronize()
    return [evs[s][l][0].elapsed_ms(evs[s][l][1]) for s in range(steps) for l in range(L)]


def run_decode(args, cfg, layers):
    import numpy as np
    import torch
    from quantized_moe_router_amd import ops
    from workloads import gen as G

    L = len(layers)
    T, H = cfg.tokens, cfg.hidden
    dims = layers[0][0].dims
    ws = ops.workspace(dims, T)
    outs = [torch.empty(T, H, dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    xs = [layer_inputs(cfg, s, L, T) for s in range(args.steps + 1)]

    # eager warm-up, then graphs: one per timed step (own inputs; an event pair around the
    # dominant kernel of one layer, a different layer each step)
    idx = [torch.empty(T, cfg.top_k, dtype=torch.int32, device="cuda") for _ in range(L)]
    for l, (pl, _) in enumerate(layers):
        ops.layer_forward(pl.weights, xs[0][l], ws, out=outs[l], topk_idx=idx[l])
    torch.cuda.synchronize()
    distinct = [len(np.unique(i.cpu().numpy())) for i in idx]
    g_plain = capture_step(ops, layers, xs[0], outs, ws)
    evs = [(ops.Event(), ops.Event()) for _ in range(args.steps)]
    try:
        graphs = [capture_step(ops, layers, xs[s + 1], outs, ws, evs[s], s % L)
                  for s in range(args.steps)]
        graph_events = True
    except Exception as e:
        log(f"event nodes could not be captured ({e}); graphs without events")
        ops.set_profile_events(None, None)
        torch.cuda.synchronize()
        graphs = [capture_step(ops, layers, xs[s + 1], outs, ws) for s in range(args.steps)]
        graph_events = False
    torch.cuda.synchronize()
    for s in range(args.warmup):
        g_plain.replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for s in range(args.steps):
        graphs[s].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # dominant kernel: the event pairs recorded around it inside the timed replays
    durs = None
    if graph_events:
        try:
            if T == 1:      # one pair around the step's L back-to-back layer kernels
                durs = [evs[s][0].elapsed_ms(evs[s][1]) / L for s in range(args.steps)]
                timing_src = ("HIP event nodes before the first and after the last of the "
                              f"{L} layer kernels of each timed graph replay, divided by {L}")
            else:
                durs = [evs[s][0].elapsed_ms(evs[s][1]) for s in range(args.steps)]
                timing_src = ("HIP event nodes around the kernel (one layer per step) in the "
                              "timed graph replays")
        except Exception as e:      # event nodes not timed by this runtime: eager instrumented pass
            log(f"graph event timing unavailable ({e})")
    if durs is None:
        durs = eager_kernel_times(ops, layers, xs, outs, ws, args.steps)
        timing_src = "HIP events around the kernel in eager calls (same inputs, after the timed region)"
    kern_ms = sum(durs) / len(durs)

    # the same stack without any timing events, for reference
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for s in range(args.steps):
        g_plain.replay()
    torch.cuda.synchronize()
    ms_plain = (time.perf_counter() - t2) * 1e3 / args.steps

    n_dist = float(np.mean(distinct))
    credited = G.credited_expert_bytes(cfg, n_dist)                   # routed bytes per layer
    all_bytes = credited + G.expert_bytes(cfg, cfg.shared_inter) + G.router_bytes(cfg)
    if T == 1:
        kernel = "decode_layer_kernel (the whole one-token layer in one launch)"
        kern_bytes = all_bytes
        traffic = stored_traffic(f"decode_layer_kernel_{cfg.name}")
    else:
        kernel = "gu_pf_kernel (routed and shared gate/up + SwiGLU, matrix cores)"
        kern_bytes = (n_dist * 2 * G.matrix_bytes(cfg.inter, H)
                      + 2 * G.matrix_bytes(cfg.shared_inter, H))
        traffic = None
    tok_s_layer = T * L / (ms_step / 1e3)
    layer_s = ms_step / 1e3 / L
    kern_gbps = kern_bytes / (kern_ms / 1e3) / 1e9
    return dict(
        ms_step=ms_step, ms_plain=ms_plain, tok_s_layer=tok_s_layer, L=L, T=T,
        kern_ms=kern_ms, kern_bytes=kern_bytes, kern_gbps=kern_gbps, kernel=kernel,
        layer_credited_gbps=credited / layer_s / 1e9,
        layer_all_gbps=all_bytes / layer_s / 1e9,
        credited=credited, all_bytes=all_bytes, distinct=n_dist, timing_src=timing_src,
        traffic=traffic,
    )


def time_stack(ops, weights, xs, ws, steps):
    """Seconds per layer call of one graph replaying the stack (xs[l] -> its own output)."""
    import torch
    outs = [torch.empty_like(x) for x in xs]
    for w, x, o in zip(weights, xs, outs):
        ops.layer_forward(w, x, ws, out=o)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for w, x, o in zip(weights, xs, outs):
            ops.layer_forward(w, x, ws, out=o)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps / len(weights)


def post_weights(layers, cfg):
    """The stack's layers with the post-combine norm and layer scalar switched on (the
    LayerWeights keep their gain and scalar tensors alive)."""
    import torch
    from quantized_moe_router_amd import ops
    from workloads import gen as G
    weights = []
    for l, (pl, _) in enumerate(layers):
        gain, scalar = G.make_post(cfg, l)
        g = torch.from_numpy(gain).cuda()
        sc = torch.tensor([scalar], dtype=torch.float32, device="cuda")
        weights.append(ops.LayerWeights(pl.dims, pl.router, pl.store, pl.stride, pl.shared,
                                        post_norm_gain=g, layer_scalar=sc))
    return weights


def run_post(layers, cfg, steps):
    """The decode stack with the post-combine norm and layer scalar switched on."""
    from quantized_moe_router_amd import ops
    weights = post_weights(layers, cfg)
    xs = [x for x in layer_inputs(cfg, 0, len(layers), cfg.tokens)]
    ws = ops.workspace(layers[0][0].dims, cfg.tokens)
    return time_stack(ops, weights, xs, ws, steps)


def time_graph(fn, steps):
    """Seconds per replay of a graph holding fn()."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def run_chain(layers, cfg, steps):
    """One token through the whole stack with each layer's input the previous layer's output:
    as one chained launch (qmoe_decode_stack) and as one-token layer calls in a graph.  The
    layers carry the post-combine norm and layer scalar, which keep the chained residual
    stream of the synthetic weights in range."""
    import torch
    from quantized_moe_router_amd import ops
    weights = post_weights(layers, cfg)
    L, H = len(weights), cfg.hidden
    x = layer_inputs(cfg, 0, 1, 1)[0]
    ws = ops.workspace(layers[0][0].dims, 1)
    out_s = torch.empty(L, H, dtype=torch.bfloat16, device="cuda")
    out_c = torch.empty(L, H, dtype=torch.bfloat16, device="cuda")

    def chained_calls():
        cur = x
        for l, w in enumerate(weights):
            ops.layer_forward(w, cur, ws, out=out_c[l:l + 1])
            cur = out_c[l:l + 1]

    t_stack = time_graph(lambda: ops.decode_stack(weights, x, ws, out=out_s), steps)
    t_calls = time_graph(chained_calls, steps)
    same = bool(torch.equal(out_s.view(torch.int16), out_c.view(torch.int16)))
    finite = bool(torch.isfinite(out_s.float()).all())
    return {"us_per_layer": round(t_stack * 1e6 / L, 3), "outputs_finite": finite,
            "tokens_per_s_per_layer": round(L / t_stack, 1),
            "chained_layer_calls_us_per_layer": round(t_calls * 1e6 / L, 3),
            "outputs_equal_chained_calls": same, "layers": L}


def run_other_configs(n_layers, steps):
    """Per-layer time of the other workload shapes on a short stack of their own layers."""
    from quantized_moe_router_amd import ops
    from workloads import gen as G
    res = {}
    for name, src in [("qwen3_next_80b_a3b_decode_b1", None),
                      ("qwen3_next_80b_a3b_decode_b16", "qwen3_next_80b_a3b_decode_b1"),
                      ("qwen3_6_35b_a3b_long_prefill", None),
                      ("gemma4_26b_a4b_int8_decode", None)]:
        cfg = G.config(name)
        layers = build_stack(G.config(src or name), n_layers)
        xs = [x for x in layer_inputs(cfg, 0, n_layers, cfg.tokens)]
        ws = ops.workspace(layers[0][0].dims, cfg.tokens)
        sec = time_stack(ops, [pl.weights for pl, _ in layers], xs, ws, steps)
        res[name] = {"tokens_per_call": cfg.tokens, "us_per_layer_call": round(sec * 1e6, 2),
                     "tokens_per_s_per_layer": round(cfg.tokens / sec, 1),
                     "expert_bits": cfg.expert_bits,
                     "stack": f"{n_layers} layers of this shape (of {cfg.layers})"}
        del layers, xs, ws
        import torch
        torch.cuda.empty_cache()
    return res


def run_tiered(layers, cfg, slots, steps):
    """One-token steps through the first layers of the stack with their routed experts in pinned
    host memory and `slots` device slots per layer: per-layer time, hit rate, copy rate."""
    import torch
    from quantized_moe_router_amd import ops
    from workloads import gen as G
    caches, keep = [], []
    for pl, _ in layers:
        host = torch.empty(pl.store.numel(), dtype=torch.uint8, pin_memory=True)
        host.copy_(pl.store)
        slot_store = torch.empty(slots * pl.stride, dtype=torch.uint8, device="cuda")
        keep += [host, slot_store]
        caches.append(ops.ExpertCache(pl.dims, host, pl.stride, slot_store, pl.stride, slots))
    ws = ops.workspace(layers[0][0].dims, 1)
    xs = [layer_inputs(cfg, s, len(layers), 1) for s in range(steps + 2)]
    out = torch.empty(1, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    for s in range(2):      # warm-up: fills the caches
        for l, (pl, _) in enumerate(layers):
            ops.layer_forward_tiered(pl.weights, caches[l], xs[s][l], ws, out=out)
    torch.cuda.synchronize()
    h0 = [c.stats() for c in caches]
    t0 = time.perf_counter()
    for s in range(steps):
        for l, (pl, _) in enumerate(layers):
            ops.layer_forward_tiered(pl.weights, caches[l], xs[s + 2][l], ws, out=out)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps / len(layers)
    hits = sum(c.stats()[0] - h[0] for c, h in zip(caches, h0))
    misses = sum(c.stats()[1] - h[1] for c, h in zip(caches, h0))
    copied = misses * G.expert_bytes(cfg) / (steps * len(layers))
    return dict(us_per_layer=round(sec * 1e6, 1), slots_per_layer=slots,
                hit_rate=round(hits / max(hits + misses, 1), 3),
                copied_MB_per_layer=round(copied / 1e6, 2),
                host_to_device_GBps=round(copied / sec / 1e9, 1),
                stack=f"first {len(layers)} layers, 1 token per step, {steps} steps")


def run_prefill(layers, cfg_pf, reps=3):
    """One 128-token chunk per layer through the same stack (prefill shape), graph-replayed."""
    import numpy as np
    import torch
    from quantized_moe_router_amd import ops
    from workloads import gen as G

    L = len(layers)
    T, H = cfg_pf.tokens, cfg_pf.hidden
    dims = layers[0][0].dims
    ws = ops.workspace(dims, T)
    outs = [torch.empty(T, H, dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    xs = [layer_inputs(cfg_pf, 100 + r, L, T) for r in range(reps + 1)]
    idx = [torch.empty(T, cfg_pf.top_k, dtype=torch.int32, device="cuda") for _ in range(L)]
    for l, (pl, _) in enumerate(layers):
        ops.layer_forward(pl.weights, xs[0][l], ws, out=outs[l], topk_idx=idx[l])
    torch.cuda.synchronize()
    distinct = [len(np.unique(i.cpu().numpy())) for i in idx]
    # one graph per input set (the chunk through every layer), replayed as the decode stack is
    graphs = []
    for r in range(reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l, (pl, _) in enumerate(layers):
                ops.layer_forward(pl.weights, xs[r + 1][l], ws, out=outs[l])
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    ms_chunk_stack = (time.perf_counter() - t0) * 1e3 / reps
    layer_s = ms_chunk_stack / 1e3 / L
    credited = G.credited_expert_bytes(cfg_pf, float(np.mean(distinct)))
    return dict(tok_s_layer=T / layer_s, us_per_chunk_layer=layer_s * 1e6,
                credited_gbps=credited / layer_s / 1e9, distinct_mean=float(np.mean(distinct)))


def cpu_baseline(cfg, n_samples):
    """The oracle on the host: token-layers of the same workload, each with its own input."""
    import numpy as np
    import oracle as O
    from workloads import gen as G
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    times = []
    for l in range(n_samples):
        x = G.make_hidden(cfg, l)            # each layer gets its own N(0,1) hidden states
        li = G.make_router(cfg, l)
        top, _, _ = O.router(x, li, cfg.top_k)          # untimed: which experts to draw
        for e in np.unique(top):
            li.expert(int(e))
        li.shared()
        t0 = time.perf_counter()
        r = O.layer_forward(x, li, cfg.top_k)
        times.append(time.perf_counter() - t0)
        assert r["out"].shape == x.shape
    s_per_unit = float(np.median(times))
    return dict(value=cfg.tokens / s_per_unit, unit="tokens/s per MoE layer", cores=int(threads),
                kind="oracle",
                sample=f"{n_samples} token-layers ({cfg.name}, layers 0..{n_samples - 1}, 1 token "
                       f"each); median {s_per_unit:.3f} s per token-layer; drawing the synthetic "
                       f"experts is excluded")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the layer is measured on a "
              f"single MI355X and a multi-GPU figure is not produced.", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        torch.cuda.set_device(0)
        copy_calibration(args.copy_calibration)
        return
    import __graft_entry__ as GE
    GE._ensure_built()
    from workloads import gen as G

    torch.cuda.set_device(0)
    cfg = G.config(args.workload)
    n_layers = args.layers or cfg.layers
    log(f"building {cfg.name}: {n_layers} layers")
    layers = build_stack(cfg, n_layers)
    log("decode timing")
    d = run_decode(args, cfg, layers)
    log(f"decode: {d['ms_step']:.3f} ms/step ({d['ms_plain']:.3f} without events), "
        f"{d['kernel'].split()[0]} {d['kern_ms'] * 1e3:.2f} us = {d['kern_gbps']:.0f} GB/s")
    pf = None
    if not args.no_prefill and cfg.name == "gemma4_26b_a4b_decode":
        log("prefill timing")
        pf = run_prefill(layers, G.config("gemma4_26b_a4b_prefill"))
    post = other = tiered = chain = None
    if not args.no_extra and cfg.tokens == 1:
        log("post-combine norm stack timing")
        post = run_post(layers, cfg, args.steps)
        log("chained launch over the stack")
        chain = run_chain(layers, cfg, args.steps)
        log(f"chained launch: {chain['us_per_layer']} us/layer "
            f"(chained layer calls {chain['chained_layer_calls_us_per_layer']})")
        if cfg.name == "gemma4_26b_a4b_decode":
            log("tiered residency (16 slots per layer)")
            tiered = run_tiered(layers[:4], cfg, 16, args.steps)
            log("other workload shapes (4-layer stacks)")
            other = run_other_configs(4, args.steps)
    cb = None
    if not args.no_cpu_baseline:
        log("cpu oracle timing")
        cb = cpu_baseline(cfg, args.cpu_sample)
    out = {
        "metric": METRIC,
        "value": round(d["tok_s_layer"], 1),
        "unit": "tokens/s per MoE layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded Philox draws, quantised to MLX affine int4/int8)",
        "config": {
            "workload": f"{cfg.name}: hidden {cfg.hidden}, {cfg.experts} experts top-{cfg.top_k}, "
                        f"expert inter {cfg.inter}, shared inter {cfg.shared_inter}, "
                        f"{d['L']} stacked layers, {cfg.tokens} token/step",
            "tokens_per_step": cfg.tokens, "layers": d["L"], "graph_replay": True,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": d["kernel"],
            "achieved": round(d["kern_gbps"], 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(d["kern_gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": d["traffic"],
            "bytes_per_launch": int(d["kern_bytes"]),
            "avg_launch_us": round(d["kern_ms"] * 1e3, 3),
            "timing": d["timing_src"],
        },
        "layer": {
            "credited_GBps": round(d["layer_credited_gbps"], 1),
            "credited_frac_of_peak": round(d["layer_credited_gbps"] / HBM_PEAK_GBPS, 4),
            "all_bytes_GBps": round(d["layer_all_gbps"], 1),
            "us_per_layer": round(d["ms_step"] * 1e3 / d["L"], 3),
            "us_per_layer_without_events": round(d["ms_plain"] * 1e3 / d["L"], 3),
            "distinct_experts_per_layer": round(d["distinct"], 2),
        },
    }
    if pf:
        out["prefill"] = {
            "workload": "gemma4_26b_a4b_prefill: one 128-token chunk through the same stack (graph replay)",
            "tokens_per_s_per_layer": round(pf["tok_s_layer"], 1),
            "us_per_chunk_layer": round(pf["us_per_chunk_layer"], 2),
            "credited_GBps": round(pf["credited_gbps"], 1),
            "distinct_experts_per_chunk": round(pf["distinct_mean"], 2),
        }
    if post:
        out["post_combine_norm"] = {
            "workload": f"{cfg.name} with the post-combine RMS norm (gain) and layer scalar",
            "us_per_layer": round(post * 1e6, 3),
        }
    if chain:
        out["chained_stack"] = dict(chain, workload=f"{cfg.name} with the post-combine norm and "
                                    f"layer scalar: one token through all {chain['layers']} "
                                    "layers, x of each layer the bf16 output of the one before, "
                                    "in one launch (qmoe_decode_stack)")
    if tiered:
        out["tiered_residency"] = dict(tiered, workload=f"{cfg.name}: routed experts in pinned host "
                                       "memory, LFU-with-recency device cache per layer")
    if other:
        out["other_workloads"] = other
    if cb:
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
