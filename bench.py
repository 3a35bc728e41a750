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
on the host.  Beside the headline it reports every other workload at its configured size
("configs": the tiny layer, the Gemma-shaped prefill chunk, the 48-layer Qwen3-Next-shaped
stack at batch 1 and 16, the 40-layer Qwen3.6-shaped stack with one 10,240-token prompt per
layer and its bucket sizes, int8 experts), each with its dominant kernel's roofline and the
oracle timed on a bounded sample, and the plain streaming-read reference.

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
    p.add_argument("--timeline", action="store_true",
                   help="only run the one-token stack once with the profiling build's phase "
                        "timestamps and write profiles/decode_timeline_<workload>.md")
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

    status = ops.workspace_status(ws)      # 0: no wait of the timed one-token calls timed out
    if status != 0:
        raise RuntimeError(f"workspace status {status} after the timed replays: a one-token "
                           "call gave up waiting, its results are not valid")
    n_dist = float(np.mean(distinct))
    credited = G.credited_expert_bytes(cfg, n_dist)                   # routed bytes per layer
    all_bytes = credited + G.expert_bytes(cfg, cfg.shared_inter) + G.router_bytes(cfg)
    if T == 1:
        # credited bytes only: the distinct routed experts' codes, scales and biases (the
        # shared expert and the router are reported beside, not credited)
        kernel = "decode_layer_kernel (the whole one-token layer in one launch)"
        kern_bytes = credited
        traffic = stored_traffic(f"decode_layer_kernel_{cfg.name}")
    else:
        kernel = "gu_pf_kernel (routed and shared gate/up + SwiGLU, matrix cores)"
        kern_bytes = (n_dist * 2 * G.matrix_bytes(cfg.inter, H)
                      + 2 * G.matrix_bytes(cfg.shared_inter, H))
        traffic = stored_traffic(f"prefill_kernels_{cfg.name}")
    tok_s_layer = T * L / (ms_step / 1e3)
    layer_s = ms_step / 1e3 / L
    kern_gbps = kern_bytes / (kern_ms / 1e3) / 1e9
    # credited (routed-only) bytes of the dominant kernel
    kern_credited = credited if T == 1 else n_dist * 2 * G.matrix_bytes(cfg.inter, H)
    return dict(
        ms_step=ms_step, ms_plain=ms_plain, tok_s_layer=tok_s_layer, L=L, T=T, status=status,
        kern_ms=kern_ms, kern_bytes=kern_bytes, kern_gbps=kern_gbps, kernel=kernel,
        kern_credited=kern_credited,
        layer_credited_gbps=credited / layer_s / 1e9,
        layer_all_gbps=all_bytes / layer_s / 1e9,
        credited=credited, all_bytes=all_bytes, distinct=n_dist, timing_src=timing_src,
        traffic=traffic, buckets=bucket_histogram([i.cpu().numpy() for i in idx], cfg.experts)
        if T > 1 else None,
    )


def bucket_histogram(idx_layers, E, chunk=128):
    """Bucket sizes of the routing (rows per expert per chunk of at most 128 tokens): the mean
    and the maximum over chunks of the largest bucket, the mean number of non-empty buckets and
    the mean rows per non-empty bucket."""
    import numpy as np
    mx, ne, rows = [], [], []
    for idx in idx_layers:
        for c0 in range(0, idx.shape[0], chunk):
            cnt = np.bincount(idx[c0:c0 + chunk].ravel(), minlength=E)
            mx.append(int(cnt.max()))
            ne.append(int((cnt > 0).sum()))
            rows.append(float(cnt[cnt > 0].mean()))
    return {"chunks": len(mx), "max_bucket_mean": round(float(np.mean(mx)), 2),
            "max_bucket_max": int(np.max(mx)), "nonempty_mean": round(float(np.mean(ne)), 2),
            "rows_per_nonempty_mean": round(float(np.mean(rows)), 2)}


def config_entry(d, cfg, note=None):
    """One workload's line: throughput per MoE layer and the dominant kernel's roofline."""
    from workloads import gen as G
    e = {"workload": f"{cfg.name}: hidden {cfg.hidden}, {cfg.experts} experts top-{cfg.top_k}, "
                     f"expert inter {cfg.inter}, shared inter {cfg.shared_inter}, "
                     f"{cfg.expert_bits}-bit experts, {d['L']} stacked layers (of {cfg.layers}), "
                     f"{d['T']} tokens per call",
         "tokens_per_s_per_layer": round(d["tok_s_layer"], 1),
         "us_per_layer_call": round(d["ms_step"] * 1e3 / d["L"], 3),
         "credited_GBps": round(d["layer_credited_gbps"], 1),
         "distinct_experts_per_call": round(d["distinct"], 2),
         "roofline": {"bound": "hbm", "kernel": d["kernel"],
                      "achieved": round(d["kern_credited"] / (d["kern_ms"] / 1e3) / 1e9, 1),
                      "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                      "frac": round(d["kern_credited"] / (d["kern_ms"] / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                      "bytes": "credited routed bytes of the kernel",
                      "all_bytes_frac": round((d["all_bytes"] if d["T"] == 1 else d["kern_bytes"])
                                              / (d["kern_ms"] / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                      "avg_launch_us": round(d["kern_ms"] * 1e3, 3), "timing": d["timing_src"],
                      "traffic": d["traffic"]}}
    if d.get("buckets"):
        e["buckets"] = d["buckets"]
    if note:
        e["note"] = note
    return e


def run_long_prefill(args, cfg, layers):
    """The long prompt of the Zipf-biased Qwen3.6-shaped config: one prompt of cfg.prompt tokens
    through every layer of the stack, each layer call taking the whole prompt (processed per
    128-token chunk inside the call), all layers in one graph.  Every layer gets its own N(0,1)
    prompt states.  The dominant kernel (routed + shared gate/up) is timed with HIP event nodes
    around it in a graph of one 128-token chunk of each layer's prompt."""
    import numpy as np
    import torch
    from quantized_moe_router_amd import ops
    from workloads import gen as G
    import stacks
    L, P, H, k = len(layers), cfg.prompt, cfg.hidden, cfg.top_k
    ws = ops.workspace(layers[0][0].dims, min(P, 128))
    xs = [stacks.hidden(cfg, 500 + l, P)[1] for l in range(L)]
    out = torch.empty(P, H, dtype=torch.bfloat16, device="cuda")
    idx = [torch.empty(P, k, dtype=torch.int32, device="cuda") for _ in range(L)]
    for l, (pl, _) in enumerate(layers):
        ops.layer_forward(pl.weights, xs[l], ws, out=out, topk_idx=idx[l])
    torch.cuda.synchronize()
    idx_n = [i.cpu().numpy() for i in idx]
    buckets = bucket_histogram(idx_n, cfg.experts)
    distinct = float(np.mean([len(np.unique(i[c:c + 128])) for i in idx_n for c in range(0, P, 128)]))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l, (pl, _) in enumerate(layers):
            ops.layer_forward(pl.weights, xs[l], ws, out=out)
    g.replay()
    torch.cuda.synchronize()
    reps = 2
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / reps
    n_chunks = (P + 127) // 128
    chunk_layer_s = sec / (L * n_chunks)
    # the dominant kernel, one chunk per layer (the event pair around layer s's gate/up kernel)
    evs = [(ops.Event(), ops.Event()) for _ in range(L)]
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        for l, (pl, _) in enumerate(layers):
            ops.set_profile_events(*evs[l])
            ops.layer_forward(pl.weights, xs[l][40 * 128:41 * 128], ws, out=out[:128])
            ops.set_profile_events(None, None)
    g2.replay()
    torch.cuda.synchronize()
    g2.replay()
    torch.cuda.synchronize()
    kern_ms = float(np.mean([a.elapsed_ms(b) for a, b in evs]))
    d40 = float(np.mean([len(np.unique(i[40 * 128:41 * 128])) for i in idx_n]))
    kern_credited = d40 * 2 * G.matrix_bytes(cfg.inter, H)
    kern_all = kern_credited + 2 * G.matrix_bytes(cfg.shared_inter, H)
    credited = G.credited_expert_bytes(cfg, distinct)
    return {"workload": f"{cfg.name}: hidden {H}, {cfg.experts} experts top-{k} with the Zipf("
                        f"{cfg.zipf_s}) router bias, expert inter {cfg.inter}, shared inter "
                        f"{cfg.shared_inter}, {L} stacked layers, one {P}-token prompt per layer "
                        f"({n_chunks} chunks of 128 tokens per layer call)",
            "tokens_per_s_per_layer": round(P / (sec / L), 1),
            "us_per_chunk_layer": round(chunk_layer_s * 1e6, 3),
            "prompt_ms_all_layers": round(sec * 1e3, 3),
            "credited_GBps": round(credited / chunk_layer_s / 1e9, 1),
            "distinct_experts_per_chunk": round(distinct, 2), "buckets": buckets,
            "roofline": {"bound": "hbm", "kernel": "gu_pf_kernel (routed and shared gate/up + "
                         "SwiGLU, matrix cores)",
                         "achieved": round(kern_credited / (kern_ms / 1e3) / 1e9, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(kern_credited / (kern_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "bytes": "credited routed bytes of the kernel",
                         "all_bytes_frac": round(kern_all / (kern_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "avg_launch_us": round(kern_ms * 1e3, 3),
                         "timing": f"HIP event nodes around the kernel of chunk 40 of each of the {L} "
                                   "layers' prompts, one graph",
                         "traffic": stored_traffic(f"prefill_kernels_{cfg.name}")}}


def oracle_sample(cfg, samples):
    """The oracle on the host, timed on `samples` = [(layer, step, tokens)]: median seconds per
    call (drawing the synthetic experts excluded)."""
    import numpy as np
    import oracle as O
    from workloads import gen as G
    times = []
    for layer, step, T in samples:
        x = G.make_hidden(cfg, step, T)
        li = G.make_router(cfg, layer)
        top, _, _ = O.router(x, li, cfg.top_k)
        li.prefetch(np.unique(top))
        li.shared()
        t0 = time.perf_counter()
        r = O.layer_forward(x, li, cfg.top_k)
        times.append(time.perf_counter() - t0)
        assert r["out"].shape == x.shape
    return float(np.median(times))


def run_read_ceiling(layers, cfg, reps=5):
    """The plain streaming read (qmoe_read_blocks) as the achievable-bandwidth reference: the
    same volume and access shape as one decode layer's routed weights -- the distinct experts a
    token of each layer selects, whole fixed-stride blocks of the layer's store -- read once per
    layer of the stack in one graph (HIP event nodes before the first and after the last read,
    divided by the layer count, as the layer kernel is timed), and a 1 GiB contiguous read."""
    import numpy as np
    import torch
    from quantized_moe_router_amd import ops
    from workloads import gen as G
    L = len(layers)
    nbytes = G.expert_bytes(cfg)
    nbytes -= nbytes % 16
    xs = layer_inputs(cfg, 7, L, 1)
    ws = ops.workspace(layers[0][0].dims, 1)
    ids = []
    for l, (pl, _) in enumerate(layers):
        idx = torch.empty(1, cfg.top_k, dtype=torch.int32, device="cuda")
        ops.layer_forward(pl.weights, xs[l], ws, topk_idx=idx)
        ids.append(sorted(set(idx.cpu().numpy().ravel().tolist())))
    nmax = max(len(i) for i in ids) * ((nbytes + 16383) // 16384)
    sink = torch.empty(nmax, dtype=torch.int32, device="cuda")
    ev0, ev1 = ops.Event(), ops.Event()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ev0.record()
        for (pl, _), i in zip(layers, ids):
            ops.read_blocks(pl.store, pl.stride, i, nbytes, sink)
        ev1.record()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        g.replay()
        torch.cuda.synchronize()
        per.append(ev0.elapsed_ms(ev1) / L)
    us = float(np.median(per)) * 1e3
    moved = float(np.mean([len(i) for i in ids])) * nbytes
    big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    sink2 = torch.empty((1 << 30) // 16384, dtype=torch.int32, device="cuda")
    t = []
    for _ in range(reps + 1):
        a, b = ops.Event(), ops.Event()
        a.record()
        ops.read_blocks(big, 0, [0], 1 << 30, sink2)
        b.record()
        torch.cuda.synchronize()
        t.append(a.elapsed_ms(b))
    gib_us = float(np.median(t[1:])) * 1e3
    del big
    return {"blocks_per_read": round(float(np.mean([len(i) for i in ids])), 2),
            "bytes_per_read": int(moved), "us_per_read": round(us, 3),
            "GBps": round(moved / (us * 1e-6) / 1e9, 1),
            "contiguous_1GiB_GBps": round((1 << 30) / (gib_us * 1e-6) / 1e9, 1),
            "kernel": "stream_read_kernel (qmoe_read_blocks): 16 KiB per wave, 8 non-temporal "
                      "16-byte loads in flight per lane",
            "timing": f"graph of {L} reads (one per layer), HIP event nodes around them, "
                      f"divided by {L}; the 1 GiB read: HIP events around one launch"}


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


def run_other_configs(args):
    """The other workloads at their configured sizes (each stack built, timed and freed in
    turn), each with its oracle timed on a bounded sample."""
    import torch
    from workloads import gen as G
    res = {}

    def cpu(cfg, samples, unit, what):
        if args.no_cpu_baseline:
            return None
        sec = oracle_sample(cfg, samples)
        return {"value": round(samples[0][2] / sec, 3), "unit": f"tokens/s per MoE layer ({unit})",
                "s_per_call": round(sec, 4), "kind": "oracle", "sample": what}

    def done(*stacks_):
        for st in stacks_:
            del st[:]
        torch.cuda.empty_cache()

    # tiny single layer, 4 tokens (the whole configuration)
    c1 = G.config("tiny")
    log("tiny layer")
    lay = build_stack(c1, 1)
    res[c1.name] = config_entry(run_decode(args, c1, lay), c1)
    res[c1.name]["cpu_baseline"] = cpu(c1, [(0, s, 4) for s in range(5)], "4-token call",
                                       "the 4-token call, 5 inputs, median")
    done(lay)
    # Qwen3-Next-shaped stack, 48 layers (43.5 GB), batch 1 and batch 16
    b1, b16 = G.config("qwen3_next_80b_a3b_decode_b1"), G.config("qwen3_next_80b_a3b_decode_b16")
    log(f"{b1.name}: building {b1.layers} layers")
    lay = build_stack(b1, b1.layers)
    for c, smp, unit, what in [(b1, [(l, l, 1) for l in range(4)], "token-layer",
                                "layers 0..3, one token each, median"),
                               (b16, [(0, 0, 16)], "16-token step-layer",
                                "layer 0, one 16-token step")]:
        log(f"{c.name} timing")
        res[c.name] = config_entry(run_decode(args, c, lay), c)
        res[c.name]["cpu_baseline"] = cpu(c, smp, unit, what)
    done(lay)
    # Qwen3.6-shaped long prefill: 40 layers, one 10,240-token prompt per layer
    c5 = G.config("qwen3_6_35b_a3b_long_prefill")
    log(f"{c5.name}: building {c5.layers} layers")
    lay = build_stack(c5, c5.layers)
    log(f"{c5.name}: {c5.prompt}-token prompt")
    res[c5.name] = run_long_prefill(args, c5, lay)
    res[c5.name]["cpu_baseline"] = cpu(c5, [(0, 500, 128)], "128-token chunk-layer",
                                       "chunk 0 of layer 0's prompt")
    done(lay)
    # int8 experts (Gemma-4 shape), a 4-layer stack
    c8 = G.config("gemma4_26b_a4b_int8_decode")
    log(f"{c8.name}: 4 layers")
    lay = build_stack(c8, 4)
    res[c8.name] = config_entry(run_decode(args, c8, lay), c8,
                                note="int8 experts, a 4-layer stack of the 30-layer shape")
    done(lay)
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
    host = dict(os_cpu_count=os.cpu_count(), affinity_cores=len(os.sched_getaffinity(0)),
                blas_threads=int(threads))
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
                kind="oracle", host=host,
                sample=f"{n_samples} token-layers ({cfg.name}, layers 0..{n_samples - 1}, 1 token "
                       f"each); median {s_per_unit:.3f} s per token-layer; drawing the synthetic "
                       f"experts is excluded")


TL_POINTS = 8
TL_ROLES = {1: ("router", {1: "logits published"}),
            2: ("shared gate/up", {1: "x staged"}),
            3: ("routed gate/up", {1: "x staged", 2: "expert known", 3: "weights consumed"}),
            4: ("shared down", {1: "router seen", 2: "weights in", 3: "h staged"}),
            5: ("routed down", {1: "top-k known", 2: "weights in", 3: "h staged",
                                4: "products done", 5: "combine inputs in"})}


def run_timeline(args, cfg, layers):
    """Phase timestamps of the one-token layer (profiling build, QMOE_LIBRARY=timeline): the
    stack captured in one graph with a timestamp buffer per layer, replayed a few times, then
    once more into zeroed buffers.  Per role and point: the median and the maximum over the
    role's workgroups of the time since the layer kernel's first workgroup started, each
    taken as the median over the layers.  Routed window: from the first routed gate/up
    workgroup that knows its expert (its weight loads start) to the last routed weight byte in
    (the last routed gate/up workgroup's weights consumed, or the last routed down
    workgroup's down weights in); credited routed bytes over that window."""
    import numpy as np
    import torch
    from quantized_moe_router_amd import ops
    from workloads import gen as G
    L, T, H = len(layers), 1, cfg.hidden
    ws = ops.workspace(layers[0][0].dims, T)
    outs = [torch.empty(T, H, dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    xs = layer_inputs(cfg, 0, L, T)
    idx = [torch.empty(T, cfg.top_k, dtype=torch.int32, device="cuda") for _ in range(L)]
    for l, (pl, _) in enumerate(layers):
        ops.layer_forward(pl.weights, xs[l], ws, out=outs[l], topk_idx=idx[l])
    torch.cuda.synchronize()
    distinct = float(np.mean([len(np.unique(i.cpu().numpy())) for i in idx]))
    max_blocks = 8192
    buf = torch.zeros(L, max_blocks * TL_POINTS, dtype=torch.int64, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l, (pl, _) in enumerate(layers):
            ops.timeline_set(buf[l])
            ops.layer_forward(pl.weights, xs[l], ws, out=outs[l])
        ops.timeline_set(None)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    buf.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    status = ops.workspace_status(ws)
    tl = buf.cpu().numpy().reshape(L, max_blocks, TL_POINTS)
    per_layer = {}
    windows, kern = [], []
    for l in range(L):
        rows = tl[l]
        role = rows[:, TL_POINTS - 1]
        used = role > 0
        t0 = rows[used, 0].min()
        us = (rows[:, :TL_POINTS - 1] - t0) / 100.0          # 100 MHz clock -> microseconds
        kern.append(us[used, 6].max())
        for r, (name, pts) in TL_ROLES.items():
            m = role == r
            if not m.any():
                continue
            for p in [0] + sorted(pts) + [6]:
                mp = m & (rows[:, p] > 0)       # workgroups that record this point
                if mp.any():
                    per_layer.setdefault((r, p), []).append((np.median(us[mp, p]), us[mp, p].max(),
                                                             int(mp.sum())))
        rg, cd = role == 3, (role == 5) & (rows[:, 2] > 0)
        start = us[rg, 2].min()
        end = max(us[rg, 3].max(), us[cd, 2].max() if cd.any() else 0.0)
        windows.append((start, end))
    credited = G.credited_expert_bytes(cfg, distinct)
    w0 = float(np.median([w[0] for w in windows]))
    w1 = float(np.median([w[1] for w in windows]))
    win_gbps = credited / ((w1 - w0) * 1e-6) / 1e9
    lines = []
    for (r, p), v in sorted(per_layer.items()):
        name, pts = TL_ROLES[r]
        label = {0: "start", 6: "end"}.get(p, pts.get(p, str(p)))
        lines.append((name, label, float(np.median([x[0] for x in v])),
                      float(np.median([x[1] for x in v])), v[0][2]))
    return dict(lines=lines, window=(w0, w1), window_gbps=win_gbps, credited=credited,
                kernel_us=float(np.median(kern)), distinct=distinct, status=status, L=L)


def write_timeline(cfg, t, cmd):
    path = os.path.join(ROOT, "profiles", f"decode_timeline_{cfg.name}.md")
    w0, w1 = t["window"]
    with open(path, "w") as f:
        f.write(f"# Phase timeline of decode_layer_kernel -- {cfg.name} ({t['L']} stacked layers, "
                "1 token)\n\n")
        f.write("Profiling build (`libqmoe_timeline.so`: the same sources with QMOE_TIMELINE, thread "
                "0 of every workgroup recording the 100 MHz device clock at fixed points of its "
                "role), one graph replay of the stack after three warm-up replays:\n\n")
        f.write(f"```\n{cmd}\n```\n\n")
        f.write("Times in microseconds since the layer kernel's first workgroup started; per role "
                "and point the median and the maximum over the role's workgroups, each the median "
                "over the layers.\n\n")
        f.write("| role | workgroups | point | median us | max us |\n|---|---|---|---|---|\n")
        for name, label, med, mx, n in t["lines"]:
            f.write(f"| {name} | {n} | {label} | {med:.2f} | {mx:.2f} |\n")
        f.write(f"\nKernel (first workgroup start to last workgroup end): {t['kernel_us']:.2f} us "
                "(median over layers; the launch's dispatch before the first workgroup is not "
                "in it).\n\n")
        f.write(f"Routed weight window: {w0:.2f} us (the first routed gate/up workgroup knows its "
                f"expert and starts its weight loads) to {w1:.2f} us (the last routed weight in: "
                "gate/up weights consumed or routed down weights loaded), "
                f"{w1 - w0:.2f} us for {t['credited'] / 1e6:.2f} MB of credited routed bytes "
                f"({t['distinct']:.1f} distinct experts x {G_expert_mb(cfg):.4f} MB): "
                f"**{t['window_gbps']:.0f} GB/s = {t['window_gbps'] / HBM_PEAK_GBPS:.3f} of "
                "8 TB/s**.\n\n")
        f.write(f"Workspace status after the run: {t['status']} (0 = no wait timed out).\n")
    return path


def G_expert_mb(cfg):
    from workloads import gen as G
    return G.expert_bytes(cfg) / 1e6


def main():
    args = parse()
    if args.timeline:
        os.environ["QMOE_LIBRARY"] = "timeline"
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
    if args.timeline:
        if cfg.tokens != 1:
            sys.exit("--timeline covers the one-token layer")
        t = run_timeline(args, cfg, layers)
        path = write_timeline(cfg, t, "python3 bench.py --timeline --workload " + cfg.name +
                              (f" --layers {n_layers}" if args.layers else ""))
        log(f"timeline: kernel {t['kernel_us']:.2f} us, routed window {t['window'][0]:.2f}.."
            f"{t['window'][1]:.2f} us = {t['window_gbps']:.0f} GB/s, status {t['status']}; "
            f"written to {path}")
        for name, label, med, mx, n in t["lines"]:
            log(f"  {name:16s} {label:20s} {med:7.2f} {mx:7.2f}")
        return
    log("decode timing")
    d = run_decode(args, cfg, layers)
    log(f"decode: {d['ms_step']:.3f} ms/step ({d['ms_plain']:.3f} without events), "
        f"{d['kernel'].split()[0]} {d['kern_ms'] * 1e3:.2f} us = {d['kern_gbps']:.0f} GB/s")
    ceiling = None
    if cfg.tokens == 1:
        log("streaming-read ceiling")
        ceiling = run_read_ceiling(layers, cfg)
        log(f"read ceiling: {ceiling['us_per_read']} us per {ceiling['bytes_per_read'] / 1e6:.2f} MB "
            f"= {ceiling['GBps']} GB/s; 1 GiB contiguous {ceiling['contiguous_1GiB_GBps']} GB/s")
    configs = {}
    if not args.no_prefill and cfg.name == "gemma4_26b_a4b_decode":
        log("prefill timing (one 128-token chunk per layer of the same stack)")
        cfg_pf = G.config("gemma4_26b_a4b_prefill")
        dp = run_decode(args, cfg_pf, layers)
        configs[cfg_pf.name] = config_entry(dp, cfg_pf)
        log(f"prefill: {dp['ms_step'] * 1e3 / dp['L']:.1f} us per chunk-layer, gu_pf_kernel "
            f"{dp['kern_ms'] * 1e3:.1f} us")
        if not args.no_cpu_baseline:
            sec = oracle_sample(cfg_pf, [(0, 100, 128)])
            configs[cfg_pf.name]["cpu_baseline"] = {
                "value": round(128 / sec, 3), "unit": "tokens/s per MoE layer (128-token chunk-layer)",
                "s_per_call": round(sec, 4), "kind": "oracle", "sample": "one 128-token chunk of layer 0"}
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
    cb = None
    if not args.no_cpu_baseline:
        log("cpu oracle timing")
        cb = cpu_baseline(cfg, args.cpu_sample)
    if not args.no_extra and cfg.name == "gemma4_26b_a4b_decode":
        del layers
        torch.cuda.empty_cache()
        configs.update(run_other_configs(args))
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
            "bytes": "credited: distinct routed experts x (int4 codes + bf16 scale and bias)",
            "all_bytes_per_launch": int(d["all_bytes"]) if d["T"] == 1 else None,
            "all_bytes_frac": (round(d["all_bytes"] / (d["kern_ms"] / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)
                               if d["T"] == 1 else None),
            "avg_launch_us": round(d["kern_ms"] * 1e3, 3),
            "timing": d["timing_src"],
            "workspace_status": d["status"],
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
    if ceiling:
        out["read_ceiling"] = ceiling
        out["roofline"]["frac_of_read_ceiling"] = round(d["kern_gbps"] / ceiling["GBps"], 4)
    if configs:
        out["configs"] = configs
    if post:
        out["post_combine_norm"] = {
            "workload": f"{cfg.name} with the post-combine RMS norm (gain) and layer scalar",
            "us_per_layer": round(post * 1e6, 3),
        }
    if chain:
        out["chained_stack"] = dict(chain, workload=f"{cfg.name} with the post-combine norm and "
                                    f"layer scalar: one token through all {chain['layers']} "
                                    "layers, x of each layer the bf16 output of the one before, "
                                    "in one launch (qmoe_decode_stack)",
                                    mode="non-default: slower on this GPU than the same chain as "
                                         "graph-replayed one-token calls (chained_layer_calls)")
    if tiered:
        out["tiered_residency"] = dict(tiered, workload=f"{cfg.name}: routed experts in pinned host "
                                       "memory, LFU-with-recency device cache per layer")

    if cb:
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
