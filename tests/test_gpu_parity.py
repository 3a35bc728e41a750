"""Parity of the HIP path (through the C ABI) against the fp64 oracle.  Needs an MI355X."""
import copy

import numpy as np
import pytest
import torch

import oracle as O
from parity import (assert_close_f32, check_out_bf16, compare_topk, rel_err_rows)
from workloads import gen as G

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_moe_router_amd import _lib
    _lib.lib()          # fails loudly if the HIP library is not built


def _ops():
    from quantized_moe_router_amd import ops
    return ops


def _stacks():
    import stacks
    return stacks


_cache = {}


def layer(name, idx=0):
    key = (name, idx)
    if key not in _cache:
        cfg = G.config(name)
        _cache[key] = _stacks().build_layer(cfg, idx, DEV)
    return _cache[key]


def np16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ------------------------------------------------------------------ generator and store

@pytest.mark.parametrize("name,experts", [("tiny", [0, 7, 15]), ("gemma4_26b_a4b_decode", [0, 77]),
                                          ("qwen3_next_80b_a3b_decode_b1", [511]),
                                          ("tiny_int8", [0, 7, 15]),
                                          ("gemma4_26b_a4b_int8_decode", [5])])
def test_device_generator_matches_host(name, experts):
    from workloads import device as D
    cfg = G.config(name)
    canon = D.CanonLayerExperts(cfg, 3, device=DEV)
    for e in experts:
        want = G.make_expert(cfg, 3, e).arrays()
        for got, w in zip(canon.expert(e), want):
            g = got.cpu().numpy()
            g = g.view(np.uint16) if w.dtype == np.uint16 else g
            assert np.array_equal(g, w), (name, e)


@pytest.mark.parametrize("name", ["tiny", "gemma4_26b_a4b_decode", "tiny_int8",
                                  "gemma4_26b_a4b_int8_decode"])
def test_pack_unpack_round_trip(name):
    ops = _ops()
    cfg = G.config(name)
    pl, li = layer(name)
    for e, ew, inter, blk in [(5, li.expert(5), cfg.inter, pl.store[5 * pl.stride:6 * pl.stride]),
                              ("sh", li.shared(), cfg.shared_inter, pl.shared)]:
        outs = [torch.empty_like(torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a),
                                 device=DEV) for a in ew.arrays()]
        ops.unpack_expert(pl.dims, inter, blk, *outs)
        for got, w in zip(outs, ew.arrays()):
            g = got.cpu().numpy()
            g = g.view(np.uint16) if w.dtype == np.uint16 else g
            assert np.array_equal(g, w), (name, e)


def test_pack_is_layout_only_byte_count():
    ops = _ops()
    cfg = G.config("gemma4_26b_a4b_decode")
    pl, _ = layer("gemma4_26b_a4b_decode")
    assert ops.expert_stride(pl.dims, cfg.inter) == 3346432          # 3,345,408 rounded to 4 KiB
    assert G.expert_bytes(cfg) == 3345408


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("name,T", [("tiny", 4), ("gemma4_26b_a4b_decode", 1),
                                    ("gemma4_26b_a4b_prefill", 128),
                                    ("qwen3_next_80b_a3b_decode_b16", 16),
                                    ("qwen3_6_35b_a3b_long_prefill", 128), ("tiny", 131)])
def test_router_parity(name, T):
    ops = _ops()
    cfg = G.config(name)
    pl, li = layer(name) if name != "gemma4_26b_a4b_prefill" else layer("gemma4_26b_a4b_decode")
    xb, x = _stacks().hidden(cfg, 0, T)
    ws = ops.workspace(pl.dims, T)
    logits = torch.empty(T, cfg.experts, dtype=torch.float32, device=DEV)
    idx, w = ops.router_topk(pl.dims, pl.router, x, ws, logits=logits)
    torch.cuda.synchronize()
    top, wr, l64 = O.router(xb, li, cfg.top_k)
    assert_close_f32(logits.cpu().numpy(), l64, "logits", rel=1e-4)
    ties, differ = compare_topk(idx.cpu().numpy(), w.cpu().numpy(), l64, top, wr)
    print(f"{name} T={T}: near-tie tokens {ties}, differing sets {len(differ)}")


def test_router_duplicate_rows_tie_to_lower_index():
    ops = _ops()
    st = _stacks()
    cfg = G.config("tiny")
    li = G.make_router(cfg, 0)
    xb, x = st.hidden(cfg, 0)
    top0, _, _ = O.router(xb, li, 2)
    e = int(top0[0, 0])
    d = 15 if e != 15 else 0
    for a in ("router_q", "router_s", "router_b"):
        getattr(li, a)[d] = getattr(li, a)[e]
    r = st.router_weights(li, DEV)
    from quantized_moe_router_amd._lib import make_dims
    dims = make_dims(cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter)
    ws = ops.workspace(dims, 4)
    idx, _ = ops.router_topk(dims, r, x[:1].contiguous(), ws)
    assert idx.cpu().numpy()[0].tolist() == sorted([e, d])


def test_router_zero_input():
    ops = _ops()
    cfg = G.config("tiny")
    pl, li = layer("tiny")
    x = torch.zeros(3, cfg.hidden, dtype=torch.int16, device=DEV)
    ws = ops.workspace(pl.dims, 3)
    idx, w = ops.router_topk(pl.dims, pl.router, x, ws)
    assert idx.cpu().numpy().tolist() == [[0, 1]] * 3
    assert np.allclose(w.cpu().numpy(), np.tile(li.pes[:2] / 2, (3, 1)), rtol=1e-6)


@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("name", ["tiny", "gemma4_26b_a4b_decode", "qwen3_next_80b_a3b_decode_b1"])
def test_exact_ties_take_the_lower_ids(name, T):
    """The selection on logits with exact ties, in the one-token layer (T = 1: by rank for up to
    128 experts, round by round above) and in the router kernel of calls of several tokens
    (T = 3): zero input makes every logit its bias (or 0), and a bias drawn from three values
    puts equal logits on both sides of the k-th place.  The ids must be the oracle's (larger
    logit first, the lower index first among equal ones) and the weights its softmax times
    per_expert_scale."""
    ops = _ops()
    cfg = G.config(name)
    pl, li = layer(name)
    E, k, H = cfg.experts, cfg.top_k, cfg.hidden
    codes, scales, biases, pes, rscale, _ = pl.router.tensors
    bias = (np.random.default_rng(7).integers(0, 3, size=E) * 0.25).astype(np.float32)
    ws = ops.workspace(pl.dims, T)
    x = torch.zeros(T, H, dtype=torch.int16, device=DEV)
    for lb in (None, bias):
        router = ops.RouterWeights(codes, scales, biases, pes, rscale,
                                   None if lb is None else torch.from_numpy(lb).to(DEV))
        lw = ops.LayerWeights(pl.dims, router, pl.store, pl.stride, pl.shared)
        idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        w = torch.empty(T, k, dtype=torch.float32, device=DEV)
        ops.layer_forward(lw, x, ws, topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        logits = np.zeros((T, E)) if lb is None else np.tile(lb.astype(np.float64), (T, 1))
        top = O.topk_select(logits, k)
        if lb is not None:      # the case really has ties across the k-th place
            kth = logits[0, top[0, -1]]
            assert (logits[0] == kth).sum() > (logits[0, top[0]] == kth).sum()
        assert idx.cpu().numpy().tolist() == top.tolist(), f"{name} T={T} bias={lb is not None}"
        want = O.topk_weights(logits, top, li.pes)
        assert np.allclose(w.cpu().numpy(), want, rtol=1e-5, atol=0), f"{name} T={T} weights"
    assert ops.workspace_status(ws) == 0


def test_nonfinite_input_routes_to_valid_experts():
    """Regression: NaN logits once left an out-of-range expert id in the top-k."""
    ops = _ops()
    cfg = G.config("gemma4_26b_a4b_decode")
    pl, _ = layer("gemma4_26b_a4b_decode")
    x = torch.zeros(3, cfg.hidden, dtype=torch.int16, device=DEV)
    x[0] = 0x7FC0                               # NaN everywhere
    x[1, :7] = 0x7F80                           # a few +inf
    xb, xr = _stacks().hidden(cfg, 5, 1)
    x[2] = xr[0]
    ws = ops.workspace(pl.dims, 3)
    idx, w = ops.router_topk(pl.dims, pl.router, x, ws)
    out = ops.layer_forward(pl.weights, x, ws)
    torch.cuda.synchronize()
    i = idx.cpu().numpy()
    assert np.all((i >= 0) & (i < cfg.experts))
    assert i[0].tolist() == list(range(cfg.top_k))        # all NaN: ties -> lowest ids
    assert all(len(set(r)) == cfg.top_k for r in i.tolist())
    assert out.shape == (3, cfg.hidden)


def test_bucket_drops_out_of_range_ids():
    ops = _ops()
    from quantized_moe_router_amd._lib import make_dims
    idx = np.array([[3, 7], [-1, 3], [16, 2], [7, 2]], np.int32)
    dims = make_dims(64, 16, 2, 64, 0)
    counts, offsets, srt, active, n_active = ops.bucket(dims, torch.from_numpy(idx).to(DEV))
    c = counts.cpu().numpy()
    assert c[[2, 3, 7]].tolist() == [2, 2, 2] and c.sum() == 6
    assert offsets.cpu().numpy()[-1] == 6
    assert srt.cpu().numpy()[:6].tolist() == [5, 7, 0, 3, 1, 6]
    assert int(n_active.cpu()[0]) == 3


# ------------------------------------------------------------------ bucket

# the first eight cases take the segmented bucketing (at most 4096 assignments and 16384
# segment x expert cells), the last two the general one; `repeat` lets a token name the same
# expert several times (the standalone entry point accepts any ids)
@pytest.mark.parametrize("T,k,E,repeat", [(1, 8, 128, False), (4, 2, 16, False),
                                          (16, 10, 512, False), (128, 8, 128, False),
                                          (128, 8, 256, False), (37, 3, 7, False),
                                          (1000, 4, 64, False), (0, 2, 16, False),
                                          (100, 8, 16, True), (2048, 4, 64, False),
                                          (64, 32, 1024, False), (1500, 4, 8, True)])
def test_bucket_parity(T, k, E, repeat):
    ops = _ops()
    from quantized_moe_router_amd._lib import make_dims
    rng = np.random.default_rng(T * 131 + k * 7 + E)
    # Zipf-skewed picks so that some buckets are large and many empty
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    idx = np.stack([rng.choice(E, size=k, replace=repeat, p=p) for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, k), np.int32)
    dims = make_dims(64, E, k, 64, 0)
    counts, offsets, srt, active, n_active = ops.bucket(dims, torch.from_numpy(idx).to(DEV))
    c, o, s, a = O.bucket(idx, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(srt.cpu().numpy(), s)
    na = int(n_active.cpu().numpy()[0])
    assert na == len(a) and np.array_equal(active.cpu().numpy()[:na], a)


# ------------------------------------------------------------------ expert FFN + combine

def _bucket_of(ops, dims, idx):
    return ops.bucket(dims, idx)


def _ffn_ref(li, xf, idx_n, k):
    """Oracle y [T*k, H] for the GPU's routing (teacher forcing): each expert dequantised
    once, over every row routed to it."""
    T, H = xf.shape
    y = np.zeros((T * k, H))
    flat = idx_n.reshape(-1)
    li.prefetch(np.unique(flat))
    for e in np.unique(flat):
        ids = np.nonzero(flat == e)[0]
        y[ids] = O.expert_ffn(xf[ids // k], li.expert(int(e)))
    return y


# Every chunk of two or more tokens takes the matrix-core kernels (T = 200: two chunks,
# the second of 72 tokens); one token takes the VALU kernels of the standalone FFN call.
@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 37), ("tiny", 200), ("tiny_int8", 1),
                                    ("tiny_int8", 37), ("gemma4_26b_a4b_int8_decode", 1),
                                    ("gemma4_26b_a4b_decode", 1), ("gemma4_26b_a4b_prefill", 128),
                                    ("qwen3_next_80b_a3b_decode_b16", 16),
                                    ("qwen3_6_35b_a3b_long_prefill", 128)])
def test_expert_ffn_and_combine_parity(name, T):
    ops = _ops()
    cfg = G.config(name)
    pl, li = layer({"gemma4_26b_a4b_prefill": "gemma4_26b_a4b_decode",
                    "qwen3_next_80b_a3b_decode_b16": "qwen3_next_80b_a3b_decode_b1"}.get(name, name))
    xb, x = _stacks().hidden(cfg, 1, T)
    ws = ops.workspace(pl.dims, T)
    idx, w = ops.router_topk(pl.dims, pl.router, x, ws)
    counts, offsets, srt, active, n_active = ops.bucket(pl.dims, idx)
    y, y_sh = ops.expert_ffn(pl.weights, x, offsets, srt, active, n_active, ws)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    out = ops.combine(pl.dims, x, y, w, y_sh, out_f32=out_f32)
    torch.cuda.synchronize()
    k = cfg.top_k
    idx_n, w_n = idx.cpu().numpy(), w.cpu().numpy()
    y_n, ysh_n = y.cpu().numpy(), y_sh.cpu().numpy()
    out_n, of_n = np16(out), out_f32.cpu().numpy()
    xf = O.bf16_to_f64(xb)
    ys = _ffn_ref(li, xf, idx_n, k)            # per assignment, with the GPU's routing
    sh = O.expert_ffn(xf, li.shared())
    assert_close_f32(y_n, ys, "y")
    assert_close_f32(ysh_n, sh, "y_shared")
    ref = xf + sh + np.einsum("tk,tkh->th", w_n.astype(np.float64), ys.reshape(T, k, cfg.hidden))
    assert_close_f32(of_n, ref, "out_f32")
    flips = check_out_bf16(out_n, of_n, ref, "out")
    print(f"{name} T={T}: every token; bf16 1-ulp flips {flips}")


# ------------------------------------------------------------------ whole layer

def _layer_check(cfg, li, xb, out, out_f32, idx, w, toks):
    T = xb.shape[0]
    idx_n = idx.cpu().numpy()
    top0, _, _ = O.router(xb[list(toks)], li, cfg.top_k)
    li.prefetch(np.union1d(np.unique(top0), np.unique(idx_n[list(toks)])))
    ref = O.layer_forward(xb[list(toks)], li, cfg.top_k)
    ties, differ = compare_topk(idx_n[list(toks)], w.cpu().numpy()[list(toks)], ref["logits"],
                                ref["top"], ref["w"])
    out_n, of_n = np16(out), out_f32.cpu().numpy()
    flips = 0
    for n, t in enumerate(toks):
        r = ref
        if n in differ:      # near tie: re-evaluate the oracle with the GPU's valid selection
            r = O.layer_forward(xb[t:t + 1], li, cfg.top_k, top_override=idx_n[t:t + 1])
            rn = 0
        else:
            rn = n
        assert_close_f32(of_n[t], r["out"][rn], f"layer out_f32 token {t}")
        flips += check_out_bf16(out_n[t], of_n[t], r["out"][rn], f"layer out token {t}")
    return ties, len(differ), flips


@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 1), ("tiny", 64), ("tiny", 130),
                                    ("gemma4_26b_a4b_decode", 1), ("gemma4_26b_a4b_prefill", 128),
                                    ("qwen3_next_80b_a3b_decode_b1", 1),
                                    ("qwen3_next_80b_a3b_decode_b16", 16),
                                    ("qwen3_6_35b_a3b_long_prefill", 128),
                                    ("tiny_int8", 1), ("tiny_int8", 4), ("tiny_int8", 64),
                                    ("gemma4_26b_a4b_int8_decode", 1),
                                    ("gemma4_26b_a4b_int8_decode", 128)])
def test_layer_forward_parity(name, T):
    ops = _ops()
    cfg = G.config(name)
    src = {"gemma4_26b_a4b_prefill": "gemma4_26b_a4b_decode",
           "qwen3_next_80b_a3b_decode_b16": "qwen3_next_80b_a3b_decode_b1"}.get(name, name)
    pl, li = layer(src)
    xb, x = _stacks().hidden(cfg, 2, T)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
    out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, range(T))
    print(f"{name} T={T}: every token; near ties {ties}, re-evaluated {nd}, bf16 flips {flips}")


@pytest.mark.parametrize("inter,bits", [(3136, 4), (1600, 8)])
def test_one_token_layer_too_wide_for_the_single_launch(inter, bits):
    """One token through a layer whose routed expert is wider than the one-token launch holds
    (more than 48 k-steps per gate/up row: inter > 3072 for 4-bit codes, > 1536 for 8-bit) takes
    the VALU kernels of the chunked path; checked against the oracle."""
    ops = _ops()
    cfg = G.Config(f"wide_{bits}", 256, 8, 2, inter, 128, layers=1, tokens=1, expert_bits=bits)
    pl, li = _stacks().build_layer(cfg, 0, DEV)
    for step in range(3):
        xb, x = _stacks().hidden(cfg, 60 + step, 1)
        ws = ops.workspace(pl.dims, 1)
        out_f32 = torch.empty(1, cfg.hidden, dtype=torch.float32, device=DEV)
        idx = torch.empty(1, cfg.top_k, dtype=torch.int32, device=DEV)
        w = torch.empty(1, cfg.top_k, dtype=torch.float32, device=DEV)
        out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, range(1))
        print(f"inter {inter} bits {bits} step {step}: near ties {ties}, bf16 flips {flips}")


@pytest.mark.parametrize("E,k", [(200, 8), (520, 10), (1024, 32)])
def test_one_token_top_k_over_many_experts(E, k):
    """One token through layers of more than 128 experts, where every wave of a gate/up
    workgroup selects the top-k of a quarter of the experts and the four lists are merged by
    rank (quarters with fewer than k experts and empty quarters included): against the oracle
    on random inputs, and a zero input (every logit equal) selecting experts 0..k-1 with
    weights per_expert_scale / k."""
    ops = _ops()
    cfg = G.Config(f"many_{E}", 256, E, k, 128, 128, layers=1, tokens=1)
    pl, li = _stacks().build_layer(cfg, 0, DEV)
    ws = ops.workspace(pl.dims, 1)
    for step in range(3):
        xb, x = _stacks().hidden(cfg, 70 + step, 1)
        out_f32 = torch.empty(1, cfg.hidden, dtype=torch.float32, device=DEV)
        idx = torch.empty(1, k, dtype=torch.int32, device=DEV)
        w = torch.empty(1, k, dtype=torch.float32, device=DEV)
        out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, range(1))
        print(f"E {E} k {k} step {step}: near ties {ties}")
    x0 = torch.zeros(1, cfg.hidden, dtype=torch.bfloat16, device=DEV)
    idx = torch.empty(1, k, dtype=torch.int32, device=DEV)
    w = torch.empty(1, k, dtype=torch.float32, device=DEV)
    ops.layer_forward(pl.weights, x0, ws, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    assert idx.cpu().numpy()[0].tolist() == list(range(k))
    np.testing.assert_allclose(w.cpu().numpy()[0], li.pes[:k] / k, rtol=1e-6)


@pytest.mark.parametrize("T", [37, 130])
def test_chunked_layer_with_the_most_experts_and_the_largest_top_k(T):
    """Calls of several tokens at the largest expert count and top-k the library accepts
    (1024 experts, top-32): the multi-token router's widest register selection, the bucketing
    of up to 4096 assignments in its general form (more segment x expert cells than the
    segmented form holds), a slot table of 1280 blocks, and for T = 130 a full chunk followed by
    a two-token one.  Every token against the oracle."""
    ops = _ops()
    cfg = G.Config("many_1024_multi", 256, 1024, 32, 128, 128, layers=1, tokens=T)
    pl, li = _stacks().build_layer(cfg, 0, DEV)
    xb, x = _stacks().hidden(cfg, 5, T)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
    out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, range(T))
    print(f"E 1024 k 32 T={T}: every token; near ties {ties}, re-evaluated {nd}, bf16 flips {flips}")


@pytest.mark.parametrize("T", [1, 20])
def test_layer_at_the_largest_hidden_size(T):
    """Hidden size 8192, the largest the library accepts: the one-token layer (x staged in LDS,
    router codes in three batches) and a chunk of 20 tokens (32 router splits, 128 k-steps
    per gate/up tile), every token against the oracle."""
    ops = _ops()
    cfg = G.Config("hidden_8192", 8192, 16, 4, 256, 256, layers=1, tokens=T)
    pl, li = _stacks().build_layer(cfg, 0, DEV)
    xb, x = _stacks().hidden(cfg, 9, T)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
    for _ in range(2):
        out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, range(T))
    assert ops.workspace_status(ws) == 0
    print(f"H 8192 T={T}: every token; near ties {ties}, re-evaluated {nd}, bf16 flips {flips}")


@pytest.mark.parametrize("T,bits", [(1, 4), (20, 4), (20, 8)])
def test_layer_at_the_largest_expert_width(T, bits):
    """Expert and shared inner width 4096, the largest the library accepts (4- and 8-bit
    experts): 128 gate/up tiles per expert and 64 (4-bit) or 128 (8-bit) down k-steps per output
    tile; every token against the oracle."""
    ops = _ops()
    cfg = G.Config(f"inter_4096_{bits}", 256, 8, 2, 4096, 4096, layers=1, tokens=T, expert_bits=bits)
    pl, li = _stacks().build_layer(cfg, 0, DEV)
    xb, x = _stacks().hidden(cfg, 11, T)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
    out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, range(T))
    assert ops.workspace_status(ws) == 0
    print(f"inter 4096 bits {bits} T={T}: every token; near ties {ties}, bf16 flips {flips}")


@pytest.mark.parametrize("E,k,T", [(1, 1, 1), (1, 1, 5), (8, 8, 1), (8, 8, 5), (3, 2, 33)])
def test_layer_degenerate_routing(E, k, T):
    """Degenerate routing: a single expert (always selected, weight per_expert_scale[0]), every
    expert selected (top-k = E: the softmax runs over all logits), and an odd expert count;
    every token against the oracle."""
    ops = _ops()
    cfg = G.Config(f"degenerate_{E}_{k}", 256, E, k, 128, 128, layers=1, tokens=T)
    pl, li = _stacks().build_layer(cfg, 0, DEV)
    xb, x = _stacks().hidden(cfg, 13, T)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, range(T))
    assert sorted(set(idx.cpu().numpy().reshape(-1).tolist())) <= list(range(E))
    if k == E:
        assert all(sorted(r) == list(range(E)) for r in idx.cpu().numpy().tolist())
        # the softmax runs over all E logits: the weights over per_expert_scale sum to one
        ratio = w.cpu().numpy() / li.pes[idx.cpu().numpy()]
        np.testing.assert_allclose(ratio.sum(axis=1), 1.0, rtol=1e-6)
    if E == 1:
        np.testing.assert_array_equal(w.cpu().numpy(), np.full((T, 1), li.pes[0], np.float32))
    print(f"E {E} k {k} T={T}: near ties {ties}, bf16 flips {flips}")


@pytest.mark.parametrize("H,E,k,T", [(256, 16, 2, 1), (256, 16, 2, 4), (256, 16, 2, 130),
                                     (2048, 64, 4, 1), (2048, 64, 4, 40)])
def test_layer_without_a_shared_expert(H, E, k, T):
    """A layer with no shared expert (its branch absent, not zero) through the resident path:
    the one-token layer without its shared roles and the chunked kernels without shared
    workgroups; every token against the oracle."""
    ops = _ops()
    cfg = G.Config(f"no_shared_{H}_{E}", H, E, k, 256 if H > 256 else 128, 0, layers=1, tokens=T)
    pl, li = _stacks().build_layer(cfg, 0, DEV)
    assert pl.shared is None
    xb, x = _stacks().hidden(cfg, 17, T)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, range(T))
    assert ops.workspace_status(ws) == 0
    print(f"no shared H {H} E {E} T={T}: near ties {ties}, bf16 flips {flips}")


@pytest.mark.parametrize("name,T", [("gemma4_26b_a4b_decode", 1), ("gemma4_26b_a4b_decode", 20),
                                    ("tiny", 1), ("tiny", 6)])
def test_layer_with_a_per_channel_router_scale(name, T):
    """router_scale as a per-channel vector (every workload uses ones; here U(0.5, 2) per
    hidden channel, so that a misplaced or transposed scale would change the logits): the
    one-token layer's router and the matrix-core router of a chunk, every token against the
    oracle, which reads the same vector."""
    ops = _ops()
    cfg = G.config(name)
    pl, li = layer(name)
    li2 = copy.copy(li)
    li2.router_scale = np.random.default_rng(23).uniform(0.5, 2.0, cfg.hidden).astype(np.float32)
    lw = ops.LayerWeights(pl.dims, _stacks().router_weights(li2, DEV), pl.store, pl.stride,
                          pl.shared)
    xb, x = _stacks().hidden(cfg, 19, T)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
    out = ops.layer_forward(lw, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    ties, nd, flips = _layer_check(cfg, li2, xb, out, out_f32, idx, w, range(T))
    # the scale matters: the oracle's logits with unit scales are far from these
    l1, l2 = O.router(xb, li, cfg.top_k)[2], O.router(xb, li2, cfg.top_k)[2]
    assert np.abs(l1 - l2).max() > 1e-2 * np.abs(l2).max()
    print(f"{name} T={T} per-channel router_scale: near ties {ties}, bf16 flips {flips}")


@pytest.mark.parametrize("name,T", [("gemma4_26b_a4b_decode", 1), ("gemma4_26b_a4b_decode", 24),
                                    ("qwen3_next_80b_a3b_decode_b1", 1)])
def test_layer_with_outlier_and_tiny_activations(name, T):
    """Hidden states with a wide dynamic range, as activations with outlier channels have:
    N(0, 1) values, eight channels scaled by 300, and one in sixteen values scaled by 1e-6.
    The matrix-core operands stay exact (bf16 x, hi/lo planes of h), so the bar is the same;
    every token against the oracle."""
    ops = _ops()
    cfg = G.config(name)
    pl, li = layer(name)
    rng = np.random.default_rng(29)
    xf = rng.standard_normal((T, cfg.hidden)).astype(np.float32)
    xf[:, rng.choice(cfg.hidden, 8, replace=False)] *= 300.0
    xf[rng.random((T, cfg.hidden)) < 1.0 / 16] *= 1e-6
    xb = G.bf16_bits_from_f32(xf)
    x = torch.from_numpy(xb.view(np.int16)).to(DEV)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
    out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, range(T))
    print(f"{name} T={T} outlier activations: near ties {ties}, bf16 flips {flips}")


@pytest.mark.parametrize("T", [1, 20])
def test_calls_on_side_streams_from_two_threads(T):
    """The entry points are asynchronous on the caller's stream and reentrant: two host threads,
    each with its own stream (default priority) and workspace, run the same layer calls
    concurrently; every output is bit-equal to the same call on the default stream."""
    import threading
    ops = _ops()
    name = "gemma4_26b_a4b_decode"
    cfg = G.config(name)
    pl, li = layer(name)
    xs = [_stacks().hidden(cfg, 40 + i, T)[1] for i in range(4)]
    ws0 = ops.workspace(pl.dims, T)
    want = [ops.layer_forward(pl.weights, x, ws0).clone() for x in xs]
    torch.cuda.synchronize()
    got = [[None] * len(xs) for _ in range(2)]
    errors = []

    def worker(j):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                ws = ops.workspace(pl.dims, T)
                for rep in range(3):
                    for i, x in enumerate(xs):
                        got[j][i] = ops.layer_forward(pl.weights, x, ws)
            s.synchronize()
        except Exception as e:     # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j in range(2):
        for i in range(len(xs)):
            assert torch.equal(got[j][i].view(torch.int16), want[i].view(torch.int16)), (j, i)


def test_bucket_at_the_largest_call():
    """The standalone bucketing at the largest call the library accepts: 65,536 tokens of
    top-32 over 1024 experts (2^21 assignments, the limit of the scan's packed fields), skewed
    so that some buckets are large; bit-exact against the oracle."""
    ops = _ops()
    from quantized_moe_router_amd._lib import make_dims
    T, k, E = 65536, 32, 1024
    rng = np.random.default_rng(41)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    # distinct experts per token: a random permutation's first k, drawn in a skewed order
    idx = np.empty((T, k), np.int32)
    for t0 in range(0, T, 4096):
        keys = rng.random((4096, E)) ** (1.0 / p[None, :])
        idx[t0:t0 + 4096] = np.argpartition(-keys, k, axis=1)[:, :k]
    dims = make_dims(64, E, k, 64, 0)
    counts, offsets, srt, active, n_active = ops.bucket(dims, torch.from_numpy(idx).to(DEV))
    c, o, srt_ref, a = O.bucket(idx, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(srt.cpu().numpy(), srt_ref)
    na = int(n_active.cpu().numpy()[0])
    assert na == len(a) and np.array_equal(active.cpu().numpy()[:na], a)


def test_layer_at_the_largest_token_count():
    """A layer call of 65,536 tokens (512 chunks), the largest the library accepts: 96 tokens
    spread over the call (first and last chunk included) against the oracle, and the whole
    output bit-equal to the same tokens run as separate calls of 4,096."""
    ops = _ops()
    T = 65536
    cfg = G.Config("tiny_long", 256, 16, 2, 128, 128, layers=1, tokens=T)
    pl, li = _stacks().build_layer(cfg, 0, DEV)
    xb, x = _stacks().hidden(cfg, 43, T)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
    out = ops.layer_forward(pl.weights, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    assert ops.workspace_status(ws) == 0
    toks = sorted(set(np.random.default_rng(47).choice(T, 90, replace=False).tolist())
                  | {0, 1, 127, 128, T - 2, T - 1})
    ties, nd, flips = _layer_check(cfg, li, xb, out, out_f32, idx, w, toks)
    ws2 = ops.workspace(pl.dims, 4096)
    for c0 in range(0, T, 4096):
        part = ops.layer_forward(pl.weights, x[c0:c0 + 4096], ws2)
        assert torch.equal(part.view(torch.int16), out[c0:c0 + 4096].view(torch.int16)), c0
    print(f"T={T}: {len(toks)} tokens against the oracle, near ties {ties}, bf16 flips {flips}")


def test_layer_forward_matches_stepwise_and_is_deterministic():
    ops = _ops()
    cfg = G.config("gemma4_26b_a4b_prefill")
    pl, li = layer("gemma4_26b_a4b_decode")
    xb, x = _stacks().hidden(cfg, 3, 128)
    ws = ops.workspace(pl.dims, 128)
    o32a = torch.empty(128, cfg.hidden, dtype=torch.float32, device=DEV)
    o32b = torch.empty_like(o32a)
    outa = ops.layer_forward(pl.weights, x, ws, out_f32=o32a)
    outb = ops.layer_forward(pl.weights, x, ws, out_f32=o32b)
    idx, w = ops.router_topk(pl.dims, pl.router, x, ws)
    counts, offsets, srt, active, n_active = ops.bucket(pl.dims, idx)
    y, y_sh = ops.expert_ffn(pl.weights, x, offsets, srt, active, n_active, ws)
    o32c = torch.empty_like(o32a)
    ops.combine(pl.dims, x, y, w, y_sh, out_f32=o32c)
    torch.cuda.synchronize()
    assert torch.equal(outa.view(torch.int16), outb.view(torch.int16))
    assert torch.equal(o32a, o32b)
    assert rel_err_rows(o32a.cpu().numpy(), o32c.cpu().numpy().astype(np.float64)) <= 1e-5


def test_layer_forward_chunks_equal_single_calls():
    ops = _ops()
    cfg = G.config("tiny")
    pl, li = layer("tiny")
    xb, x = _stacks().hidden(cfg, 4, 300)
    ws = ops.workspace(pl.dims, 300)
    o_all = torch.empty(300, cfg.hidden, dtype=torch.float32, device=DEV)
    ops.layer_forward(pl.weights, x, ws, out_f32=o_all)
    parts = []
    for a, b in [(0, 128), (128, 256), (256, 300)]:
        o = torch.empty(b - a, cfg.hidden, dtype=torch.float32, device=DEV)
        ops.layer_forward(pl.weights, x[a:b].contiguous(), ws, out_f32=o)
        parts.append(o)
    torch.cuda.synchronize()
    assert torch.equal(o_all, torch.cat(parts))


def test_zero_tokens_is_noop():
    ops = _ops()
    pl, _ = layer("tiny")
    x = torch.empty(0, 256, dtype=torch.int16, device=DEV)
    ws = ops.workspace(pl.dims, 1)
    out = ops.layer_forward(pl.weights, x, ws)
    assert out.shape == (0, 256)


# ------------------------------------------------------------------ one-token launches and graphs

@pytest.mark.parametrize("name", ["tiny", "gemma4_26b_a4b_decode", "qwen3_next_80b_a3b_decode_b1",
                                  "gemma4_26b_a4b_int8_decode"])
def test_one_token_calls_repeat_and_report_no_timeout(name):
    """Back-to-back one-token calls on one workspace (each advances its epoch) give the same
    bits as a fresh workspace, and the workspace status reports no timed-out wait."""
    ops = _ops()
    cfg = G.config(name)
    pl, li = layer(name)
    xb, x = _stacks().hidden(cfg, 7, 1)
    ws = ops.workspace(pl.dims, 1)
    outs = [ops.layer_forward(pl.weights, x, ws) for _ in range(5)]
    ws2 = ops.workspace(pl.dims, 1)
    o32 = torch.empty(1, cfg.hidden, dtype=torch.float32, device=DEV)
    fresh = ops.layer_forward(pl.weights, x, ws2, out_f32=o32)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), fresh.view(torch.int16))
    assert ops.workspace_status(ws) == 0 and ops.workspace_status(ws2) == 0
    ref = O.layer_forward(xb, li, cfg.top_k)
    assert_close_f32(o32.cpu().numpy()[0], ref["out"][0], "one-token out_f32")
    check_out_bf16(np16(fresh)[0], o32.cpu().numpy()[0], ref["out"][0], "one-token out")


def test_one_token_calls_after_a_chunk_share_the_workspace():
    """A workspace sized for a 128-token chunk serves chunk calls and one-token calls in turn:
    the one-token results equal a fresh workspace's bit for bit and the oracle's (the one-token
    hand-off words sit where no chunk call writes, so a chunk's data never poses as a fresh
    word)."""
    ops = _ops()
    cfg = G.config("gemma4_26b_a4b_decode")
    pl, li = layer("gemma4_26b_a4b_decode")
    ws = ops.workspace(pl.dims, 128)
    xb128, x128 = _stacks().hidden(cfg, 40, 128)
    xs = [_stacks().hidden(cfg, 41 + j, 1) for j in range(3)]
    fresh = [ops.layer_forward(pl.weights, x, ops.workspace(pl.dims, 1)) for _, x in xs]
    o32 = torch.empty(1, cfg.hidden, dtype=torch.float32, device=DEV)
    for rep in range(3):
        ops.layer_forward(pl.weights, x128, ws)
        for j, (_, x) in enumerate(xs):
            out = ops.layer_forward(pl.weights, x, ws, out_f32=o32)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), fresh[j].view(torch.int16)), (rep, j)
    assert ops.workspace_status(ws) == 0
    ref = O.layer_forward(xs[-1][0], li, cfg.top_k)
    assert_close_f32(o32.cpu().numpy()[0], ref["out"][0], "one-token out_f32 after chunks")


# ------------------------------------------------------------------ post-combine steps (cb2)

class _WithPost:
    """Oracle view of a layer that carries the post-combine norm gain and layer scalar."""

    def __init__(self, li, gain, scalar):
        self._li, self.post_gain, self.layer_scalar = li, gain, scalar

    def __getattr__(self, name):
        return getattr(self._li, name)


def post_layer(name, steps="both"):
    """(LayerWeights with the post steps, oracle layer view) sharing layer(name)'s store."""
    ops = _ops()
    cfg = G.config(name)
    pl, li = layer(name)
    gain, scalar = G.make_post(cfg, 0)
    g = torch.from_numpy(gain).to(DEV) if steps in ("both", "gain") else None
    sc = torch.tensor([scalar], dtype=torch.float32, device=DEV) if steps in ("both", "scalar") else None
    lw = ops.LayerWeights(pl.dims, pl.router, pl.store, pl.stride, pl.shared,
                          post_norm_gain=g, layer_scalar=sc)
    view = _WithPost(li, gain if g is not None else None, scalar if sc is not None else None)
    return pl, lw, view


@pytest.mark.parametrize("name,T,steps", [
    ("tiny", 4, "both"), ("tiny", 1, "both"), ("tiny", 1, "scalar"), ("tiny", 64, "gain"),
    ("tiny", 37, "scalar"), ("gemma4_26b_a4b_decode", 1, "both"),
    ("gemma4_26b_a4b_decode", 128, "both"), ("qwen3_next_80b_a3b_decode_b1", 1, "both"),
    ("qwen3_6_35b_a3b_long_prefill", 128, "gain")])
def test_layer_forward_post_parity(name, T, steps):
    """The layer with cb2's post-combine steps (one-token kernel and chunked path)."""
    ops = _ops()
    cfg = G.config(name)
    pl, lw, view = post_layer(name, steps)
    xb, x = _stacks().hidden(cfg, 5, T)
    ws = ops.workspace(pl.dims, T)
    out_f32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
    out = ops.layer_forward(lw, x, ws, out_f32=out_f32, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    assert ops.workspace_status(ws) == 0
    ties, nd, flips = _layer_check(cfg, view, xb, out, out_f32, idx, w, range(T))
    print(f"{name} T={T} post={steps}: near ties {ties}, re-evaluated {nd}, bf16 flips {flips}")


def test_combine_post_against_oracle_and_plain_combine():
    ops = _ops()
    cfg = G.config("gemma4_26b_a4b_prefill")
    T, H, k = 9, cfg.hidden, cfg.top_k
    rng = np.random.default_rng(11)
    xb = O.bf16_rne_bits(rng.standard_normal((T, H)))
    x = _stacks().t16(xb, DEV)
    y = torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).to(DEV)
    ysh = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(DEV)
    w = torch.from_numpy(rng.uniform(0.05, 0.3, (T, k)).astype(np.float32)).to(DEV)
    gain, scalar = G.make_post(cfg, 3)
    g = torch.from_numpy(gain).to(DEV)
    sc = torch.tensor([scalar], dtype=torch.float32, device=DEV)
    dims = layer("gemma4_26b_a4b_decode")[0].dims
    o32 = torch.empty(T, H, dtype=torch.float32, device=DEV)
    out = ops.combine_post(dims, x, y, w, ysh, g, sc, out_f32=o32)
    p32 = torch.empty_like(o32)
    plain = ops.combine_post(dims, x, y, w, ysh, out_f32=p32)
    c32 = torch.empty_like(o32)
    ref_plain = ops.combine(dims, x, y, w, ysh, out_f32=c32)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), ref_plain.view(torch.int16))
    assert torch.equal(p32, c32)
    want, _ = O.combine_post(xb, y.cpu().numpy().astype(np.float64).reshape(T, k, H),
                             w.cpu().numpy(), ysh.cpu().numpy().astype(np.float64), gain, scalar)
    o_n = o32.cpu().numpy()
    for t in range(T):
        assert_close_f32(o_n[t], want[t], f"combine_post out_f32 token {t}")
        check_out_bf16(np16(out)[t], o_n[t], want[t], f"combine_post out token {t}")


@pytest.mark.parametrize("name", ["tiny", "gemma4_26b_a4b_decode"])
def test_one_token_post_calls_repeat(name):
    """Back-to-back one-token calls with the post-combine norm give the same bits as a fresh
    workspace and report no timed-out wait."""
    ops = _ops()
    cfg = G.config(name)
    pl, lw, view = post_layer(name)
    xb, x = _stacks().hidden(cfg, 8, 1)
    ws = ops.workspace(pl.dims, 1)
    outs = [ops.layer_forward(lw, x, ws) for _ in range(4)]
    plain = ops.layer_forward(pl.weights, x, ws)
    outs.append(ops.layer_forward(lw, x, ws))
    ws2 = ops.workspace(pl.dims, 1)
    fresh = ops.layer_forward(lw, x, ws2)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), fresh.view(torch.int16))
    assert not torch.equal(plain.view(torch.int16), fresh.view(torch.int16))
    assert ops.workspace_status(ws) == 0 and ops.workspace_status(ws2) == 0


# ------------------------------------------------------------------ tiered residency

def _tiered(name, slots):
    ops = _ops()
    pl, li = layer(name)
    host = torch.empty(pl.store.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(pl.store)
    slot_store = torch.empty(slots * pl.stride, dtype=torch.uint8, device=DEV)
    cache = ops.ExpertCache(pl.dims, host, pl.stride, slot_store, pl.stride, slots)
    return pl, li, cache


@pytest.mark.parametrize("name,T,slots,steps", [("tiny", 4, 8, 6), ("tiny", 1, 2, 8),
                                                ("tiny", 130, 16, 2), ("tiny_int8", 4, 8, 3),
                                                ("gemma4_26b_a4b_decode", 1, 16, 6),
                                                ("gemma4_26b_a4b_decode", 128, 128, 2)])
def test_tiered_layer_equals_resident_stepwise(name, T, slots, steps):
    """Experts streamed from host memory through the device cache give the bits of the
    resident step-by-step path, and the cache counts follow the replacement rule."""
    from cache_model import Model
    ops = _ops()
    cfg = G.config(name)
    pl, li, cache = _tiered(name, slots)
    ws = ops.workspace(pl.dims, T)
    ws2 = ops.workspace(pl.dims, T)
    model = Model(cfg.experts, slots)
    for step in range(steps):
        xb, x = _stacks().hidden(cfg, 20 + step, T)
        o32t = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
        idx_t = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
        w_t = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
        out_t = ops.layer_forward_tiered(pl.weights, cache, x, ws, out_f32=o32t, topk_idx=idx_t,
                                         topk_w=w_t)
        idx, w = ops.router_topk(pl.dims, pl.router, x, ws2)
        counts, offsets, srt, active, n_active = ops.bucket(pl.dims, idx)
        y, ysh = ops.expert_ffn(pl.weights, x, offsets, srt, active, n_active, ws2)
        o32r = torch.empty_like(o32t)
        out_r = ops.combine(pl.dims, x, y, w, ysh, out_f32=o32r)
        torch.cuda.synchronize()
        assert torch.equal(idx_t, idx) and torch.equal(w_t, w)
        assert torch.equal(out_t.view(torch.int16), out_r.view(torch.int16))
        assert torch.equal(o32t, o32r)
        ids = idx.cpu().numpy()
        for c0 in range(0, T, 128):
            model.plan(ids[c0:c0 + 128].ravel())
    assert cache.stats() == (model.hits, model.misses)
    print(f"{name} T={T} slots={slots}: hits {model.hits}, misses {model.misses}")


@pytest.mark.parametrize("T,steps", [(1, 6), (4, 4)])
def test_tiered_layer_without_shared_expert(T, steps):
    """A layer with no shared expert through the tiered mode, including calls whose every
    expert misses the cache (nothing runs while the copies are in flight): the bits of the
    resident step-by-step path."""
    ops = _ops()
    cfg = G.Config("tiny_no_shared", 256, 16, 2, 128, 0, layers=1, tokens=T)
    pl, li = _stacks().build_layer(cfg, 0, DEV)
    host = torch.empty(pl.store.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(pl.store)
    slot_store = torch.empty(8 * pl.stride, dtype=torch.uint8, device=DEV)
    cache = ops.ExpertCache(pl.dims, host, pl.stride, slot_store, pl.stride, 8)
    ws, ws2 = ops.workspace(pl.dims, T), ops.workspace(pl.dims, T)
    for step in range(steps):
        xb, x = _stacks().hidden(cfg, 40 + step, T)
        o32t = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
        out_t = ops.layer_forward_tiered(pl.weights, cache, x, ws, out_f32=o32t)
        idx, w = ops.router_topk(pl.dims, pl.router, x, ws2)
        counts, offsets, srt, active, n_active = ops.bucket(pl.dims, idx)
        y, ysh = ops.expert_ffn(pl.weights, x, offsets, srt, active, n_active, ws2)
        o32r = torch.empty_like(o32t)
        out_r = ops.combine(pl.dims, x, y, w, ysh, out_f32=o32r)
        torch.cuda.synchronize()
        assert torch.equal(out_t.view(torch.int16), out_r.view(torch.int16))
        assert torch.equal(o32t, o32r)
    hits, misses = cache.stats()
    assert misses > 0


def test_tiered_layer_with_post_steps_and_too_few_slots():
    ops = _ops()
    cfg = G.config("tiny")
    pl, lw, view = post_layer("tiny")
    _, _, cache = _tiered("tiny", 4)
    xb, x = _stacks().hidden(cfg, 31, 1)
    ws = ops.workspace(pl.dims, 4)
    o32 = torch.empty(1, cfg.hidden, dtype=torch.float32, device=DEV)
    out = ops.layer_forward_tiered(lw, cache, x, ws, out_f32=o32)
    torch.cuda.synchronize()
    ref = O.layer_forward(xb, view, cfg.top_k)
    assert_close_f32(o32.cpu().numpy()[0], ref["out"][0], "tiered post out_f32")
    check_out_bf16(np16(out)[0], o32.cpu().numpy()[0], ref["out"][0], "tiered post out")
    # four tokens name up to eight experts: more than the four slots
    _, _, small = _tiered("tiny", 2)
    xb4, x4 = _stacks().hidden(cfg, 32, 4)
    from quantized_moe_router_amd import QmoeError
    with pytest.raises(QmoeError):
        ops.layer_forward_tiered(pl.weights, small, x4, ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 128])
def test_graph_replays_match_eager(T):
    """A captured layer call replayed several times, with eager work in between, reproduces the
    eager result on every replay."""
    ops = _ops()
    cfg = G.config("gemma4_26b_a4b_decode")
    pl, _ = layer("gemma4_26b_a4b_decode")
    ws = ops.workspace(pl.dims, T)
    xs = [_stacks().hidden(cfg, 20 + i, T)[1] for i in range(3)]
    x_static = xs[0].clone()
    out_static = torch.empty(T, cfg.hidden, dtype=torch.bfloat16, device=DEV)
    ref = [ops.layer_forward(pl.weights, xi, ws).clone() for xi in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.layer_forward(pl.weights, x_static, ws, out=out_static)
    for rep in range(6):
        i = rep % 3
        x_static.copy_(xs[i])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_static.view(torch.int16), ref[i].view(torch.int16)), rep
        # eager work on the same workspace between replays
        e = ops.layer_forward(pl.weights, xs[(i + 1) % 3], ws)
        torch.cuda.synchronize()
        assert torch.equal(e.view(torch.int16), ref[(i + 1) % 3].view(torch.int16))
    assert ops.workspace_status(ws) == 0
