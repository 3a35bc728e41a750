"""The chained one-token launch (qmoe_decode_stack) through the C ABI.  Needs an MI355X.

Its per-layer arithmetic is the one-token layer's, so every layer's output, fp32 output and
routing must equal the same layers run as chained qmoe_layer_forward calls bit for bit; against
the oracle the chain is followed layer by layer from the same input."""
import numpy as np
import pytest
import torch

import oracle as O
from parity import assert_close_f32, check_out_bf16, compare_topk
from workloads import gen as G

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_moe_router_amd import _lib
    _lib.lib()


def _ops():
    from quantized_moe_router_amd import ops
    return ops


def _stacks():
    import stacks
    return stacks


_cache = {}


def layer(name, idx):
    key = (name, idx)
    if key not in _cache:
        _cache[key] = _stacks().build_layer(G.config(name), idx, DEV)
    return _cache[key]


def np16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class _View:
    """Oracle view of a layer, optionally with the post-combine steps."""

    def __init__(self, li, gain=None, scalar=None):
        self._li, self.post_gain, self.layer_scalar = li, gain, scalar

    def __getattr__(self, name):
        return getattr(self._li, name)


def chain(name, n, post=(), shared=True):
    """n layers of config `name` (layer index i for layer i); layers listed in `post` carry the
    post-combine gain and layer scalar.  Returns (LayerWeights list, oracle views)."""
    ops = _ops()
    cfg = G.config(name)
    lws, views = [], []
    for i in range(n):
        pl, li = layer(name, i)
        g = sc = None
        gain = scalar = None
        if i in post:
            gain, scalar = G.make_post(cfg, i)
            g = torch.from_numpy(gain).to(DEV)
            sc = torch.tensor([scalar], dtype=torch.float32, device=DEV)
        lws.append(ops.LayerWeights(pl.dims, pl.router, pl.store, pl.stride,
                                    pl.shared if shared else None, post_norm_gain=g,
                                    layer_scalar=sc))
        views.append(_View(li, gain, scalar))
    return lws, views


def run_chained_calls(lws, x, ws):
    """The same chain as separate one-token qmoe_layer_forward calls."""
    ops = _ops()
    H, k = lws[0].dims.hidden, lws[0].dims.top_k
    n = len(lws)
    out = torch.empty(n, H, dtype=torch.bfloat16, device=DEV)
    o32 = torch.empty(n, H, dtype=torch.float32, device=DEV)
    idx = torch.empty(n, k, dtype=torch.int32, device=DEV)
    w = torch.empty(n, k, dtype=torch.float32, device=DEV)
    cur = x
    for i, lw in enumerate(lws):
        ops.layer_forward(lw, cur, ws, out=out[i:i + 1], out_f32=o32[i:i + 1],
                          topk_idx=idx[i:i + 1], topk_w=w[i:i + 1])
        cur = out[i:i + 1]
    return out, o32, idx, w


def run_stack(lws, x, ws):
    ops = _ops()
    H, k = lws[0].dims.hidden, lws[0].dims.top_k
    n = len(lws)
    o32 = torch.empty(n, H, dtype=torch.float32, device=DEV)
    idx = torch.empty(n, k, dtype=torch.int32, device=DEV)
    w = torch.empty(n, k, dtype=torch.float32, device=DEV)
    out = ops.decode_stack(lws, x, ws, out_f32=o32, topk_idx=idx, topk_w=w)
    return out, o32, idx, w


def assert_same(a, b, what):
    for i, (p, q) in enumerate(zip(a, b)):
        if p.dtype == torch.bfloat16:
            p, q = p.view(torch.int16), q.view(torch.int16)
        assert torch.equal(p, q), f"{what}: output {i} differs"


@pytest.mark.parametrize("name,n,post,shared", [
    ("tiny", 5, (), True), ("tiny", 1, (), True), ("tiny", 6, (1, 2, 5), True),
    ("tiny", 3, (), False), ("tiny_int8", 3, (0,), True),
    ("gemma4_26b_a4b_decode", 4, (), True), ("gemma4_26b_a4b_decode", 3, (0, 2), True),
    ("qwen3_next_80b_a3b_decode_b1", 3, (), True), ("gemma4_26b_a4b_int8_decode", 2, (), True),
    ("tiny", 64, tuple(range(64)), True)])
def test_stack_equals_chained_layer_calls(name, n, post, shared):
    ops = _ops()
    cfg = G.config(name)
    lws, _ = chain(name, n, post, shared)
    _, x = _stacks().hidden(cfg, 31, 1)
    ws = ops.workspace(lws[0].dims, 1)
    ref = run_chained_calls(lws, x, ws)
    ws2 = ops.workspace(lws[0].dims, 1)
    got = run_stack(lws, x, ws2)
    torch.cuda.synchronize()
    assert_same(got, ref, f"{name} x{n}")
    assert ops.workspace_status(ws) == 0 and ops.workspace_status(ws2) == 0


def test_stack_longer_than_the_table_is_rejected():
    """A chain of more layers than one launch's table holds (64) is rejected before any launch."""
    ops = _ops()
    from quantized_moe_router_amd import QmoeError
    cfg = G.config("tiny")
    lws, _ = chain("tiny", 65, tuple(range(65)))
    _, x = _stacks().hidden(cfg, 34, 1)
    ws = ops.workspace(lws[0].dims, 1)
    with pytest.raises(QmoeError):
        run_stack(lws, x, ws)
    torch.cuda.synchronize()
    assert ops.workspace_status(ws) == 0


def test_stack_repeats_and_shares_the_workspace_with_layer_calls():
    """Stack calls advance the epoch by their layer count: back-to-back stack calls and
    one-token layer calls on one workspace keep giving the results of fresh workspaces."""
    ops = _ops()
    cfg = G.config("gemma4_26b_a4b_decode")
    lws, _ = chain("gemma4_26b_a4b_decode", 3, (1,))
    _, x = _stacks().hidden(cfg, 32, 1)
    _, x2 = _stacks().hidden(cfg, 33, 1)
    ws = ops.workspace(lws[0].dims, 1)
    ref = run_stack(lws, x, ops.workspace(lws[0].dims, 1))
    ref2 = run_stack(lws[:2], x2, ops.workspace(lws[0].dims, 1))
    single = ops.layer_forward(lws[0], x, ops.workspace(lws[0].dims, 1))
    for rep in range(3):
        got = run_stack(lws, x, ws)
        s = ops.layer_forward(lws[0], x, ws)
        got2 = run_stack(lws[:2], x2, ws)
        torch.cuda.synchronize()
        assert_same(got, ref, f"stack rep {rep}")
        assert_same(got2, ref2, f"short stack rep {rep}")
        assert torch.equal(s.view(torch.int16), single.view(torch.int16))
    assert ops.workspace_status(ws) == 0


def test_stack_graph_replays_match_eager():
    ops = _ops()
    cfg = G.config("gemma4_26b_a4b_decode")
    lws, _ = chain("gemma4_26b_a4b_decode", 4, (3,))
    ws = ops.workspace(lws[0].dims, 1)
    xs = [_stacks().hidden(cfg, 40 + i, 1)[1] for i in range(3)]
    refs = [run_stack(lws, xi, ws)[0].clone() for xi in xs]
    torch.cuda.synchronize()
    x_static = xs[0].clone()
    out_static = torch.empty(4, cfg.hidden, dtype=torch.bfloat16, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.decode_stack(lws, x_static, ws, out=out_static)
    for rep in range(6):
        i = rep % 3
        x_static.copy_(xs[i])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_static.view(torch.int16), refs[i].view(torch.int16)), rep
        e = ops.decode_stack(lws, xs[(i + 1) % 3], ws)
        torch.cuda.synchronize()
        assert torch.equal(e.view(torch.int16), refs[(i + 1) % 3].view(torch.int16))
    assert ops.workspace_status(ws) == 0


@pytest.mark.parametrize("name,n,post", [("tiny", 5, (2,)), ("gemma4_26b_a4b_decode", 4, (1, 3)),
                                         ("qwen3_next_80b_a3b_decode_b1", 3, (0, 1, 2)),
                                         ("gemma4_26b_a4b_int8_decode", 2, (1,))])
def test_stack_against_oracle_chain(name, n, post):
    """Layer by layer against the oracle, teacher-forced: oracle layer l takes the stack's own
    input to layer l (the bf16 output of its layer l - 1), so every layer is held to the full
    layer bar -- the top-k bit-exact apart from near ties (oracle gap < 1e-5, counted), the
    fp32 output element by element within 2e-3 and the bf16 output by the bf16 rule."""
    ops = _ops()
    cfg = G.config(name)
    lws, views = chain(name, n, post)
    xb, x = _stacks().hidden(cfg, 34, 1)
    ws = ops.workspace(lws[0].dims, 1)
    out, o32, idx, w = run_stack(lws, x, ws)
    torch.cuda.synchronize()
    out_n, o32_n, idx_n, w_n = np16(out), o32.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    xs = np.asarray(xb, np.uint16)          # the stack's input to layer l
    n_ties = n_differ = flips = 0
    for l in range(n):
        ref = O.layer_forward(xs, views[l], cfg.top_k)
        ties, differ = compare_topk(idx_n[l:l + 1], w_n[l:l + 1], ref["logits"], ref["top"],
                                    ref["w"])
        n_ties += ties
        if differ:          # near tie: the oracle re-evaluated with the GPU's valid selection
            n_differ += 1
            ref = O.layer_forward(xs, views[l], cfg.top_k, top_override=idx_n[l:l + 1])
        assert_close_f32(o32_n[l], ref["out"][0], f"{name} layer {l} out_f32")
        flips += check_out_bf16(out_n[l], o32_n[l], ref["out"][0], f"{name} layer {l} out")
        xs = out_n[l:l + 1]
    print(f"{name} x{n} teacher-forced: near ties {n_ties}, re-evaluated {n_differ}, "
          f"bf16 flips {flips}")
    assert ops.workspace_status(ws) == 0
