"""The allocation-free layer entry point (qmoe_layer_forward_noalloc) through the C ABI.

It runs the kernels of qmoe_layer_forward on the library's fixed per-device scratch instead of a
caller's workspace, so its results must equal that entry point's bit for bit; checked on two
calls in a row, the second with fewer tokens (a chunk call, then a one-token call, which reuse
the same scratch), and against the oracle.  Needs an MI355X."""
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


def _call(fn, cfg, T):
    out = torch.empty(T, cfg.hidden, dtype=torch.bfloat16, device=DEV)
    o32 = torch.empty(T, cfg.hidden, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=DEV)
    fn(out, o32, idx, w)
    return out, o32, idx, w


@pytest.mark.parametrize("name,Ts", [("gemma4_26b_a4b_decode", (128, 1)), ("tiny", (64, 4)),
                                     ("qwen3_next_80b_a3b_decode_b1", (16, 1))])
def test_noalloc_equals_workspace_entry_point(name, Ts):
    import stacks
    from quantized_moe_router_amd import ops
    cfg = G.config(name)
    pl, li = stacks.build_layer(cfg, 0, DEV)
    ws = ops.workspace(pl.dims, max(Ts))
    for n, T in enumerate(Ts):
        xb, x = stacks.hidden(cfg, 70 + n, T)
        ref = _call(lambda o, f, i, w: ops.layer_forward(pl.weights, x, ws, out=o, out_f32=f,
                                                        topk_idx=i, topk_w=w), cfg, T)
        got = _call(lambda o, f, i, w: ops.layer_forward_noalloc(pl.weights, x, o, out_f32=f,
                                                                topk_idx=i, topk_w=w), cfg, T)
        torch.cuda.synchronize()
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)), (name, T)
        for g, r in zip(got[1:], ref[1:]):
            assert torch.equal(g, r), (name, T)
        # and the oracle's bar on the last token of the call
        t = T - 1
        r = O.layer_forward(xb[t:t + 1], li, cfg.top_k)
        ties, differ = compare_topk(got[2].cpu().numpy()[t:t + 1], got[3].cpu().numpy()[t:t + 1],
                                    r["logits"], r["top"], r["w"])
        if not differ:
            assert_close_f32(got[1].cpu().numpy()[t], r["out"][0], f"{name} T={T} out_f32")
            check_out_bf16(got[0].view(torch.int16).cpu().numpy().view(np.uint16)[t],
                           got[1].cpu().numpy()[t], r["out"][0], f"{name} T={T} out")
    assert ops.workspace_status(ws) == 0
