"""Pins of the fp64 oracle against closed forms, brute force, textbook special cases and
hand-built fixtures (tests/golden).  CPU only.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign,
a swapped nibble, a transposed operand, a wrong reduction axis) fails at least one test.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle as O
from conftest import golden_lines
from workloads import gen as G


class Layer:
    """Minimal duck-typed layer for hand-built cases."""

    def __init__(self, router_q, router_s, router_b, pes, experts=None, shared=None,
                 router_scale=None, bias=None):
        self.router_q, self.router_s, self.router_b = router_q, router_s, router_b
        self.pes = np.asarray(pes, np.float32)
        self.router_scale = router_scale
        self.bias = bias
        self._experts = experts or {}
        self._shared = shared

    def expert(self, e):
        return self._experts[e]

    def shared(self):
        return self._shared


def _bits(v):
    return np.array([int(v, 16)], dtype=np.uint16)


# ------------------------------------------------------------------ bf16

def test_bf16_rounding_golden():
    for val, bits in golden_lines("bf16_rounding.txt"):
        got = O.bf16_rne_bits(np.array([float.fromhex(val)]))[0]
        assert got == int(bits, 16), (val, hex(got), bits)


def test_bf16_widen_golden():
    for bits, val in golden_lines("bf16_widen.txt"):
        assert O.bf16_to_f64(_bits(bits))[0] == float.fromhex(val), bits


def test_bf16_round_trip_all_finite_patterns():
    # every finite bf16 value is a fixed point of rounding
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_to_f64(b)
    fin = np.isfinite(v)
    got = O.bf16_rne_bits(v[fin])
    assert np.array_equal(got, b[fin])


# ------------------------------------------------------------------ dequantisation

def _parse_affine_fixture(name):
    codes, scale, bias, rows = {}, {}, {}, []
    for parts in golden_lines(name):
        tag, r = parts[0], int(parts[1])
        if tag == "codes":
            codes[r] = np.array([int(t, 16) for t in parts[2:]], dtype=np.uint8)
        elif tag == "scale":
            scale[r] = [int(t, 16) for t in parts[2:]]
        elif tag == "bias":
            bias[r] = [int(t, 16) for t in parts[2:]]
        else:
            rows.append(parts)
    n = len(codes)
    q = np.stack([codes[r] for r in range(n)])
    s = np.array([scale[r] for r in range(n)], dtype=np.uint16)
    b = np.array([bias[r] for r in range(n)], dtype=np.uint16)
    return q, s, b, rows


def test_dequant_int4_golden():
    q, s, b, rows = _parse_affine_fixture("dequant_int4.txt")
    w = O.dequant_int4(q, s, b)
    assert w.shape == (2, 128)
    seen = 0
    for parts in rows:
        assert parts[0] == "period16"
        r, g = int(parts[1]), int(parts[2])
        pat = np.array([float(t) for t in parts[3:]])
        want = np.tile(pat, 4)
        assert np.array_equal(w[r, 64 * g:64 * (g + 1)], want), (r, g)
        seen += 1
    assert seen == 4


def test_dequant_int8_golden():
    q, s, b, rows = _parse_affine_fixture("dequant_int8.txt")
    w = O.dequant_int8(q, s, b)
    for parts in rows:
        assert parts[0] == "expect"
        r = int(parts[1])
        assert np.array_equal(w[r], np.array([float(t) for t in parts[2:]])), r


def test_nibble_pack_unpack_identity():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(7, 128), dtype=np.uint8)
    assert np.array_equal(O.unpack_nibbles(G.pack_nibbles(q)), q)


# ------------------------------------------------------------------ quantiser of the synthetic data

def test_quantiser_error_bound_and_requant():
    w = G.normal_f32(123, 7, 64 * 300, 0.02).reshape(300, 64)
    q, s, b = G.quantize_groups(w, 4)
    deq = O.dequant(q, s, b)
    sf = O.bf16_to_f64(s)[:, 0]
    bf = O.bf16_to_f64(b)[:, 0]
    wmin = w.min(axis=1).astype(np.float64)
    wmax = w.max(axis=1).astype(np.float64)
    # error of the nearest code is at most half a step, plus what the bf16 rounding of
    # b (above wmin) and of s (15 s below the range) push outside the code range
    slack = np.maximum(bf - wmin, 0) + np.maximum((wmax - wmin) - 15 * sf, 0)
    err = np.abs(deq - w.astype(np.float64)).max(axis=1)
    assert np.all(err <= 0.5 * sf + slack + 1e-9)
    # bf16 keeps 8 significant bits: b is within 2^-9 |wmin| of wmin and s within 2^-9 s
    assert np.all(slack <= 2.0 ** -8 * np.abs(wmin) + 15 * 2.0 ** -8 * sf)
    # re-quantising the dequantised weights with the same (s, b) gives the same codes:
    # q' = nearest integer to (w' - b)/s
    t = (deq - bf[:, None]) / sf[:, None]
    assert np.array_equal(np.clip(np.rint(t), 0, 15).astype(np.uint8), q)


def test_quantiser_codes_use_full_range():
    w = G.normal_f32(9, 9, 64 * 100, 0.02).reshape(100, 64)
    q, s, b = G.quantize_groups(w, 4)
    # min maps to 0 and max to 15 (or 14 when bf16 rounding shrinks the step range)
    assert np.all(q.min(axis=1) == 0)
    assert np.all(q.max(axis=1) >= 14)


# ------------------------------------------------------------------ router

def _router_fixture_layer(scale):
    H = 64
    rq = np.zeros((3, H), np.uint8)
    rq[0] = 1
    rq[2, 0::2] = 2
    rs = np.array([[0x3F80]] * 3, np.uint16)
    rb = np.array([[0x0000], [0xBF80], [0xBF80]], np.uint16)
    return Layer(rq, rs, rb, pes=np.ones(3), router_scale=scale)


def test_router_logits_closed_form():
    want = {p[0]: [float(v) for v in p[1:]] for p in golden_lines("router_closed_form.txt")}
    x = np.full((1, 64), 0x3F80, np.uint16)
    la = O.router_logits(x, _router_fixture_layer(None))
    assert np.allclose(la[0], want["caseA"], rtol=0, atol=1e-12)
    sc = np.where(np.arange(64) < 32, 2.0, 1.0).astype(np.float32)
    lb = O.router_logits(x, _router_fixture_layer(sc))
    assert np.allclose(lb[0], want["caseB"], rtol=0, atol=1e-12)


def test_router_rmsnorm_scale_invariance():
    # rmsnorm removes a positive scale of the input (up to eps): logits of x and 4x agree
    cfg = G.config("tiny")
    li = G.make_router(cfg, 0)
    x = G.make_hidden(cfg, 0)
    x4 = (x.astype(np.uint32) + (2 << 7)).astype(np.uint16)    # exponent + 2 -> x * 4 exactly
    l1 = O.router_logits(x, li)
    l4 = O.router_logits(x4, li)
    assert np.allclose(l1, l4, rtol=1e-6, atol=1e-9)


def test_topk_brute_force_subsets():
    rng = np.random.default_rng(0)
    for E, k in [(16, 2), (8, 3), (6, 1), (5, 5)]:
        logits = rng.standard_normal((40, E))
        top = O.topk_select(logits, k)
        for t in range(40):
            best = max(itertools.combinations(range(E), k), key=lambda S: sum(logits[t, list(S)]))
            assert set(top[t]) == set(best)
            assert np.all(np.diff(logits[t, top[t]]) <= 0)      # descending order


def test_topk_exact_ties_lower_index_first():
    logits = np.array([[0.5, 0.9, 0.9, 0.1], [0.0, 0.0, 0.0, 0.0], [1.0, 2.0, 1.0, 2.0]])
    assert O.topk_select(logits, 2).tolist() == [[1, 2], [0, 1], [1, 3]]
    assert O.topk_select(logits, 1).tolist() == [[1], [0], [1]]
    assert O.topk_select(logits, 3).tolist() == [[1, 2, 0], [0, 1, 2], [1, 3, 0]]


def test_duplicate_router_rows_tie_to_lower_index():
    cfg = G.config("tiny")
    li = G.make_router(cfg, 0)
    x = G.make_hidden(cfg, 0)
    top0, _, l0 = O.router(x, li, 2)
    # copy the winning expert's router row onto a higher-indexed expert: exact tie
    for t in range(x.shape[0]):
        e = int(top0[t, 0])
        d = cfg.experts - 1 if e != cfg.experts - 1 else 0
        li2 = G.make_router(cfg, 0)
        for a in ("router_q", "router_s", "router_b"):
            getattr(li2, a)[d] = getattr(li2, a)[e]
        top, w, lg = O.router(x[t:t + 1], li2, 2)
        assert lg[0, d] == lg[0, e]
        assert top[0].tolist() == sorted([e, d])
        assert w[0, 0] * li2.pes[top[0, 1]] == pytest.approx(w[0, 1] * li2.pes[top[0, 0]], rel=1e-15)


def test_softmax_sums_to_one_and_matches_renormalised_full_softmax():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((50, 16)) * 3
    top = O.topk_select(logits, 4)
    p = O.topk_weights(logits, top, np.ones(16))
    assert np.all(np.abs(p.sum(axis=1) - 1) <= 1e-12)
    full = scipy.special.softmax(logits, axis=1)
    kept = np.take_along_axis(full, top.astype(np.int64), axis=1)
    assert np.allclose(p, kept / kept.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)


def test_per_expert_scale_multiplies_after_softmax():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((20, 8))
    pes = rng.uniform(0.5, 1.5, 8)
    top = O.topk_select(logits, 3)
    p = O.topk_weights(logits, top, np.ones(8))
    w = O.topk_weights(logits, top, pes)
    assert np.allclose(w, p * pes[top], rtol=1e-15)
    # k = 1: the weight is exactly the expert's scale
    t1 = O.topk_select(logits, 1)
    assert np.array_equal(O.topk_weights(logits, t1, pes)[:, 0], pes[t1[:, 0]])


def test_near_tie_mask():
    logits = np.array([[1.0, 0.5, 0.5 - 5e-6, 0.0], [1.0, 0.5, 0.4, 0.0]])
    assert O.near_tie_mask(logits, 2).tolist() == [True, False]
    assert O.near_tie_mask(logits, 4).tolist() == [False, False]


# ------------------------------------------------------------------ bucketing

def test_bucket_brute_force():
    rng = np.random.default_rng(3)
    for T, k, E in [(1, 1, 4), (4, 2, 16), (33, 3, 7), (128, 8, 128), (0, 2, 5)]:
        top = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]) if T else \
            np.zeros((0, k), np.int64)
        counts, offsets, srt, active = O.bucket(top, E)
        flat = top.reshape(-1)
        assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
        pos = 0
        for e in range(E):
            ids = [i for i in range(T * k) if flat[i] == e]        # ascending flat id
            assert counts[e] == len(ids) and offsets[e] == pos
            assert list(srt[pos:pos + len(ids)]) == ids
            pos += len(ids)
        assert list(active) == [e for e in range(E) if counts[e]]


# ------------------------------------------------------------------ expert FFN

def _identity_expert():
    H = 64
    eye = np.eye(H, dtype=np.uint8)
    shift = int([p for p in golden_lines("swiglu_identity.txt") if p[0] == "down_shift"][0][1])
    perm = np.zeros((H, H), np.uint8)
    perm[np.arange(H), (np.arange(H) + shift) % H] = 1
    one = np.full((H, 1), 0x3F80, np.uint16)
    two = np.full((H, 1), 0x4000, np.uint16)
    zero = np.zeros((H, 1), np.uint16)
    return G.ExpertWeights(G.pack_nibbles(eye), one, zero, G.pack_nibbles(eye), two, zero,
                           G.pack_nibbles(perm), one, zero)


def test_swiglu_identity_closed_form():
    lines = golden_lines("swiglu_identity.txt")
    x = np.zeros((1, 64))
    for p in lines:
        if p[0] == "x":
            x[0, int(p[1])] = float(p[2])
    want = np.zeros(64)
    for p in lines:
        if p[0] == "y":
            want[int(p[1])] = float(p[2])
    y = O.expert_ffn(x, _identity_expert())
    assert np.allclose(y[0], want, rtol=1e-14, atol=1e-15)


def _identity_expert_int8():
    """The same closed-form expert with 8-bit codes that use both nibbles and a bias:
    gate codes 192 on the diagonal and 64 elsewhere with s = 1/128, b = -0.5 (so W_g = I);
    up 192 / 64 with s = 1/64, b = -1 (W_u = 2 I); down 160 on the shifted diagonal and 32
    elsewhere with s = 1/128, b = -0.25 (the permutation)."""
    H = 64
    shift = int([p for p in golden_lines("swiglu_identity.txt") if p[0] == "down_shift"][0][1])
    diag = np.where(np.eye(H, dtype=bool), 192, 64).astype(np.uint8)
    perm = np.full((H, H), 32, np.uint8)
    perm[np.arange(H), (np.arange(H) + shift) % H] = 160

    def col(v):
        return np.full((H, 1), v, np.uint16)

    return G.ExpertWeights(diag, col(0x3C00), col(0xBF00), diag, col(0x3C80), col(0xBF80),
                           perm, col(0x3C00), col(0xBE80), bits=8)


def test_swiglu_identity_closed_form_int8_experts():
    lines = golden_lines("swiglu_identity.txt")
    x = np.zeros((1, 64))
    for p in lines:
        if p[0] == "x":
            x[0, int(p[1])] = float(p[2])
    want = np.zeros(64)
    for p in lines:
        if p[0] == "y":
            want[int(p[1])] = float(p[2])
    y = O.expert_ffn(x, _identity_expert_int8())
    assert np.allclose(y[0], want, rtol=1e-14, atol=1e-15)


def test_int8_expert_generator_codes_span_the_range():
    cfg = G.config("tiny_int8")
    ew = G.make_expert(cfg, 0, 3)
    assert ew.bits == 8 and ew.gate_q.shape == (cfg.inter, cfg.hidden)
    assert ew.gate_q.min() == 0 and ew.gate_q.max() == 255


def test_expert_ffn_zero_input_is_zero():
    cfg = G.config("tiny")
    y = O.expert_ffn(np.zeros((2, cfg.hidden)), G.make_expert(cfg, 0, 3))
    assert np.all(y == 0)


# ------------------------------------------------------------------ combine and whole layer

def test_combine_closed_form():
    d = {p[0]: [float(v) for v in p[1:]] for p in golden_lines("combine_closed_form.txt")}
    xb = O.bf16_rne_bits(np.array([d["x"]]))
    y = np.array([[d["y0"], d["y1"]]])
    out, out_b = O.combine(xb, y, np.array([d["w"]]), np.array([d["yshared"]]))
    assert np.array_equal(out[0], np.array(d["out"]))
    assert np.array_equal(O.bf16_to_f64(out_b[0]), np.array(d["out"]))


# ------------------------------------------------------------------ post-combine steps (cb2)

def _post_case():
    d = {p[0]: [float(v) for v in p[1:]] for p in golden_lines("post_combine_example.txt")}
    xb = O.bf16_rne_bits(np.array([d["x"]]))
    y = np.array([[d["y0"]]])
    return d, xb, y


def test_post_combine_hand_example():
    """Order (norm of the combined branches, then residual, then scalar) and the gain."""
    d, xb, y = _post_case()
    out, out_b = O.combine_post(xb, y, np.array([d["w"]]), np.array([d["yshared"]]),
                                np.array(d["gain"]), d["scalar"][0])
    assert np.allclose(out[0], d["out"], rtol=1e-15, atol=0)
    assert np.array_equal(out_b, O.bf16_rne_bits(out))


def test_post_combine_without_steps_is_combine():
    d, xb, y = _post_case()
    a, ab = O.combine_post(xb, y, np.array([d["w"]]), np.array([d["yshared"]]))
    b, bb = O.combine(xb, y, np.array([d["w"]]), np.array([d["yshared"]]))
    assert np.array_equal(a, b) and np.array_equal(ab, bb)


def test_post_norm_unit_gain_has_unit_rms():
    """gain 1, scalar 1: the added term has RMS sqrt(ms / (ms + eps)) over the hidden axis."""
    rng = np.random.default_rng(7)
    T, H = 5, 256
    xb = O.bf16_rne_bits(rng.standard_normal((T, H)))
    m = rng.standard_normal((T, H)) * np.array([[0.01], [0.1], [1.0], [10.0], [100.0]])
    out, _ = O.post_combine(xb, m, np.ones(H), None)
    added = out - O.bf16_to_f64(xb)
    ms = np.mean(m * m, axis=1)
    want = np.sqrt(ms / (ms + O.EPS))
    assert np.allclose(np.sqrt(np.mean(added * added, axis=1)), want, rtol=1e-12)


def test_post_norm_scale_invariance_and_scalar_linearity():
    rng = np.random.default_rng(8)
    T, H = 3, 128
    xb = O.bf16_rne_bits(rng.standard_normal((T, H)))
    m = rng.standard_normal((T, H))
    g = 1.0 + 0.1 * rng.standard_normal(H)
    a, _ = O.post_combine(xb, m, g, None)
    b, _ = O.post_combine(xb, 1000.0 * m, g, None, eps=1e6 * O.EPS)   # scale m by c, eps by c^2
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)
    c1, _ = O.post_combine(xb, m, g, 1.0)
    c3, _ = O.post_combine(xb, m, g, 0.75)
    assert np.allclose(c3, 0.75 * c1, rtol=1e-15, atol=0)
    z, _ = O.post_combine(xb, m, np.zeros(H), 0.5)       # zero gain: scaled residual only
    assert np.array_equal(z, 0.5 * O.bf16_to_f64(xb))


def test_layer_forward_post_steps_match_post_combine():
    cfg = G.config("tiny")
    li = G.make_layer_small(cfg, 0)
    xb = G.make_hidden(cfg, 0)
    plain = O.layer_forward(xb, li, cfg.top_k)
    li.post_gain, li.layer_scalar = G.make_post(cfg, 0)
    post = O.layer_forward(xb, li, cfg.top_k)
    m = plain["out"] - O.bf16_to_f64(xb)
    want, _ = O.post_combine(xb, m, li.post_gain, li.layer_scalar)
    assert np.array_equal(post["top"], plain["top"])
    assert np.allclose(post["out"], want, rtol=1e-12, atol=1e-12)


def test_zero_input_routes_to_first_k_experts():
    cfg = G.config("tiny")
    li = G.make_layer_small(cfg, 0)
    x = np.zeros((3, cfg.hidden), np.uint16)
    r = O.layer_forward(x, li, cfg.top_k)
    assert np.all(r["logits"] == 0)
    assert r["top"].tolist() == [[0, 1]] * 3
    assert np.allclose(r["w"], li.pes[:2][None, :] / 2, rtol=1e-15)
    assert np.all(r["out"] == 0)


def _tiny_layer():
    cfg = G.config("tiny")
    return cfg, G.make_layer_small(cfg, 0), G.make_hidden(cfg, 0)


def test_token_independence():
    cfg, li, x = _tiny_layer()
    full = O.layer_forward(x, li, cfg.top_k)
    for t in range(x.shape[0]):
        one = O.layer_forward(x[t:t + 1], li, cfg.top_k)
        assert np.allclose(one["out"][0], full["out"][t], rtol=1e-12, atol=1e-12)
        assert one["top"][0].tolist() == full["top"][t].tolist()


def test_expert_permutation_invariance():
    cfg, li, x = _tiny_layer()
    base = O.layer_forward(x, li, cfg.top_k)
    perm = np.random.default_rng(4).permutation(cfg.experts)        # new label of expert e
    inv = np.argsort(perm)
    li2 = Layer(li.router_q[inv], li.router_s[inv], li.router_b[inv], li.pes[inv],
                experts={int(perm[e]): li.expert(e) for e in range(cfg.experts)},
                shared=li.shared(), router_scale=li.router_scale)
    r = O.layer_forward(x, li2, cfg.top_k)
    assert np.allclose(r["out"], base["out"], rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["top"], perm[base["top"]])


def test_per_expert_scale_linearity():
    cfg, li, x = _tiny_layer()
    base = O.layer_forward(x, li, cfg.top_k)
    # pes * 2 is exact in fp32
    li3 = Layer(li.router_q, li.router_s, li.router_b, li.pes * np.float32(2),
                experts={e: li.expert(e) for e in range(cfg.experts)}, shared=li.shared())
    r = O.layer_forward(x, li3, cfg.top_k)
    xf = O.bf16_to_f64(x)
    routed0 = base["out"] - xf - base["y_shared"]
    routed2 = r["out"] - xf - r["y_shared"]
    assert np.allclose(routed2, 2 * routed0, rtol=1e-12, atol=1e-14)


def test_dense_top_e_equals_softmax_gated_mixture():
    # k = E: every expert is kept, so the layer is a dense softmax-gated mixture
    cfg, li, x = _tiny_layer()
    E = cfg.experts
    r = O.layer_forward(x, li, E)
    logits = r["logits"]
    gate = scipy.special.softmax(logits, axis=1) * li.pes.astype(np.float64)[None, :]
    xf = O.bf16_to_f64(x)
    want = xf + O.expert_ffn(xf, li.shared())
    for e in range(E):
        want = want + gate[:, e:e + 1] * O.expert_ffn(xf, li.expert(e))
    assert np.allclose(r["out"], want, rtol=1e-12, atol=1e-12)


def test_empty_call():
    cfg, li, _ = _tiny_layer()
    r = O.layer_forward(np.zeros((0, cfg.hidden), np.uint16), li, cfg.top_k)
    assert r["out"].shape == (0, cfg.hidden) and r["top"].shape == (0, cfg.top_k)


# ------------------------------------------------------------------ sizes

def test_container_sizes_match_pages():
    rows = golden_lines("container_sizes.txt")
    total, expected = {}, {}
    for row in rows:
        if row[0] == "ratio":
            continue
        name, dense, exp, tol = row
        cfg = G.config(name)
        total[name] = cfg.layers * cfg.experts * G.expert_bytes(cfg) + float(dense)
        expected[name] = float(exp)
        assert abs(total[name] / expected[name] - 1) <= float(tol), (name, total[name])
    ratios = [r for r in rows if r[0] == "ratio"]
    assert ratios
    for _, num, den, tol in ratios:
        got = total[num] / total[den]
        want = expected[num] / expected[den]
        assert abs(got / want - 1) <= float(tol), (num, den, got, want)
    # the format's 0.5625 B per weight matters: 0.5 B per weight (codes only) misses the
    # Gemma install by more than the tolerance
    cfg = G.config("gemma4_26b_a4b_decode")
    codes_only = cfg.layers * cfg.experts * 3 * cfg.hidden * cfg.inter * 0.5 + 1.35e9
    assert abs(codes_only / 14.3e9 - 1) > 0.10


def test_silu_orientation_and_swiglu_against_logistic():
    # h = silu(gate) * up: swapping gate and up changes the result (pinned in the fixture)
    s15 = float([p for p in golden_lines("swiglu_identity.txt") if p[:2] == ["logistic", "1.5"]][0][2])
    assert math.isclose(s15, 1 / (1 + math.exp(-1.5)), rel_tol=1e-15)


# ------------------------------------------------------------------ router logit bias
# (optional per-expert bias added to the logits before the top-k and kept in the softmax:
# the plain linear-layer reading of the Zipf-biased router of the long-prefill workload;
# the router listing of the TurboFieldfare post, section "TurboFieldfare의 전문가 스트리밍
# 구조", has no bias term, so the reading is pinned by closed forms here.)

def _bias_only_layer(bias, pes):
    """Router rows of zero weight (codes 0, s = 1, b = 0): every logit is its bias."""
    H, E = 64, len(bias)
    return Layer(np.zeros((E, H), np.uint8), np.full((E, 1), 0x3F80, np.uint16),
                 np.zeros((E, 1), np.uint16), pes=pes, bias=np.asarray(bias, np.float32))


def test_logit_bias_zero_input_closed_form():
    """x = 0 gives u = 0, so logits == bias exactly.  Biases (0, 1, 1, 2, 0.5), k = 2: the
    selection is expert 3 (bias 2), then expert 1 (bias 1, lower index of the tie with 2),
    and the weights are the softmax of (2, 1) -- e/(e+1) and 1/(e+1) -- times the experts'
    scales.  A flipped sign selects (0, 4); a bias used only for selection gives 1/2, 1/2."""
    pes = np.array([0.5, 0.75, 1.25, 1.5, 1.0], np.float32)
    li = _bias_only_layer([0.0, 1.0, 1.0, 2.0, 0.5], pes)
    x = np.zeros((2, 64), np.uint16)
    top, w, logits = O.router(x, li, 2)
    assert np.array_equal(logits, np.tile([0.0, 1.0, 1.0, 2.0, 0.5], (2, 1)))
    assert top.tolist() == [[3, 1], [3, 1]]
    e = math.e
    want = np.array([e / (e + 1) * 1.5, 1 / (e + 1) * 0.75])
    assert np.allclose(w, np.tile(want, (2, 1)), rtol=1e-15, atol=0)
    # k = 3 takes the tied expert 2 next; its weight uses the same bias as expert 1
    top3, w3, _ = O.router(x, li, 3)
    assert top3[0].tolist() == [3, 1, 2]
    z = e * e + 2 * e
    assert np.allclose(w3[0], [e * e / z * 1.5, e / z * 0.75, e / z * 1.25], rtol=1e-15, atol=0)


def test_logit_bias_adds_to_projected_logits():
    """The closed-form router of tests/golden/router_closed_form.txt (case A: logits
    8/sqrt(1+eps), -8/sqrt(1+eps), 0 for x = 1) with the bias (-8, 8.5, 0.25): the logits are
    the sums, which reverses the order of experts 0 and 1 and puts expert 2 in between."""
    want_a = [float(v) for p in golden_lines("router_closed_form.txt") if p[0] == "caseA"
              for v in p[1:]]
    li = _router_fixture_layer(None)
    li.bias = np.array([-8.0, 8.5, 0.25], np.float32)
    x = np.full((1, 64), 0x3F80, np.uint16)
    top, w, logits = O.router(x, li, 2)
    want = np.array(want_a) + np.array([-8.0, 8.5, 0.25])
    assert np.allclose(logits[0], want, rtol=0, atol=1e-12)
    assert top[0].tolist() == [1, 2]
    d = want[1] - want[2]
    assert np.allclose(w[0], [1 / (1 + math.exp(-d)), 1 / (1 + math.exp(d))], rtol=1e-14, atol=0)


def test_logit_bias_none_equals_zero_bias():
    cfg, li, x = _tiny_layer()
    base = O.layer_forward(x, li, cfg.top_k)
    li0 = Layer(li.router_q, li.router_s, li.router_b, li.pes,
                experts={e: li.expert(e) for e in range(cfg.experts)}, shared=li.shared(),
                bias=np.zeros(cfg.experts, np.float32))
    r = O.layer_forward(x, li0, cfg.top_k)
    assert np.array_equal(r["top"], base["top"]) and np.array_equal(r["out"], base["out"])


# ------------------------------------------------------------------ selection override
# (layer_forward(top_override=...) re-evaluates a near-tied token with another valid
# selection; the parity tests use it, so it is pinned here.)

def test_top_override_with_own_selection_is_identity():
    cfg, li, x = _tiny_layer()
    base = O.layer_forward(x, li, cfg.top_k)
    again = O.layer_forward(x, li, cfg.top_k, top_override=base["top"])
    for key in ("logits", "top", "w", "counts", "offsets", "sorted", "active", "y",
                "y_shared", "out", "out_bf16"):
        assert np.array_equal(again[key], base[key]), key


def test_top_override_alternative_selection():
    """Another selection: its weights are the softmax of the overriding experts' own logits
    (times their scales) and its routed rows are those experts' FFN outputs."""
    cfg, li, x = _tiny_layer()
    k = cfg.top_k
    base = O.layer_forward(x, li, k)
    alt = base["top"].copy()
    for t in range(x.shape[0]):   # keep the first choice, replace the second by an unchosen expert
        alt[t, 1] = next(e for e in range(cfg.experts) if e not in base["top"][t])
    r = O.layer_forward(x, li, k, top_override=alt)
    assert np.array_equal(r["top"], alt)
    xf = O.bf16_to_f64(x)
    for t in range(x.shape[0]):
        lg = base["logits"][t, alt[t]]
        p = np.exp(lg - lg.max())
        p /= p.sum()
        assert np.allclose(r["w"][t], p * li.pes[alt[t]].astype(np.float64), rtol=1e-14, atol=0)
        for j in range(k):
            want = O.expert_ffn(xf[t:t + 1], li.expert(int(alt[t, j])))[0]
            assert np.allclose(r["y"][t * k + j], want, rtol=1e-12, atol=1e-15)
    want_out = xf + r["y_shared"] + np.einsum("tk,tkh->th", r["w"], r["y"].reshape(-1, k, cfg.hidden))
    assert np.allclose(r["out"], want_out, rtol=1e-14, atol=1e-14)
