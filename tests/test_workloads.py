"""The seeded input generator: Philox known answers and the draw recipe (CPU only)."""
import numpy as np

from conftest import golden_lines
from workloads import gen as G
from workloads.philox import philox4x32_10


def test_philox_known_answers():
    for p in golden_lines("philox4x32_10_kat.txt"):
        v = [int(t, 16) for t in p]
        got = philox4x32_10(*v[:6])
        assert [int(g) for g in got] == v[6:], p


def test_philox_vectorised_matches_scalar():
    ctr = np.arange(50, dtype=np.uint64) * np.uint64(0x9E3779B1)
    a = philox4x32_10(ctr, 7, 0, 3, 11, 12)
    for i in range(0, 50, 7):
        b = philox4x32_10(int(ctr[i]) & 0xFFFFFFFF, 7, 0, 3, 11, 12)
        assert [int(x[i]) for x in a] == [int(y) for y in b]


def test_normal_draw_moments_and_determinism():
    z = G.normal_f32(1, 2, 1 << 20, 1.0)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert np.abs(z).max() <= 131070 * (1 / G.IH_STD) * 1.0001
    assert np.array_equal(z, G.normal_f32(1, 2, 1 << 20, 1.0))
    assert not np.array_equal(z[:100], G.normal_f32(1, 3, 100, 1.0))
    # element 2p and 2p+1 come from pair p: a prefix of a longer draw is the shorter draw
    assert np.array_equal(G.normal_f32(1, 2, 64, 1.0), z[:64])


def test_uniform_pes_range():
    u = G.uniform_f32(3, G.Tag.PES, 4096, 0.5, 1.5)
    assert u.dtype == np.float32 and u.min() >= 0.5 and u.max() < 1.5
    assert abs(u.mean() - 1.0) < 0.02


def test_expert_shapes_and_code_histogram():
    cfg = G.config("tiny")
    e = G.make_expert(cfg, 0, 5)
    H, I = cfg.hidden, cfg.inter
    assert e.gate_q.shape == (I, H // 2) and e.gate_s.shape == (I, H // 64)
    assert e.down_q.shape == (H, I // 2) and e.down_s.shape == (H, I // 64)
    lo = (e.gate_q & 15).ravel()
    hist = np.bincount(lo, minlength=16)
    assert hist[7] + hist[8] > hist[0] + hist[15]      # bell-shaped codes


def test_zipf_bias_skews_routing():
    cfg = G.config("qwen3_6_35b_a3b_long_prefill")
    b = G.zipf_bias(cfg, 0)
    assert b.shape == (cfg.experts,) and len(set(b.tolist())) == cfg.experts
    rank_order = np.argsort(-b)
    # the most popular expert's bias exceeds the least popular by (s ln E) * 0.02 * sqrt(6)/pi
    spread = b[rank_order[0]] - b[rank_order[-1]]
    assert abs(spread - 1.1 * np.log(cfg.experts) * 0.02 * np.sqrt(6) / np.pi) < 1e-6


def test_hidden_is_bf16_of_normal():
    cfg = G.config("tiny")
    x = G.make_hidden(cfg, 0)
    assert x.dtype == np.uint16 and x.shape == (cfg.tokens, cfg.hidden)
    assert not np.array_equal(x, G.make_hidden(cfg, 1))


def test_host_c_generator_matches_numpy_recipe():
    """The C draw + quantiser (workloads/hostgen.py) equals the numpy recipe bit for bit."""
    from workloads import hostgen as H
    if H.lib() is None:
        H.build()
    for k0, k1, rows, cols, std, bits in [(0, 16, 128, 256, 0.02, 4), (3, 77, 96, 2816, 0.02, 4),
                                          (5, 1, 128, 2816, 0.02, 8), (1, 9, 256, 128, 0.02, 8),
                                          (2 ** 32 - 1, 123, 64, 64, 1.0, 4)]:
        w = G.normal_f32(k0, k1, rows * cols, std).reshape(rows, cols)
        q, s, b = G.quantize_groups(w, bits)
        if bits == 4:
            q = G.pack_nibbles(q)
        q2, s2, b2 = H.matrix(k0, k1, rows, cols, std, bits)
        assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(b, b2), \
            (k0, k1, rows, cols, bits)
        assert np.array_equal(H.normal_f32(k0, k1, rows * cols, std), w.reshape(-1))
