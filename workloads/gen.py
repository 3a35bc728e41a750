"""Workload configurations and the seeded synthetic input recipe.

Every tensor is drawn from Philox4x32-10 (workloads/philox.py) under a key
(k0, k1) = (seed + layer, tag), with counter (pair, 0, 0, 0) for element pair
``pair`` of the tensor in row-major order.  One Philox call yields four 32-bit
words, i.e. eight 16-bit uniforms; four uniforms summed (Irwin-Hall, n=4) give
one approximately normal integer z in [-131070, 131070], so a call yields the
two elements 2*pair (words 0,1) and 2*pair+1 (words 2,3).  The float value is
fp32(z) * fp32(sigma / std(z)): a single IEEE round-to-nearest-even product,
so a HIP implementation of the same recipe reproduces it bit for bit.

Synthetic weights are then quantised per group of 64 consecutive input
elements into MLX-style affine codes (w ~ s*q + b, unsigned q, bf16 s and b),
the format [TF] describes for its checkpoint (4-bit experts, 8-bit router).
The pages copy codes from a checkpoint; this quantiser exists only to make
synthetic data of that shape and value distribution, and every step of it is
exact-integer or a single IEEE fp32 rounding (so the HIP re-implementation
agrees bit for bit):
    wmin, wmax = min, max of the group (fp32)
    s = bf16_rne( fp32(wmax - wmin) * fp32(1 / (2^bits - 1)) )
    b = bf16_rne( wmin )
    t = fp32( w - b )
    q = the integer in [0, 2^bits - 1] nearest to the real ratio t / s, ties to even
        (q = 0 everywhere when s == 0)

Shapes follow [TF] (128 experts, top-8, Gemma 4 26B-A4B) and [SW] (512 experts
top-10; 256 experts top-8).  Hidden sizes and expert widths of those models
are not on the pages; they are the public model shapes.
"""
from dataclasses import dataclass, field
import math
import os
from typing import Optional

import numpy as np

from .philox import philox4x32_10

GROUP = 64
IH_STD = math.sqrt((65536.0 * 65536.0 - 1.0) / 3.0)   # std of a sum of 4 uniform 16-bit ints
IH_MEAN = 4 * 32767.5                                  # = 131070


class Tag:
    """Second Philox key word: which tensor of a layer is drawn."""
    ROUTER = 1
    PES = 2
    HIDDEN = 3
    ZIPF = 4
    POST_GAIN = 5
    POST_SCALAR = 6
    SHARED = 8          # + 0 gate, 1 up, 2 down
    EXPERT = 16         # + 3*e + m, m: 0 gate, 1 up, 2 down

    @staticmethod
    def expert(e, m):
        return 16 + 3 * int(e) + int(m)

    @staticmethod
    def shared(m):
        return 8 + int(m)


@dataclass(frozen=True)
class Config:
    name: str
    hidden: int
    experts: int
    top_k: int
    inter: int
    shared_inter: int
    layers: int
    tokens: int                 # tokens per call (decode batch or prefill chunk)
    seed: int = 0
    zipf_s: Optional[float] = None
    prompt: int = 0             # long-prefill prompt length (0 = none)
    weight_std: float = 0.02
    hidden_std: float = 1.0
    pes_lo: float = 0.5
    pes_hi: float = 1.5
    expert_bits: int = 4        # routed and shared expert codes: 4 or 8 (MLX int8 groups)
    desc: str = ""


CONFIGS = {
    c.name: c for c in [
        Config("tiny", 256, 16, 2, 128, 128, layers=1, tokens=4,
               desc="tiny single MoE layer, 4 tokens"),
        Config("gemma4_26b_a4b_decode", 2816, 128, 8, 704, 2112, layers=30, tokens=1,
               desc="Gemma-4-26B-A4B-shaped decode, 1 token/step, 30 stacked layers"),
        Config("gemma4_26b_a4b_prefill", 2816, 128, 8, 704, 2112, layers=30, tokens=128,
               desc="Gemma-4-26B-A4B-shaped prefill, 128-token chunk"),
        Config("qwen3_next_80b_a3b_decode_b1", 2048, 512, 10, 512, 512, layers=48, tokens=1,
               desc="Qwen3-Next-80B-A3B-shaped decode, batch 1, 48 stacked layers"),
        Config("qwen3_next_80b_a3b_decode_b16", 2048, 512, 10, 512, 512, layers=48, tokens=16,
               desc="Qwen3-Next-80B-A3B-shaped decode, batch 16, 48 stacked layers"),
        Config("qwen3_6_35b_a3b_long_prefill", 2048, 256, 8, 512, 512, layers=40, tokens=128,
               zipf_s=1.1, prompt=10240,
               desc="Qwen3.6-35B-A3B-shaped long prefill, 10,240 tokens in 128-token "
                    "chunks, Zipf(1.1) router bias, 40 stacked layers"),
        Config("tiny_int8", 256, 16, 2, 128, 128, layers=1, tokens=4, expert_bits=8,
               desc="tiny single MoE layer with int8 experts, 4 tokens"),
        Config("gemma4_26b_a4b_int8_decode", 2816, 128, 8, 704, 2112, layers=30, tokens=1,
               expert_bits=8,
               desc="Gemma-4-26B-A4B-shaped decode with int8 experts, 1 token/step"),
    ]
}


def config(name):
    return CONFIGS[name]


# ---------------------------------------------------------------- bf16 bits

def bf16_bits_from_f32(a):
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def _bf16_bits_to_f32(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- draws

def normal_f32(k0, k1, n, std):
    """n approximately-N(0, std^2) fp32 values of tensor key (k0, k1), row-major order."""
    if n % 2:
        raise ValueError("element count must be even")
    pairs = np.arange(n // 2, dtype=np.uint64)
    r0, r1, r2, r3 = philox4x32_10(pairs & np.uint64(0xFFFFFFFF), pairs >> np.uint64(32), 0, 0, k0, k1)
    out = np.empty(n, dtype=np.int64)

    def isum(a, b):
        a = a.astype(np.int64)
        b = b.astype(np.int64)
        return (a & 0xFFFF) + (a >> 16) + (b & 0xFFFF) + (b >> 16)

    out[0::2] = isum(r0, r1)
    out[1::2] = isum(r2, r3)
    z = (out - int(IH_MEAN)).astype(np.float32)          # |z| < 2^18: exact
    c = np.float32(std / IH_STD)
    return z * c


def uniform_f32(k0, k1, n, lo, hi):
    """n fp32 values lo + u * (hi - lo), u = (word0 >> 8) * 2^-24, counter (i, 0, 0, 0)."""
    idx = np.arange(n, dtype=np.uint64)
    r0, _, _, _ = philox4x32_10(idx, 0, 0, 0, k0, k1)
    u = (r0 >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)
    return np.float32(lo) + u * np.float32(hi - lo)


def quantize_groups(w, bits):
    """Quantise fp32 w[rows, cols] per 64 consecutive columns (recipe in the module doc).

    Returns (q uint8 [rows, cols] unpacked codes, s uint16 [rows, cols/64], b uint16 [...]).
    """
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    if cols % GROUP:
        raise ValueError("columns must be a multiple of 64")
    qmax = (1 << bits) - 1
    g = w.reshape(rows, cols // GROUP, GROUP)
    wmin = g.min(axis=2)
    wmax = g.max(axis=2)
    rng = (wmax - wmin).astype(np.float32)
    s32 = rng * np.float32(1.0 / qmax)
    s16 = bf16_bits_from_f32(s32)
    b16 = bf16_bits_from_f32(wmin)
    sf = _bf16_bits_to_f32(s16)[:, :, None].astype(np.float64)
    bf = _bf16_bits_to_f32(b16)[:, :, None]
    t = (g - bf).astype(np.float32).astype(np.float64)
    safe = np.where(sf > 0, sf, 1.0)
    q = np.floor(t / safe)
    # exact corrections: afterwards q*s <= t < (q+1)*s holds exactly (products of a
    # bf16 and a small integer are exact in fp64)
    q = np.where(t < q * safe, q - 1, q)
    q = np.where(t >= (q + 1) * safe, q + 1, q)
    mid = (q + 0.5) * safe
    up = (t > mid) | ((t == mid) & (np.mod(q, 2) == 1))
    q = q + up
    q = np.clip(q, 0, qmax)
    q = np.where(sf > 0, q, 0).astype(np.uint8)
    return q.reshape(rows, cols), s16, b16


def pack_nibbles(q):
    """uint8 codes 0..15 [rows, cols] -> bytes [rows, cols/2]; element 2m in the low nibble of byte m."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------- layer tensors

@dataclass
class ExpertWeights:
    """Canonical MLX-style expert: int4 codes packed two per byte (low nibble first), or
    int8 codes one per byte when bits == 8 (shapes [I, H] and [H, I] then)."""
    gate_q: np.ndarray   # uint8 [I, H/2]
    gate_s: np.ndarray   # uint16 bf16 bits [I, H/64]
    gate_b: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    up_b: np.ndarray
    down_q: np.ndarray   # uint8 [H, I/2]
    down_s: np.ndarray   # uint16 [H, I/64]
    down_b: np.ndarray
    bits: int = 4

    def arrays(self):
        return (self.gate_q, self.gate_s, self.gate_b, self.up_q, self.up_s, self.up_b,
                self.down_q, self.down_s, self.down_b)


@dataclass
class LayerInputs:
    """Router tensors of one layer (experts are drawn on demand)."""
    cfg: Config
    layer: int
    router_q: np.ndarray       # uint8 [E, H]
    router_s: np.ndarray       # uint16 [E, H/64]
    router_b: np.ndarray
    router_scale: np.ndarray   # fp32 [H]
    pes: np.ndarray            # fp32 [E]
    bias: Optional[np.ndarray]  # fp32 [E] or None
    _cache: dict = field(default_factory=dict, repr=False)

    def expert(self, e):
        if e not in self._cache:
            self._cache[e] = make_expert(self.cfg, self.layer, e)
        return self._cache[e]

    def prefetch(self, experts, workers=None):
        """Draw the listed experts (not yet drawn) on several threads; the C draw releases
        the interpreter lock, so they run in parallel."""
        import concurrent.futures
        todo = sorted({int(e) for e in experts} - set(self._cache))
        if not todo:
            return
        n = workers or min(16, len(os.sched_getaffinity(0)))
        with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
            for e, ew in zip(todo, ex.map(lambda e: make_expert(self.cfg, self.layer, e), todo)):
                self._cache[e] = ew

    def shared(self):
        if not self.cfg.shared_inter:   # a layer without a shared expert
            return None
        if "shared" not in self._cache:
            self._cache["shared"] = make_shared(self.cfg, self.layer)
        return self._cache["shared"]


def layer_key(cfg, layer):
    return (cfg.seed + layer) & 0xFFFFFFFF


def _hostgen():
    """The C implementation of the draw and the quantiser (hostgen.py), or None when it is not
    built; it returns the same bits as normal_f32 / quantize_groups above."""
    from . import hostgen
    return hostgen if hostgen.lib() is not None else None


def quantized_matrix(k0, k1, rows, cols, std, bits):
    """normal_f32 draw of a [rows, cols] matrix, quantised with quantize_groups; codes packed
    two per byte for 4 bits."""
    fast = _hostgen()
    if fast is not None:
        return fast.matrix(k0, k1, rows, cols, std, bits)
    w = normal_f32(k0, k1, rows * cols, std).reshape(rows, cols)
    q, s, b = quantize_groups(w, bits)
    return (q if bits == 8 else pack_nibbles(q)), s, b


def _expert_matrix(cfg, layer, tag, rows, cols):
    return quantized_matrix(layer_key(cfg, layer), tag, rows, cols, cfg.weight_std, cfg.expert_bits)


def _ffn_block(cfg, layer, tags, inter):
    H = cfg.hidden
    gq, gs, gb = _expert_matrix(cfg, layer, tags[0], inter, H)
    uq, us, ub = _expert_matrix(cfg, layer, tags[1], inter, H)
    dq, ds, db = _expert_matrix(cfg, layer, tags[2], H, inter)
    return ExpertWeights(gq, gs, gb, uq, us, ub, dq, ds, db, bits=cfg.expert_bits)


def make_expert(cfg, layer, e):
    return _ffn_block(cfg, layer, [Tag.expert(e, m) for m in range(3)], cfg.inter)


def make_shared(cfg, layer):
    return _ffn_block(cfg, layer, [Tag.shared(m) for m in range(3)], cfg.shared_inter)


def zipf_bias(cfg, layer, sigma=None):
    """Router logit bias that skews expert popularity towards a Zipf(s) law.

    A seeded permutation gives each expert a rank r in 1..E; p_e = r^-s / sum;
    bias_e = ln(p_e) * sigma * sqrt(6) / pi, i.e. the log-popularity rescaled to
    the spread of a Gumbel variable whose std equals sigma, the std of the
    unbiased logits.  With N(0, std^2) router weights and a unit-norm scaled
    router input, that std is the weight std (0.02).
    """
    E = cfg.experts
    sigma = cfg.weight_std if sigma is None else sigma
    idx = np.arange(E, dtype=np.uint64)
    r0, r1, _, _ = philox4x32_10(idx, 0, 0, 0, layer_key(cfg, layer), Tag.ZIPF)
    keys = (r0.astype(np.uint64) << np.uint64(32)) | r1.astype(np.uint64)
    order = np.argsort(keys, kind="stable")
    rank = np.empty(E, dtype=np.int64)
    rank[order] = np.arange(1, E + 1)
    logp = -cfg.zipf_s * np.log(rank.astype(np.float64))
    logp -= np.log(np.exp(logp).sum())
    return (logp * sigma * math.sqrt(6.0) / math.pi).astype(np.float32)


def make_router(cfg, layer):
    E, H = cfg.experts, cfg.hidden
    q, s, b = quantized_matrix(layer_key(cfg, layer), Tag.ROUTER, E, H, cfg.weight_std, 8)
    pes = uniform_f32(layer_key(cfg, layer), Tag.PES, E, cfg.pes_lo, cfg.pes_hi)
    bias = zipf_bias(cfg, layer) if cfg.zipf_s else None
    return LayerInputs(cfg, layer, q, s, b, np.ones(H, np.float32), pes, bias)


def make_post(cfg, layer):
    """Post-combine norm gain (fp32 [H], 1 + N(0, 0.1^2)) and layer scalar (fp32,
    U(0.5, 1.0)) of one layer."""
    g = normal_f32(layer_key(cfg, layer), Tag.POST_GAIN, cfg.hidden, 0.1)
    gain = (np.float32(1.0) + g).astype(np.float32)
    scalar = uniform_f32(layer_key(cfg, layer), Tag.POST_SCALAR, 1, 0.5, 1.0)[0]
    return gain, np.float32(scalar)


def make_hidden(cfg, step, tokens=None, std=None):
    """bf16 bit patterns [T, H] of the hidden states entering the first layer at ``step``."""
    T = cfg.tokens if tokens is None else tokens
    k0 = (cfg.seed + 1_000_003 + step) & 0xFFFFFFFF
    fast = _hostgen()
    draw = fast.normal_f32 if fast is not None else normal_f32
    x = draw(k0, Tag.HIDDEN, T * cfg.hidden, cfg.hidden_std if std is None else std)
    return bf16_bits_from_f32(x).reshape(T, cfg.hidden)


def make_layer_small(cfg, layer):
    """Router tensors plus every expert and the shared block (small configs only)."""
    li = make_router(cfg, layer)
    for e in range(cfg.experts):
        li.expert(e)
    li.shared()
    return li


# ---------------------------------------------------------------- byte accounting

def matrix_bytes(rows, cols, bits=4):
    """Codes + bf16 scale + bf16 bias of one group-quantised matrix."""
    return rows * cols * bits // 8 + rows * (cols // GROUP) * 4


def expert_bytes(cfg, inter=None):
    """Bytes of one routed expert (gate, up, down) in the canonical format."""
    I = cfg.inter if inter is None else inter
    b = cfg.expert_bits
    return 2 * matrix_bytes(I, cfg.hidden, b) + matrix_bytes(cfg.hidden, I, b)


def credited_expert_bytes(cfg, n_distinct):
    """Algorithmic bytes of a call: distinct routed experts touched x expert bytes."""
    return int(n_distinct) * expert_bytes(cfg)


def router_bytes(cfg):
    return matrix_bytes(cfg.experts, cfg.hidden, bits=8)
