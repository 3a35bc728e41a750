"""fp64 CPU oracle of the routed int4 MoE layer (test infrastructure only).

Sources (the pages this follows; cited by short name below):
  [TF-struct]  TurboFieldfare post on discuss.pytorch.kr, section
               "TurboFieldfare의 전문가 스트리밍 구조" (expert-streaming structure):
               128 routed experts with top-8 per token plus an always-on shared
               expert added with no routing weight; the router listing (scale-free
               RMS norm, scaling by router_scale / sqrt(hidden), an 8-bit affine
               projection to one logit per expert, top-8, softmax over the kept
               logits, times per_expert_scale); cb2 combining the routed
               branches by router weight with the shared branch and the residual;
               prefill in chunks of at most 128 tokens.
  [TF-mem]     same post, section "TurboFieldfare가 메모리를 아끼는 방식": MLX affine
               4-bit weights, one bf16 scale and one bf16 bias per group of 64
               weights; only the router projection is 8-bit.
  [SW-mem]     Swiftlet article on tech.utomolab.com, section "같은 모델을 왜 이렇게
               적은 메모리로 돌릴 수 있나": 512 experts / top-10 and 256 / top-8.

Readings where the pages are silent (each is listed with its reason in the
project's design notes):
  * rmsnorm epsilon 1e-6, mean over the hidden axis, no gain.
  * MLX affine: w = s * q + b with unsigned codes q (0..15 for 4-bit, 0..255
    for 8-bit); groups are 64 consecutive elements along each matrix's input
    (reduction) axis; element 2m of a 4-bit row is the low nibble of byte m.
  * The expert FFN is SwiGLU: h = silu(x W_g^T) * (x W_u^T), y = h W_d^T,
    silu(z) = z / (1 + exp(-z)); no biases.  The shared expert uses the same
    form and format and is added with weight 1.
  * The layer output is x + m with m = shared + sum_j w_j y_j.  When a layer
    carries cb2's post-combine steps, they run in the order the post lists
    them -- normalisation, residual, layer scalar:
        out = (x + gain * m / sqrt(mean(m^2) + 1e-6)) * scalar
    (RMS over the hidden axis, a per-channel gain multiplying the normalised
    value directly, one scalar per layer).  Without a gain the norm step is
    skipped; without a scalar it is 1.
  * Top-k order: descending logit; exact ties go to the lower expert index.
  * Optional per-expert logit bias (absent on the pages) is added to the
    logits before top-k and enters the softmax.
  * Buckets: assignments (flat id t*k + j) grouped by expert in ascending
    expert order, stable (ascending flat id within an expert).
Everything is fp64 except the final bf16 rounding of the layer output.
"""
import numpy as np

EPS = 1e-6
GROUP = 64


# ------------------------------------------------------------------ bf16

def bf16_to_f64(bits):
    """bf16 bit patterns -> fp64.  A bf16 is the upper half of an IEEE fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_rne_bits(v):
    """Round fp64 values to the nearest bf16 (ties to even), directly from fp64.

    bf16 keeps 8 significant bits, exponent range of fp32, subnormal quantum
    2^-133.  Rounding is done once, on the fp64 value (no detour through fp32).
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    finite = np.isfinite(v)
    m, e = np.frexp(np.where(finite, v, 0.0))          # v = m * 2^e, 0.5 <= |m| < 1
    quantum_exp = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(np.where(finite, v, 0.0), -quantum_exp))   # exact scaling
    r = np.ldexp(r, quantum_exp)
    over = np.abs(r) >= 2.0 ** 128
    r = np.where(over, np.copysign(np.inf, v), r)
    r = np.where(finite, r, v)
    bits32 = r.astype(np.float32).view(np.uint32)       # r is exactly a bf16 value
    out[...] = (bits32 >> np.uint32(16)).astype(np.uint16)
    return out


# ------------------------------------------------------------------ quantised weights

def unpack_nibbles(packed):
    """uint8 [rows, n] -> int codes [rows, 2n]; element 2m = low nibble of byte m."""
    p = np.asarray(packed, dtype=np.uint8)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    q[..., 0::2] = p & 0x0F
    q[..., 1::2] = p >> 4
    return q


def dequant(codes, s_bits, b_bits):
    """w[r, c] = s[r, c//64] * q[r, c] + b[r, c//64] in fp64 ([TF-mem], MLX affine)."""
    q = np.asarray(codes, dtype=np.float64)
    rows, cols = q.shape
    s = bf16_to_f64(s_bits).reshape(rows, cols // GROUP, 1)
    b = bf16_to_f64(b_bits).reshape(rows, cols // GROUP, 1)
    return (s * q.reshape(rows, cols // GROUP, GROUP) + b).reshape(rows, cols)


def dequant_int4(packed, s_bits, b_bits):
    return dequant(unpack_nibbles(packed), s_bits, b_bits)


def dequant_int8(codes, s_bits, b_bits):
    return dequant(np.asarray(codes, dtype=np.uint8).astype(np.int64), s_bits, b_bits)


# ------------------------------------------------------------------ router ([TF-struct])

def rmsnorm_no_scale(x, eps=EPS):
    """x / sqrt(mean_h x^2 + eps), per row, no learnable gain."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def router_logits(x_bits, layer, eps=EPS):
    """Per-expert router logits [T, E] in fp64.

    Steps of the router listing: scale-free RMS norm of the bf16 hidden state,
    multiply by router_scale / sqrt(hidden), project with the 8-bit affine
    router matrix (one row per expert), plus the optional logit bias.
    """
    x = bf16_to_f64(x_bits)
    H = x.shape[-1]
    u = rmsnorm_no_scale(x, eps)
    rs = np.ones(H) if layer.router_scale is None else np.asarray(layer.router_scale, np.float64)
    u = u * rs / np.sqrt(H)
    W = dequant_int8(layer.router_q, layer.router_s, layer.router_b)     # [E, H]
    logits = u @ W.T
    if getattr(layer, "bias", None) is not None:
        logits = logits + np.asarray(layer.bias, np.float64)
    return logits


def topk_select(logits, k):
    """Indices [T, k] of the k largest logits, by descending logit, ties to the lower index."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    out = np.empty((T, k), dtype=np.int32)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -logits[t]))          # primary: -logit, secondary: index
        out[t] = order[:k]
    return out


def topk_weights(logits, top, pes):
    """softmax over the kept logits only, then times per_expert_scale of each kept expert."""
    kept = np.take_along_axis(np.asarray(logits, np.float64), top.astype(np.int64), axis=1)
    z = np.exp(kept - kept.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    return p * np.asarray(pes, np.float64)[top]


def router(x_bits, layer, k, eps=EPS):
    """Returns (top [T,k] int32, w [T,k] fp64, logits [T,E] fp64)."""
    logits = router_logits(x_bits, layer, eps)
    top = topk_select(logits, k)
    return top, topk_weights(logits, top, layer.pes), logits


def near_tie_mask(logits, k, gap=1e-5):
    """Tokens whose k-th and (k+1)-th largest logits differ by less than ``gap``."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=1)
    if s.shape[1] <= k:
        return np.zeros(s.shape[0], dtype=bool)
    return (s[:, k - 1] - s[:, k]) < gap


# ------------------------------------------------------------------ bucketing

def bucket(top, n_experts):
    """Group the T*k assignments by expert.

    Returns counts [E], offsets [E+1] (exclusive prefix sum), sorted [T*k] (flat
    assignment ids t*k+j, experts ascending, flat id ascending within an
    expert), active [n_active] (experts with a non-zero count, ascending).
    """
    flat = np.asarray(top, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_ids = np.argsort(flat, kind="stable").astype(np.int32)
    active = np.nonzero(counts)[0].astype(np.int32)
    return counts, offsets, sorted_ids, active


# ------------------------------------------------------------------ expert FFN

def expert_ffn(x, weights, return_h=False):
    """SwiGLU expert on fp64 rows x [m, H]; weights dequantised on the fly (int4 codes, or
    int8 codes when weights.bits == 8: the MLX 8-bit group format of [SW-mem]'s runtime).

    g = x W_g^T, v = x W_u^T, h = silu(g) * v, y = h W_d^T with W = s*q + b.
    """
    x = np.asarray(x, dtype=np.float64)
    deq = dequant_int8 if getattr(weights, "bits", 4) == 8 else dequant_int4
    Wg = deq(weights.gate_q, weights.gate_s, weights.gate_b)   # [I, H]
    Wu = deq(weights.up_q, weights.up_s, weights.up_b)         # [I, H]
    Wd = deq(weights.down_q, weights.down_s, weights.down_b)   # [H, I]
    g = x @ Wg.T
    v = x @ Wu.T
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * v
    y = h @ Wd.T
    return (y, h) if return_h else y


# ------------------------------------------------------------------ combine ([TF-struct], cb2)

def combine(x_bits, y_routed, w, y_shared):
    """out_t = x_t + y_shared_t + sum_j w_tj * y_routed_tj (fp64), and its bf16 rounding.

    y_routed [T, k, H]; w [T, k]; y_shared [T, H] or None.
    """
    x = bf16_to_f64(x_bits)
    acc = np.einsum("tk,tkh->th", np.asarray(w, np.float64), np.asarray(y_routed, np.float64))
    out = x + acc
    if y_shared is not None:
        out = out + y_shared
    return out, bf16_rne_bits(out)


def post_combine(x_bits, m, gain=None, scalar=None, eps=EPS):
    """cb2's last steps on the combined branches m [T, H] (fp64): normalisation, residual,
    layer scalar, in that order ([TF-struct] cb2).

        n   = gain * m / sqrt(mean_h(m^2) + eps)     (gain None: n = m, no norm)
        out = (x + n) * scalar                       (scalar None: 1)
    Returns the fp64 result and its bf16 rounding.
    """
    x = bf16_to_f64(x_bits)
    m = np.asarray(m, np.float64)
    n = m
    if gain is not None:
        rms = np.sqrt(np.mean(m * m, axis=-1, keepdims=True) + eps)
        n = np.asarray(gain, np.float64) * (m / rms)
    out = x + n
    if scalar is not None:
        out = out * float(scalar)
    return out, bf16_rne_bits(out)


def combine_post(x_bits, y_routed, w, y_shared, gain=None, scalar=None, eps=EPS):
    """m = y_shared + sum_j w_j y_routed_j, then post_combine (fp64)."""
    m = np.einsum("tk,tkh->th", np.asarray(w, np.float64), np.asarray(y_routed, np.float64))
    if y_shared is not None:
        m = m + y_shared
    return post_combine(x_bits, m, gain, scalar, eps)


# ------------------------------------------------------------------ whole layer

def layer_forward(x_bits, layer, k, eps=EPS, top_override=None):
    """One routed MoE layer on bf16 input rows x_bits [T, H].

    ``layer`` provides router_q/s/b, router_scale, pes, bias, expert(e) and
    shared() (or None for no shared expert), and optionally post_gain [H] and
    layer_scalar for cb2's post-combine steps.  ``top_override`` replaces the
    router's selection (used to re-evaluate near-tied tokens with another
    valid selection); the weights are then recomputed from the logits.
    Returns a dict of every intermediate.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    logits = router_logits(x_bits, layer, eps)
    top = topk_select(logits, k) if top_override is None else np.asarray(top_override, np.int32)
    w = topk_weights(logits, top, layer.pes)
    E = np.asarray(layer.pes).shape[0]
    counts, offsets, sorted_ids, active = bucket(top, E)
    x = bf16_to_f64(x_bits)
    y = np.zeros((T * k, H))
    h_rows = {}
    for e in active:
        ids = sorted_ids[offsets[e]:offsets[e + 1]]
        tok = ids // k
        ye, he = expert_ffn(x[tok], layer.expert(int(e)), return_h=True)
        y[ids] = ye
        h_rows[int(e)] = he
    sh = layer.shared() if hasattr(layer, "shared") else None
    y_sh = expert_ffn(x, sh) if sh is not None else None
    gain, scalar = getattr(layer, "post_gain", None), getattr(layer, "layer_scalar", None)
    if gain is None and scalar is None:
        out64, out_bf16 = combine(x_bits, y.reshape(T, k, H), w, y_sh)
    else:
        out64, out_bf16 = combine_post(x_bits, y.reshape(T, k, H), w, y_sh, gain, scalar, eps)
    return dict(logits=logits, top=top, w=w, counts=counts, offsets=offsets, sorted=sorted_ids,
                active=active, y=y, y_shared=y_sh, h=h_rows, out=out64, out_bf16=out_bf16)
