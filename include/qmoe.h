/*
 * qmoe.h -- C ABI of the routed int4 Mixture-of-Experts layer for AMD MI355X (gfx950).
 *
 * Sources of the operations (the pages the library implements):
 *   [TF-struct] TurboFieldfare post on discuss.pytorch.kr, section "TurboFieldfare의
 *               전문가 스트리밍 구조" (expert-streaming structure): each layer has 128
 *               routed experts, 8 chosen per token, plus a shared expert added without a
 *               routing weight; the router listing (scale-free RMS norm, scaling by
 *               router_scale / sqrt(hidden), 8-bit affine projection to per-expert
 *               logits, top-8, softmax over the kept logits, times per_expert_scale);
 *               cb2 combines the routed branches by router weight with the shared branch
 *               and the residual; prompts are prefilled in chunks of at most 128 tokens,
 *               so one expert read serves every row routed to it.
 *   [TF-mem]    same post, section "TurboFieldfare가 메모리를 아끼는 방식": MLX affine
 *               4-bit weights with one bf16 scale and one bf16 bias per 64 weights; only
 *               the router projection is 8-bit.
 *   [TF-inst]   same post, section "TurboFieldfare의 스트리밍 설치 방식": quantised values
 *               are copied with a layout change only, never dequantised and requantised.
 *   [SW-mem]    Swiftlet article on tech.utomolab.com, section "같은 모델을 왜 이렇게 적은
 *               메모리로 돌릴 수 있나": routed experts stored as fixed-stride blocks so that
 *               fetching one expert is a single read; 512 experts/top-10, 256/top-8.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller, unless stated otherwise.
 *    Descriptor structs (qmoe_dims, qmoe_router, qmoe_layer) live in HOST memory and are
 *    read during the call only.  The library never allocates device memory; scratch
 *    space comes from a caller-provided device workspace (see qmoe_workspace_bytes).
 *  - Every compute call is enqueued asynchronously on the caller's hipStream_t (NULL is
 *    the default stream).  No call synchronises or copies device->host, so every call
 *    can be captured into a HIP graph.  Nothing is cleared with memset.
 *  - bf16 values travel as uint16_t bit patterns.  Matrices are row-major.
 *  - Status: every int-returning entry returns QMOE_OK (0) or a negative QMOE_ERR_*.
 *    On error nothing is enqueued and qmoe_last_error() returns a thread-local message.
 *    Arguments are validated on the host before any device call, so argument errors are
 *    reported on machines without a GPU too.
 *  - Calls keep no state between invocations (apart from the workspace contents, which
 *    belong to the call using them); calls on different streams may run concurrently if
 *    they use different workspaces and outputs.  Outputs must not alias inputs.
 *  - T = 0 (no tokens) is a valid no-op that returns QMOE_OK.
 *  - Shape limits: hidden, inter and shared_inter are multiples of 64; hidden <= 8192,
 *    inter and shared_inter <= 4096; group == 64; expert_bits 0, 4 or 8; 1 <= top_k <= min(n_experts, 32); 1 <= n_experts <= 1024;
 *    T <= 65536 per call.  Store base pointers and strides are 256-byte aligned; x and the
 *    router codes are 16-byte aligned (the kernels read them with 16-byte loads).
 *
 * Quantised formats (canonical, as the pages describe them)
 * ---------------------------------------------------------
 *  int4 matrix [R, K]: codes uint8 [R, K/2], element 2m in the LOW nibble of byte m,
 *  scale and bias bf16 [R, K/64]; value = scale[r, c/64] * code[r, c] + bias[r, c/64]
 *  with unsigned codes 0..15.  int8 router [E, H]: codes uint8 [E, H] (0..255), scale and
 *  bias bf16 [E, H/64], value = s * q + b.
 *  An expert is gate [I, H], up [I, H] and down [H, I] int4 matrices (SwiGLU:
 *  h = silu(x gate^T) * (x up^T), y = h down^T, silu(z) = z / (1 + exp(-z))).
 *  With qmoe_dims.expert_bits = 8 the expert matrices are int8 like the router (codes
 *  uint8 [R, K], MLX int8 group quantisation as in [SW-mem]'s runtime): the store then
 *  holds every 64-weight group as two 4-bit k-steps (high nibbles with scale 16*s and bias
 *  b, low nibbles with scale s and bias 0), twice the k-steps of a 4-bit block.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *qmoe_stream_t; /* the caller's hipStream_t */

enum {
    QMOE_OK = 0,
    QMOE_ERR_ARG = -1,       /* null pointer, bad enum/flag, aliasing outputs */
    QMOE_ERR_SHAPE = -2,     /* a dimension outside the limits above */
    QMOE_ERR_WORKSPACE = -3, /* workspace null or smaller than qmoe_workspace_bytes */
    QMOE_ERR_ARCH = -4,      /* current device is not gfx950 */
    QMOE_ERR_HIP = -5        /* a HIP runtime call or kernel launch failed */
};

/* Layer dimensions. group must be 64. shared_inter = 0 means the layer has no shared expert. */
typedef struct {
    int32_t hidden;        /* H */
    int32_t n_experts;     /* E */
    int32_t top_k;         /* k */
    int32_t inter;         /* I, routed expert width */
    int32_t shared_inter;  /* Is, shared expert width (0: none) */
    int32_t group;         /* 64 */
    int32_t expert_bits;   /* bits of the routed and shared expert codes: 0 or 4 (MLX int4),
                              8 (MLX int8, [SW-mem]); the router is always 8-bit */
} qmoe_dims;

/* Router weights of one layer [TF-struct] router listing, [TF-mem] 8-bit projection. */
typedef struct {
    const uint8_t *codes;            /* [E, H] uint8 codes */
    const uint16_t *scales;          /* [E, H/64] bf16 */
    const uint16_t *biases;          /* [E, H/64] bf16 */
    const float *router_scale;       /* [H] fp32 multiplier after the norm (16-byte aligned), or
                                        NULL for all ones */
    const float *per_expert_scale;   /* [E] fp32, multiplies the softmax weights */
    const float *logit_bias;         /* [E] fp32 added to the logits before top-k, or NULL */
} qmoe_router;

/* One layer: router + packed expert store (qmoe_pack_expert layout) + optional shared block. */
typedef struct {
    qmoe_dims d;
    qmoe_router r;
    const void *experts;     /* base of E blocks, block e at experts + e * expert_stride */
    size_t expert_stride;    /* >= qmoe_expert_stride(&d, d.inter), multiple of 256 */
    const void *shared;      /* one block packed with inter = shared_inter, or NULL */
    /* cb2's post-combine steps ([TF-struct] cb2: normalisation, residual, layer scalar), both
     * optional; with both NULL the layer ends at the residual add. */
    const float *post_norm_gain; /* [H] fp32 (16-byte aligned) gain of the RMS norm of the
                                    combined branches, or NULL: no norm */
    const float *layer_scalar;   /* [1] fp32 multiplier of the layer output, or NULL: 1 */
} qmoe_layer;

/* ---------------------------------------------------------------- host-only queries */

/* Library ABI version (major*10000 + minor*100 + patch): 200 = 0.2.0. */
int qmoe_version(void);

/* Thread-local text of the last error (empty string if none). Never NULL. */
const char *qmoe_last_error(void);

/* Bytes of one packed expert block of width `inter` (4 KiB-rounded), 0 on invalid dims.
 * [SW-mem]: experts are fixed-stride blocks, so expert e starts at base + e * stride. */
size_t qmoe_expert_stride(const qmoe_dims *d, int32_t inter);

/* Workspace bytes needed by qmoe_router_topk / qmoe_bucket / qmoe_expert_ffn /
 * qmoe_layer_forward for calls with up to max_tokens tokens (0 on invalid dims).  The
 * workspace is device memory owned by the caller and must be zero before its first use:
 * initialise a new workspace once with qmoe_workspace_init (or a zero fill).  Every call leaves
 * it ready for the next one (counters return to zero; the one-token path advances an epoch
 * word that tags its hand-off data), so later calls need no re-initialisation.  Calls that
 * share one workspace must be ordered (same stream, or synchronised). */
size_t qmoe_workspace_bytes(const qmoe_dims *d, int32_t max_tokens);

/* Zero the whole workspace with a kernel on `stream` (graph-capturable).  Needed once per new
 * workspace: the counters and the epoch-tagged hand-off words of the one-token path must start
 * at zero. */
int qmoe_workspace_init(void *ws, size_t ws_bytes, qmoe_stream_t stream);

/* ---------------------------------------------------------------- expert store */

/* Copy one expert from the canonical int4 (or, with d->expert_bits = 8, int8) arrays (gate/up
 * [inter, H], down [H, inter], see the formats above; all device pointers) into `dst_block` (device, qmoe_expert_stride bytes,
 * 256-byte aligned) in the store's tiled order.  Layout change only: every code, scale and
 * bias bit is copied, nothing is dequantised or requantised [TF-inst].  `inter` is d->inter
 * for a routed expert or d->shared_inter for the shared block. */
int qmoe_pack_expert(const qmoe_dims *d, int32_t inter,
                     const uint8_t *gate_q, const uint16_t *gate_s, const uint16_t *gate_b,
                     const uint8_t *up_q, const uint16_t *up_s, const uint16_t *up_b,
                     const uint8_t *down_q, const uint16_t *down_s, const uint16_t *down_b,
                     void *dst_block, qmoe_stream_t stream);

/* Exact inverse of qmoe_pack_expert: canonical arrays back from a packed block. */
int qmoe_unpack_expert(const qmoe_dims *d, int32_t inter, const void *src_block,
                       uint8_t *gate_q, uint16_t *gate_s, uint16_t *gate_b,
                       uint8_t *up_q, uint16_t *up_s, uint16_t *up_b,
                       uint8_t *down_q, uint16_t *down_s, uint16_t *down_b,
                       qmoe_stream_t stream);

/* ---------------------------------------------------------------- the four steps */

/* Step 1, router [TF-struct] router listing.  For each token t of x [T, H] (bf16):
 * (a NaN logit ranks below every number, so topk_idx always holds valid expert ids)
 *   u = x / sqrt(mean(x^2) + 1e-6) * router_scale / sqrt(H)   (fp32)
 *   logit_e = sum_h (s*q+b)[e,h] * u_h + logit_bias_e          (fp32 accumulate)
 *   topk_idx[t, :] = the k largest logits, descending; equal logits -> lower expert index
 *   topk_w[t, j] = softmax over the k kept logits, times per_expert_scale[topk_idx[t, j]]
 * Outputs: topk_idx int32 [T, k], topk_w fp32 [T, k], logits fp32 [T, E] (optional, may be
 * NULL).  ws: device workspace of qmoe_workspace_bytes(d, T) bytes.  Runs per chunk of at most
 * 128 tokens, two launches each: the logits on the matrix cores (fp32 products of
 * x*router_scale with s*q+b over tiles of 16 tokens x 16 experts, the hidden axis split over
 * workgroups), then the partial tiles summed in a fixed order, the norm factor and bias
 * applied, and the top-k selected, one wave per token. */
int qmoe_router_topk(const qmoe_dims *d, const qmoe_router *r, const uint16_t *x, int32_t T,
                     int32_t *topk_idx, float *topk_w, float *logits_or_null,
                     void *ws, size_t ws_bytes, qmoe_stream_t stream);

/* Step 2, bucketing: one expert read serves every row routed to it [TF-struct] (chunked
 * prefill).  Groups the T*k assignments (flat id f = t*k + j, expert topk_idx[f]) by expert:
 *   counts [E]      rows per expert
 *   offsets [E+1]   exclusive prefix sum of counts (offsets[E] = T*k)
 *   sorted [T*k]    flat ids grouped by ascending expert, ascending flat id within an expert
 *   active [E]      the experts with a non-zero count, ascending (first *n_active entries valid)
 *   n_active [1]    number of active experts
 * Deterministic (bit-identical across runs).  Assignments whose expert id lies outside
 * [0, E) are dropped: not counted and not listed (offsets[E] is then below T*k).  With T = 0 the outputs are still written (all counts zero) and
 * topk_idx may be NULL.  ws is not used and may be NULL. */
int qmoe_bucket(const qmoe_dims *d, const int32_t *topk_idx, int32_t T,
                int32_t *counts, int32_t *offsets, int32_t *sorted, int32_t *active,
                int32_t *n_active, void *ws, size_t ws_bytes, qmoe_stream_t stream);

/* Step 3, expert FFN over the bucketed assignments [TF-struct], weights in the packed store
 * (int4 codes decoded in registers, never written out [TF-mem]).  For every assignment f
 * (flat id, expert e = topk_idx[f], token t = f / k):
 *   y[f, :] = down_e( silu(gate_e(x_t)) * up_e(x_t) )       fp32 [T*k, H]
 * and, if the layer has a shared block and y_shared_or_null != NULL, for every token
 *   y_shared[t, :] = shared FFN of x_t                        fp32 [T, H]
 * offsets/sorted/active/n_active come from qmoe_bucket (device pointers); slots whose bucket
 * data would index outside the store or the assignment list are skipped, and their y rows are
 * left unwritten. */
int qmoe_expert_ffn(const qmoe_layer *L, const uint16_t *x, int32_t T,
                    const int32_t *offsets, const int32_t *sorted, const int32_t *active,
                    const int32_t *n_active, float *y, float *y_shared_or_null,
                    void *ws, size_t ws_bytes, qmoe_stream_t stream);

/* Step 4, combine (cb2 of [TF-struct] up to the residual add):
 *   out[t, :] = bf16_rne( x[t] + y_shared[t] + sum_j topk_w[t, j] * y[t*k + j] )
 * summed in fp32 in the order j = 0..k-1, then the shared branch, then the residual.
 * y_shared may be NULL (no shared expert); out_f32_or_null receives the fp32 sum. */
int qmoe_combine(const qmoe_dims *d, const uint16_t *x, const float *y, const float *topk_w,
                 const float *y_shared_or_null, int32_t T, uint16_t *out,
                 float *out_f32_or_null, qmoe_stream_t stream);

/* Step 4 with cb2's post-combine steps ([TF-struct] cb2, in the order listed there:
 * normalisation, residual, layer scalar):
 *   m[t, :]   = y_shared[t] + sum_j topk_w[t, j] * y[t*k + j]         (fp32, j ascending, then
 *                                                                      the shared branch)
 *   n[t, :]   = gain * m[t] / sqrt(mean(m[t]^2) + 1e-6)                (gain NULL: n = m)
 *   out[t, :] = bf16_rne( (x[t] + n[t]) * layer_scalar )               (layer_scalar NULL: 1)
 * gain: fp32 [H], 16-byte aligned; layer_scalar: fp32 [1]; both device pointers.  With both
 * NULL the result equals qmoe_combine's bit for bit. */
int qmoe_combine_post(const qmoe_dims *d, const uint16_t *x, const float *y, const float *topk_w,
                      const float *y_shared_or_null, const float *post_norm_gain_or_null,
                      const float *layer_scalar_or_null, int32_t T, uint16_t *out,
                      float *out_f32_or_null, qmoe_stream_t stream);

/* The whole layer (steps 1-4, plus the layer's post-combine steps when it carries them) with
 * no host round trip.  A one-token call runs as a single launch whose workgroups take the
 * roles router, shared gate/up, routed gate/up, shared down and routed down, handing data to
 * each other through the workspace (each role starts loading its weights as soon as it knows
 * them); the routed-down workgroups of the last slot combine.  Larger calls run per chunk of
 * at most 128 tokens as five launches:
 *   kernels 1-2: router logits (as qmoe_router_topk) and the 64-column group sums of x, then
 *             top-k, softmax and (last workgroup) bucketing into a table of 16-row blocks;
 *   kernel 3: routed and shared gate/up projection + SwiGLU on the matrix cores;
 *   kernel 4: routed and shared down projection on the matrix cores;
 *   kernel 5: combine (qmoe_combine / qmoe_combine_post arithmetic).
 * out: bf16 [T, H]; out_f32_or_null: fp32 [T, H]; topk_idx_or_null / topk_w_or_null receive
 * the routing ([T, k]).  Results equal qmoe_router_topk -> qmoe_bucket -> qmoe_expert_ffn ->
 * qmoe_combine_post up to fp32 summation order.  T may exceed 128; callers that follow the
 * pages' chunked prefill pass chunks of at most 128 tokens. */
int qmoe_layer_forward(const qmoe_layer *L, const uint16_t *x, int32_t T, uint16_t *out,
                       float *out_f32_or_null, int32_t *topk_idx_or_null,
                       float *topk_w_or_null, void *ws, size_t ws_bytes,
                       qmoe_stream_t stream);

/* qmoe_layer_forward without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, arithmetic and results (bit for bit) as qmoe_layer_forward; the workspace is a
 * fixed 32 MiB device array inside the library, one per GPU it runs on, held until the process
 * ends (zero when the library is loaded, left ready for the next call by every call).  Calls no
 * allocator.  Fails with QMOE_ERR_WORKSPACE, before enqueueing anything, when the shape needs
 * more scratch than that (qmoe_workspace_bytes(&L->d, min(T, 128)) > 32 MiB; every shape of
 * this library's configured models needs at most about 18 MiB).  All calls on one GPU share
 * that GPU's array: calls that overlap on one GPU (different streams or threads, not ordered)
 * race and must not be issued; calls ordered on one stream are fine. */
int qmoe_layer_forward_noalloc(const qmoe_layer *L, const uint16_t *x, int32_t T, uint16_t *out,
                               float *out_f32_or_null, int32_t *topk_idx_or_null,
                               float *topk_w_or_null, qmoe_stream_t stream);

/* ---------------------------------------------------------------- chained one-token layers */

#define QMOE_MAX_STACK 64

/* One token through n_layers layers in one launch, each layer's input being the bf16 output of
 * the one before: x_0 = x, x_{l+1} = out[l].  The per-layer arithmetic is that of a one-token
 * qmoe_layer_forward call (results equal n_layers such calls chained, bit for bit); the chain
 * overlaps the layers' phases as the pages' decode loop does ([TF-struct]: the next layer's
 * resident work starts while the current one's routed work is still running): workgroups of
 * layer l + 1 start loading their weights while layer l runs and wait only for its output.
 *   layers: host array of n_layers descriptors (read during the call), all with the same dims
 *           and either all or none with a shared block; the one-token launch must fit the
 *           shape (routed inter and bits as for qmoe_layer_forward's single launch, else
 *           QMOE_ERR_SHAPE).  n_layers in [0, QMOE_MAX_STACK]; 0 is a no-op.
 *   x: bf16 [H] device; out: bf16 [n_layers, H] device (every layer's output; the last row is
 *   the chain's result); out_f32_or_null: fp32 [n_layers, H]; topk_idx_or_null /
 *   topk_w_or_null: [n_layers, k], both or neither.
 *   ws: a workspace for one token (qmoe_workspace_bytes(d, >= 1)); calls that share it must
 *   run on one stream in order, as for qmoe_layer_forward.
 * Capturable in a graph (the per-layer table is written by kernels whose arguments carry it). */
int qmoe_decode_stack(const qmoe_layer *layers, int32_t n_layers, const uint16_t *x,
                      uint16_t *out, float *out_f32_or_null, int32_t *topk_idx_or_null,
                      float *topk_w_or_null, void *ws, size_t ws_bytes, qmoe_stream_t stream);

/* ---------------------------------------------------------------- tiered expert residency */

/* For layers whose routed experts do not all stay in device memory: the experts live in host
 * memory in the store's block layout (the cold tier; the pages keep them on SSD and read one
 * fixed-stride block per expert [TF-struct] io phase, [SW-mem]), and `slots` device blocks
 * cache the ones in use, replaced LFU with recency as the pages describe: a hit adds one use
 * and refreshes the last use; a miss takes an empty slot, else the slot not used by the same
 * call with the fewest uses, then the oldest last use, then the lowest index, and starts at one
 * use.  Counts belong to the slot (no ageing). */
typedef struct qmoe_expert_cache qmoe_expert_cache;

/* host_store: host memory (pinned for full copy speed) with expert e's block at
 * host_store + e * host_stride; device_slots: device memory with slot s at
 * device_slots + s * slot_stride.  Both strides >= qmoe_expert_stride(d, d->inter) and multiples
 * of 256; slots in [top_k, n_experts].  The cache object is host memory owned by the library
 * (the pointers are kept, nothing is touched until a forward call). */
int qmoe_cache_create(const qmoe_dims *d, const void *host_store, size_t host_stride,
                      void *device_slots, size_t slot_stride, int32_t slots,
                      qmoe_expert_cache **cache_out);
int qmoe_cache_destroy(qmoe_expert_cache *cache);

/* Host only: the cache's decision for one call naming the expert ids ids[0..n) -- the slot of
 * every id (slot_of_out[n]) and the blocks to copy (fill_expert_out / fill_slot_out, at most
 * `slots` entries, count in *n_fills_out).  Updates the cache state exactly as a forward call
 * does.  Fails (QMOE_ERR_ARG) on an id outside [0, E) or more distinct ids than slots. */
int qmoe_cache_plan(qmoe_expert_cache *cache, const int32_t *ids, int32_t n, int32_t *slot_of_out,
                    int32_t *fill_expert_out, int32_t *fill_slot_out, int32_t *n_fills_out);

/* Lookups so far (hits + misses = distinct experts per call, summed over calls). */
int qmoe_cache_stats(const qmoe_expert_cache *cache, int64_t *hits_out, int64_t *misses_out);

/* The layer with its routed experts streamed through the cache, per chunk of at most 128
 * tokens: router and top-k on the GPU; the ids copied to the host (the one synchronisation of
 * `stream`, where the pages' CPU reads the router's choice); the cache plan; one host-to-device
 * copy per missing expert block, on two copy streams of the cache's own; the slot ids copied
 * back; bucketing; the expert FFN of the shared block (L->shared) and of the experts already in
 * their slots on `stream` while the copies run, then, once the copies have landed, the FFN of
 * the refilled slots (the pages overlap the expert reads with the shared and cached experts'
 * work: TurboFieldfare post, section "TurboFieldfare의 전문가 스트리밍 구조"); combine (with
 * L's post-combine steps if set) as in qmoe_layer_forward.  L->experts and L->expert_stride are
 * not used.  The chunk's distinct experts must fit in the slots.  The cache's copy streams and
 * pinned staging are made on the device current at the first forward call; later calls on
 * another device fail (QMOE_ERR_ARG).  Not for use under graph capture.  Results equal
 * qmoe_router_topk -> qmoe_bucket -> qmoe_expert_ffn -> qmoe_combine_post on a resident store
 * bit for bit. */
int qmoe_layer_forward_tiered(const qmoe_layer *L, qmoe_expert_cache *cache, const uint16_t *x,
                              int32_t T, uint16_t *out, float *out_f32_or_null,
                              int32_t *topk_idx_or_null, float *topk_w_or_null, void *ws,
                              size_t ws_bytes, qmoe_stream_t stream);

/* Diagnostic: copy the workspace's status word to *status_out (0 = no fault; 1 = a one-token
 * layer call gave up waiting for another workgroup, so its results are not valid).
 * Synchronises `stream`; not for use under graph capture. */
int qmoe_workspace_status(const void *ws, size_t ws_bytes, int32_t *status_out,
                          qmoe_stream_t stream);

/* ---------------------------------------------------------------- timing helpers */

/* Thin wrappers over HIP events so that callers can time individual kernels of
 * qmoe_layer_forward on the stream they run on.  qmoe_set_profile_events(start, stop)
 * makes subsequent qmoe_layer_forward calls on this thread record `start` (if not NULL) right
 * before and `stop` (if not NULL) right after their dominant kernel: the single kernel of a
 * one-token call, else the routed gate/up kernel (pass NULL, NULL to stop).  Under stream
 * capture the records become graph event nodes.  Events are created with qmoe_event_create
 * and read with qmoe_event_elapsed_ms (which synchronises on `stop`). */
int qmoe_event_create(void **event_out);
int qmoe_event_destroy(void *event);
int qmoe_event_record(void *event, qmoe_stream_t stream);
int qmoe_event_elapsed_ms(void *start, void *stop, float *ms_out);
int qmoe_set_profile_events(void *start, void *stop);

/* ---------------------------------------------------------------- measurement reference */

/* A plain streaming read, the achievable-bandwidth reference against which the layer's weight
 * streams are measured: reads the first `bytes` bytes of each of the n blocks
 * base + ids[i] * stride (the access shape of fetching n experts of the fixed-stride store
 * [SW-mem]) with 16-byte non-temporal loads, each wave a contiguous 16 KiB chunk, and writes one
 * word per wave to sink (device, at least n * ceil(bytes / 16384) words; its values mean
 * nothing).  ids: HOST array of n block ids (n <= 64); base device, 16-byte aligned; stride
 * and bytes multiples of 16.  The caller keeps every block inside its allocation.
 * Asynchronous on `stream`. */
int qmoe_read_blocks(const void *base, size_t stride, const int32_t *ids, int32_t n, size_t bytes,
                     uint32_t *sink, qmoe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
