// Host side of the qmoe C ABI: argument validation, workspace layout and kernel launches.
// Every entry point validates its arguments on the host before touching the device, returns
// a status code and never lets a C++ exception cross the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "qmoe.h"
#include "common.h"
#include "store.h"
#include "router.h"
#include "ffn.h"
#include "decode.h"
#include "router_mf.h"
#include "cache.h"
#include "diag.h"

using namespace qmoe;

namespace {

constexpr int VERSION = 200;               // 0.2.0
constexpr size_t COUNTER_BYTES = 512 * 1024;
constexpr int GU_W = 8;     // waves per routed gate/up workgroup (split-K)
constexpr int D_W = 8;      // waves per down workgroup (split-K)
constexpr int KB = 12;      // k-steps loaded per batch by a wave
constexpr int DEC_SYNC_WORD = 32768;       // first word of the one-token decode sync area
constexpr int MAX_T = 65536;

thread_local std::string g_err;
#ifdef QMOE_TIMELINE
thread_local unsigned long long *g_tl = nullptr;   // phase timestamps of the next one-token call
#endif
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return QMOE_OK;
}

#define QMOE_HIP(call)                                                                  \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) return fail(QMOE_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define QMOE_LAUNCHED()                                                                 \
  do {                                                                                  \
    hipError_t e_ = hipGetLastError();                                                  \
    if (e_ != hipSuccess) return fail(QMOE_ERR_HIP, "kernel launch: %s", hipGetErrorString(e_)); \
  } while (0)

inline bool mult64(int v) { return v > 0 && v % 64 == 0; }

int check_dims(const qmoe_dims *d) {
  if (!d) return fail(QMOE_ERR_ARG, "dims is NULL");
  if (d->group != GROUP) return fail(QMOE_ERR_SHAPE, "group must be 64 (got %d)", d->group);
  if (!mult64(d->hidden) || d->hidden > 8192)
    return fail(QMOE_ERR_SHAPE, "hidden must be a positive multiple of 64 <= 8192 (got %d)", d->hidden);
  if (!mult64(d->inter) || d->inter > 4096)
    return fail(QMOE_ERR_SHAPE, "inter must be a positive multiple of 64 <= 4096 (got %d)", d->inter);
  if (d->shared_inter != 0 && (!mult64(d->shared_inter) || d->shared_inter > 4096))
    return fail(QMOE_ERR_SHAPE, "shared_inter must be 0 or a multiple of 64 <= 4096 (got %d)",
                d->shared_inter);
  if (d->n_experts < 1 || d->n_experts > MAX_EXPERTS)
    return fail(QMOE_ERR_SHAPE, "n_experts must be in [1, %d] (got %d)", MAX_EXPERTS, d->n_experts);
  if (d->top_k < 1 || d->top_k > MAX_TOPK || d->top_k > d->n_experts)
    return fail(QMOE_ERR_SHAPE, "top_k must be in [1, min(n_experts, 32)] (got %d)", d->top_k);
  if (d->expert_bits != 0 && d->expert_bits != 4 && d->expert_bits != 8)
    return fail(QMOE_ERR_SHAPE, "expert_bits must be 0 or 4 (4-bit) or 8 (got %d)", d->expert_bits);
  return QMOE_OK;
}

// k-steps per quantisation group of the expert store: 1 for 4-bit experts, 2 for 8-bit ones
inline int kshift_of(const qmoe_dims *d) { return d->expert_bits == 8 ? 1 : 0; }

int check_T(int32_t T) {
  if (T < 0 || T > MAX_T) return fail(QMOE_ERR_SHAPE, "T must be in [0, %d] (got %d)", MAX_T, T);
  return QMOE_OK;
}

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Current device must be gfx950.  Cached per device ordinal.
int check_arch() {
  static std::mutex mu;
  static int state[64] = {0};  // 0 unknown, 1 ok, 2 bad
  int dev = 0;
  QMOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(QMOE_ERR_ARCH, "device ordinal %d out of range", dev);
  {
    std::lock_guard<std::mutex> lk(mu);
    if (state[dev] == 0) {
      hipDeviceProp_t prop;
      hipError_t e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return fail(QMOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
      state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
      if (state[dev] == 2)
        return fail(QMOE_ERR_ARCH, "device %d is %s, this library is built for gfx950", dev,
                    prop.gcnArchName);
    }
  }
  if (state[dev] != 1) return fail(QMOE_ERR_ARCH, "device %d is not gfx950", dev);
  return QMOE_OK;
}

inline size_t al(size_t v) { return (v + 255) & ~(size_t)255; }

// Down-projection workgroups per output tile for the shared block in the layer path: the
// shared width is cut into chunks about as wide as a routed expert, so that every workgroup
// of the launch has a similar amount of work.
inline int shared_chunks(const qmoe_dims *d) {
  if (d->shared_inter == 0) return 0;
  const int ks = d->shared_inter / GROUP;
  const int c = (d->shared_inter + d->inter / 2) / d->inter;
  return std::max(1, std::min(c, ks));
}

// The same for the one-token decode launch, whose shared down workgroups split one output
// tile's k-steps over their four waves (at most DEC_W * KB_DEC k-steps per chunk).
inline int dec_shared_chunks(const qmoe_dims *d) {
  if (d->shared_inter == 0) return 0;
  const int groups = d->shared_inter / GROUP, per = (DEC_W * KB_DEC) >> kshift_of(d);
  return (groups + per - 1) / per;
}

struct WsLayout {
  size_t cnt, logits, tidx, tw, counts, offsets, sorted, active, nact, slot_tab;
  size_t hr_hi, hr_lo, hs_hi, hs_lo, y, ysh, gx, ghr, ghs, slot_ids;
  size_t dec_logits, dec_hr, dec_hsh, dec_yr, dec_ysh, dec_nrm, dec_tk, dec_x, dec_tab, rpart, rss,
      total = 0;
  // every region in order, for the bounds checks of the debug build
  struct Region {
    const char *name;
    size_t off, bytes;
  };
  static constexpr int MAX_REGIONS = 32;
  Region reg[MAX_REGIONS];
  int n_reg = 0;
  size_t put(const char *name, size_t bytes) {
    QMOE_BOUNDS(n_reg < MAX_REGIONS && bytes % 256 == 0);
    reg[n_reg++] = Region{name, total, bytes};
    total += bytes;
    return total - bytes;
  }
  // bytes of the region that starts at off (empty regions share their offset with the next
  // one; 0: no region of any size starts there)
  size_t bytes_at(size_t off) const {
    size_t b = 0;
    for (int i = 0; i < n_reg; ++i)
      if (reg[i].off == off) b += reg[i].bytes;
    return b;
  }
};

WsLayout ws_layout(const qmoe_dims *d, int Tmax) {
  WsLayout w;
  const size_t T = (size_t)Tmax, k = d->top_k, E = d->n_experts, H = d->hidden;
  const size_t Tc = std::min<size_t>(T, CHUNK_TOKENS);
  w.cnt = w.put("cnt", COUNTER_BYTES);
  // The one-token path's tagged hand-off areas come first, at offsets that do not depend on
  // the token count: a workspace sized for a chunk may serve one-token calls too, and no
  // multi-token call ever writes into these areas (a stale word there can only be an older
  // one-token call's, whose tag is an older epoch).
  w.dec_logits = w.put("dec_logits", (size_t)LOGIT_COPIES * dec_copy_stride(E));
  w.dec_hr = w.put("dec_hr", (size_t)H_COPIES * dec_copy_stride(k * d->inter));
  w.dec_hsh = w.put("dec_hsh", (size_t)H_COPIES * dec_copy_stride((size_t)d->shared_inter));
  w.dec_yr = w.put("dec_yr", al((k - 1) * H * 8));
  w.dec_ysh = w.put("dec_ysh", al((size_t)dec_shared_chunks(d) * H * 8));
  w.dec_nrm = w.put("dec_nrm", al((H / TILE_ROWS) * 8));
  w.dec_tk = w.put("dec_tk", al((size_t)TK_COPIES * 2 * MAX_TOPK * 8));
  w.dec_x = w.put("dec_x", 2 * (size_t)X_COPIES * dec_x_copy_bytes((int)H));
  w.dec_tab = w.put("dec_tab", al((size_t)MAX_STACK * sizeof(DecLayer)));
  w.logits = w.put("logits", al(T * E * 4));
  w.tidx = w.put("tidx", al(T * k * 4));
  w.tw = w.put("tw", al(T * k * 4));
  w.counts = w.put("counts", al(E * 4));
  w.offsets = w.put("offsets", al((E + 1) * 4));
  w.sorted = w.put("sorted", al(T * k * 4));
  w.active = w.put("active", al(E * 4));
  w.nact = w.put("nact", al(4));
  w.slot_tab = w.put("slot_tab", al((size_t)bucket_max_blocks((int)(Tc * k), (int)E) * 16));
  w.slot_ids = w.put("slot_ids", al(Tc * k * 4));
  w.hr_hi = w.put("hr_hi", al(T * k * d->inter * 2));
  w.hr_lo = w.put("hr_lo", al(T * k * d->inter * 2));
  w.hs_hi = w.put("hs_hi", al(T * (size_t)d->shared_inter * 2));
  w.hs_lo = w.put("hs_lo", al(T * (size_t)d->shared_inter * 2));
  w.y = w.put("y", al(Tc * k * H * 4));
  w.ysh = w.put("ysh", al(Tc * H * 4));
  w.gx = w.put("gx", al(T * (H / GROUP) * 4));
  w.ghr = w.put("ghr", al(T * k * (size_t)(d->inter / GROUP) * 4));
  w.ghs = w.put("ghs", al(T * (size_t)(d->shared_inter / GROUP) * 4));
  w.rpart = w.put("rpart", al((size_t)rmf_splits((int)H) * Tc * E * 4));   // router partial tiles
  w.rss = w.put("rss", al((size_t)rmf_splits((int)H) * Tc * 4));         // and sums of x^2
  return w;
}

template <class T>
inline T *at(void *ws, size_t off) { return (T *)((char *)ws + off); }

int check_ws(const qmoe_dims *d, int T, void *ws, size_t ws_bytes) {
  if (!ws) return fail(QMOE_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(QMOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const size_t need = ws_layout(d, T).total;
  if (ws_bytes < need)
    return fail(QMOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed for T=%d", ws_bytes, need, T);
  return QMOE_OK;
}

int check_router(const qmoe_router *r) {
  if (!r || !r->codes || !r->scales || !r->biases || !r->per_expert_scale)
    return fail(QMOE_ERR_ARG, "router codes/scales/biases/per_expert_scale must not be NULL");
  if (!aligned(r->codes, 16)) return fail(QMOE_ERR_ARG, "router codes must be 16-byte aligned");
  if (r->router_scale && !aligned(r->router_scale, 16))
    return fail(QMOE_ERR_ARG, "router_scale must be 16-byte aligned");
  return QMOE_OK;
}

int check_layer(const qmoe_layer *L) {
  if (!L) return fail(QMOE_ERR_ARG, "layer is NULL");
  int rc = check_dims(&L->d);
  if (rc || (rc = check_router(&L->r))) return rc;
  if (!L->experts) return fail(QMOE_ERR_ARG, "expert store is NULL");
  if (!aligned(L->experts, 256) || L->expert_stride % 256)
    return fail(QMOE_ERR_ARG, "expert store base and stride must be 256-byte aligned");
  if (L->expert_stride < block_stride_bytes(L->d.hidden, L->d.inter, kshift_of(&L->d)))
    return fail(QMOE_ERR_ARG, "expert_stride %zu smaller than the packed block (%zu)",
                L->expert_stride, block_stride_bytes(L->d.hidden, L->d.inter, kshift_of(&L->d)));
  if (L->shared && L->d.shared_inter == 0)
    return fail(QMOE_ERR_ARG, "shared block given but shared_inter is 0");
  if (L->shared && !aligned(L->shared, 256))
    return fail(QMOE_ERR_ARG, "shared block must be 256-byte aligned");
  if (L->post_norm_gain && !aligned(L->post_norm_gain, 16))
    return fail(QMOE_ERR_ARG, "post_norm_gain must be 16-byte aligned");
  return QMOE_OK;
}

// Raise a kernel's dynamic LDS limit once per (device, kernel) to the largest size used.
template <class K>
int set_lds(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return QMOE_OK;
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, size_t> done;
  int dev = 0;
  QMOE_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(mu);
  size_t &have = done[{dev, (const void *)kernel}];
  if (bytes <= have) return QMOE_OK;
  hipError_t e = hipFuncSetAttribute((const void *)kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess)
    return fail(QMOE_ERR_HIP, "hipFuncSetAttribute(lds=%zu): %s", bytes, hipGetErrorString(e));
  have = bytes;
  return QMOE_OK;
}

// dynamic LDS of the top-k / bucketing launch
size_t router_smem(const qmoe_dims *d, int T) {
  return bucket_lds_bytes(T * d->top_k, d->n_experts);
}

RouterArgs make_router_args(const qmoe_dims *d, const qmoe_router *r, const uint16_t *x, int T,
                            float *logits, int32_t *idx, float *w, void *ws) {
  RouterArgs a;
  memset(&a, 0, sizeof a);
  a.x = x; a.rq = r->codes; a.rs = r->scales; a.rb = r->biases;
  a.rscale = r->router_scale; a.pes = r->per_expert_scale; a.lbias = r->logit_bias;
  a.T = T; a.H = d->hidden; a.E = d->n_experts; a.k = d->top_k;
  a.inv_sqrt_h = (float)(1.0 / std::sqrt((double)d->hidden));
  a.logits = logits; a.topk_idx = idx; a.topk_w = w;
  const WsLayout wl = ws_layout(d, T);
  a.cnt_all = at<unsigned>(ws, wl.cnt);
  return a;
}

// Router of a call of T tokens (router_mf.h): logits on the matrix cores, then top-k (and, with
// a.counts set, bucketing) in a second launch.
// (a.T <= CHUNK_TOKENS: the partial tiles live in the workspace regions rpart / rss)
int launch_router(const RouterArgs &a, size_t smem, void *ws, const WsLayout &wl, hipStream_t s) {
  float *part = at<float>(ws, wl.rpart), *ssq = at<float>(ws, wl.rss);
  const unsigned nb = (unsigned)(((a.T + RMF_ROWS - 1) / RMF_ROWS) *
                                 ((a.E + RMF_COLS - 1) / RMF_COLS) * rmf_splits(a.H));
  hipLaunchKernelGGL(router_mf_kernel, dim3(nb), dim3(RMF_THREADS), 0, s, a, part, ssq);
  QMOE_LAUNCHED();
  if (!a.counts) smem = 0;
  int rc = set_lds(router_topk_kernel, smem);
  if (rc) return rc;
  hipLaunchKernelGGL(router_topk_kernel, dim3((unsigned)((a.T + ROUTER_WAVES - 1) / ROUTER_WAVES)),
                     dim3(ROUTER_THREADS), smem, s, a, (const float *)part, (const float *)ssq);
  QMOE_LAUNCHED();
  return QMOE_OK;
}

static_assert(BUCKET_BLOCK_ROWS == PF_MT, "one matrix-core pass per bucket block");
static_assert((long)MAX_T * MAX_TOPK <= BUCKET_MAX_N, "bucket scan fields hold every call");
static_assert((size_t)(DEC_SYNC_WORD + SY_LINES * SY_LINE) * 4 <= COUNTER_BYTES,
              "decode sync area inside the counter area");

// Record an event; under stream capture it is added as an event-record node of the graph
// after the captured work so far, and later captured work depends on it.
int record_event(hipEvent_t e, hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  QMOE_HIP(hipStreamIsCapturing(s, &st));
  if (st != hipStreamCaptureStatusActive) {
    QMOE_HIP(hipEventRecord(e, s));
    return QMOE_OK;
  }
  hipGraph_t g = nullptr;
  const hipGraphNode_t *deps = nullptr;
  size_t ndeps = 0;
  QMOE_HIP(hipStreamGetCaptureInfo_v2(s, &st, nullptr, &g, &deps, &ndeps));
  hipGraphNode_t node;
  QMOE_HIP(hipGraphAddEventRecordNode(&node, g, deps, ndeps, e));
  QMOE_HIP(hipStreamUpdateCaptureDependencies(s, &node, 1, hipStreamSetCaptureDependencies));
  return QMOE_OK;
}


static FfnArgs make_ffn_args(const qmoe_layer *L, const uint16_t *x, int T, const int32_t *offsets,
                             const int32_t *sorted, const int32_t *active, const int32_t *n_active,
                             float *y, float *y_sh, void *ws, int Tws) {
  FfnArgs a;
  memset(&a, 0, sizeof a);
  const WsLayout wl = ws_layout(&L->d, Tws);
  a.experts = (const uint8_t *)L->experts;
  a.stride = L->expert_stride;
  a.shared = (const uint8_t *)L->shared;
  a.H = L->d.hidden; a.I = L->d.inter; a.Is = L->d.shared_inter; a.k = L->d.top_k; a.T = T;
  a.n_experts = L->d.n_experts;
  a.x = x;
  a.offsets = offsets; a.sorted = sorted; a.active = active; a.n_active = n_active;
  a.n_slots = std::min(L->d.n_experts, T * L->d.top_k);
  a.kshift = kshift_of(&L->d);
  a.hr_hi = at<uint16_t>(ws, wl.hr_hi); a.hr_lo = at<uint16_t>(ws, wl.hr_lo);
  a.hs_hi = at<uint16_t>(ws, wl.hs_hi); a.hs_lo = at<uint16_t>(ws, wl.hs_lo);
  a.y = y; a.y_sh = y_sh;
  a.gx = at<float>(ws, wl.gx);
  a.gh_r = at<float>(ws, wl.ghr);
  a.gh_s = at<float>(ws, wl.ghs);
  a.n_sh_chunks = 1;
  return a;
}

template <int MB>
static int launch_gu_t(const FfnArgs &a, int n, hipStream_t s) {
  const size_t smem = gu_lds_bytes<GU_W, MB>(a.H);
  int rc = set_lds(gu_kernel<GU_W, MB, KB>, smem);
  if (rc) return rc;
  hipLaunchKernelGGL((gu_kernel<GU_W, MB, KB>), dim3(n), dim3(GU_W * WAVE), smem, s, a);
  QMOE_LAUNCHED();
  return QMOE_OK;
}

// routed tiles, plus the shared block's tiles when a.shared and a.y_sh are set
static int launch_gu(FfnArgs a, hipStream_t s) {
  const int tiles_r = a.I / 16;
  const bool sh = a.shared && a.y_sh;
  const int n = a.n_slots * tiles_r + (sh ? a.Is / 16 : 0);
  if (!sh) a.shared = nullptr;
  if (n == 0) return QMOE_OK;
  return launch_gu_t<1>(a, n, s);
}

template <int MB>
static int launch_d_t(const FfnArgs &a, int slots, int Kc, hipStream_t s) {
  const size_t smem = d_lds_bytes<D_W, MB>(Kc);
  int rc = set_lds(d_kernel<D_W, MB, KB>, smem);
  if (rc) return rc;
  hipLaunchKernelGGL((d_kernel<D_W, MB, KB>), dim3(a.H / TILE_ROWS, slots), dim3(D_W * WAVE),
                     smem, s, a);
  QMOE_LAUNCHED();
  return QMOE_OK;
}

// Down projection: routed slots plus a.n_sh_chunks shared chunks when with_shared.  The LDS
// holds the h columns of the widest workgroup.
static int launch_d(FfnArgs a, bool with_shared, hipStream_t s) {
  if (!with_shared) a.shared = nullptr;
  const int slots = a.n_slots + (with_shared ? a.n_sh_chunks : 0);
  if (slots == 0) return QMOE_OK;
  int Kc = a.I;
  if (with_shared) {
    const int KSs = a.Is / GROUP;
    Kc = std::max(Kc, GROUP * ((KSs + a.n_sh_chunks - 1) / a.n_sh_chunks));
  }
  return launch_d_t<1>(a, slots, Kc, s);
}

// Matrix-core grouped GEMM (mfma.h): gate/up then down.  Routed rows go to a.y, shared rows
// (if a.shared) to a.y_sh; a.gx must hold the group sums of x.  Profile events (if set)
// bracket the gate/up kernel.
static int launch_pf(const FfnArgs &a, hipStream_t s) {
  int rc;
  const int ntb = (a.T + PF_MT - 1) / PF_MT;
  const int n_gu = (a.shared ? pf_xcd_blocks(a.Is / GROUP, ntb) : 0) + a.n_slots * (a.I / GROUP);
  if (g_prof_start && (rc = record_event(g_prof_start, s))) return rc;
  if (n_gu > 0) {
    hipLaunchKernelGGL(gu_pf_kernel, dim3(n_gu), dim3(GU_WAVES * WAVE), 0, s, a);
    QMOE_LAUNCHED();
  }
  if (g_prof_stop && (rc = record_event(g_prof_stop, s))) return rc;
  const int tgroups = (a.H / TILE_ROWS + D_WAVES * D_NT - 1) / (D_WAVES * D_NT);
  const int n_d = (a.shared ? pf_xcd_blocks(tgroups, ntb) : 0) + pf_xcd_blocks(a.n_slots, tgroups);
  if (n_d > 0) {
    hipLaunchKernelGGL(d_pf_kernel, dim3(n_d), dim3(D_WAVES * WAVE), 0, s, a);
    QMOE_LAUNCHED();
  }
  return QMOE_OK;
}

// Chunks with fewer tokens than this take the VALU kernels (ffn.h), which stage one activation
// row: the matrix-core blocks would be mostly padding rows.
constexpr int PF_MIN_TOKENS = 2;
static bool valu_ffn(int T) { return T < PF_MIN_TOKENS; }
static_assert(PF_MIN_TOKENS == 2, "the VALU launchers are instantiated for one row only");

static int launch_gsum(const uint16_t *x, int T, int H, float *g, hipStream_t s) {
  const int n = T * (H / GROUP);
  hipLaunchKernelGGL(gsum_kernel, dim3((n + 255) / 256), dim3(256), 0, s, x, n, g);
  QMOE_LAUNCHED();
  return QMOE_OK;
}

static int launch_combine_post(const uint16_t *x, const float *y, const float *w,
                               const float *y_sh, const float *gain, const float *scalar, int T,
                               int H, int k, uint16_t *out, float *out_f32, hipStream_t s) {
  hipLaunchKernelGGL(combine_post_kernel, dim3(T), dim3(POST_THREADS), 0, s, x, y, w, y_sh, gain,
                     scalar, H, k, out, out_f32);
  QMOE_LAUNCHED();
  return QMOE_OK;
}

static int launch_combine_pf(const uint16_t *x, const float *y, const float *w, const float *y_sh,
                             int T, int H, int k, uint16_t *out, float *out_f32, hipStream_t s) {
  const size_t n4 = (size_t)T * H / 4;
  const unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(combine_pf_kernel, dim3(blocks), dim3(256), 0, s, x, y, w, y_sh, T, H, k,
                     out, out_f32);
  QMOE_LAUNCHED();
  return QMOE_OK;
}

// One-token decode in a single launch (decode.h) when every down-projection wave's k-steps
// fit in its register batch.  Routed down tiles take 1, 2 or 4 waves (wpt): the fewest that
// give each wave at most KB_DEC / 2 k-steps (the dot products of a wave are a serial chain on
// the critical path), else the fewest that fit KB_DEC; the shared down width is cut into
// chunks of at most DEC_W * KB_DEC k-steps.
static int dec_wpt(const qmoe_dims *d) {
  const int ks = (d->inter / GROUP) << kshift_of(d);
  for (int lim : {KB_DEC / 2, KB_DEC})
    for (int w = 1; w <= DEC_W; w *= 2)
      if ((ks + w - 1) / w <= lim) return w;
  return 0;
}

static bool decode_fits(const qmoe_dims *d) {
  return dec_wpt(d) > 0 && d->top_k <= MAX_TOPK && d->n_experts <= MAX_EXPERTS;
}

static DecLds dec_lds_of(const qmoe_dims *d, bool sh) {
  const int nc = sh ? dec_shared_chunks(d) : 0;
  const int kc = sh ? GROUP * ((d->shared_inter / GROUP + nc - 1) / nc) : 0;
  return dec_lds(d->hidden, d->n_experts, d->top_k, d->inter, kc, nc, dec_wpt(d));
}

static DecodeArgs make_decode_args(const qmoe_layer *L, const uint16_t *x, uint16_t *out,
                                   float *out_f32, int32_t *idx, float *w, void *ws,
                                   const WsLayout &wl) {
  const qmoe_dims *d = &L->d;
  const bool sh = L->shared != nullptr;
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.x = x; a.rq = L->r.codes; a.rs = L->r.scales; a.rb = L->r.biases;
  a.rscale = L->r.router_scale; a.pes = L->r.per_expert_scale; a.lbias = L->r.logit_bias;
  a.experts = (const uint8_t *)L->experts; a.stride = L->expert_stride;
  a.shared = sh ? (const uint8_t *)L->shared : nullptr;
  a.H = d->hidden; a.E = d->n_experts; a.k = d->top_k; a.I = d->inter;
  a.kshift = kshift_of(d);
  a.Is = sh ? d->shared_inter : 0;
  a.nc = sh ? dec_shared_chunks(d) : 0;
  a.wpt = dec_wpt(d);
  a.inv_sqrt_h = (float)(1.0 / std::sqrt((double)d->hidden));
  a.sync = at<unsigned>(ws, wl.cnt) + DEC_SYNC_WORD;
  a.logits = at<uint64_t>(ws, wl.dec_logits);
  a.logit_copy = dec_copy_stride(a.E) / 8;
  a.h_r = at<uint64_t>(ws, wl.dec_hr);
  a.hr_copy = dec_copy_stride((size_t)a.k * a.I) / 8;
  a.h_sh = at<uint64_t>(ws, wl.dec_hsh);
  a.hsh_copy = dec_copy_stride((size_t)a.Is) / 8;
  a.y_r = at<uint64_t>(ws, wl.dec_yr);
  a.y_sh = at<uint64_t>(ws, wl.dec_ysh);
  a.topk_idx = idx; a.topk_w = w; a.out = out; a.out_f32 = out_f32;
  a.gain = L->post_norm_gain; a.lscale = L->layer_scalar;
  a.nrm = at<uint64_t>(ws, wl.dec_nrm);
  a.tk = at<uint64_t>(ws, wl.dec_tk);
  const int tiles_d = a.H / TILE_ROWS, tpw = dec_tiles_per_wg(a.wpt);
  a.nR = (a.E + ROUTER_WAVES - 1) / ROUTER_WAVES;   // one expert per wave
  a.nSG = sh ? a.Is / 16 : 0;
  a.nRG = a.k * (a.I / 16);
  a.nSD = sh ? tiles_d * a.nc : 0;
  a.nRD = a.k * ((tiles_d + tpw - 1) / tpw);
  a.lcnt = a.sync + (size_t)SY_DONE * SY_LINE;
  a.advance = 1;
  // every copy of every hand-off area inside its workspace region
  QMOE_BOUNDS(((size_t)(LOGIT_COPIES - 1) * a.logit_copy + a.E) * 8 <= wl.bytes_at(wl.dec_logits));
  QMOE_BOUNDS(((size_t)(H_COPIES - 1) * a.hr_copy + (size_t)a.k * a.I) * 8 <= wl.bytes_at(wl.dec_hr));
  QMOE_BOUNDS(!sh || ((size_t)(H_COPIES - 1) * a.hsh_copy + a.Is) * 8 <= wl.bytes_at(wl.dec_hsh));
  QMOE_BOUNDS((size_t)(a.k - 1) * a.H * 8 <= wl.bytes_at(wl.dec_yr) || a.k == 1);
  QMOE_BOUNDS((size_t)a.nc * a.H * 8 <= wl.bytes_at(wl.dec_ysh) || a.nc == 0);
  QMOE_BOUNDS((size_t)tiles_d * 8 <= wl.bytes_at(wl.dec_nrm));
  QMOE_BOUNDS((size_t)TK_COPIES * 2 * MAX_TOPK * 8 <= wl.bytes_at(wl.dec_tk));
  QMOE_BOUNDS((size_t)(DEC_SYNC_WORD + SY_LINES * SY_LINE) * 4 <= wl.bytes_at(wl.cnt));
  QMOE_BOUNDS(dec_lds_of(d, sh).total <= 160 * 1024);
#ifdef QMOE_TIMELINE
  a.tl = g_tl;
#endif
  return a;
}

static int launch_decode(const qmoe_layer *L, const uint16_t *x, uint16_t *out, float *out_f32,
                         int32_t *idx, float *w, void *ws, const WsLayout &wl, hipStream_t s) {
  const DecodeArgs a = make_decode_args(L, x, out, out_f32, idx, w, ws, wl);
  const size_t lds = std::max(router_lds_bytes(a.H, 1), dec_lds_of(&L->d, a.shared != nullptr).total);
  int rc = set_lds(decode_layer_kernel, lds);
  if (rc) return rc;
  const int n = a.nR + a.nSG + a.nRG + a.nSD + a.nRD;
  hipLaunchKernelGGL(decode_layer_kernel, dim3(n), dim3(DEC_THREADS), lds, s, a);
  QMOE_LAUNCHED();
  return QMOE_OK;
}

// Layer chain of one token in one launch (decode.h): the per-layer table is written by small
// kernels whose arguments carry it (so that the call can be captured in a graph), then the
// chained kernel runs every layer.
static int launch_decode_stack(const qmoe_layer *layers, int n, const uint16_t *x, uint16_t *out,
                               float *out_f32, int32_t *idx, float *w, bool tk_per_layer, void *ws,
                               const WsLayout &wl, hipStream_t s) {
  DecLayer *tab = at<DecLayer>(ws, wl.dec_tab);
  for (int f = 0; f < n; f += DEC_TAB_CHUNK) {
    DecTabChunk c;
    memset(&c, 0, sizeof c);
    const int m = std::min(DEC_TAB_CHUNK, n - f);
    for (int i = 0; i < m; ++i) {
      const qmoe_layer &Li = layers[f + i];
      c.L[i] = DecLayer{Li.r.codes, Li.r.scales, Li.r.biases, Li.r.router_scale,
                        Li.r.per_expert_scale, Li.r.logit_bias, (const uint8_t *)Li.experts,
                        (const uint8_t *)Li.shared, Li.post_norm_gain, Li.layer_scalar};
    }
    hipLaunchKernelGGL(dec_table_kernel, dim3(1), dim3(DEC_TAB_CHUNK), 0, s, c, tab, f, m);
    QMOE_LAUNCHED();
  }
  DecodeArgs a = make_decode_args(&layers[0], x, out, out_f32, idx, w, ws, wl);
  a.x_copy = dec_x_copy_bytes(a.H) / 8;
  uint64_t *xb0 = at<uint64_t>(ws, wl.dec_x);
  uint64_t *xb1 = xb0 + (size_t)X_COPIES * a.x_copy;
  const size_t lds = std::max(al16(router_lds_bytes(a.H, 1)) + (size_t)a.H * 2,
                              dec_lds_of(&layers[0].d, a.shared != nullptr).total);
  int rc = set_lds(decode_stack_kernel, lds);
  if (rc) return rc;
  const int per = a.nR + a.nSG + a.nRG + a.nSD + a.nRD;
  hipLaunchKernelGGL(decode_stack_kernel, dim3((unsigned)(per * n)), dim3(DEC_THREADS), lds, s, a,
                     (const DecLayer *)tab, xb0, xb1, n, tk_per_layer ? 1 : 0);
  QMOE_LAUNCHED();
  return QMOE_OK;
}

}  // namespace

// The tiered-residency cache object behind the opaque qmoe_expert_cache handle.
struct qmoe_expert_cache {
  qmoe_dims d;
  const uint8_t *host_store;
  size_t host_stride;
  uint8_t *slots_mem;
  size_t slot_stride;
  int n_slots;
  qmoe::ExpertCachePolicy policy;
  // made on the first forward call, on the device current then: pinned staging for the ids,
  // the slot ids and the slot lists, and two copy streams (default priority) with an event each
  int32_t *h_ids = nullptr, *h_slots = nullptr, *h_lists = nullptr;
  hipStream_t copy_s[2] = {nullptr, nullptr};
  hipEvent_t copied[2] = {nullptr, nullptr};
  int device = -1;
  qmoe_expert_cache(const qmoe_dims &dd, const void *hs, size_t hst, void *ds, size_t dst, int n)
      : d(dd), host_store((const uint8_t *)hs), host_stride(hst), slots_mem((uint8_t *)ds),
        slot_stride(dst), n_slots(n), policy(dd.n_experts, n) {}
};

// ====================================================================== exported entry points
extern "C" {

int qmoe_version(void) { return VERSION; }

const char *qmoe_last_error(void) { return g_err.c_str(); }

size_t qmoe_expert_stride(const qmoe_dims *d, int32_t inter) {
  if (check_dims(d)) return 0;
  if (!mult64(inter) || inter > 4096) {
    fail(QMOE_ERR_SHAPE, "inter must be a positive multiple of 64 <= 4096 (got %d)", inter);
    return 0;
  }
  return block_stride_bytes(d->hidden, inter, kshift_of(d));
}

size_t qmoe_workspace_bytes(const qmoe_dims *d, int32_t max_tokens) {
  if (check_dims(d) || check_T(max_tokens)) return 0;
  return ws_layout(d, std::max(max_tokens, 1)).total;
}

int qmoe_workspace_init(void *ws, size_t ws_bytes, qmoe_stream_t stream) {
  if (!ws) return fail(QMOE_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(QMOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  int rc = check_arch();
  if (rc) return rc;
  const size_t n = ws_bytes / 4;
  if (n == 0) return ok();
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, (uint32_t *)ws, n);
  QMOE_LAUNCHED();
  return ok();
}

int qmoe_pack_expert(const qmoe_dims *d, int32_t inter, const uint8_t *gate_q,
                     const uint16_t *gate_s, const uint16_t *gate_b, const uint8_t *up_q,
                     const uint16_t *up_s, const uint16_t *up_b, const uint8_t *down_q,
                     const uint16_t *down_s, const uint16_t *down_b, void *dst_block,
                     qmoe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!mult64(inter) || inter > 4096)
    return fail(QMOE_ERR_SHAPE, "inter must be a positive multiple of 64 <= 4096 (got %d)", inter);
  if (!gate_q || !gate_s || !gate_b || !up_q || !up_s || !up_b || !down_q || !down_s || !down_b ||
      !dst_block)
    return fail(QMOE_ERR_ARG, "pack_expert: NULL pointer");
  if (!aligned(dst_block, 256)) return fail(QMOE_ERR_ARG, "dst_block must be 256-byte aligned");
  if ((rc = check_arch())) return rc;
  CanonExpert c{gate_q, up_q, down_q, gate_s, gate_b, up_s, up_b, down_s, down_b};
  const BlockGeom g = block_geom(d->hidden, inter, kshift_of(d));
  const long n = (long)(g.gu_tiles * g.gu_ks + g.d_tiles * g.d_ks) * 64;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, c, d->hidden, inter, kshift_of(d), (uint8_t *)dst_block);
  QMOE_LAUNCHED();
  return ok();
}

int qmoe_unpack_expert(const qmoe_dims *d, int32_t inter, const void *src_block, uint8_t *gate_q,
                       uint16_t *gate_s, uint16_t *gate_b, uint8_t *up_q, uint16_t *up_s,
                       uint16_t *up_b, uint8_t *down_q, uint16_t *down_s, uint16_t *down_b,
                       qmoe_stream_t stream) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!mult64(inter) || inter > 4096)
    return fail(QMOE_ERR_SHAPE, "inter must be a positive multiple of 64 <= 4096 (got %d)", inter);
  if (!gate_q || !gate_s || !gate_b || !up_q || !up_s || !up_b || !down_q || !down_s || !down_b ||
      !src_block)
    return fail(QMOE_ERR_ARG, "unpack_expert: NULL pointer");
  if (!aligned(src_block, 256)) return fail(QMOE_ERR_ARG, "src_block must be 256-byte aligned");
  if ((rc = check_arch())) return rc;
  CanonExpertOut c{gate_q, up_q, down_q, gate_s, gate_b, up_s, up_b, down_s, down_b};
  const BlockGeom g = block_geom(d->hidden, inter, kshift_of(d));
  const long n = (long)(g.gu_tiles * g.gu_ks + g.d_tiles * g.d_ks) * 64;
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, (const uint8_t *)src_block, d->hidden, inter,
                     kshift_of(d), c);
  QMOE_LAUNCHED();
  return ok();
}

int qmoe_router_topk(const qmoe_dims *d, const qmoe_router *r, const uint16_t *x, int32_t T,
                     int32_t *topk_idx, float *topk_w, float *logits_or_null, void *ws,
                     size_t ws_bytes, qmoe_stream_t stream) {
  int rc = check_dims(d);
  if (rc || (rc = check_T(T)) || (rc = check_router(r))) return rc;
  if (T == 0) return ok();
  if (!x || !topk_idx || !topk_w) return fail(QMOE_ERR_ARG, "x/topk_idx/topk_w must not be NULL");
  if (!aligned(x, 16)) return fail(QMOE_ERR_ARG, "x must be 16-byte aligned");
  if ((rc = check_ws(d, T, ws, ws_bytes))) return rc;
  if ((rc = check_arch())) return rc;
  const WsLayout wl = ws_layout(d, T);
  float *logits = logits_or_null ? logits_or_null : at<float>(ws, wl.logits);
  // per chunk of at most CHUNK_TOKENS tokens (the partial tiles of the router are sized for one)
  for (int c0 = 0; c0 < T; c0 += CHUNK_TOKENS) {
    const int Tc = std::min(CHUNK_TOKENS, T - c0);
    RouterArgs a = make_router_args(d, r, x + (size_t)c0 * d->hidden, Tc,
                                    logits + (size_t)c0 * d->n_experts, topk_idx + (size_t)c0 * d->top_k,
                                    topk_w + (size_t)c0 * d->top_k, ws);
    if ((rc = launch_router(a, router_smem(d, Tc), ws, wl, (hipStream_t)stream))) return rc;
  }
  return ok();
}

int qmoe_bucket(const qmoe_dims *d, const int32_t *topk_idx, int32_t T, int32_t *counts,
                int32_t *offsets, int32_t *sorted, int32_t *active, int32_t *n_active, void *ws,
                size_t ws_bytes, qmoe_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_dims(d);
  if (rc || (rc = check_T(T))) return rc;
  if ((!topk_idx && T > 0) || !counts || !offsets || !sorted || !active || !n_active)
    return fail(QMOE_ERR_ARG, "bucket: NULL pointer");
  if ((rc = check_arch())) return rc;
  const size_t lds = bucket_lds_bytes(T * d->top_k, d->n_experts);
  QMOE_BOUNDS((long)T * d->top_k <= BUCKET_MAX_N && lds <= 160 * 1024);
  if ((rc = set_lds(bucket_kernel, lds))) return rc;
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(256), lds, (hipStream_t)stream, topk_idx,
                     T * d->top_k, d->n_experts, counts, offsets, sorted, active, n_active);
  QMOE_LAUNCHED();
  return ok();
}

int qmoe_expert_ffn(const qmoe_layer *L, const uint16_t *x, int32_t T, const int32_t *offsets,
                    const int32_t *sorted, const int32_t *active, const int32_t *n_active,
                    float *y, float *y_shared_or_null, void *ws, size_t ws_bytes,
                    qmoe_stream_t stream) {
  int rc = check_layer(L);
  if (rc || (rc = check_T(T))) return rc;
  if (y_shared_or_null && !L->shared)
    return fail(QMOE_ERR_ARG, "y_shared given but the layer has no shared block");
  if (T == 0) return ok();
  if (!x || !offsets || !sorted || !active || !n_active || !y)
    return fail(QMOE_ERR_ARG, "expert_ffn: NULL pointer");
  if (!aligned(x, 16)) return fail(QMOE_ERR_ARG, "x must be 16-byte aligned");
  if ((rc = check_ws(&L->d, T, ws, ws_bytes))) return rc;
  if ((rc = check_arch())) return rc;
  FfnArgs a = make_ffn_args(L, x, T, offsets, sorted, active, n_active, y, y_shared_or_null, ws, T);
  hipStream_t s = (hipStream_t)stream;
  if (valu_ffn(T)) {
    if ((rc = launch_gu(a, s))) return rc;
    const bool sh = L->shared && y_shared_or_null;
    if (!sh) a.shared = nullptr;
    if ((rc = launch_d(a, sh, s))) return rc;
    return ok();
  }
  if (!y_shared_or_null) a.shared = nullptr;
  if ((rc = launch_gsum(x, T, L->d.hidden, at<float>(ws, ws_layout(&L->d, T).gx), s))) return rc;
  if ((rc = launch_pf(a, s))) return rc;
  return ok();
}

int qmoe_combine(const qmoe_dims *d, const uint16_t *x, const float *y, const float *topk_w,
                 const float *y_shared_or_null, int32_t T, uint16_t *out, float *out_f32_or_null,
                 qmoe_stream_t stream) {
  int rc = check_dims(d);
  if (rc || (rc = check_T(T))) return rc;
  if (T == 0) return ok();
  if (!x || !y || !topk_w || !out) return fail(QMOE_ERR_ARG, "combine: NULL pointer");
  if ((rc = check_arch())) return rc;
  const size_t n = (size_t)T * d->hidden;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, x, y,
                     topk_w, y_shared_or_null, T, d->hidden, d->top_k, out, out_f32_or_null);
  QMOE_LAUNCHED();
  return ok();
}

int qmoe_combine_post(const qmoe_dims *d, const uint16_t *x, const float *y, const float *topk_w,
                      const float *y_shared_or_null, const float *post_norm_gain_or_null,
                      const float *layer_scalar_or_null, int32_t T, uint16_t *out,
                      float *out_f32_or_null, qmoe_stream_t stream) {
  int rc = check_dims(d);
  if (rc || (rc = check_T(T))) return rc;
  if (T == 0) return ok();
  if (!x || !y || !topk_w || !out) return fail(QMOE_ERR_ARG, "combine_post: NULL pointer");
  if (post_norm_gain_or_null && !aligned(post_norm_gain_or_null, 16))
    return fail(QMOE_ERR_ARG, "post_norm_gain must be 16-byte aligned");
  if ((rc = check_arch())) return rc;
  if ((rc = launch_combine_post(x, y, topk_w, y_shared_or_null, post_norm_gain_or_null,
                                layer_scalar_or_null, T, d->hidden, d->top_k, out,
                                out_f32_or_null, (hipStream_t)stream)))
    return rc;
  return ok();
}

}  // extern "C"

namespace {

// The layer on workspace ws (validated by the caller), per chunk of at most CHUNK_TOKENS tokens.
int layer_forward_impl(const qmoe_layer *L, const uint16_t *x, int32_t T, uint16_t *out,
                       float *out_f32_or_null, int32_t *topk_idx_or_null, float *topk_w_or_null,
                       void *ws, qmoe_stream_t stream) {
  int rc;
  const int Tc_max = std::min<int>(T, CHUNK_TOKENS);
  const qmoe_dims *d = &L->d;
  hipStream_t s = (hipStream_t)stream;
  const WsLayout wl = ws_layout(d, Tc_max);
  const int H = d->hidden, k = d->top_k;
  const bool sh = L->shared != nullptr;
  const bool post = L->post_norm_gain || L->layer_scalar;
  if (T == 1 && decode_fits(d)) {
    int32_t *idx = topk_idx_or_null ? topk_idx_or_null : at<int32_t>(ws, wl.tidx);
    float *w = topk_w_or_null ? topk_w_or_null : at<float>(ws, wl.tw);
    if (g_prof_start && (rc = record_event(g_prof_start, s))) return rc;
    if ((rc = launch_decode(L, x, out, out_f32_or_null, idx, w, ws, wl, s))) return rc;
    if (g_prof_stop && (rc = record_event(g_prof_stop, s))) return rc;
    return ok();
  }
  for (int c0 = 0; c0 < T; c0 += CHUNK_TOKENS) {
    const int Tc = std::min(CHUNK_TOKENS, T - c0);
    const uint16_t *xc = x + (size_t)c0 * H;
    int32_t *idx = topk_idx_or_null ? topk_idx_or_null + (size_t)c0 * k : at<int32_t>(ws, wl.tidx);
    float *w = topk_w_or_null ? topk_w_or_null + (size_t)c0 * k : at<float>(ws, wl.tw);
    // kernel 1: router, top-k and bucketing (with the slot table)
    RouterArgs ra = make_router_args(d, &L->r, xc, Tc, at<float>(ws, wl.logits), idx, w, ws);
    ra.counts = at<int32_t>(ws, wl.counts);
    ra.offsets = at<int32_t>(ws, wl.offsets);
    ra.sorted = at<int32_t>(ws, wl.sorted);
    ra.active = at<int32_t>(ws, wl.active);
    ra.n_active = at<int32_t>(ws, wl.nact);
    ra.slot_tab = at<int32_t>(ws, wl.slot_tab);
    FfnArgs fa = make_ffn_args(L, xc, Tc, ra.offsets, ra.sorted, ra.active, ra.n_active,
                               at<float>(ws, wl.y), nullptr, ws, Tc_max);
    fa.slot_tab = ra.slot_tab;
    fa.n_slots = bucket_max_blocks(Tc * k, d->n_experts);
    ra.n_slots = fa.n_slots;
    QMOE_BOUNDS(Tc <= Tc_max && (size_t)fa.n_slots * 16 <= wl.bytes_at(wl.slot_tab));
    QMOE_BOUNDS((size_t)Tc * k * H * 4 <= wl.bytes_at(wl.y) && (size_t)Tc * k * 4 <= wl.bytes_at(wl.sorted));
    QMOE_BOUNDS(router_smem(d, Tc) <= 160 * 1024);
    const bool mfma = !valu_ffn(Tc);
    if (mfma) ra.gsum = at<float>(ws, wl.gx);
    if ((rc = launch_router(ra, router_smem(d, Tc), ws, wl, s))) return rc;
    uint16_t *oc = out + (size_t)c0 * H;
    float *oc32 = out_f32_or_null ? out_f32_or_null + (size_t)c0 * H : nullptr;
    if (mfma) {
      // kernels 2-4: gate/up, down (matrix cores), combine with the shared rows and residual
      fa.y_sh = sh ? at<float>(ws, wl.ysh) : nullptr;
      if (!sh) fa.shared = nullptr;
      if ((rc = launch_pf(fa, s))) return rc;
      if (post) rc = launch_combine_post(xc, fa.y, w, fa.y_sh, L->post_norm_gain, L->layer_scalar,
                                         Tc, H, k, oc, oc32, s);
      else rc = launch_combine_pf(xc, fa.y, w, fa.y_sh, Tc, H, k, oc, oc32, s);
      if (rc) return rc;
    } else {
      // VALU kernels: gate/up (routed + shared), down (routed + shared, one chunk), combine
      fa.y_sh = sh ? at<float>(ws, wl.ysh) : nullptr;
      if (!sh) fa.shared = nullptr;
      if (g_prof_start && (rc = record_event(g_prof_start, s))) return rc;
      if ((rc = launch_gu(fa, s))) return rc;
      if (g_prof_stop && (rc = record_event(g_prof_stop, s))) return rc;
      if ((rc = launch_d(fa, sh, s))) return rc;
      if (post) {
        if ((rc = launch_combine_post(xc, fa.y, w, fa.y_sh, L->post_norm_gain, L->layer_scalar,
                                      Tc, H, k, oc, oc32, s)))
          return rc;
      } else {
        const size_t n = (size_t)Tc * H;
        const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
        hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, xc, fa.y, w, fa.y_sh,
                           Tc, H, k, oc, oc32);
        QMOE_LAUNCHED();
      }
    }
  }
  return ok();
}

// Arguments of a layer call, checked on the host before any device call.
int check_layer_call(const qmoe_layer *L, const uint16_t *x, int32_t T, const uint16_t *out) {
  int rc = check_layer(L);
  if (rc || (rc = check_T(T))) return rc;
  if (T == 0) return QMOE_OK;
  if (!x || !out) return fail(QMOE_ERR_ARG, "layer_forward: x/out must not be NULL");
  if (!aligned(x, 16)) return fail(QMOE_ERR_ARG, "x must be 16-byte aligned");
  return QMOE_OK;
}

// ------------------------------------------------------------ allocation-free variant
// Workspace of qmoe_layer_forward_noalloc: one fixed device array, a copy of which every GPU the
// library runs on holds until the process ends.  Like every device global without an
// initialiser it is zero when the code object is loaded, which is the state a new workspace
// must start in; every call leaves it ready for the next one (counters back at zero, the epoch
// of the one-token path advanced).  Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

// The current device's address of `scratch` (looked up on its first use on that device).
int scratch_address(void **out) {
  int dev = 0;
  QMOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(QMOE_ERR_ARCH, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(QMOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QMOE_OK;
}

}  // namespace

extern "C" {

int qmoe_layer_forward(const qmoe_layer *L, const uint16_t *x, int32_t T, uint16_t *out,
                       float *out_f32_or_null, int32_t *topk_idx_or_null, float *topk_w_or_null,
                       void *ws, size_t ws_bytes, qmoe_stream_t stream) {
  int rc = check_layer_call(L, x, T, out);
  if (rc || T == 0) return rc ? rc : ok();
  if ((rc = check_ws(&L->d, std::min<int>(T, CHUNK_TOKENS), ws, ws_bytes))) return rc;
  if ((rc = check_arch())) return rc;
  return layer_forward_impl(L, x, T, out, out_f32_or_null, topk_idx_or_null, topk_w_or_null, ws,
                            stream);
}

int qmoe_layer_forward_noalloc(const qmoe_layer *L, const uint16_t *x, int32_t T, uint16_t *out,
                               float *out_f32_or_null, int32_t *topk_idx_or_null,
                               float *topk_w_or_null, qmoe_stream_t stream) {
  int rc = check_layer_call(L, x, T, out);
  if (rc || T == 0) return rc ? rc : ok();
  const size_t need = ws_layout(&L->d, std::min<int>(T, CHUNK_TOKENS)).total;
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(QMOE_ERR_WORKSPACE, "layer_forward_noalloc: this shape needs %zu bytes of scratch, "
                "more than the %zu the library holds per device; use qmoe_layer_forward with a "
                "workspace", need, NOALLOC_SCRATCH_BYTES);
  if ((rc = check_arch())) return rc;
  void *ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return layer_forward_impl(L, x, T, out, out_f32_or_null, topk_idx_or_null, topk_w_or_null, ws,
                            stream);
}

int qmoe_cache_create(const qmoe_dims *d, const void *host_store, size_t host_stride,
                      void *device_slots, size_t slot_stride, int32_t slots,
                      qmoe_expert_cache **cache_out) {
  int rc = check_dims(d);
  if (rc) return rc;
  if (!cache_out) return fail(QMOE_ERR_ARG, "cache_out is NULL");
  *cache_out = nullptr;
  if (!host_store || !device_slots) return fail(QMOE_ERR_ARG, "cache: NULL store or slots");
  const size_t blk = block_stride_bytes(d->hidden, d->inter, kshift_of(d));
  if (host_stride < blk || slot_stride < blk || host_stride % 256 || slot_stride % 256)
    return fail(QMOE_ERR_ARG, "cache strides must be multiples of 256 and >= %zu", blk);
  if (!aligned(device_slots, 256)) return fail(QMOE_ERR_ARG, "device_slots must be 256-byte aligned");
  if (slots < d->top_k || slots > d->n_experts)
    return fail(QMOE_ERR_SHAPE, "slots must be in [top_k, n_experts] (got %d)", slots);
  *cache_out = new qmoe_expert_cache(*d, host_store, host_stride, device_slots, slot_stride, slots);
  return ok();
}

int qmoe_cache_destroy(qmoe_expert_cache *cache) {
  if (!cache) return ok();
  for (int i = 0; i < 2; ++i) {
    if (cache->copy_s[i]) {
      (void)hipStreamSynchronize(cache->copy_s[i]);
      (void)hipStreamDestroy(cache->copy_s[i]);
    }
    if (cache->copied[i]) (void)hipEventDestroy(cache->copied[i]);
  }
  if (cache->h_ids) (void)hipHostFree(cache->h_ids);
  if (cache->h_slots) (void)hipHostFree(cache->h_slots);
  if (cache->h_lists) (void)hipHostFree(cache->h_lists);
  delete cache;
  return ok();
}

int qmoe_cache_plan(qmoe_expert_cache *cache, const int32_t *ids, int32_t n, int32_t *slot_of_out,
                    int32_t *fill_expert_out, int32_t *fill_slot_out, int32_t *n_fills_out) {
  if (!cache || (!ids && n > 0) || (!slot_of_out && n > 0) || !fill_expert_out || !fill_slot_out ||
      !n_fills_out)
    return fail(QMOE_ERR_ARG, "cache_plan: NULL pointer");
  if (n < 0) return fail(QMOE_ERR_ARG, "cache_plan: n < 0");
  CachePlan p;
  if (!cache->policy.plan(ids, n, p))
    return fail(QMOE_ERR_ARG, "cache_plan: an id outside [0, %d) or more distinct ids than the %d slots",
                cache->d.n_experts, cache->n_slots);
  for (int i = 0; i < n; ++i) slot_of_out[i] = p.slot_of[i];
  for (size_t j = 0; j < p.fill_slot.size(); ++j) {
    fill_expert_out[j] = p.fill_expert[j];
    fill_slot_out[j] = p.fill_slot[j];
  }
  *n_fills_out = (int32_t)p.fill_slot.size();
  return ok();
}

int qmoe_cache_stats(const qmoe_expert_cache *cache, int64_t *hits_out, int64_t *misses_out) {
  if (!cache || !hits_out || !misses_out) return fail(QMOE_ERR_ARG, "cache_stats: NULL pointer");
  *hits_out = cache->policy.hits();
  *misses_out = cache->policy.misses();
  return ok();
}

int qmoe_decode_stack(const qmoe_layer *layers, int32_t n_layers, const uint16_t *x,
                      uint16_t *out, float *out_f32_or_null, int32_t *topk_idx_or_null,
                      float *topk_w_or_null, void *ws, size_t ws_bytes, qmoe_stream_t stream) {
  if (!layers) return fail(QMOE_ERR_ARG, "decode_stack: layers is NULL");
  if (n_layers < 0 || n_layers > QMOE_MAX_STACK)
    return fail(QMOE_ERR_SHAPE, "decode_stack: n_layers must be in [0, %d] (got %d)", QMOE_MAX_STACK,
                n_layers);
  if (n_layers == 0) return ok();
  int rc;
  for (int i = 0; i < n_layers; ++i) {
    if ((rc = check_layer(&layers[i]))) return rc;
    if (memcmp(&layers[i].d, &layers[0].d, sizeof(qmoe_dims)) != 0)
      return fail(QMOE_ERR_SHAPE, "decode_stack: dims of layer %d differ from layer 0", i);
    if ((layers[i].shared != nullptr) != (layers[0].shared != nullptr))
      return fail(QMOE_ERR_ARG, "decode_stack: every layer or none must have a shared block");
  }
  if (!x || !out) return fail(QMOE_ERR_ARG, "decode_stack: x/out must not be NULL");
  if (!aligned(x, 16)) return fail(QMOE_ERR_ARG, "x must be 16-byte aligned");
  if ((topk_idx_or_null == nullptr) != (topk_w_or_null == nullptr))
    return fail(QMOE_ERR_ARG, "decode_stack: give both top-k outputs or neither");
  const qmoe_dims *d = &layers[0].d;
  if (!decode_fits(d))
    return fail(QMOE_ERR_SHAPE, "decode_stack: inter %d with %d-bit experts is too wide for the "
                "one-token launch", d->inter, d->expert_bits == 8 ? 8 : 4);
  if ((rc = check_ws(d, 1, ws, ws_bytes))) return rc;
  if ((rc = check_arch())) return rc;
  const WsLayout wl = ws_layout(d, 1);
  const bool tk = topk_idx_or_null != nullptr;
  int32_t *idx = tk ? topk_idx_or_null : at<int32_t>(ws, wl.tidx);
  float *w = tk ? topk_w_or_null : at<float>(ws, wl.tw);
  hipStream_t s = (hipStream_t)stream;
  if (g_prof_start && (rc = record_event(g_prof_start, s))) return rc;
  if ((rc = launch_decode_stack(layers, n_layers, x, out, out_f32_or_null, idx, w, tk, ws, wl, s)))
    return rc;
  if (g_prof_stop && (rc = record_event(g_prof_stop, s))) return rc;
  return ok();
}

int qmoe_layer_forward_tiered(const qmoe_layer *L, qmoe_expert_cache *C, const uint16_t *x,
                              int32_t T, uint16_t *out, float *out_f32_or_null,
                              int32_t *topk_idx_or_null, float *topk_w_or_null, void *ws,
                              size_t ws_bytes, qmoe_stream_t stream) {
  if (!L) return fail(QMOE_ERR_ARG, "layer is NULL");
  int rc = check_dims(&L->d);
  if (rc || (rc = check_router(&L->r)) || (rc = check_T(T))) return rc;
  if (!C) return fail(QMOE_ERR_ARG, "cache is NULL");
  const qmoe_dims *d = &L->d;
  if (C->d.hidden != d->hidden || C->d.n_experts != d->n_experts || C->d.top_k != d->top_k ||
      C->d.inter != d->inter || kshift_of(&C->d) != kshift_of(d))
    return fail(QMOE_ERR_ARG, "cache was made for other layer dims");
  if (L->shared && (d->shared_inter == 0 || !aligned(L->shared, 256)))
    return fail(QMOE_ERR_ARG, "shared block needs shared_inter > 0 and 256-byte alignment");
  if (L->post_norm_gain && !aligned(L->post_norm_gain, 16))
    return fail(QMOE_ERR_ARG, "post_norm_gain must be 16-byte aligned");
  if (T == 0) return ok();
  if (!x || !out) return fail(QMOE_ERR_ARG, "layer_forward_tiered: x/out must not be NULL");
  if (!aligned(x, 16)) return fail(QMOE_ERR_ARG, "x must be 16-byte aligned");
  const int Tc_max = std::min<int>(T, CHUNK_TOKENS);
  if ((rc = check_ws(d, Tc_max, ws, ws_bytes))) return rc;
  if ((rc = check_arch())) return rc;
  int dev = 0;
  QMOE_HIP(hipGetDevice(&dev));
  if (C->device < 0) {
    QMOE_HIP(hipHostMalloc((void **)&C->h_ids, (size_t)CHUNK_TOKENS * MAX_TOPK * 4));
    QMOE_HIP(hipHostMalloc((void **)&C->h_slots, (size_t)CHUNK_TOKENS * MAX_TOPK * 4));
    QMOE_HIP(hipHostMalloc((void **)&C->h_lists, (size_t)(C->n_slots + 2) * 4));
    for (int i = 0; i < 2; ++i) {
      QMOE_HIP(hipStreamCreateWithFlags(&C->copy_s[i], hipStreamNonBlocking));
      QMOE_HIP(hipEventCreateWithFlags(&C->copied[i], hipEventDisableTiming));
    }
    C->device = dev;
  } else if (C->device != dev) {
    return fail(QMOE_ERR_ARG, "cache was first used on device %d, current device is %d", C->device,
                dev);
  }
  hipStream_t s = (hipStream_t)stream;
  const WsLayout wl = ws_layout(d, Tc_max);
  const int H = d->hidden, k = d->top_k;
  const bool sh = L->shared != nullptr;
  const bool post = L->post_norm_gain || L->layer_scalar;
  const size_t blk = block_stride_bytes(d->hidden, d->inter, kshift_of(d));
  for (int c0 = 0; c0 < T; c0 += CHUNK_TOKENS) {
    const int Tc = std::min(CHUNK_TOKENS, T - c0), N = Tc * k;
    const uint16_t *xc = x + (size_t)c0 * H;
    int32_t *idx = topk_idx_or_null ? topk_idx_or_null + (size_t)c0 * k : at<int32_t>(ws, wl.tidx);
    float *w = topk_w_or_null ? topk_w_or_null + (size_t)c0 * k : at<float>(ws, wl.tw);
    // router and top-k, then the ids to the host
    RouterArgs ra = make_router_args(d, &L->r, xc, Tc, at<float>(ws, wl.logits), idx, w, ws);
    if ((rc = launch_router(ra, router_smem(d, Tc), ws, wl, s))) return rc;
    QMOE_HIP(hipMemcpyAsync(C->h_ids, idx, (size_t)N * 4, hipMemcpyDeviceToHost, s));
    QMOE_HIP(hipStreamSynchronize(s));
    CachePlan p;
    if (!C->policy.plan(C->h_ids, N, p))
      return fail(QMOE_ERR_ARG, "a chunk names more distinct experts than the cache's %d slots",
                  C->n_slots);
    // One copy per missing block, alternating over the two copy streams (the io phase of
    // TurboFieldfare post, section "TurboFieldfare의 전문가 스트리밍 구조").  The caller's
    // stream is idle here (synchronised for the ids above), so no earlier kernel still reads a
    // slot being refilled, and this call's kernels read a refilled slot only after its copy.
    const int nf = (int)p.fill_slot.size();
    for (int j = 0; j < nf; ++j)
      QMOE_HIP(hipMemcpyAsync(C->slots_mem + (size_t)p.fill_slot[j] * C->slot_stride,
                              C->host_store + (size_t)p.fill_expert[j] * C->host_stride, blk,
                              hipMemcpyHostToDevice, C->copy_s[j & 1]));
    for (int i = 0; i < 2 && i < nf; ++i) QMOE_HIP(hipEventRecord(C->copied[i], C->copy_s[i]));
    for (int i = 0; i < N; ++i) C->h_slots[i] = p.slot_of[i];
    // the call's distinct slots: those it hit first, then those being filled
    std::vector<char> mark(C->n_slots, 0);   // 1: listed as hit, 2: being filled
    for (int j = 0; j < nf; ++j) mark[p.fill_slot[j]] = 2;
    int nh = 0;
    for (int i = 0; i < N; ++i) {
      const int sl = p.slot_of[i];
      if (!mark[sl]) {
        mark[sl] = 1;
        C->h_lists[2 + nh++] = sl;
      }
    }
    for (int j = 0; j < nf; ++j) C->h_lists[2 + nh + j] = p.fill_slot[j];
    C->h_lists[0] = nh;
    C->h_lists[1] = nf;
    int32_t *slot_ids = at<int32_t>(ws, wl.slot_ids);
    QMOE_HIP(hipMemcpyAsync(slot_ids, C->h_slots, (size_t)N * 4, hipMemcpyHostToDevice, s));
    // bucketing over the slots; its list of active slots is then replaced by the two lists
    int32_t *counts = at<int32_t>(ws, wl.counts), *offsets = at<int32_t>(ws, wl.offsets);
    int32_t *sorted = at<int32_t>(ws, wl.sorted), *active = at<int32_t>(ws, wl.active);
    int32_t *nact = at<int32_t>(ws, wl.nact);
    QMOE_BOUNDS((size_t)(nh + nf) * 4 <= wl.bytes_at(wl.active) && 8 <= wl.bytes_at(wl.nact));
    const size_t lds = bucket_lds_bytes(N, C->n_slots);
    if ((rc = set_lds(bucket_kernel, lds))) return rc;
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(256), lds, s, (const int32_t *)slot_ids, N,
                       C->n_slots, counts, offsets, sorted, active, nact);
    QMOE_LAUNCHED();
    QMOE_HIP(hipMemcpyAsync(active, C->h_lists + 2, (size_t)(nh + nf) * 4, hipMemcpyHostToDevice, s));
    QMOE_HIP(hipMemcpyAsync(nact, C->h_lists, 8, hipMemcpyHostToDevice, s));
    // the FFN of the shared expert and the hit slots while the copies run, then, once they
    // have landed, the FFN of the filled slots (the pages overlap the reads with the shared
    // and cached experts' work); every row's arithmetic is the same as in one launch
    FfnArgs fa = make_ffn_args(L, xc, Tc, offsets, sorted, active, nact, at<float>(ws, wl.y),
                               sh ? at<float>(ws, wl.ysh) : nullptr, ws, Tc_max);
    fa.experts = C->slots_mem;
    fa.stride = C->slot_stride;
    fa.n_experts = C->n_slots;
    fa.n_slots = nh;
    if (!sh) fa.shared = nullptr;
    FfnArgs fb = fa;
    fb.active = active + nh;
    fb.n_active = nact + 1;
    fb.n_slots = nf;
    fb.shared = nullptr;
    uint16_t *oc = out + (size_t)c0 * H;
    float *oc32 = out_f32_or_null ? out_f32_or_null + (size_t)c0 * H : nullptr;
    const bool valu = valu_ffn(Tc);
    if (!valu && (rc = launch_gsum(xc, Tc, H, at<float>(ws, wl.gx), s))) return rc;
    if (valu) {
      if ((rc = launch_gu(fa, s))) return rc;
      if ((rc = launch_d(fa, sh, s))) return rc;
    } else if ((rc = launch_pf(fa, s))) {
      return rc;
    }
    if (nf > 0) {
      for (int i = 0; i < 2 && i < nf; ++i) QMOE_HIP(hipStreamWaitEvent(s, C->copied[i], 0));
      if (valu) {
        if ((rc = launch_gu(fb, s))) return rc;
        if ((rc = launch_d(fb, false, s))) return rc;
      } else if ((rc = launch_pf(fb, s))) {
        return rc;
      }
    }
    if (post) rc = launch_combine_post(xc, fa.y, w, fa.y_sh, L->post_norm_gain, L->layer_scalar, Tc,
                                       H, k, oc, oc32, s);
    else rc = launch_combine_pf(xc, fa.y, w, fa.y_sh, Tc, H, k, oc, oc32, s);
    if (rc) return rc;
  }
  return ok();
}

int qmoe_event_create(void **event_out) {
  if (!event_out) return fail(QMOE_ERR_ARG, "event_out is NULL");
  hipEvent_t e;
  QMOE_HIP(hipEventCreate(&e));
  *event_out = (void *)e;
  return ok();
}

int qmoe_event_destroy(void *event) {
  if (!event) return fail(QMOE_ERR_ARG, "event is NULL");
  QMOE_HIP(hipEventDestroy((hipEvent_t)event));
  return ok();
}

int qmoe_event_record(void *event, qmoe_stream_t stream) {
  if (!event) return fail(QMOE_ERR_ARG, "event is NULL");
  int rc = record_event((hipEvent_t)event, (hipStream_t)stream);
  return rc ? rc : ok();
}

int qmoe_event_elapsed_ms(void *start, void *stop, float *ms_out) {
  if (!start || !stop || !ms_out) return fail(QMOE_ERR_ARG, "event_elapsed_ms: NULL argument");
  QMOE_HIP(hipEventSynchronize((hipEvent_t)stop));
  QMOE_HIP(hipEventElapsedTime(ms_out, (hipEvent_t)start, (hipEvent_t)stop));
  return ok();
}

int qmoe_workspace_status(const void *ws, size_t ws_bytes, int32_t *status_out,
                          qmoe_stream_t stream) {
  if (!ws || !status_out) return fail(QMOE_ERR_ARG, "workspace_status: NULL argument");
  if (ws_bytes < COUNTER_BYTES) return fail(QMOE_ERR_WORKSPACE, "workspace smaller than its counter area");
  int rc = check_arch();
  if (rc) return rc;
  unsigned v = 0;
  const unsigned *p = (const unsigned *)ws + DEC_SYNC_WORD + SY_STATUS * SY_LINE;
  QMOE_HIP(hipMemcpyAsync(&v, p, sizeof v, hipMemcpyDeviceToHost, (hipStream_t)stream));
  QMOE_HIP(hipStreamSynchronize((hipStream_t)stream));
  *status_out = (int32_t)v;
  return ok();
}

#ifdef QMOE_TIMELINE
// Timeline builds only: device buffer of TL_POINTS 64-bit words per workgroup that the next
// one-token layer calls on this thread (and the launches captured from them) write their phase
// timestamps to (NULL: none).
int qmoe_timeline_set(void *buf) {
  g_tl = (unsigned long long *)buf;
  return ok();
}
#endif

int qmoe_read_blocks(const void *base, size_t stride, const int32_t *ids, int32_t n, size_t bytes,
                     uint32_t *sink, qmoe_stream_t stream) {
  if (!base || !ids || !sink) return fail(QMOE_ERR_ARG, "read_blocks: NULL pointer");
  if (n < 0 || n > READ_MAX_BLOCKS)
    return fail(QMOE_ERR_SHAPE, "read_blocks: n must be in [0, %d] (got %d)", READ_MAX_BLOCKS, n);
  if (bytes % 16 || !aligned(base, 16) || stride % 16)
    return fail(QMOE_ERR_ARG, "read_blocks: base, stride and bytes must be multiples of 16");
  if (n == 0 || bytes == 0) return ok();
  int rc = check_arch();
  if (rc) return rc;
  ReadArgs a;
  memset(&a, 0, sizeof a);
  a.base = (const uint8_t *)base;
  a.stride = stride;
  a.bytes = bytes;
  a.n = n;
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0) return fail(QMOE_ERR_ARG, "read_blocks: negative block id");
    a.ids[i] = ids[i];
  }
  a.sink = sink;
  const size_t waves = stream_read_waves(bytes, n);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                     (hipStream_t)stream, a);
  QMOE_LAUNCHED();
  return ok();
}

int qmoe_set_profile_events(void *start, void *stop) {
  g_prof_start = (hipEvent_t)start;
  g_prof_stop = (hipEvent_t)stop;
  return ok();
}

}  // extern "C"
