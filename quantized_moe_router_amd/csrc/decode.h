// One-token decode of a whole routed MoE layer in a single launch.
//
// The layer's steps (TurboFieldfare post, section "TurboFieldfare의 전문가 스트리밍 구조":
// router -> expert reads/compute -> cb2 combine with the shared branch and the residual) are
// run by workgroups with different roles, ordered by block index:
//   R   router: 4 experts' logits each
//   SG  shared gate/up: 16 rows of h_shared each
//   RG  routed gate/up: (slot, 16-row tile); it ranks the logits itself to find the slot's
//       expert (the first RG workgroup also writes the top-k outputs)
//   SD  shared down: (32-row output tile, K chunk)
//   RD  routed down: (slot, group of output tiles); it ranks the logits itself, loads its
//       weights, then waits for the slot's h; its rows are scaled by the slot's router weight.
//       The RD workgroups of the last slot also combine: routed rows of every slot + shared
//       rows + residual -> output rows.
//
// Hand-off without counters or fences: every value that one workgroup passes to another is
// published as a tagged word (common.h) whose tag is this launch's epoch, and a consumer
// waits until every word it needs carries the epoch.  The epoch is read from the workspace at
// the start and advanced by the last combining workgroup (the only counter of the launch), so
// stale words of an earlier call never match.
//
// A workgroup only ever waits for words written by workgroups with smaller block indices, and
// the hardware dispatches workgroups of a launch in index order, so every wait ends; each wait
// is also bounded and reports a timeout in the status word instead of spinning on.
//
// Layer chain (decode_stack_kernel): one launch runs a token through several layers of the
// same shape, x of layer l + 1 being the bf16 output of layer l.  Block b belongs to layer
// b / (blocks per layer), with the roles above in the same order inside each layer, so the
// argument above still holds: a layer's router, shared and routed gate/up workgroups wait for
// the previous layer's output, which comes from workgroups of smaller index.  Layer l's words
// carry tag epoch + l; its combining workgroups publish the output as tagged bf16 pairs (two
// buffers, alternating by layer), which readers poll through the first word of each
// combining workgroup's rows before fetching them all.  Workgroups of layer l + 1
// are dispatched while layer l still runs and issue their weight loads before they wait, which
// takes the router's cold loads and the launch gap off the chain between layers (the overlap
// of the pages' cb1 / io / cb2 phases, TurboFieldfare post, section "TurboFieldfare의 전문가
// 스트리밍 구조").  Every hand-off buffer of a layer is reused by the next one only after all
// of its readers are done: each of them feeds, through the chain of waits, the output that
// the next layer waits for.
#pragma once
#include "common.h"
#include "store.h"
#include "router.h"
#include "ffn.h"
#include "mfma.h"

namespace qmoe {

// Phase timestamps (only in the library built with QMOE_TIMELINE, for profiling): thread 0 of
// a workgroup records the device's 100 MHz clock at numbered points of its role into
// tl[block * TL_POINTS + point], and the role's number at point TL_ROLE.  Points: 0 start;
// router 1 logits published; shared gate/up 1 x staged; routed gate/up 1 x staged, 2 expert
// known, 3 weights consumed; shared down 1 router seen, 2 weights in, 3 h staged; routed down
// 1 top-k known, 2 weights in, 3 h staged, 4 products done, 5 combine inputs in (last slot);
// every role 6 end.
constexpr int TL_POINTS = 8, TL_ROLE = 7;
enum : int { TL_R = 1, TL_SG = 2, TL_RG = 3, TL_SD = 4, TL_RD = 5 };
#ifdef QMOE_TIMELINE
#define QMOE_TL(a, point)                                                                  \
  do {                                                                                     \
    if (threadIdx.x == 0 && (a).tl) (a).tl[(size_t)blockIdx.x * TL_POINTS + (point)] = wall_clock64(); \
  } while (0)
#define QMOE_TL_ROLE(a, role)                                                              \
  do {                                                                                     \
    if (threadIdx.x == 0 && (a).tl) (a).tl[(size_t)blockIdx.x * TL_POINTS + TL_ROLE] = (role); \
  } while (0)
#else
#define QMOE_TL(a, point) \
  do {                    \
  } while (0)
#define QMOE_TL_ROLE(a, role) \
  do {                        \
  } while (0)
#endif

// Sync area of the workspace (zero-initialised, one 256-byte line each)
constexpr int SY_LINE = 64;                    // words per line
enum : int { SY_EPOCH = 0, SY_STATUS = 1, SY_DONE = 2, SY_LINES = 3 };
constexpr int MAX_STACK = 64;                  // layers of one chained launch
constexpr unsigned WAIT_LIMIT = 1u << 20;      // polls: well over a second
constexpr int DEC_W = 4;                       // waves per workgroup (every role)
constexpr int KB_DEC = 12;                     // k-steps a down wave holds in registers
constexpr int KB_GU = 12;                      // k-steps a gate/up wave loads per batch
constexpr int DEC_THREADS = DEC_W * WAVE;
// Values that many workgroups wait for are published in several copies, each on its own
// memory pages, and a reader polls one of them, so that polling does not pile onto a few
// memory lines: the logits in LOGIT_COPIES copies, h (routed and shared) in H_COPIES.  More
// copies spread the polling but cost the router more stores before its logits are all out;
// eight copies measured fastest for the logits (32 and 64 were slower, as were 1 to 4).
constexpr int LOGIT_COPIES = 8, H_COPIES = 4, X_COPIES = 8, TK_COPIES = 8;
inline __host__ __device__ size_t dec_copy_stride(size_t words) {
  return ((words * 8 + 4095) / 4096) * 4096;   // bytes
}

struct DecodeArgs {
  const uint16_t *x;            // [H] bf16
  const uint8_t *rq;
  const uint16_t *rs, *rb;
  const float *rscale, *pes, *lbias;
  const uint8_t *experts;
  size_t stride;
  const uint8_t *shared;        // null: no shared expert
  int H, E, k, I, Is;
  int kshift;                   // k-steps per expert-code group: 0 (4-bit) or 1 (8-bit)
  int nc;                       // shared down K chunks per output tile
  int wpt;                      // waves per routed down tile (1, 2 or 4)
  float inv_sqrt_h;
  unsigned *sync;               // [SY_LINES * SY_LINE]
  uint64_t *logits;             // [LOGIT_COPIES][E] tagged, copies logit_copy words apart
  uint64_t *h_r;                // [H_COPIES][k][I] tagged, copies hr_copy words apart
  uint64_t *h_sh;               // [H_COPIES][Is] tagged, copies hsh_copy words apart
  size_t logit_copy, hr_copy, hsh_copy;
  uint64_t *y_r;                // [k-1][H] tagged routed rows of slots 0..k-2, router-weighted
  uint64_t *y_sh;               // [nc][H] tagged shared rows
  int32_t *topk_idx;            // [k]
  float *topk_w;                // [k]
  uint16_t *out;                // [H]
  float *out_f32;               // [H] or null
  const float *gain;            // [H] post-combine norm gain, or null (no norm)
  const float *lscale;          // [1] layer scalar, or null (1)
  uint64_t *nrm;                // [combining workgroups] tagged partial sums of m^2
  uint64_t *tk;                 // [TK_COPIES][2 MAX_TOPK] tagged top-k (expert bits, weight) of
                                //   the layer, published by the first routed gate/up workgroup
  int nR, nSG, nRG, nSD, nRD;
  // layer chain
  const uint64_t *xin;          // [X_COPIES] tagged x (bf16 pairs) from the previous layer, or null
  uint64_t *xout;               // [X_COPIES] tagged output for the next layer, or null
  size_t x_copy;                // words between x copies
  unsigned *lcnt;               // arrival counter of the combining workgroups (the SY_DONE line)
  unsigned long long *tl;       // phase timestamps (QMOE_TIMELINE builds), or null
  int advance;                  // this layer's combining workgroups count their arrivals, and
                                // the last of them advances the epoch (the launch's last layer)
};

// Per-layer pointers of a chained launch (a table in device memory).
struct DecLayer {
  const uint8_t *rq;
  const uint16_t *rs, *rb;
  const float *rscale, *pes, *lbias;
  const uint8_t *experts, *shared;
  const float *gain, *lscale;
};

inline __host__ __device__ size_t dec_x_copy_bytes(int H) { return dec_copy_stride((size_t)H / 2); }

// LDS map (bytes) shared by every role: [top-k ranking][per-expert scales][reduction]
// [union: staged x | staged h + combine rows]
struct DecLds {
  size_t tk, tks, pes, red, nrm, xw, x, xs, hf, hh, hl, hs, comb, total;
};
inline __host__ __device__ size_t al16(size_t v) { return (v + 15) & ~(size_t)15; }
inline __host__ __device__ int dec_tiles_per_wg(int wpt) { return DEC_W / wpt; }
inline __host__ __device__ DecLds dec_lds(int H, int E, int k, int I, int Kc_sh, int nc, int wpt) {
  DecLds L;
  size_t o = 0;
  L.tk = o; o = al16(o + (topk_chunks(E) <= 2 ? (size_t)topk_chunks(E) * WAVE * 8
                                                : (size_t)topk_chunks(E) * WAVE * 4 + DEC_W * MAX_TOPK * 8));
  L.tks = o; o = al16(o + (size_t)2 * MAX_TOPK * 4);
  L.pes = o; o = al16(o + (size_t)E * 4 + 16);
  L.red = o; o = al16(o + (size_t)DEC_W * 32 * 4);
  L.nrm = o; o = al16(o + (size_t)(DEC_W + H / TILE_ROWS) * 4);
  L.xw = o; o = al16(o + (size_t)TILE_ROWS * DEC_W / 2 * 4);
  const size_t u = o;
  L.x = u;
  L.xs = al16(L.x + (size_t)H * 2);
  const size_t xend = al16(L.xs + (size_t)(H / 32) * 4);
  const int K = I > Kc_sh ? I : Kc_sh;
  L.hf = u;
  L.hh = al16(L.hf + (size_t)K * 4);
  L.hl = al16(L.hh + (size_t)K * 2);
  L.hs = al16(L.hl + (size_t)K * 2);
  L.comb = al16(L.hs + (size_t)(K / 32) * 4);
  const size_t hend = al16(L.comb + (size_t)(k - 1 + nc) * TILE_ROWS * dec_tiles_per_wg(wpt) * 4);
  L.total = xend > hend ? xend : hend;
  return L;
}

QMOE_DEV void st_sys_u(unsigned *p, unsigned v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); }
QMOE_DEV unsigned ld_sys_u(const unsigned *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); }
QMOE_DEV unsigned *sy(const DecodeArgs &a, int line) { return a.sync + (size_t)line * SY_LINE; }
QMOE_DEV void give_up(const DecodeArgs &a) { st_sys_u(sy(a, SY_STATUS), 1u); }

// Bounded wait of the whole workgroup until the n tagged words p[i * stride] carry tag ep
// (used on one word per producer, as a cheap first test before a full fetch).
QMOE_DEV void wait_tags(const DecodeArgs &a, const uint64_t *p, int n, int stride, unsigned ep) {
  for (unsigned it = 0;; ++it) {
    bool ok = true;
    for (int i = threadIdx.x; i < n; i += DEC_THREADS) ok &= tag_is(ld_tag(p + (size_t)i * stride), ep);
    if (__syncthreads_and(ok)) return;
    if (it == WAIT_LIMIT) {
      if (threadIdx.x == 0) give_up(a);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Bounded fetch, by the whole workgroup, of n tagged words (word i at addr(i)): f(i, value)
// is called for every word that carries tag ep (possibly more than once), and the fetch is
// repeated until all of them do.  PT words per thread are loaded together per pass.
template <int PT, class Addr, class F>
QMOE_DEV void fetch_tags(const DecodeArgs &a, int n, unsigned ep, Addr addr, F f) {
  for (int base = 0; base < n; base += DEC_THREADS * PT) {
    for (unsigned it = 0;; ++it) {
      uint64_t v[PT];
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const int i = base + (int)threadIdx.x + j * DEC_THREADS;
        v[j] = (i < n) ? ld_tag(addr(i)) : 0;
      }
      bool ok = true;
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const int i = base + (int)threadIdx.x + j * DEC_THREADS;
        if (i < n) {
          if (tag_is(v[j], ep)) f(i, tag_val(v[j]));
          else ok = false;
        }
      }
      if (__syncthreads_and(ok)) break;
      if (it == WAIT_LIMIT) {
        if (threadIdx.x == 0) give_up(a);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

// Whole workgroup: wait until the first word of every combining workgroup of the previous
// layer carries its tag (ep - 1), then fetch the H bf16 outputs into dst.
QMOE_DEV void dec_fetch_x(const DecodeArgs &a, unsigned ep, uint16_t *dst) {
  const uint64_t *src = a.xin + (size_t)(blockIdx.x % X_COPIES) * a.x_copy;
  const unsigned tg = ep - 1u;
  const int rows = TILE_ROWS * dec_tiles_per_wg(a.wpt);
  wait_tags(a, src, (a.H + rows - 1) / rows, rows / 2, tg);
  fetch_tags<6>(a, a.H / 2, tg, [&](int i) { return src + i; },
                [&](int i, float v) { ((uint32_t *)dst)[i] = __float_as_uint(v); });
}

// ---------------------------------------------------------------- R: router
template <bool ST>
QMOE_DEV void dec_router(const DecodeArgs &a, int rb, unsigned ep, char *smem) {
  QMOE_TL_ROLE(a, TL_R);
  RouterArgs ra;
  ra.x = a.x; ra.rq = a.rq; ra.rs = a.rs; ra.rb = a.rb; ra.rscale = a.rscale; ra.pes = a.pes;
  ra.lbias = a.lbias; ra.T = 1; ra.H = a.H; ra.E = a.E; ra.k = a.k; ra.inv_sqrt_h = a.inv_sqrt_h;
  ra.logits = nullptr; ra.logits_tag = a.logits; ra.tag = ep;
  ra.tag_copies = LOGIT_COPIES; ra.tag_copy_stride = a.logit_copy;
  ra.topk_idx = nullptr; ra.topk_w = nullptr;
  ra.cnt_all = nullptr; ra.counts = nullptr; ra.offsets = nullptr;
  ra.sorted = nullptr; ra.active = nullptr; ra.n_active = nullptr; ra.slot_tab = nullptr;
  ra.n_slots = 0; ra.gsum = nullptr;
  if (ST && a.xin) {
    // x staged after the router's own LDS, fetched once the codes are in flight
    uint16_t *xs = (uint16_t *)(smem + al16(router_lds_bytes(a.H, 1)));
    ra.x = xs;
    router_logits_block<1, 1>(ra, 0, rb, smem, [&]() { dec_fetch_x(a, ep, xs); });
  } else {
    router_logits_block<1, 1>(ra, 0, rb, smem);
  }
}

// ---------------------------------------------------------------- top-k (every wave)
// Top-k of the workgroup's routed gate/up (all waves), for E <= 128, by rank: expert i gets
// the 64-bit key (ordered logit << 32) | ~i.  The keys are distinct and their order is the
// order in which the round-by-round selection takes the experts (larger logit first, the
// lower index first among equal logits), so the expert whose key has r keys above it is the
// r-th selection.  Each wave ranks E_pad / 4 experts, every lane of it against one of the
// E_pad / (E_pad / 4) equal parts of the keys (broadcast LDS reads), and the parts' counts are
// added by lane swaps; the experts of rank < k write themselves to their place.  Every wave
// then forms the k weights itself.
template <int NCH>
QMOE_DEV void dec_rank_select(const uint64_t *key, int k, int32_t *tk_e, float *tk_l) {
  constexpr int EP = NCH * WAVE, CPW = EP / DEC_W, PP = WAVE / CPW, SPAN = EP / PP;
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  const int c = CPW * wv + lane % CPW, part = lane / CPW;
  const uint64_t mine = key[c];
  const uint64_t *kp = key + SPAN * part;
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < SPAN; ++j) r += kp[j] > mine ? 1u : 0u;
  if (PP == 4) r += (uint32_t)__float_as_int(xor16(__int_as_float((int)r)));
  r += (uint32_t)__float_as_int(xor32(__int_as_float((int)r)));
  if (part == 0 && mine != 0 && r < (uint32_t)k) {
    tk_e[r] = c;
    tk_l[r] = topk_ord_logit((uint32_t)(mine >> 32));
  }
}

// The workgroup's expert for routing slot `slot`, returned to every thread (its routing
// weight is applied by the routed down workgroups); with publish, the top-k ids and weights
// are also written out for the routed down workgroups and the caller.  The E logits are
// fetched (tagged) into LDS; for E <= 128 the whole workgroup ranks them as above, otherwise
// every wave runs the round-by-round selection in registers over a quarter of them and the
// four lists are merged by rank.
QMOE_DEV int dec_topk(const DecodeArgs &a, unsigned ep, int slot, bool publish, char *smem,
                      const DecLds &L) {
  const int tid = threadIdx.x, wv = tid / WAVE, lane = tid % WAVE;
  const int E = a.E, k = a.k, nch = topk_chunks(E);
  float *pes = (float *)(smem + L.pes);
  int32_t *tk_e = (int32_t *)(smem + L.tks);
  float *tk_l = (float *)(tk_e + MAX_TOPK);
  const bool chosen = __builtin_amdgcn_readfirstlane(wv) == (int)(blockIdx.x % DEC_W);
  // per-expert scales into LDS (loads in flight while the logits are fetched; only the
  // publishing workgroup forms weights)
  constexpr int PJ = MAX_EXPERTS / DEC_THREADS;
  float pv[PJ];
#pragma unroll
  for (int j = 0; j < PJ; ++j) {
    const int i = tid + j * DEC_THREADS;
    pv[j] = (publish && i < E) ? a.pes[i] : 0.f;
  }
  const uint64_t *lg = a.logits + (size_t)(blockIdx.x % LOGIT_COPIES) * a.logit_copy;
  int my_e = 0;
  float my_l = 0.f;
  if (nch <= 2) {
    uint64_t *key = (uint64_t *)(smem + L.tk);
    for (int i = E + tid; i < nch * WAVE; i += DEC_THREADS) key[i] = 0u;
    fetch_tags<PJ>(a, E, ep, [&](int i) { return lg + i; }, [&](int i, float v) {
      key[i] = ((uint64_t)topk_ord(v) << 32) | (uint32_t)~i;
    });
    if (publish) {
#pragma unroll
      for (int j = 0; j < PJ; ++j) {
        const int i = tid + j * DEC_THREADS;
        if (i < E) pes[i] = pv[j];
      }
    }
    __syncthreads();
    if (nch <= 1) dec_rank_select<1>(key, k, tk_e, tk_l);
    else dec_rank_select<2>(key, k, tk_e, tk_l);
    __syncthreads();
    const int e_out = min(max(tk_e[slot], 0), E - 1);
    if (!publish || !chosen) return e_out;
    my_e = lane < k ? tk_e[lane] : 0;
    my_l = lane < k ? tk_l[lane] : 0.f;
  } else {
    uint32_t *ord = (uint32_t *)(smem + L.tk);
    for (int i = E + tid; i < nch * WAVE; i += DEC_THREADS) ord[i] = 0u;
    fetch_tags<PJ>(a, E, ep, [&](int i) { return lg + i; },
                   [&](int i, float v) { ord[i] = topk_ord(v); });
    if (publish) {
#pragma unroll
      for (int j = 0; j < PJ; ++j) {
        const int i = tid + j * DEC_THREADS;
        if (i < E) pes[i] = pv[j];
      }
    }
    __syncthreads();
    // two levels: each wave selects the top-k of its quarter of the chunks (in registers, the
    // four waves at once), then the k of the union of the four lists by rank.  The union holds
    // every expert of the overall top-k, and an expert's rank in it is its overall rank.
    uint64_t *cand = (uint64_t *)(ord + nch * WAVE);   // [DEC_W][k] keys, 0: none
    const int cpw = (nch + DEC_W - 1) / DEC_W, c0 = wv * cpw;
    int le;
    float ll;
    topk_select(cpw, [&](int c) { return c < cpw && c0 + c < nch ? ord[(c0 + c) * WAVE + lane] : 0u; },
                k, le, ll);
    if (lane < k) {
      // selections past the quarter's expert count took padding or a taken entry: none
      const int n_sub = min(E, (c0 + cpw) * WAVE) - c0 * WAVE, e = c0 * WAVE + le;
      cand[wv * k + lane] = lane < n_sub ? (((uint64_t)ord[e] << 32) | (uint32_t)~e) : 0ull;
    }
    __syncthreads();
    if (tid < DEC_W * k) {
      const uint64_t mine = cand[tid];
      uint32_t r = 0;
      for (int j = 0; j < DEC_W * k; ++j) r += cand[j] > mine ? 1u : 0u;
      if (mine != 0 && r < (uint32_t)k) {
        tk_e[r] = (int)~(uint32_t)mine;
        tk_l[r] = topk_ord_logit((uint32_t)(mine >> 32));
      }
    }
    __syncthreads();
    const int e_out = min(max(tk_e[slot], 0), E - 1);
    if (!publish || !chosen) return e_out;
    my_e = lane < k ? tk_e[lane] : 0;
    my_l = lane < k ? tk_l[lane] : 0.f;
  }
  const float my_w = topk_weight(my_e, my_l, k, pes);
  if (lane < k) {
    a.topk_idx[lane] = my_e;
    a.topk_w[lane] = my_w;
    // and for the routed down workgroups, which take their expert from these words
    for (int c = 0; c < TK_COPIES; ++c) {
      st_tag(a.tk + (size_t)c * 2 * MAX_TOPK + lane, ep, __int_as_float(my_e));
      st_tag(a.tk + (size_t)c * 2 * MAX_TOPK + MAX_TOPK + lane, ep, my_w);
    }
  }
  return min(max(tk_e[slot], 0), E - 1);
}

// ---------------------------------------------------------------- gate/up of one tile, one token
template <bool ST>
QMOE_DEV void dec_stage_x(const DecodeArgs &a, unsigned ep, char *smem, const DecLds &L) {
  uint16_t *xl = (uint16_t *)(smem + L.x);
  if (ST && a.xin) {
    dec_fetch_x(a, ep, xl);
    // in place: the same 32-column sums as for x read from memory
    stage_rows_bf16<DEC_THREADS>(xl, a.H, 1, [](int) { return 0; }, xl, (float *)(smem + L.xs));
  } else {
    stage_rows_bf16<DEC_THREADS>(a.x, a.H, 1, [](int) { return 0; }, xl, (float *)(smem + L.xs));
  }
}

// ---------------------------------------------------------------- k-steps on the matrix cores
// A wave's batch of loaded k-steps (codes and scale|bias words, load_batch layout).
struct DownRegs {
  qmoe_u32x4 cv[KB_DEC];
  uint32_t sb[KB_DEC];
  int nk;
};

// One k-step (u of the wave's batch d, k-step kb0 + u, activations at column block
// ((kb0 + u) >> kshift) - g0) of a 32-row tile on the matrix cores.  A operand: lane l gives
// row l % 16, columns 8 (l / 16) + [0, 8) of each column half, from arow (zero where zero_a);
// B operand: the k-step's codes after four lane swaps (mfma.h).  Row 0 receives the bias
// term (b - 128 s) times the group sum of the A rows (hs: 32-column sums).  acc0 / acc1:
// tile rows 0..15 / 16..31, lane l < 16 holding A rows 0 and 1 of tile row l (+ 16).
QMOE_DEV void dec_kstep_mf(const DownRegs &d, int u, int nk, int kb0, int g0, int kshift,
                            const uint16_t *arow, const float *hs, bool zero_a,
                            qmoe_f32x4 &acc0, qmoe_f32x4 &acc1) {
  // steps past the wave's count re-read the last one and are scaled by 0
  const bool valid = u < nk;
  const int col = (((kb0 + min(u, nk - 1)) >> kshift) - g0) * GROUP;
  qmoe_u32x4 xa0 = *(const qmoe_u32x4 *)(arow + col);
  qmoe_u32x4 xa1 = *(const qmoe_u32x4 *)(arow + col + 32);
  if (zero_a) {
    xa0 = qmoe_u32x4{0u, 0u, 0u, 0u};
    xa1 = qmoe_u32x4{0u, 0u, 0u, 0u};
  }
  const qmoe_u32x4 cv = d.cv[u];
  const auto x02 = __builtin_amdgcn_permlane32_swap(cv.x, cv.z, false, false);
  const auto x13 = __builtin_amdgcn_permlane32_swap(cv.y, cv.w, false, false);
  const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
  const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
  qmoe_f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
  t0 = mfma16(xa0, y01[0], t0);
  t1 = mfma16(xa0, y01[1], t1);
  t0 = mfma16(xa1, y23[0], t0);
  t1 = mfma16(xa1, y23[1], t1);
  // lane l < 16 holds rows 0, 1 of output column l: tile row l (block 0) and 16 + l
  // (block 1), whose scale|bias word lane l + 16 loaded
  const uint32_t sb0 = d.sb[u], sb1 = __float_as_uint(xor16(__uint_as_float(sb0)));
  const float s0 = valid ? bf16lo(sb0) : 0.f, s1 = valid ? bf16lo(sb1) : 0.f;
  const float c0 = valid ? fmaf(-128.f, bf16lo(sb0), bf16hi(sb0)) : 0.f;
  const float c1 = valid ? fmaf(-128.f, bf16lo(sb1), bf16hi(sb1)) : 0.f;
  const float g = hs[col / 32] + hs[col / 32 + 1];
  acc0[0] = fmaf(s0, t0[0], acc0[0]);
  acc0[1] = fmaf(s0, t0[1], acc0[1]);
  acc1[0] = fmaf(s1, t1[0], acc1[0]);
  acc1[1] = fmaf(s1, t1[1], acc1[1]);
  acc0[0] = fmaf(c0, g, acc0[0]);
  acc1[0] = fmaf(c1, g, acc1[0]);
}

// 16 gate + 16 up rows of store tile `tile` of block `blk` against the staged x (split-K over
// the four waves); the 16 values silu(g)*u are published (tagged) at h_out[16*tile + r] of
// each of the H_COPIES copies.
QMOE_DEV void dec_gate_up(const DecodeArgs &a, const uint8_t *blk, int tile, uint64_t *h_out,
                          size_t copy_stride, unsigned ep, char *smem, const DecLds &L) {
  const int H = a.H, KS = (H / GROUP) << a.kshift;
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int rr = lane % 32, half = lane / 32;
  const uint16_t *xl = (const uint16_t *)(smem + L.x);
  const float *xs = (const float *)(smem + L.xs);
  float *red = (float *)(smem + L.red);
  const uint8_t *tbase = blk + (size_t)tile * KS * KSTEP_BYTES;
  const int ks0 = (KS * wv) / DEC_W, nk = (KS * (wv + 1)) / DEC_W - ks0;
  // each batch's k-steps in straight-line chunks of four (steps past the count re-read the
  // last one and add 0), so that their products overlap
  float acc = 0.f;
  for (int kc = 0; kc < nk; kc += KB_GU) {
    qmoe_u32x4 cv[KB_GU];
    uint32_t sb[KB_GU];
    load_batch<KB_GU>(tbase, ks0, kc, nk, lane, rr, cv, sb);
    const int nb = __builtin_amdgcn_readfirstlane(min(KB_GU, nk - kc));
#pragma unroll
    for (int c = 0; c < KB_GU; c += 4)
      if (c < nb) {
#pragma unroll
        for (int u = c; u < c + 4; ++u) {
          const int col = ((ks0 + kc + min(u, nb - 1)) >> a.kshift) * GROUP + half * 32;
          const float r = kstep_bf16(cv[u], sb[u], xl + col, xs[col / 32]);
          acc += u < nb ? r : 0.f;
        }
      }
  }
  acc += xor32(acc);
  QMOE_TL(a, 3);
  if (half == 0) red[wv * 32 + rr] = acc;
  __syncthreads();
  if (tid < 16 * H_COPIES) {
    const int r = tid % 16, c = tid / 16;
    float g = 0.f, u = 0.f;
    for (int w = 0; w < DEC_W; ++w) { g += red[w * 32 + r]; u += red[w * 32 + 16 + r]; }
    st_tag(h_out + (size_t)c * copy_stride + 16 * tile + r, ep, silu(g) * u);
  }
}

// This wave's k-steps [kb0, kb0 + nk) (nk <= KB_DEC) of output tile `tile` of the down
// section of block `blk` (input width K).
QMOE_DEV void dec_down_load(const DecodeArgs &a, const uint8_t *blk, int K, int tile, int kb0,
                            int nk, DownRegs &d) {
  const int lane = threadIdx.x % WAVE;
  const BlockGeom geo = block_geom(a.H, K, a.kshift);
  const uint8_t *tbase = blk + geo.gu_bytes + (size_t)tile * geo.d_ks * KSTEP_BYTES;
  d.nk = nk;
  if (nk > 0) load_batch<KB_DEC>(tbase, kb0, 0, nk, lane, lane % 32, d.cv, d.sb);
}

// Fetch the n tagged h values src[0..n) (n a multiple of 64) and stage them as hi/lo bf16
// planes with 32-column sums of hi + lo.  Called after the caller's weight loads were issued:
// those are awaited first, so that polling starts about when h is due.
QMOE_DEV void dec_stage_h(const DecodeArgs &a, const uint64_t *src, int n, unsigned ep, char *smem,
                          const DecLds &L) {
  float *hf = (float *)(smem + L.hf);
  uint16_t *hh = (uint16_t *)(smem + L.hh), *hl = (uint16_t *)(smem + L.hl);
  float *hs = (float *)(smem + L.hs);
  drain_memory();
  fetch_tags<4>(a, n, ep, [&](int i) { return src + i; }, [&](int i, float v) { hf[i] = v; });
  for (int c = threadIdx.x; c < n / 8; c += DEC_THREADS) {
    uint32_t hi2[4], lo2[4];
    float p = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v0 = hf[8 * c + 2 * q], v1 = hf[8 * c + 2 * q + 1];
      const uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
      const uint32_t l0 = f32_to_bf16_bits(v0 - __uint_as_float(h0 << 16));
      const uint32_t l1 = f32_to_bf16_bits(v1 - __uint_as_float(h1 << 16));
      hi2[q] = h0 | (h1 << 16);
      lo2[q] = l0 | (l1 << 16);
      p += (__uint_as_float(h0 << 16) + __uint_as_float(l0 << 16)) +
           (__uint_as_float(h1 << 16) + __uint_as_float(l1 << 16));
    }
    *(qmoe_u32x4 *)(hh + 8 * c) = qmoe_u32x4{hi2[0], hi2[1], hi2[2], hi2[3]};
    *(qmoe_u32x4 *)(hl + 8 * c) = qmoe_u32x4{lo2[0], lo2[1], lo2[2], lo2[3]};
    p += xor1(p);
    p += xor2(p);
    if ((c & 3) == 0) hs[c / 4] = p;
  }
  __syncthreads();
}

// This wave's partial dot products for its 32 rows over its loaded k-steps, on the matrix
// cores; local k-step u of the wave is k-step kb0 + u, whose activations are column block
// ((kb0 + u) >> kshift) - g0 of the staged h (staged from group g0 on).  The A operand holds
// the one token's h as two rows, the hi plane in row 0 and the lo plane in row 1 (the other
// 14 rows zero); the B operand is the k-step's codes, re-laid by four lane swaps as in the
// multi-token kernels (mfma.h).  Per k-step and 16-row block the products of the two column
// halves are scaled by the row's scale, and (b - 128 s) times the group's sum of hi + lo is
// added to row 0; rows 0 and 1 added give the 32 sums, which go to red[wave][row].
QMOE_DEV void dec_down_dot(const DownRegs &d, int kb0, int g0, int kshift, char *smem,
                           const DecLds &L) {
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  const int m = lane % 16, kc = lane / 16;
  const uint16_t *hh = (const uint16_t *)(smem + L.hh), *hl = (const uint16_t *)(smem + L.hl);
  const uint16_t *arow = (m == 1 ? hl : hh) + 8 * kc;   // rows >= 2 read row 0 and zero it
  const float *hs = (const float *)(smem + L.hs);
  float *red = (float *)(smem + L.red);
  const int nk = __builtin_amdgcn_readfirstlane(d.nk);
  qmoe_f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  if (nk > 0) {
    // straight-line code for the first half of the batch (the usual count), so that the
    // steps' products overlap; the second half only where a wave has more
#pragma unroll
    for (int u = 0; u < KB_DEC / 2; ++u)
      dec_kstep_mf(d, u, nk, kb0, g0, kshift, arow, hs, m >= 2, acc0, acc1);
    if (nk > KB_DEC / 2) {
#pragma unroll
      for (int u = KB_DEC / 2; u < KB_DEC; ++u)
        dec_kstep_mf(d, u, nk, kb0, g0, kshift, arow, hs, m >= 2, acc0, acc1);
    }
  }
  if (lane < 16) {
    red[wv * 32 + lane] = acc0[0] + acc0[1];
    red[wv * 32 + 16 + lane] = acc1[0] + acc1[1];
  }
}

// ---------------------------------------------------------------- roles
QMOE_DEV void dec_shared_down(const DecodeArgs &a, int b, unsigned ep, char *smem, const DecLds &L) {
  const int tiles_d = a.H / TILE_ROWS;
  const int tile = b % tiles_d, c = b / tiles_d;
  const int NG = a.Is / GROUP;
  const int g0 = (NG * c) / a.nc, g1 = (NG * (c + 1)) / a.nc;   // this chunk's groups
  const int kb0 = g0 << a.kshift, kb1 = g1 << a.kshift;        // and its k-steps
  const int wv = threadIdx.x / WAVE;
  const int n = kb1 - kb0;
  const int w0 = (n * wv) / DEC_W, w1 = (n * (wv + 1)) / DEC_W;
  // once the first router workgroup has published (so that the router's loads go first; the
  // last one's word comes later and then leaves these loads to compete with the routed gate/up
  // stream), load the weights, then wait for h_shared
  QMOE_TL_ROLE(a, TL_SD);
  wait_tags(a, a.logits + (size_t)(blockIdx.x % LOGIT_COPIES) * a.logit_copy, 1, 1, ep);
  QMOE_TL(a, 1);
  DownRegs d;
  dec_down_load(a, a.shared, a.Is, tile, kb0 + w0, w1 - w0, d);
  drain_memory();
  QMOE_TL(a, 2);
  dec_stage_h(a, a.h_sh + (size_t)(tile % H_COPIES) * a.hsh_copy + (size_t)g0 * GROUP,
              (g1 - g0) * GROUP, ep, smem, L);
  QMOE_TL(a, 3);
  dec_down_dot(d, kb0 + w0, g0, a.kshift, smem, L);
  __syncthreads();
  if (threadIdx.x < 32) {
    const float *red = (const float *)(smem + L.red);
    float yv = 0.f;
    for (int w = 0; w < DEC_W; ++w) yv += red[w * 32 + threadIdx.x];
    st_tag(a.y_sh + (size_t)c * a.H + TILE_ROWS * tile + threadIdx.x, ep, yv);
  }
}

template <bool ST>
QMOE_DEV void dec_routed_down(const DecodeArgs &a, int b, unsigned ep, char *smem, const DecLds &L) {
  const int tiles_d = a.H / TILE_ROWS, tpw = dec_tiles_per_wg(a.wpt);
  const int groups = (tiles_d + tpw - 1) / tpw;
  const int slot = b / groups, g = b % groups;
  const int tid = threadIdx.x, wv = tid / WAVE;
  // expert and weight of the slot from the top-k the first routed gate/up workgroup published
  // (selected from the same logits by the same code: these workgroups have time to spare and
  // leave the SIMDs to the gate/up workgroups, whose selection is on the critical path)
  QMOE_TL_ROLE(a, TL_RD);
  int32_t *tk_e = (int32_t *)(smem + L.tks);
  float *tk_w = (float *)(tk_e + MAX_TOPK);
  const uint64_t *tks = a.tk + (size_t)(blockIdx.x % TK_COPIES) * 2 * MAX_TOPK;
  fetch_tags<1>(a, 2 * a.k, ep,
                [&](int i) { return tks + (i < a.k ? i : MAX_TOPK + i - a.k); },
                [&](int i, float v) {
                  if (i < a.k) tk_e[i] = __float_as_int(v); else tk_w[i - a.k] = v;
                });
  QMOE_TL(a, 1);
  const int e = min(max(tk_e[slot], 0), a.E - 1);
  const float w = tk_w[slot];
  const int KS = (a.I / GROUP) << a.kshift;
  const int tile = g * tpw + wv / a.wpt, part = wv % a.wpt;
  const int kb0 = (KS * part) / a.wpt, kb1 = (KS * (part + 1)) / a.wpt;
  DownRegs d;
  dec_down_load(a, a.experts + (size_t)e * a.stride, a.I, min(tile, tiles_d - 1), kb0,
                tile < tiles_d ? kb1 - kb0 : 0, d);
  drain_memory();
  QMOE_TL(a, 2);
  dec_stage_h(a, a.h_r + (size_t)(g % H_COPIES) * a.hr_copy + (size_t)slot * a.I, a.I, ep, smem, L);
  QMOE_TL(a, 3);
  dec_down_dot(d, kb0, 0, a.kshift, smem, L);
  __syncthreads();
  QMOE_TL(a, 4);
  // row r of this group (tile r / 32 of the group): the wpt waves of its tile add up
  const float *red = (const float *)(smem + L.red);
  const int row0 = g * TILE_ROWS * tpw;
  const int nr = min(TILE_ROWS * tpw, a.H - row0);
  const int r = tid;
  const bool mine = r < nr;
  float yv = 0.f;
  if (mine) {
    const int t = r / TILE_ROWS, rw = r % TILE_ROWS;
    for (int p = 0; p < a.wpt; ++p) yv += red[(t * a.wpt + p) * 32 + rw];
    yv *= w;
  }
  if (slot < a.k - 1) {
    if (mine) st_tag(a.y_r + (size_t)slot * a.H + row0 + r, ep, yv);
    QMOE_TL(a, 6);
    return;
  }
  // last slot: combine the rows of this group.  The residual rows, the gain and the layer
  // scalar are read first, so that their loads overlap the wait for the other slots' rows.
  // Residual rows: from memory, or from the previous layer's tagged output (complete by now:
  // this workgroup's h depends on all of it).
  float xr = 0.f;
  if (ST && a.xin) {
    uint32_t *xw = (uint32_t *)(smem + L.xw);
    const uint64_t *src = a.xin + (size_t)(blockIdx.x % X_COPIES) * a.x_copy + row0 / 2;
    fetch_tags<1>(a, nr / 2, ep - 1u, [&](int i) { return src + i; },
                  [&](int i, float v) { xw[i] = __float_as_uint(v); });
    if (mine) xr = bf16_to_f32((uint16_t)(xw[r / 2] >> (16 * (r & 1))));
  } else if (mine) {
    xr = bf16_to_f32(a.x[row0 + r]);
  }
  const float gr = (a.gain && mine) ? a.gain[row0 + r] : 0.f;
  const float lsc = a.lscale ? *a.lscale : 1.f;
  const int nsrc = a.k - 1 + (a.shared ? a.nc : 0);
  float *comb = (float *)(smem + L.comb);
  fetch_tags<4>(a, nsrc * nr, ep,
                [&](int i) {
                  const int s = i / nr, rw = i % nr;
                  return (s < a.k - 1) ? a.y_r + (size_t)s * a.H + row0 + rw
                                       : a.y_sh + (size_t)(s - (a.k - 1)) * a.H + row0 + rw;
                },
                [&](int i, float v) { comb[i] = v; });
  QMOE_TL(a, 5);
  // Arrival of this combining workgroup, issued now and read at the end.  Once every
  // combining workgroup has its inputs, every workgroup of the launch has published its part
  // and so has read the epoch: the last to arrive may advance it.  (No drain first: the
  // launch's outputs reach the next launch through the kernel boundary, not through the
  // epoch.)
  unsigned old = 0u;
  if (a.advance && tid == 0)
    old = __hip_atomic_fetch_add(a.lcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float m = 0.f;  // routed rows (router-weighted) + shared row
  if (mine) {
    m = yv;
    for (int s = 0; s < a.k - 1; ++s) m += comb[s * nr + r];
    float sh = 0.f;
    for (int s = a.k - 1; s < nsrc; ++s) sh += comb[s * nr + r];
    m += sh;
  }
  float o = 0.f;
  if (a.gain) {
    // post-combine norm: every combining workgroup publishes the sum of m^2 over its rows,
    // reads all of them (summed in the same order everywhere) and finishes its rows.  These
    // are the only waits on higher workgroup indices in the launch; they cannot block, because
    // the combining workgroups are far fewer than the workgroups the device holds at once and
    // every other role finishes without waiting on them.
    float *nr_lds = (float *)(smem + L.nrm);  // [DEC_W] wave sums, then [groups] partials
    const float ss = wave_sum(mine ? m * m : 0.f);
    if (tid % WAVE == 0) nr_lds[wv] = ss;
    __syncthreads();
    if (tid == 0) {
      float p = 0.f;
      for (int i = 0; i < DEC_W; ++i) p += nr_lds[i];
      st_tag(a.nrm + g, ep, p);
    }
    float *part = nr_lds + DEC_W;
    fetch_tags<1>(a, groups, ep, [&](int i) { return a.nrm + i; },
                  [&](int i, float v) { part[i] = v; });
    float tot = 0.f;
    for (int i = 0; i < groups; ++i) tot += part[i];
    o = xr + gr * (m * (1.f / sqrtf(tot / (float)a.H + RMS_EPS)));
  } else {
    o = xr + m;
  }
  if (a.lscale) o *= lsc;
  const uint32_t ob = mine ? f32_to_bf16_bits(o) : 0u;
  if (mine) {
    a.out[row0 + r] = (uint16_t)ob;
    if (a.out_f32) a.out_f32[row0 + r] = o;
  }
  if (ST && a.xout) {
    // rows r, r + 1 (same wave) as one tagged pair in every copy
    const uint32_t hi = (uint32_t)__shfl_down((int)ob, 1, WAVE);
    if (mine && (r & 1) == 0)
      for (int c = 0; c < X_COPIES; ++c)
        st_tag(a.xout + (size_t)c * a.x_copy + (row0 + r) / 2, ep, __uint_as_float(ob | (hi << 16)));
  }
  // the last combining workgroup of the launch to arrive advances the epoch
  if (a.advance && tid == 0 && old == (unsigned)groups - 1u) {
    __hip_atomic_store(a.lcnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st_sys_u(sy(a, SY_EPOCH), ep);
  }
  QMOE_TL(a, 6);
}

// Block b (of one layer) with tag ep.
template <bool ST>
QMOE_DEV void decode_block(const DecodeArgs &a, int b, unsigned ep, char *smem) {
  const int Kc_sh = a.shared ? GROUP * ((a.Is / GROUP + a.nc - 1) / a.nc) : 0;
  const DecLds L = dec_lds(a.H, a.E, a.k, a.I, Kc_sh, a.nc, a.wpt);
  QMOE_TL(a, 0);
  if (b < a.nR) {
    dec_router<ST>(a, b, ep, smem);
    QMOE_TL(a, 1);
    QMOE_TL(a, 6);
    return;
  }
  b -= a.nR;
  if (b < a.nSG) {
    QMOE_TL_ROLE(a, TL_SG);
    dec_stage_x<ST>(a, ep, smem, L);
    __syncthreads();   // (no wait for the router: measured slightly faster than letting it go first)
    QMOE_TL(a, 1);
    dec_gate_up(a, a.shared, b, a.h_sh, a.hsh_copy, ep, smem, L);
    QMOE_TL(a, 6);
    return;
  }
  b -= a.nSG;
  if (b < a.nRG) {
    QMOE_TL_ROLE(a, TL_RG);
    const int tiles_r = a.I / 16;
    const int slot = b / tiles_r, tile = b % tiles_r;
    dec_stage_x<ST>(a, ep, smem, L);
    QMOE_TL(a, 1);
    const int e = dec_topk(a, ep, slot, b == 0, smem, L);
    QMOE_TL(a, 2);
    dec_gate_up(a, a.experts + (size_t)e * a.stride, tile, a.h_r + (size_t)slot * a.I, a.hr_copy, ep,
                smem, L);
    QMOE_TL(a, 6);
    return;
  }
  b -= a.nRG;
  if (b < a.nSD) {
    dec_shared_down(a, b, ep, smem, L);
    QMOE_TL(a, 6);
    return;
  }
  b -= a.nSD;
  if (b < a.nRD) dec_routed_down<ST>(a, b, ep, smem, L);
}

// One layer (a.lcnt = the SY_DONE line, a.advance = 1; a.xin, a.xout unused).
__global__ void __launch_bounds__(DEC_THREADS) decode_layer_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) char smem[];
  const unsigned ep = ld_sys_u(sy(a, SY_EPOCH)) + 1u;
  decode_block<false>(a, blockIdx.x, ep, smem);
}

// n_layers chained layers of one token; a holds the shared shape and hand-off buffers, tab the
// per-layer pointers, xb[0..1] the two tagged x buffers.  out, out_f32 are [n_layers][H]; the
// top-k outputs are [n_layers][k] when tk_per_layer, else one scratch row for every layer.
__global__ void __launch_bounds__(DEC_THREADS)
decode_stack_kernel(DecodeArgs a, const DecLayer *tab, uint64_t *xb0, uint64_t *xb1, int n_layers,
                    int tk_per_layer) {
  extern __shared__ __align__(16) char smem[];
  const int per = a.nR + a.nSG + a.nRG + a.nSD + a.nRD;
  const int l = blockIdx.x / per;
  const unsigned ep = ld_sys_u(sy(a, SY_EPOCH)) + 1u + (unsigned)l;
  const DecLayer D = tab[l];
  a.rq = D.rq; a.rs = D.rs; a.rb = D.rb; a.rscale = D.rscale; a.pes = D.pes; a.lbias = D.lbias;
  a.experts = D.experts; a.shared = D.shared; a.gain = D.gain; a.lscale = D.lscale;
  a.out += (size_t)l * a.H;
  if (a.out_f32) a.out_f32 += (size_t)l * a.H;
  if (tk_per_layer) { a.topk_idx += (size_t)l * a.k; a.topk_w += (size_t)l * a.k; }
  a.xin = l > 0 ? ((l - 1) & 1 ? xb1 : xb0) : nullptr;
  a.xout = l + 1 < n_layers ? (l & 1 ? xb1 : xb0) : nullptr;
  a.lcnt = sy(a, SY_DONE);
  a.advance = l == n_layers - 1;
  decode_block<true>(a, blockIdx.x % per, ep, smem);
}

// Writes entries [first, first + n) of the per-layer table (n <= DEC_TAB_CHUNK).
constexpr int DEC_TAB_CHUNK = 32;
struct DecTabChunk {
  DecLayer L[DEC_TAB_CHUNK];
};
__global__ void dec_table_kernel(DecTabChunk c, DecLayer *tab, int first, int n) {
  if ((int)threadIdx.x < n) tab[first + threadIdx.x] = c.L[threadIdx.x];
}

}  // namespace qmoe
