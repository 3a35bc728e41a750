// Router and bucketing kernels.
//
// Router (TurboFieldfare post, section "TurboFieldfare의 전문가 스트리밍 구조", router
// listing): scale-free RMS norm of the hidden state, times router_scale / sqrt(hidden), an
// 8-bit affine projection to one logit per expert, the k largest logits, softmax over those
// k logits only, times per_expert_scale of each kept expert.  The 8-bit format is the MLX
// affine one of section "TurboFieldfare가 메모리를 아끼는 방식" (w = s*q + b, unsigned q,
// bf16 s and b per 64 inputs).
//
// Bucketing groups token->expert assignments by expert so that one expert read serves every
// row routed to it (the same post's 128-token prefill chunks).
#pragma once
#include "common.h"

namespace qmoe {

constexpr int ROUTER_WAVES = 4;
constexpr int ROUTER_THREADS = ROUTER_WAVES * WAVE;

struct RouterArgs {
  const uint16_t *x;          // [T, H] bf16
  const uint8_t *rq;          // [E, H]
  const uint16_t *rs;         // [E, H/64]
  const uint16_t *rb;         // [E, H/64]
  const float *rscale;        // [H] or null
  const float *pes;           // [E]
  const float *lbias;         // [E] or null
  int T, H, E, k;
  float inv_sqrt_h;           // fp32(1/sqrt(H))
  float *logits;              // [T, E] (unless logits_tag is set)
  uint64_t *logits_tag;       // or null: logits published as tagged words (tag << 32 | bits),
  unsigned tag;               //   tag_copies copies of [T, E], tag_copy_stride words apart
  int tag_copies;
  size_t tag_copy_stride;
  int32_t *topk_idx;          // [T, k]
  float *topk_w;              // [T, k]
  unsigned *cnt_all;          // [1] completion counter (zero on entry, zero on exit)
  // optional fused bucketing (layer path); null counts -> skip
  int32_t *counts, *offsets, *sorted, *active, *n_active;
  int32_t *slot_tab;          // [n_slots][4] block table {expert, first bucket position, rows,
                              //   first flat id or -1} (bucket_offsets)
  float *gsum;                // [T, H/64] sums of every 64-column group of x, or null
  int n_slots;
};


// ---------------------------------------------------------------- top-k selection (one wave)
// Order: larger logit first, equal logits -> lower expert index.  A NaN logit ranks as -inf
// (so every selected index is a valid expert id whatever the logits hold) and -0 as +0.
// A logit becomes 32 bits whose unsigned order is its numeric order; 0 lies below every
// logit and marks padding and taken entries.  Lane l holds experts l + 64 c (c < chunks) in
// registers; each of the k rounds takes the wave maximum (a rotate-max inside each 16-lane
// row by DPP, then the four row results read as scalars), and one ballot per chunk finds the
// lowest expert index holding it, which is then removed.  No LDS, no barrier.  The chunk
// count is compiled in (1, 2, 4, 8 or 16) so that the rounds have no runtime guards.
constexpr int TOPK_NCH = MAX_EXPERTS / WAVE;   // register chunks per lane

QMOE_DEV uint32_t topk_ord(float l) {
  if (!(l == l)) l = -INFINITY;
  if (l == 0.f) l = 0.f;
  const uint32_t u = __float_as_uint(l);
  return u ^ ((u & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u);
}
QMOE_DEV float topk_ord_logit(uint32_t v) {
  return __uint_as_float(v ^ ((v & 0x80000000u) ? 0x80000000u : 0xFFFFFFFFu));
}
inline __host__ __device__ int topk_chunks(int E) { return (E + WAVE - 1) / WAVE; }

QMOE_DEV uint32_t dpp_ror_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));  // ror 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));  // ror 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // ror 4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // ror 8
  return v;
}
QMOE_DEV uint32_t wave_max_uniform(uint32_t v) {
  v = dpp_ror_max(v);
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// The selection over NCH register chunks; load(c) gives the lane's ordered logit of expert
// lane + 64 c (0 for padding).  Lane j < k receives the j-th selection (expert, logit); the
// others receive (0, 0).
template <int NCH, class Load>
QMOE_DEV void topk_run(Load load, int k, int &my_e, float &my_l) {
  const int lane = threadIdx.x % WAVE;
  uint32_t u[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) u[c] = load(c);
  my_e = 0;
  my_l = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t lm = u[0];
#pragma unroll
    for (int c = 1; c < NCH; ++c) lm = max(lm, u[c]);
    const uint32_t M = wave_max_uniform(lm);
    int e = -1;
#pragma unroll
    for (int c = NCH - 1; c >= 0; --c) {
      const unsigned long long m = __ballot(u[c] == M);
      if (m) e = WAVE * c + __builtin_ctzll(m);
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (WAVE * c + lane == e) u[c] = 0;
    if (lane == j) {
      my_e = e;
      my_l = topk_ord_logit(M);
    }
  }
}

// nch = topk_chunks(E) chunks, rounded up to a compiled width (load(c) must give 0 past nch).
template <class Load>
QMOE_DEV void topk_select(int nch, Load load, int k, int &my_e, float &my_l) {
  if (nch <= 1) topk_run<1>(load, k, my_e, my_l);
  else if (nch <= 2) topk_run<2>(load, k, my_e, my_l);
  else if (nch <= 4) topk_run<4>(load, k, my_e, my_l);
  else if (nch <= 8) topk_run<8>(load, k, my_e, my_l);
  else topk_run<TOPK_NCH>(load, k, my_e, my_l);
}

// Softmax over the k selected logits (lane j < k holds the j-th, the largest in lane 0), times
// per_expert_scale (global or LDS).  Lanes >= k get 0.
QMOE_DEV float topk_weight(int my_e, float my_l, int k, const float *pes) {
  const int lane = threadIdx.x % WAVE;
  const float vmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const float z = (lane < k) ? expf(my_l - vmax) : 0.f;
  const float zsum = wave_sum(z);
  return (lane < k) ? (z / zsum) * pes[my_e] : 0.f;
}

// ---------------------------------------------------------------- bucketing (one workgroup)
// Stable counting sort of N = T*k assignments by expert (ids outside [0, E) are dropped):
// position of assignment f = (first position of its expert) + (number of assignments f' < f
// with the same expert).  Optionally also writes the block table used by the expert kernels
// (bucket_offsets).  get(f) returns the expert id of assignment f.

// Per-expert totals -> counts, offsets, active list, block table; cnt[e] becomes the
// expert's first position.  first[e]: smallest flat id of the expert.  The block table cuts
// the rows of every active expert, in expert order, into blocks of BUCKET_BLOCK_ROWS: entry b
// = {expert, bucket position of the block's first row, rows, flat id of that row for the
// expert's first block, else -1}; entries from the number of blocks up to n_slots have zero
// rows.
constexpr int BUCKET_BLOCK_ROWS = 16;
constexpr int BUCKET_MAX_N = 1 << 21;     // assignments of one bucketing call (T x k limits)
inline __host__ __device__ int bucket_max_blocks(int N, int E) {
  return N / BUCKET_BLOCK_ROWS + (N < E ? N : E);
}
// The exclusive scan over experts carries (rows, blocks, active flag) in one 64-bit word:
// rows in bits 40..63, blocks in bits 20..39, flags in bits 0..19.  Totals stay inside their
// fields for N <= BUCKET_MAX_N and E <= MAX_EXPERTS (blocks <= N/16 + E < 2^20).
QMOE_HD long long bucket_scan_word(long long c) {
  return (c << 40) | (((c + BUCKET_BLOCK_ROWS - 1) / BUCKET_BLOCK_ROWS) << 20) | (c > 0 ? 1 : 0);
}
QMOE_HD int bucket_scan_rows(long long v) { return (int)(v >> 40); }
QMOE_HD int bucket_scan_blocks(long long v) { return (int)((v >> 20) & 0xFFFFF); }
QMOE_HD int bucket_scan_flags(long long v) { return (int)(v & 0xFFFFF); }
// Block b of an expert with c rows starting at bucket position pos: {expert, position of the
// block's first row, rows, the expert's smallest flat id for its first block, else -1}.
QMOE_HD qmoe_u32x4 bucket_block_entry(int e, int c, int pos, int first_e, int b) {
  QMOE_BOUNDS(b >= 0 && b * BUCKET_BLOCK_ROWS < c);
  const int rows = c - b * BUCKET_BLOCK_ROWS;
  return qmoe_u32x4{(uint32_t)e, (uint32_t)(pos + b * BUCKET_BLOCK_ROWS),
                    (uint32_t)(rows < BUCKET_BLOCK_ROWS ? rows : BUCKET_BLOCK_ROWS),
                    b == 0 ? (uint32_t)first_e : 0xFFFFFFFFu};
}

template <int NT>
QMOE_DEV void bucket_offsets(int *cnt, const int *first, int E, int32_t *counts, int32_t *offsets,
                             int32_t *active, int32_t *n_active, int32_t *slot_tab, int n_slots) {
  constexpr int NW = NT / WAVE, BB = BUCKET_BLOCK_ROWS;
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  // exclusive scan of (rows, blocks, active flags) packed as rows << 40 | blocks << 20 | flags
  // (at most 2^21 assignments), E <= MAX_EXPERTS
  const int per = (E + NT - 1) / NT;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  long long own = 0;
  for (int e = e0; e < e1; ++e) own += bucket_scan_word(cnt[e]);
  long long pack = own;
  for (int o = 1; o < WAVE; o <<= 1) {
    const long long up = __shfl_up(pack, o, WAVE);
    if (lane >= o) pack += up;
  }
  __shared__ long long wtot[NW];
  if (lane == WAVE - 1) wtot[wv] = pack;
  __syncthreads();
  long long before = 0, tot = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wv) before += wtot[w];
    tot += wtot[w];
  }
  const long long excl = before + pack - own;
  int run_cnt = bucket_scan_rows(excl), run_blk = bucket_scan_blocks(excl),
      run_act = bucket_scan_flags(excl);
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    counts[e] = c;
    offsets[e] = run_cnt;
    if (c > 0) {
      active[run_act] = e;
      if (slot_tab)
        for (int b = 0; b * BB < c && run_blk + b < n_slots; ++b)
          *(qmoe_u32x4 *)(slot_tab + 4 * (run_blk + b)) = bucket_block_entry(e, c, run_cnt, first[e], b);
      run_blk += (c + BB - 1) / BB;
      ++run_act;
    }
    cnt[e] = run_cnt;
    run_cnt += c;
  }
  const int na = bucket_scan_flags(tot), nb = bucket_scan_blocks(tot);
  if (tid == NT - 1) {
    offsets[E] = bucket_scan_rows(tot);
    *n_active = na;
  }
  if (slot_tab)
    for (int sl = nb + tid; sl < n_slots; sl += NT)
      *(qmoe_u32x4 *)(slot_tab + 4 * sl) = qmoe_u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
}

// Segmented form, for up to BUCKET_SEG_N assignments with segments x experts <=
// BUCKET_SEG_CELLS: the assignments are cut into 64-long segments (one wave each); an
// assignment's rank among the same expert's earlier ones is its rank inside its segment (one
// ballot per bit of the expert id) plus the expert's counts in the earlier segments (a prefix
// per expert).
// Every step is parallel.  lds: bucket_lds_bytes(N, E).
constexpr int BUCKET_SEG_N = 4096, BUCKET_SEG_CELLS = 16384;
inline __host__ __device__ bool bucket_seg_ok(int N, int E) {
  return N <= BUCKET_SEG_N && ((N + WAVE - 1) / WAVE) * E <= BUCKET_SEG_CELLS;
}
inline __host__ __device__ size_t bucket_lds_bytes(int N, int E) {
  return bucket_seg_ok(N, E) ? ((size_t)((N + WAVE - 1) / WAVE) * E + 2 * (size_t)E + N) * 4
                             : (size_t)2 * E * 4;
}

template <int NT, class Get>
QMOE_DEV void bucket_block_seg(Get get, int N, int E, int32_t *counts, int32_t *offsets,
                               int32_t *sorted, int32_t *active, int32_t *n_active,
                               int32_t *slot_tab, int n_slots, int *lds) {
  constexpr int NW = NT / WAVE;
  const int S = (N + WAVE - 1) / WAVE;
  int *cnt = lds;                   // [S][E] counts per segment, then prefix over segments
  int *tot = cnt + S * E;           // [E] totals, then first positions
  int *first = tot + E;             // [E] smallest flat id
  int *er = first + E;              // [N] expert << 8 | rank inside the segment (-1: dropped)
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  for (int i = tid; i < S * E; i += NT) cnt[i] = 0;
  for (int e = tid; e < E; e += NT) first[e] = 0x7FFFFFFF;
  // every id into er[], eight loads per thread in flight
  for (int base = 0; base < N; base += 8 * NT) {
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = base + tid + j * NT;
      v[j] = (f < N) ? get(f) : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = base + tid + j * NT;
      if (f < N) er[f] = v[j];
    }
  }
  __syncthreads();
  // lanes of a segment with the same expert: AND over the id bits of the ballot of that bit
  // (or of its complement), restricted to valid lanes
  const int bits = 32 - __builtin_clz((unsigned)max(E - 1, 1));
  for (int sg = wv; sg < S; sg += NW) {
    const int f = sg * WAVE + lane;
    const int e = (f < N) ? er[f] : -1;
    const bool valid = (f < N) && ((unsigned)e < (unsigned)E);
    unsigned long long same = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool set = (e >> b) & 1;
      const unsigned long long m = __ballot(set);
      same &= set ? m : ~m;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    if (f < N) er[f] = valid ? ((e << 8) | rank) : -1;
    if (valid && rank == 0) {
      // the first lane of each expert in the segment holds its count and smallest flat id
      cnt[sg * E + e] = __popcll(same);
      atomicMin(&first[e], f);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int run = 0;
    for (int sg = 0; sg < S; ++sg) {
      const int c = cnt[sg * E + e];
      cnt[sg * E + e] = run;
      run += c;
    }
    tot[e] = run;
  }
  __syncthreads();
  bucket_offsets<NT>(tot, first, E, counts, offsets, active, n_active, slot_tab, n_slots);
  for (int f = tid; f < N; f += NT) {
    const int v = er[f];
    if (v < 0) continue;
    const int e = v >> 8, rank = v & 0xFF;
    sorted[tot[e] + cnt[(f / WAVE) * E + e] + rank] = f;
  }
}

// General form (any N): LDS histogram, then a stable scatter with one ballot per distinct
// expert of a wave and a per-expert cursor advanced wave by wave.  lds: 2 * E * 4 bytes.
template <int NT, class Get>
QMOE_DEV void bucket_block(Get get, int N, int E, int32_t *counts, int32_t *offsets,
                           int32_t *sorted, int32_t *active, int32_t *n_active, int32_t *slot_tab,
                           int n_slots, int *lds) {
  if (bucket_seg_ok(N, E)) {
    bucket_block_seg<NT>(get, N, E, counts, offsets, sorted, active, n_active, slot_tab, n_slots,
                         lds);
    return;
  }
  constexpr int NW = NT / WAVE;
  int *cnt = lds;                 // [E]
  int *first = lds + E;           // [E] smallest flat id of each expert
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  for (int e = tid; e < E; e += NT) { cnt[e] = 0; first[e] = 0x7FFFFFFF; }
  __syncthreads();
  for (int f = tid; f < N; f += NT) {
    const int e = get(f);
    if ((unsigned)e < (unsigned)E) {
      atomicAdd(&cnt[e], 1);
      atomicMin(&first[e], f);
    }
  }
  __syncthreads();
  bucket_offsets<NT>(cnt, first, E, counts, offsets, active, n_active, slot_tab, n_slots);
  // stable scatter, NT assignments per round
  for (int base = 0; base < N; base += NT) {
    const int f = base + tid;
    const int e = (f < N) ? get(f) : -1;
    const bool valid = (f < N) && ((unsigned)e < (unsigned)E);
    // rank among lower lanes of this wave with the same expert, and the wave's count of it
    int rank = 0, wtotal = 0;
    unsigned long long pending = __ballot(valid);
    while (pending) {
      const int leader = __ffsll((long long)pending) - 1;
      const int el = __shfl(e, leader, WAVE);
      const unsigned long long same = __ballot(valid && e == el);
      if (valid && e == el) {
        rank = __popcll(same & ((1ull << lane) - 1ull));
        wtotal = __popcll(same);
      }
      pending &= ~same;
    }
    for (int w = 0; w < NW; ++w) {
      if (wv == w && valid) {
        const int cur = cnt[e];
        sorted[cur + rank] = f;
        __builtin_amdgcn_wave_barrier();
        if (rank == 0) cnt[e] = cur + wtotal;
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- router logits (VALU)
// The one-token layer's router role (TB = 1, EPW = 1: one expert per wave); calls of several
// tokens use the matrix-core router (router_mf.h).
// Workgroup (tb, eb): tokens [TB tb, TB tb + TB) x experts [EPB eb, EPB eb + EPB), EPW
// experts per wave.  Per token the input is staged in LDS as z = x * router_scale (fp32);
// the token's norm factor f = (1/sqrt(H)) / sqrt(mean(x^2) + eps) multiplies the finished
// dot product:
//   logit = f * sum_h (s q + b)_h z_h + bias.
// Lane l of a wave works on elements 256 j + 4 l .. + 3 of the rows, so both the code loads
// (4 bytes per lane) and the LDS reads of z (16 bytes per lane) are contiguous across lanes;
// each z read serves the wave's EPW experts.
constexpr int ROUTER_MAX_H = 8192;
constexpr int ROUTER_RB = 11;          // 256-element blocks of codes a wave loads per batch

inline __host__ __device__ size_t router_lds_bytes(int H, int nt) {
  return (size_t)nt * H * 4 + 64;
}

struct NoWait {
  QMOE_DEV void operator()() const {}
};

// xwait() is called by the whole workgroup after the first batch of codes was issued and
// before x is read (a caller whose x is produced inside the same launch waits there).
template <int TB, int EPW, class XW = NoWait>
QMOE_DEV void router_logits_block(const RouterArgs &a, int tb, int eb, char *smem,
                                  XW xwait = XW()) {
  constexpr int EPB = EPW * ROUTER_WAVES;
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int H = a.H;
  const int t0 = tb * TB;
  const int nt = min(TB, a.T - t0);
  const int e_first = eb * EPB + wv * EPW;
  const int nb = (H + 255) / 256;                  // blocks of 256 elements (last may be partial)
  // first batch of this wave's codes and group scales/biases, issued before the activations
  uint32_t cq[EPW][ROUTER_RB];
  uint32_t sbw[EPW][ROUTER_RB];
  auto load_codes = [&](int b0) {
#pragma unroll
    for (int x = 0; x < EPW; ++x) {
      const int ec = min(e_first + x, a.E - 1);
      const uint8_t *row = a.rq + (size_t)ec * H;
      const uint16_t *rs = a.rs + (size_t)ec * (H / GROUP), *rb = a.rb + (size_t)ec * (H / GROUP);
#pragma unroll
      for (int j = 0; j < ROUTER_RB; ++j) {
        const int el = min(256 * (b0 + j) + 4 * lane, H - 4);
        cq[x][j] = *(const uint32_t *)(row + el);
        sbw[x][j] = (uint32_t)rs[el / GROUP] | ((uint32_t)rb[el / GROUP] << 16);
      }
    }
  };
  load_codes(0);
  float lb[EPW];
#pragma unroll
  for (int x = 0; x < EPW; ++x) lb[x] = a.lbias ? a.lbias[min(e_first + x, a.E - 1)] : 0.f;
  // activations: thread tid stages elements 4 (tid + 256 j) .. + 3 of each token, XB chunks
  // per batch (one batch for H <= 3072); the router scales of the first batch are loaded
  // before xwait()
  constexpr int XB = 3;
  const int n4 = H / 4;
  float4 rsv[XB];
  auto load_rs = [&](int j0) {
#pragma unroll
    for (int j = 0; j < XB; ++j) {
      const int c = min(tid + ROUTER_THREADS * (j0 + j), n4 - 1);
      rsv[j] = a.rscale ? *(const float4 *)(a.rscale + 4 * c) : float4{1.f, 1.f, 1.f, 1.f};
    }
  };
  load_rs(0);
  xwait();
  float *z = (float *)smem;                                  // [nt][H]
  __shared__ float red[ROUTER_WAVES][TB];
  float ss[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) ss[i] = 0.f;
  for (int j0 = 0; j0 * ROUTER_THREADS < n4; j0 += XB) {
    uint2 xv[TB][XB];
    if (j0 > 0) load_rs(j0);
#pragma unroll
    for (int j = 0; j < XB; ++j) {
      const int c = min(tid + ROUTER_THREADS * (j0 + j), n4 - 1);
#pragma unroll
      for (int i = 0; i < TB; ++i)
        xv[i][j] = *(const uint2 *)(a.x + (size_t)(t0 + min(i, nt - 1)) * H + 4 * c);
    }
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      if (i >= nt) continue;
#pragma unroll
      for (int j = 0; j < XB; ++j) {
        const int c = tid + ROUTER_THREADS * (j0 + j);
        if (c < n4) {
          const float x0 = bf16lo(xv[i][j].x), x1 = bf16hi(xv[i][j].x);
          const float x2 = bf16lo(xv[i][j].y), x3 = bf16hi(xv[i][j].y);
          ss[i] = fmaf(x0, x0, ss[i]);
          ss[i] = fmaf(x1, x1, ss[i]);
          ss[i] = fmaf(x2, x2, ss[i]);
          ss[i] = fmaf(x3, x3, ss[i]);
          *(float4 *)(z + i * H + 4 * c) =
              float4{x0 * rsv[j].x, x1 * rsv[j].y, x2 * rsv[j].z, x3 * rsv[j].w};
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    if (i >= nt) continue;
    ss[i] = wave_sum(ss[i]);
    if (lane == 0) red[wv][i] = ss[i];
  }
  __syncthreads();
  if (e_first >= a.E) return;
  // every wave forms the norm factors itself (same sums in the same order)
  float facv[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    float tot = 0.f;
    for (int w = 0; w < ROUTER_WAVES; ++w) tot += red[w][min(i, nt - 1)];
    facv[i] = a.inv_sqrt_h / sqrtf(tot / (float)H + RMS_EPS);
  }
  float acc[EPW][TB];
#pragma unroll
  for (int x = 0; x < EPW; ++x)
#pragma unroll
    for (int i = 0; i < TB; ++i) acc[x][i] = 0.f;
  for (int b0 = 0; b0 < nb; b0 += ROUTER_RB) {
    if (b0 > 0) load_codes(b0);
#pragma unroll
    for (int j = 0; j < ROUTER_RB; ++j) {
      const int el = 256 * (b0 + j) + 4 * lane;
      if (b0 + j < nb && el < H) {
        float4 zz[TB];
#pragma unroll
        for (int i = 0; i < TB; ++i)
          if (i < nt) zz[i] = *(const float4 *)(z + i * H + el);
#pragma unroll
        for (int x = 0; x < EPW; ++x) {
          const float s = bf16_to_f32((uint16_t)(sbw[x][j] & 0xFFFFu));
          const float bb = bf16_to_f32((uint16_t)(sbw[x][j] >> 16));
          const float w0 = fmaf(s, (float)(cq[x][j] & 0xFFu), bb);
          const float w1 = fmaf(s, (float)((cq[x][j] >> 8) & 0xFFu), bb);
          const float w2 = fmaf(s, (float)((cq[x][j] >> 16) & 0xFFu), bb);
          const float w3 = fmaf(s, (float)(cq[x][j] >> 24), bb);
#pragma unroll
          for (int i = 0; i < TB; ++i) {
            if (i < nt) {
              acc[x][i] = fmaf(w0, zz[i].x, acc[x][i]);
              acc[x][i] = fmaf(w1, zz[i].y, acc[x][i]);
              acc[x][i] = fmaf(w2, zz[i].z, acc[x][i]);
              acc[x][i] = fmaf(w3, zz[i].w, acc[x][i]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int x = 0; x < EPW; ++x) {
    const int e = e_first + x;
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      if (i < nt) {
        const float tot = wave_sum(acc[x][i]);
        float l = facv[i] * tot;
        if (a.lbias) l += lb[x];
        const size_t o = (size_t)(t0 + i) * a.E + e;
        if (e < a.E) {
          if (a.logits_tag) {
            if (lane < a.tag_copies) st_tag(a.logits_tag + (size_t)lane * a.tag_copy_stride + o, a.tag, l);
          } else if (lane == 0) {
            st_sys(a.logits + o, l);
          }
        }
      }
    }
  }
}

__global__ void __launch_bounds__(256) bucket_kernel(const int32_t *idx, int N, int E,
                                                     int32_t *counts, int32_t *offsets,
                                                     int32_t *sorted, int32_t *active,
                                                     int32_t *n_active) {
  extern __shared__ __align__(16) char smem[];
  bucket_block<256>([&](int f) { return idx[f]; }, N, E, counts, offsets, sorted, active, n_active,
                    nullptr, 0, (int *)smem);
}

}  // namespace qmoe
