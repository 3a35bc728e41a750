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

constexpr int ROUTER_TB = 4;     // tokens per router workgroup
constexpr int ROUTER_EPW = 1;    // experts per wave
constexpr int ROUTER_WAVES = 4;
constexpr int ROUTER_EPB = ROUTER_EPW * ROUTER_WAVES;  // experts per router workgroup
constexpr int ROUTER_THREADS = ROUTER_WAVES * WAVE;
constexpr float RMS_EPS = 1e-6f;

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
  unsigned *cnt_tb;           // [n_tb] completion counters (zero on entry, zero on exit)
  unsigned *cnt_all;          // [1]
  int n_tb, n_eb;             // token blocks, expert blocks
  // optional fused bucketing (layer path); null counts -> skip
  int32_t *counts, *offsets, *sorted, *active, *n_active;
  int32_t *slot_tab;          // [n_slots][4] {expert, first bucket position, rows, first flat id}
  int n_slots;
};

// LDS bytes of the logits part of a router workgroup for hidden H and up to nt tokens
inline __host__ __device__ size_t router_lds_bytes(int H, int nt = ROUTER_TB) {
  return (size_t)nt * H * 4 + (size_t)nt * (H / 16) * 4 + 64;
}

// ---------------------------------------------------------------- top-k by exact ranking
// Order: larger logit first, equal logits -> lower expert index.  A NaN logit ranks as -inf
// (so every selected index is a valid expert id whatever the logits hold) and -0 as +0.
// Each (logit, expert) pair becomes one 64-bit key whose unsigned order is exactly that
// order; all keys are distinct, so the selection is a rank computation with no branches:
//   1. the keys are cut into chunks of 64; a lane ranks its key inside its chunk with 64
//      broadcast LDS reads, and the keys of rank < k ("survivors") go to slot rank of their
//      chunk's k survivor slots (every global top-k key survives its chunk);
//   2. each survivor is ranked among all survivors; rank r < k is the r-th selected expert.
// Padding keys (chunk positions >= E) sort below every real key.
QMOE_DEV uint64_t topk_key(float l, int e) {
  if (!(l == l)) l = -INFINITY;
  if (l == 0.f) l = 0.f;
  uint32_t u = __float_as_uint(l);
  u ^= (u & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u;
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
QMOE_DEV uint64_t topk_pad_key(int e) { return (uint64_t)(0xFFFFFFFFu - (uint32_t)e); }
QMOE_DEV int key_expert(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
QMOE_DEV float key_logit(uint64_t key) {
  uint32_t u = (uint32_t)(key >> 32);
  u ^= (u & 0x80000000u) ? 0x80000000u : 0xFFFFFFFFu;
  return __uint_as_float(u);
}

inline __host__ __device__ int topk_chunks(int E) { return (E + WAVE - 1) / WAVE; }
// LDS of one ranking: keys [chunks*64], survivors [chunks*k], result [k] (64-bit each)
inline __host__ __device__ size_t topk_lds_bytes(int E, int k) {
  return (size_t)8 * (topk_chunks(E) * WAVE + topk_chunks(E) * k + k);
}

// Step 1 for one chunk, by one wave: ck = the chunk's 64 keys.
QMOE_DEV void topk_rank_chunk(const uint64_t *ck, int k, uint64_t *surv) {
  const int lane = threadIdx.x % WAVE;
  const uint64_t K = ck[lane];
  int r = 0;
#pragma unroll 16
  for (int j = 0; j < WAVE; ++j) r += (ck[j] > K) ? 1 : 0;
  if (r < k) surv[r] = K;
}

// Step 2, by one wave: sel[r] = the key of rank r < k among the n survivors.
QMOE_DEV void topk_rank_survivors(const uint64_t *surv, int n, int k, uint64_t *sel) {
  for (int i = threadIdx.x % WAVE; i < n; i += WAVE) {
    const uint64_t K = surv[i];
    int r = 0;
    for (int j = 0; j < n; ++j) r += (surv[j] > K) ? 1 : 0;
    if (r < k) sel[r] = K;
  }
}

// Lane j < k of the wave gets the j-th selected expert and its weight: softmax over the kept
// logits, times per_expert_scale (pes, global or LDS) of that expert.  Other lanes get 0, 0.
QMOE_DEV void topk_weights(const uint64_t *sel, int k, const float *pes, int &myi, float &myw) {
  const int lane = threadIdx.x % WAVE;
  const uint64_t K = sel[min(lane, k - 1)];
  const float lv = key_logit(K);
  const float vmax = __shfl(lv, 0, WAVE);
  const float z = (lane < k) ? expf(lv - vmax) : 0.f;
  const float zsum = wave_sum(z);
  myi = (lane < k) ? key_expert(K) : 0;
  myw = (lane < k) ? (z / zsum) * pes[myi] : 0.f;
}

// The whole selection by one wave for one token.  lrow: E logits written by other
// workgroups of the launch (system-scope loads).  lds: topk_lds_bytes(E, k) bytes owned by
// this wave.
QMOE_DEV void topk_wave(const float *lrow, int E, int k, const float *pes, uint64_t *lds,
                        int &myi, float &myw) {
  const int lane = threadIdx.x % WAVE, nch = topk_chunks(E);
  uint64_t *keys = lds, *surv = lds + nch * WAVE, *sel = surv + nch * k;
  float v[MAX_EXPERTS / WAVE];
#pragma unroll
  for (int c = 0; c < MAX_EXPERTS / WAVE; ++c) {
    const int e = c * WAVE + lane;
    v[c] = (c < nch && e < E) ? ld_sys(lrow + e) : 0.f;
  }
#pragma unroll
  for (int c = 0; c < MAX_EXPERTS / WAVE; ++c) {
    const int e = c * WAVE + lane;
    if (c < nch) keys[e] = (e < E) ? topk_key(v[c], e) : topk_pad_key(e);
  }
  __builtin_amdgcn_wave_barrier();
  for (int c = 0; c < nch; ++c) topk_rank_chunk(keys + c * WAVE, k, surv + c * k);
  __builtin_amdgcn_wave_barrier();
  topk_rank_survivors(surv, nch * k, k, sel);
  __builtin_amdgcn_wave_barrier();
  topk_weights(sel, k, pes, myi, myw);
}

// ---------------------------------------------------------------- bucketing (one workgroup)
// Stable counting sort of N = T*k assignments by expert (ids outside [0, E) are dropped).
// Counts via an LDS histogram; the rank of an assignment among the earlier ones of its
// expert from wave ballots (one ballot per distinct expert in a wave) plus a per-expert cursor
// advanced wave by wave in order.  Optionally also writes the slot table used by the expert
// kernels: entry s = {expert, first bucket position, rows, first flat id} of the s-th active
// expert, zero rows for s in [n_active, n_slots).
// lds: at least 2 * E * 4 bytes.  get(f) returns the expert id of assignment f.
template <int NT, class Get>
QMOE_DEV void bucket_block(Get get, int N, int E, int32_t *counts, int32_t *offsets,
                           int32_t *sorted, int32_t *active, int32_t *n_active, int32_t *slot_tab,
                           int n_slots, int *lds) {
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
  // exclusive scan of counts and of (count > 0) flags, E <= MAX_EXPERTS
  const int per = (E + NT - 1) / NT;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int s_cnt = 0, s_act = 0;
  for (int e = e0; e < e1; ++e) { s_cnt += cnt[e]; s_act += cnt[e] > 0; }
  // inclusive wave scan of the pair (count total in the high bits, active flags in the low 16)
  long long pair = ((long long)s_cnt << 16) | s_act;
  for (int o = 1; o < WAVE; o <<= 1) {
    const long long up = __shfl_up(pair, o, WAVE);
    if (lane >= o) pair += up;
  }
  __shared__ long long wtot[NW];
  __shared__ int n_act_sh;
  if (lane == WAVE - 1) wtot[wv] = pair;
  __syncthreads();
  long long before = 0, tot = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wv) before += wtot[w];
    tot += wtot[w];
  }
  long long excl = before + pair - (((long long)s_cnt << 16) | s_act);
  int run_cnt = (int)(excl >> 16), run_act = (int)(excl & 0xFFFF);
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    counts[e] = c;
    offsets[e] = run_cnt;
    if (c > 0) {
      active[run_act] = e;
      if (slot_tab && run_act < n_slots)
        *(qmoe_u32x4 *)(slot_tab + 4 * run_act) =
            qmoe_u32x4{(uint32_t)e, (uint32_t)run_cnt, (uint32_t)c, (uint32_t)first[e]};
      ++run_act;
    }
    cnt[e] = run_cnt;  // becomes the cursor
    run_cnt += c;
  }
  const int na = (int)(tot & 0xFFFF);
  if (tid == NT - 1) {
    offsets[E] = (int)(tot >> 16);
    *n_active = na;
  }
  if (slot_tab)
    for (int sl = na + tid; sl < n_slots; sl += NT)
      *(qmoe_u32x4 *)(slot_tab + 4 * sl) = qmoe_u32x4{0u, 0u, 0u, 0u};
  (void)n_act_sh;
  __syncthreads();
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

// ---------------------------------------------------------------- router logits
// Workgroup (tb, eb): tokens [TB tb, TB tb + TB) x experts [4 eb, 4 eb + 4).  Per token the
// input is staged as z = x * router_scale (fp32) with per-16-element sums; the token's norm
// factor f = (1/sqrt(H)) / sqrt(mean(x^2) + eps) multiplies the finished dot product:
//   logit = f * sum_g [ s_g * sum_{h in g} q_h z_h + b_g * sum_{h in g} z_h ] + bias.
// Every global load (codes, scales, activations, router_scale) is issued before the first
// one is used, so the workgroup waits for memory once.
template <int TB>
QMOE_DEV void router_logits_block(const RouterArgs &a, int tb, int eb, char *smem) {
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int H = a.H;
  const int t0 = tb * TB;
  const int nt = min(TB, a.T - t0);
  // this wave's expert row: lane l holds chunks l, l+64, ... (16 codes each; H <= 8192 -> at
  // most 8 chunks per lane)
  constexpr int NCH = 8;
  const int n16 = H / 16;
  const int e = eb * ROUTER_EPB + wv;
  const int ec = min(e, a.E - 1);
  const uint8_t *row = a.rq + (size_t)ec * H;
  qmoe_u32x4 v[NCH];
  uint16_t sv[NCH], bv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = min(lane + WAVE * j, n16 - 1);
    v[j] = *(const qmoe_u32x4 *)(row + 16 * c);
    sv[j] = a.rs[(size_t)ec * (H / GROUP) + c / 4];
    bv[j] = a.rb[(size_t)ec * (H / GROUP) + c / 4];
  }
  const float lb = a.lbias ? a.lbias[ec] : 0.f;
  // activations: thread tid holds the 8-element chunks tid + 256 j (j < XC) of each token,
  // with the matching router_scale entries
  constexpr int XC = 4;
  const int n8 = H / 8;
  qmoe_u32x4 xv[TB][XC];
  float4 rsv[XC][2];
#pragma unroll
  for (int j = 0; j < XC; ++j) {
    const int c = min(tid + ROUTER_THREADS * j, n8 - 1);
    if (a.rscale) {
      rsv[j][0] = *(const float4 *)(a.rscale + 8 * c);
      rsv[j][1] = *(const float4 *)(a.rscale + 8 * c + 4);
    }
#pragma unroll
    for (int i = 0; i < TB; ++i)
      xv[i][j] = *(const qmoe_u32x4 *)(a.x + (size_t)(t0 + min(i, nt - 1)) * H + 8 * c);
  }
  float *z = (float *)smem;                                  // [nt][H]
  float *zs = z + nt * H;                                    // [nt][H/16]
  float *fac = zs + nt * (H / 16);                           // [nt]
  __shared__ float red[ROUTER_WAVES];
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    if (i >= nt) continue;       // nt is the same for the whole workgroup
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      const int c = tid + ROUTER_THREADS * j;
      if (c < n8) {
        const uint32_t wv4[4] = {xv[i][j].x, xv[i][j].y, xv[i][j].z, xv[i][j].w};
        const float rs8[8] = {rsv[j][0].x, rsv[j][0].y, rsv[j][0].z, rsv[j][0].w,
                              rsv[j][1].x, rsv[j][1].y, rsv[j][1].z, rsv[j][1].w};
        float part = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float x0 = bf16lo(wv4[d]), x1 = bf16hi(wv4[d]);
          ss = fmaf(x0, x0, ss);
          ss = fmaf(x1, x1, ss);
          if (a.rscale) { x0 *= rs8[2 * d]; x1 *= rs8[2 * d + 1]; }
          z[i * H + 8 * c + 2 * d] = x0;
          z[i * H + 8 * c + 2 * d + 1] = x1;
          part += x0 + x1;
        }
        // two 8-element threads make one 16-element sum (c even/odd are adjacent lanes)
        const float other = __shfl_xor(part, 1, WAVE);
        if ((c & 1) == 0) zs[i * (H / 16) + c / 2] = part + other;
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wv] = ss;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int w = 0; w < ROUTER_WAVES; ++w) tot += red[w];
      fac[i] = a.inv_sqrt_h / sqrtf(tot / (float)H + RMS_EPS);
    }
    __syncthreads();
  }
  if (e >= a.E) return;
  float acc[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + WAVE * j;
    if (c < n16) {
      const float s = bf16_to_f32(sv[j]), b = bf16_to_f32(bv[j]);
      const uint32_t w4[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      float q[16];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        q[4 * d + 0] = (float)(w4[d] & 0xFFu);
        q[4 * d + 1] = (float)((w4[d] >> 8) & 0xFFu);
        q[4 * d + 2] = (float)((w4[d] >> 16) & 0xFFu);
        q[4 * d + 3] = (float)(w4[d] >> 24);
      }
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        if (i < nt) {
          const float *zr = z + i * H + 16 * c;
          float dq = 0.f;
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) dq = fmaf(q[jj], zr[jj], dq);
          acc[i] = fmaf(s, dq, acc[i]);
          acc[i] = fmaf(b, zs[i * (H / 16) + c], acc[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    if (i < nt) {
      const float tot = wave_sum(acc[i]);
      float l = fac[i] * tot;
      if (a.lbias) l += lb;
      const size_t o = (size_t)(t0 + i) * a.E + e;
      if (a.logits_tag) {
        if (lane < a.tag_copies) st_tag(a.logits_tag + (size_t)lane * a.tag_copy_stride + o, a.tag, l);
      } else if (lane == 0) {
        st_sys(a.logits + o, l);
      }
    }
  }
}

// After a router workgroup has written its logits: the last workgroup of a token block runs
// top-k for that block; with bucketing requested, the last of those (or that workgroup
// itself when there is a single token block) runs the bucketing.
QMOE_DEV void router_finish(const RouterArgs &a, int tb, char *smem) {
  if (!arrive_last(&a.cnt_tb[tb], (unsigned)a.n_eb)) return;
  const int wv = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
  const int t0 = tb * ROUTER_TB;
  const int nt = min(ROUTER_TB, a.T - t0);
  uint64_t *lds = (uint64_t *)(smem + (size_t)wv * topk_lds_bytes(a.E, a.k));
  for (int i = wv; i < nt; i += ROUTER_WAVES) {
    const int t = t0 + i;
    int myi;
    float myw;
    topk_wave(a.logits + (size_t)t * a.E, a.E, a.k, a.pes, lds, myi, myw);
    if (lane < a.k) {
      st_sys(a.topk_idx + (size_t)t * a.k + lane, myi);
      st_sys(a.topk_w + (size_t)t * a.k + lane, myw);
    }
  }
  __syncthreads();
  if (a.counts == nullptr) return;
  if (a.n_tb == 1) {
    drain_memory();    // this workgroup wrote every assignment
    __syncthreads();
  } else if (!arrive_last(a.cnt_all, (unsigned)a.n_tb)) {
    return;
  }
  bucket_block<ROUTER_THREADS>([&](int f) { return ld_sys(a.topk_idx + f); }, a.T * a.k, a.E,
                               a.counts, a.offsets, a.sorted, a.active, a.n_active, a.slot_tab,
                               a.n_slots, (int *)smem);
}

__global__ void __launch_bounds__(ROUTER_THREADS) router_kernel(RouterArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int tb = blockIdx.x / a.n_eb, eb = blockIdx.x % a.n_eb;
  router_logits_block<ROUTER_TB>(a, tb, eb, smem);
  router_finish(a, tb, smem);
}

__global__ void __launch_bounds__(256) bucket_kernel(const int32_t *idx, int N, int E,
                                                     int32_t *counts, int32_t *offsets,
                                                     int32_t *sorted, int32_t *active,
                                                     int32_t *n_active) {
  __shared__ int lds[2 * MAX_EXPERTS];
  bucket_block<256>([&](int f) { return idx[f]; }, N, E, counts, offsets, sorted, active, n_active,
                    nullptr, 0, lds);
}

}  // namespace qmoe
