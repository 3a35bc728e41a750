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
  float *logits;              // [T, E]
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

// LDS bytes of a router workgroup for hidden H
inline size_t router_lds_bytes(int H) {
  return (size_t)ROUTER_TB * H * 4 + (size_t)ROUTER_TB * (H / 16) * 4 + 64;
}

// ---------------------------------------------------------------- top-k of one token (one wave)
// Exact order: larger logit first, equal logits -> lower expert index.  A NaN logit ranks
// as -inf, so every selected index is a valid expert id whatever the logits hold (the
// sentinel index of an empty candidate always loses to a real expert).
QMOE_DEV void topk_one_token(const float *lrow, int E, int k, const float *pes,
                             int32_t *idx_out, float *w_out) {
  const int lane = threadIdx.x % WAVE;
  float v[MAX_EXPERTS / WAVE];
#pragma unroll
  for (int j = 0; j < MAX_EXPERTS / WAVE; ++j) {
    const int e = lane + WAVE * j;
    const float l = (e < E) ? ld_sys(lrow + e) : -INFINITY;
    v[j] = (l == l) ? l : -INFINITY;
  }
  unsigned taken = 0;
  float myv = 0.f;
  int myi = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < MAX_EXPERTS / WAVE; ++j) {
      const int e = lane + WAVE * j;
      if (e < E && !((taken >> j) & 1u)) {
        if (v[j] > bv || (v[j] == bv && e < bi)) { bv = v[j]; bi = e; }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, WAVE);
      const int oi = __shfl_xor(bi, o, WAVE);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if ((bi % WAVE) == lane) taken |= 1u << (bi / WAVE);
    if (lane == r) { myv = bv; myi = bi; }
  }
  const float vmax = __shfl(myv, 0, WAVE);
  const float z = (lane < k) ? expf(myv - vmax) : 0.f;
  const float zsum = wave_sum(z);
  if (lane < k) {
    st_sys(idx_out + lane, myi);
    st_sys(w_out + lane, (z / zsum) * pes[myi]);
  }
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
// Workgroup (tb, eb): tokens [4 tb, 4 tb + 4) x experts [4 eb, 4 eb + 4).  Per token the
// input is staged as z = x * router_scale (fp32) with per-16-element sums; the token's norm
// factor f = (1/sqrt(H)) / sqrt(mean(x^2) + eps) multiplies the finished dot product:
//   logit = f * sum_g [ s_g * sum_{h in g} q_h z_h + b_g * sum_{h in g} z_h ] + bias.
QMOE_DEV void router_logits_block(const RouterArgs &a, int tb, int eb, char *smem) {
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int H = a.H;
  const int t0 = tb * ROUTER_TB;
  const int nt = min(ROUTER_TB, a.T - t0);
  // this wave's expert row: lane l holds chunks l, l+64, ... (16 codes each), loaded before
  // the activations are staged (H <= 8192 -> at most 8 chunks per lane)
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
  float *z = (float *)smem;                                  // [TB][H]
  float *zs = z + ROUTER_TB * H;                             // [TB][H/16]
  float *fac = zs + ROUTER_TB * (H / 16);                    // [TB]
  // stage z and the 16-element sums; thread handles 8 consecutive elements
  const int n8 = H / 8;
  for (int i = 0; i < nt; ++i) {
    const uint16_t *xr = a.x + (size_t)(t0 + i) * H;
    float ss = 0.f;
    for (int c = tid; c < n8; c += ROUTER_THREADS) {
      const qmoe_u32x4 v = *(const qmoe_u32x4 *)(xr + 8 * c);
      const uint32_t wv4[4] = {v.x, v.y, v.z, v.w};
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        float x0 = bf16lo(wv4[d]), x1 = bf16hi(wv4[d]);
        ss = fmaf(x0, x0, ss);
        ss = fmaf(x1, x1, ss);
        if (a.rscale) { x0 *= a.rscale[8 * c + 2 * d]; x1 *= a.rscale[8 * c + 2 * d + 1]; }
        z[i * H + 8 * c + 2 * d] = x0;
        z[i * H + 8 * c + 2 * d + 1] = x1;
        part += x0 + x1;
      }
      // two 8-element threads make one 16-element sum (c even/odd are adjacent lanes)
      const float other = __shfl_xor(part, 1, WAVE);
      if ((c & 1) == 0) zs[i * (H / 16) + c / 2] = part + other;
    }
    ss = wave_sum(ss);
    __shared__ float red[ROUTER_WAVES];
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
  float acc[ROUTER_TB];
#pragma unroll
  for (int i = 0; i < ROUTER_TB; ++i) acc[i] = 0.f;
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
      for (int i = 0; i < ROUTER_TB; ++i) {
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
  for (int i = 0; i < ROUTER_TB; ++i) {
    if (i < nt) {
      const float tot = wave_sum(acc[i]);
      if (lane == 0) {
        float l = fac[i] * tot;
        if (a.lbias) l += a.lbias[e];
        st_sys(a.logits + (size_t)(t0 + i) * a.E + e, l);
      }
    }
  }
}

// After a router workgroup has written its logits: the last workgroup of a token block runs
// top-k for that block; with bucketing requested, the last of those (or that workgroup
// itself when there is a single token block) runs the bucketing.
QMOE_DEV void router_finish(const RouterArgs &a, int tb, char *smem) {
  if (!arrive_last(&a.cnt_tb[tb], (unsigned)a.n_eb)) return;
  const int wv = threadIdx.x / WAVE;
  const int t0 = tb * ROUTER_TB;
  const int nt = min(ROUTER_TB, a.T - t0);
  for (int i = wv; i < nt; i += ROUTER_WAVES) {
    const int t = t0 + i;
    topk_one_token(a.logits + (size_t)t * a.E, a.E, a.k, a.pes, a.topk_idx + (size_t)t * a.k,
                   a.topk_w + (size_t)t * a.k);
  }
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
  router_logits_block(a, tb, eb, smem);
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
