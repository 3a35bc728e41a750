// Grouped-GEMM kernels of the expert FFN on the gfx950 matrix cores (prefill chunks of the
// TurboFieldfare post, section "TurboFieldfare의 전문가 스트리밍 구조": up to 128 tokens per
// chunk, so each expert read serves every row routed to it).
//
// Operands are exact: the int4 codes become the bf16 values 128 + q (one AND-OR per two
// codes), activations are bf16 (x) or hi/lo bf16 planes (h).  Per k-step (one 64-input group
// with scale s and bias b of each weight row) and 32x32 output block:
//   t   = sum over the group of a * (128 + q)        four v_mfma_f32_32x32x16_bf16
//   acc += s * t                                      one FMA per accumulator (VALU)
//   acc += (b - 128 s) * sum over the group of a      one v_mfma_f32_32x32x2_f32 (the
//                                                     group sum in one K entry, 0 in the
//                                                     other)
// so the result equals sum (s q + b) a with fp32 accumulation, as in the VALU path.
//
// Lane layout (v_mfma_f32_32x32x16_bf16): lane l supplies row (l % 32) of both operands for
// the 8-element sub-block (l / 32) of each 16-deep K block.  The store's k-step gives lane l
// the codes of weight row l % 32 for columns 32 (l / 32) + [0, 32), so word j of the lane's
// 16 bytes is K block j.  Activation rows (tokens) are M and weight rows are N, so every
// accumulator of a lane belongs to the lane's own weight row and uses its own scale.
// Accumulator r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//
// A wave owns one weight tile and runs over all of its k-steps.  Its activation row is read
// straight from memory (every wave of a bucket reads the same rows at the same k-steps, so
// they hit in L1/L2); nothing is staged in LDS.  The bias term needs the sum of each
// 64-column group of every activation row: for x they are computed once per chunk (by the
// router pass or gsum_kernel), for h by the gate/up kernel that writes h (the four waves of a
// gate/up workgroup own exactly one 64-column group of h).
#pragma once
#include "common.h"
#include "store.h"

namespace qmoe {

typedef __bf16 qmoe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float qmoe_f32x16 __attribute__((ext_vector_type(16)));

constexpr int PF_W = 4;                 // waves per workgroup
constexpr int PF_THREADS = PF_W * WAVE;
constexpr int PF_KB = 3;                // k-steps per load batch of a wave
constexpr int GU_MT = 32;               // rows per gate/up pass (MFMA rows)
constexpr int D_MT = 16;                // tokens per down pass (hi + lo planes: 32 MFMA rows)

QMOE_DEV int mfma_row(int lane, int r) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); }

// B operand: the 8 codes of word w as bf16 (128 + q), element order
QMOE_DEV qmoe_bf16x8 q4_operand(uint32_t w) {
  const qmoe_u32x4 v = {nib_pair(w, 0), nib_pair(w, 1), nib_pair(w, 2), nib_pair(w, 3)};
  return __builtin_bit_cast(qmoe_bf16x8, v);
}

// One k-step: t = A (128 + q) on the matrix cores, acc += s t, then acc += (b - 128 s) G with
// G the group sum of the lane's activation row (given by half-0 lanes, 0 by the others, so
// the K = 2 product adds it once).
QMOE_DEV void pf_kstep(qmoe_f32x16 &acc, const qmoe_u32x4 (&xa)[4], qmoe_u32x4 cv, float g,
                       uint32_t sb) {
  qmoe_f32x16 t = {};
  t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(qmoe_bf16x8, xa[0]),
                                              q4_operand(cv.x), t, 0, 0, 0);
  t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(qmoe_bf16x8, xa[1]),
                                              q4_operand(cv.y), t, 0, 0, 0);
  t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(qmoe_bf16x8, xa[2]),
                                              q4_operand(cv.z), t, 0, 0, 0);
  t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(qmoe_bf16x8, xa[3]),
                                              q4_operand(cv.w), t, 0, 0, 0);
  const float s = bf16lo(sb), c = fmaf(-128.f, s, bf16hi(sb));
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = fmaf(s, t[r], acc[r]);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(g, c, acc, 0, 0, 0);
}

// PF_KB consecutive k-steps from ks0 (or, with TAIL, the ones below nks; the loads past
// the end re-read the last k-step and are not used), all loads issued before any product.
template <bool TAIL>
QMOE_DEV void pf_batch(qmoe_f32x16 &acc, const uint8_t *tbase, int ks0, int nks,
                       const uint16_t *arow, const float *grow, bool gmask) {
  const int lane = threadIdx.x % WAVE, rr = lane % 32;
  qmoe_u32x4 cv[PF_KB], xa[PF_KB][4];
  uint32_t sb[PF_KB];
  float g[PF_KB];
#pragma unroll
  for (int u = 0; u < PF_KB; ++u) {
    const int ks = TAIL ? min(ks0 + u, nks - 1) : ks0 + u;
    const uint8_t *st = tbase + (size_t)ks * KSTEP_BYTES;
    cv[u] = *(const qmoe_u32x4 *)(st + 16 * lane);
    sb[u] = *(const uint32_t *)(st + 1024 + 4 * rr);
#pragma unroll
    for (int j = 0; j < 4; ++j) xa[u][j] = *(const qmoe_u32x4 *)(arow + GROUP * ks + 8 * j);
    g[u] = grow[ks];
  }
#pragma unroll
  for (int u = 0; u < PF_KB; ++u)
    if (!TAIL || ks0 + u < nks) pf_kstep(acc, xa[u], cv[u], gmask ? g[u] : 0.f, sb[u]);
}

// All nks k-steps of the tile at tbase.  arow: the lane's activation row, offset to its half
// (k-step ks covers columns 64 ks + 32 half + [0, 32)); grow: the row's group sums, used
// where gmask is set (a padding lane reads a valid row; its MFMA rows are not used).
QMOE_DEV qmoe_f32x16 pf_tile(const uint8_t *tbase, int nks, const uint16_t *arow,
                             const float *grow, bool gmask) {
  qmoe_f32x16 acc = {};
  int k0 = 0;
  for (; k0 + PF_KB <= nks; k0 += PF_KB) pf_batch<false>(acc, tbase, k0, nks, arow, grow, gmask);
  if (k0 < nks) pf_batch<true>(acc, tbase, k0, nks, arow, grow, gmask);
  return acc;
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// grid: shared workgroups first (h group, block of GU_MT tokens), then routed (slot, h group).
// Wave w computes tile 4 group + w (h columns 16 tile .. + 15); a routed workgroup loops over
// its bucket GU_MT rows at a time.  Lanes with n = lane % 32 < 16 hold gate row 16 tile + n,
// the others the matching up row.  h = silu(gate) up goes to the hi/lo planes (routed rows in
// bucket order), and the group sums of hi + lo to gh_r / gh_s.
__global__ void __launch_bounds__(PF_THREADS) gu_pf_kernel(FfnArgs a) {
  __shared__ float gpart[PF_W][GU_MT];
  const int H = a.H, KS = H / GROUP;
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE, n = lane % 32, half = lane / 32;
  const int grp_s = a.shared ? a.Is / GROUP : 0;
  const int n_sh = grp_s * ((a.T + GU_MT - 1) / GU_MT);
  int bid = blockIdx.x;
  SlotRows sr;
  int grp, m0, m1;
  if (bid < n_sh) {
    slot_rows(a, 0, true, sr);
    grp = bid % grp_s;
    m0 = (bid / grp_s) * GU_MT;
    m1 = min(a.T, m0 + GU_MT);
  } else {
    bid -= n_sh;
    const int grp_r = a.I / GROUP;
    if (!slot_rows(a, bid / grp_r, false, sr)) return;
    grp = bid % grp_r;
    m0 = 0;
    m1 = sr.m;
  }
  const int I = sr.shared ? a.Is : a.I, KI = I / GROUP;
  const int tile = PF_W * grp + wv;
  const uint8_t *tbase = sr.blk + (size_t)tile * KS * KSTEP_BYTES;
  uint16_t *hhi = sr.shared ? a.hs_hi : a.hr_hi;
  uint16_t *hlo = sr.shared ? a.hs_lo : a.hr_lo;
  float *gh = sr.shared ? a.gh_s : a.gh_r;
  const int pos0 = sr.shared ? 0 : sr.beg;
  for (int p0 = m0; p0 < m1; p0 += GU_MT) {
    const int mt = min(GU_MT, m1 - p0);
    const int i = min(n, mt - 1);  // padding lanes repeat the last row
    const int tok = sr.shared ? p0 + i : flat_of(a, sr, p0 + i) / a.k;
    const qmoe_f32x16 acc = pf_tile(tbase, KS, a.x + (size_t)tok * H + 32 * half,
                                    a.gx + (size_t)tok * KS, half == 0);
    float hs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float up = __shfl_xor(acc[r], 16, WAVE);
      const int m = mfma_row(lane, r);
      hs[r] = 0.f;
      if (n < 16 && m < mt) {
        const float h = silu(acc[r]) * up;
        const uint32_t hi = f32_to_bf16_bits(h);
        const uint32_t lo = f32_to_bf16_bits(h - __uint_as_float(hi << 16));
        const size_t row = (size_t)(pos0 + p0 + m);
        hhi[row * I + 16 * tile + n] = (uint16_t)hi;
        hlo[row * I + 16 * tile + n] = (uint16_t)lo;
        hs[r] = __uint_as_float(hi << 16) + __uint_as_float(lo << 16);
      }
    }
    // group sums: over the 16 gate lanes of each half, then over the four waves
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      hs[r] += __shfl_xor(hs[r], 1, WAVE);
      hs[r] += __shfl_xor(hs[r], 2, WAVE);
      hs[r] += __shfl_xor(hs[r], 4, WAVE);
      hs[r] += __shfl_xor(hs[r], 8, WAVE);
    }
    if (n == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) gpart[wv][mfma_row(lane, r)] = hs[r];
    }
    __syncthreads();
    if ((int)threadIdx.x < mt) {
      const int m = threadIdx.x;
      gh[(size_t)(pos0 + p0 + m) * KI + grp] =
          (gpart[0][m] + gpart[1][m]) + (gpart[2][m] + gpart[3][m]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down projection
// grid: shared workgroups first (tile group, block of D_MT tokens), then routed (slot, tile
// group).  Wave w computes output tile 4 group + w (32 rows of H) over all of K.  MFMA rows
// 0..15 are D_MT tokens' h hi planes, rows 16..31 their lo planes; a token's output is the
// sum of its two rows, accumulators r and r + 8 of the same lane.  Routed rows go to y by
// flat assignment id, shared rows to y_sh.
__global__ void __launch_bounds__(PF_THREADS) d_pf_kernel(FfnArgs a) {
  const int H = a.H, tiles = H / TILE_ROWS, tgroups = (tiles + PF_W - 1) / PF_W;
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE, rr = lane % 32, half = lane / 32;
  const int n_sh = a.shared ? tgroups * ((a.T + D_MT - 1) / D_MT) : 0;
  int bid = blockIdx.x;
  SlotRows sr;
  int tg, m0, m1;
  if (bid < n_sh) {
    slot_rows(a, 0, true, sr);
    tg = bid % tgroups;
    m0 = (bid / tgroups) * D_MT;
    m1 = min(a.T, m0 + D_MT);
  } else {
    bid -= n_sh;
    if (!slot_rows(a, bid / tgroups, false, sr)) return;
    tg = bid % tgroups;
    m0 = 0;
    m1 = sr.m;
  }
  const int tile = PF_W * tg + wv;
  if (tile >= tiles) return;  // no barrier in this kernel
  const int K = sr.shared ? a.Is : a.I, KSd = K / GROUP;
  const uint8_t *tbase = sr.blk + block_geom(H, K).gu_bytes + (size_t)tile * KSd * KSTEP_BYTES;
  const uint16_t *src = rr < 16 ? (sr.shared ? a.hs_hi : a.hr_hi) : (sr.shared ? a.hs_lo : a.hr_lo);
  const float *gh = sr.shared ? a.gh_s : a.gh_r;
  const int pos0 = sr.shared ? 0 : sr.beg;
  for (int p0 = m0; p0 < m1; p0 += D_MT) {
    const int mt = min(D_MT, m1 - p0);
    const int tok = min(rr % 16, mt - 1);  // padding lanes repeat the last row
    const size_t pos = (size_t)(pos0 + p0 + tok);
    const qmoe_f32x16 acc = pf_tile(tbase, KSd, src + pos * K + 32 * half, gh + pos * KSd,
                                    rr < 16 && half == 0);
    int flat = 0;
    if (!sr.shared && lane < mt) flat = flat_of(a, sr, p0 + lane);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int m = mfma_row(lane, r);
      const int fm = __shfl(flat, m, WAVE);
      if (m < mt) {
        const float yv = acc[r] + acc[r + 8];
        if (sr.shared)
          a.y_sh[(size_t)(p0 + m) * H + TILE_ROWS * tile + rr] = yv;
        else
          a.y[(size_t)fm * H + TILE_ROWS * tile + rr] = yv;
      }
    }
  }
}

// Sums of every 64-element group of x [T, H] (n_groups = T H / 64), the gate/up bias term's
// operand, where no router pass has produced them.
__global__ void __launch_bounds__(256) gsum_kernel(const uint16_t *x, int n_groups, float *g) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_groups) return;
  const qmoe_u32x4 *p = (const qmoe_u32x4 *)(x + (size_t)i * GROUP);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const qmoe_u32x4 v = p[j];
    s += (bf16lo(v.x) + bf16hi(v.x)) + (bf16lo(v.y) + bf16hi(v.y)) +
         (bf16lo(v.z) + bf16hi(v.z)) + (bf16lo(v.w) + bf16hi(v.w));
  }
  g[i] = s;
}

// out[t, :] = bf16( x[t, :] + sum_j w[t,j] y[t*k+j, :] + y_sh[t, :] ) in fp32, j ascending,
// then the shared row, then the residual (the order of combine_kernel); four columns per
// thread.
__global__ void __launch_bounds__(256) combine_pf_kernel(const uint16_t *x, const float *y,
                                                         const float *w, const float *y_sh,
                                                         int T, int H, int k, uint16_t *out,
                                                         float *out_f32) {
  const size_t n4 = (size_t)T * H / 4;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < n4;
       o += (size_t)gridDim.x * blockDim.x) {
    const size_t t = (o * 4) / H, col = (o * 4) % H;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const float wj = w[t * k + j];
      const float4 v = *(const float4 *)(y + (t * k + j) * H + col);
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
      acc.z = fmaf(wj, v.z, acc.z);
      acc.w = fmaf(wj, v.w, acc.w);
    }
    if (y_sh) {
      const float4 v = *(const float4 *)(y_sh + t * H + col);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const uint2 xb = *(const uint2 *)(x + t * H + col);
    acc.x += bf16lo(xb.x); acc.y += bf16hi(xb.x); acc.z += bf16lo(xb.y); acc.w += bf16hi(xb.y);
    const uint2 ob = {f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16),
                      f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16)};
    *(uint2 *)(out + t * H + col) = ob;
    if (out_f32) *(float4 *)(out_f32 + t * H + col) = acc;
  }
}

}  // namespace qmoe
