// Grouped-GEMM kernels of the expert FFN on the gfx950 matrix cores (prefill chunks of the
// TurboFieldfare post, section "TurboFieldfare의 전문가 스트리밍 구조": up to 128 tokens per
// chunk, so each expert read serves every row routed to it).
//
// Operands are exact: the int4 codes become the bf16 values 128 + q (one AND-OR per two
// codes), activations are bf16 (x) or hi/lo bf16 planes (h).  Per k-step (one 64-input group
// with scale s and bias b of each weight row) and 16x16 output block:
//   t   = sum over the group of a * (128 + q)        v_mfma_f32_16x16x32_bf16, two per
//                                                     activation plane
//   acc += s * t                                      one FMA per accumulator (VALU)
//   acc += (b - 128 s) * sum over the group of a      one v_mfma_f32_16x16x4_f32 (the group
//                                                     sum in K entry 0, zeros in the others)
// so the result equals sum (s q + b) a with fp32 accumulation, as in the VALU path.  For h the
// two planes hi and lo go through the same accumulation (the product is linear in a), and
// the group sum is that of hi + lo.
//
// Lane layout (v_mfma_f32_16x16x32_bf16): lane l supplies row l % 16 of A and column l % 16
// of B for K entries 8 (l / 16) + [0, 8); accumulator i of lane l is row 4 (l / 16) + i,
// column l % 16.  Activation rows (tokens) are M and weight rows are N.  The store's k-step
// gives lane l the 32 codes of tile row l % 32 for the columns 32 (l / 32) + [0, 32), word j
// holding columns 8 j + [0, 8) of them.  Four lane swaps (two v_permlane32_swap, two
// v_permlane16_swap) transpose the 16-lane groups against the four words, after which word
// G of lane l holds, for tile row 16 (G % 2) + l % 16, the columns 32 (G / 2) + 8 (l / 16) +
// [0, 8): exactly the B operand of weight block G % 2 for column half G / 2.
//
// A wave owns a few weight tiles (32 rows each) and runs over all of their k-steps, so one
// load of its activation rows serves all of them; the rows are read straight from memory
// (every wave of a bucket reads the same rows at the same k-steps, so they hit in L1/L2),
// nothing is staged in LDS.  The bias term needs the sum of
// each 64-column group of every activation row: for x they are computed once per chunk (by
// the router pass or gsum_kernel), for h by the gate/up kernel that writes h (the four waves
// of a gate/up workgroup own exactly one 64-column group of h).
#pragma once
#include "common.h"
#include "store.h"

namespace qmoe {

typedef __bf16 qmoe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float qmoe_f32x4 __attribute__((ext_vector_type(4)));

constexpr int PF_MT = 16;               // activation rows per pass (MFMA rows)
constexpr int GU_NT = 2;                // gate/up: tiles per wave (a workgroup of 2 waves owns
constexpr int GU_WAVES = 4 / GU_NT;     //   the 4 tiles of one 64-column group of h)
constexpr int GU_KB = 2;                //   k-steps per load batch
constexpr int D_NT = 4;                 // down: tiles per wave (the activation rows of a wave serve four tiles)
constexpr int D_WAVES = 2;              //   waves per workgroup
constexpr int D_KB = 2;                 //   k-steps per load batch

// B operand: the 8 codes of word w as bf16 (128 + q), element order
QMOE_DEV qmoe_bf16x8 q4_operand(uint32_t w) {
  const qmoe_u32x4 v = {nib_pair(w, 0), nib_pair(w, 1), nib_pair(w, 2), nib_pair(w, 3)};
  return __builtin_bit_cast(qmoe_bf16x8, v);
}

QMOE_DEV qmoe_f32x4 mfma16(qmoe_u32x4 a, uint32_t w, qmoe_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(qmoe_bf16x8, a),
                                                 q4_operand(w), c, 0, 0, 0);
}

// One k-step of NT 32-row tiles against the wave's 16 activation rows: acc[j][0] (tile j rows
// 0..15) and acc[j][1] (rows 16..31) += scale * (x . (128 + q)).  xa[p][h]: plane p, column half
// h of the lane's row; sw[j]: the scale|bias word of tile row lane % 32 (one load per tile),
// turned by one lane swap into the words of the lane's column in both blocks.  The lanes of
// group `mine` keep those words in bsel for the bias term of their k-step (pf_bias).
template <int NP, int NT>
QMOE_DEV void pf_kstep(qmoe_f32x4 (&acc)[NT][2], uint32_t (&bsel)[NT][2],
                       const qmoe_u32x4 (&cv)[NT], const qmoe_u32x4 (&xa)[NP][2],
                       const uint32_t (&sw)[NT], bool mine) {
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const auto x02 = __builtin_amdgcn_permlane32_swap(cv[j].x, cv[j].z, false, false);
    const auto x13 = __builtin_amdgcn_permlane32_swap(cv[j].y, cv[j].w, false, false);
    const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
    const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
    qmoe_f32x4 t0 = {}, t1 = {};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      t0 = mfma16(xa[p][0], y01[0], t0);
      t1 = mfma16(xa[p][0], y01[1], t1);
      t0 = mfma16(xa[p][1], y23[0], t0);
      t1 = mfma16(xa[p][1], y23[1], t1);
    }
    // lane l loaded the word of tile row l % 32: rows of 16 lanes alternate between block 0
    // and block 1, and the swap of odd and even rows gives every lane both
    const auto sb = __builtin_amdgcn_permlane16_swap(sw[j], sw[j], false, false);
    const float sc0 = bf16lo(sb[0]), sc1 = bf16lo(sb[1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[j][0][i] = fmaf(sc0, t0[i], acc[j][0][i]);
      acc[j][1][i] = fmaf(sc1, t1[i], acc[j][1][i]);
    }
    bsel[j][0] = mine ? sb[0] : bsel[j][0];
    bsel[j][1] = mine ? sb[1] : bsel[j][1];
  }
}

// The bias term of up to four k-steps in one v_mfma_f32_16x16x4_f32 per block: lane group lg
// supplies, for its k-step of the four, the group sum of its row (A, K entry lg) and
// (b - 128 s) of its column (B, K entry lg), so acc += sum over the k-steps of g c.  Lane
// groups without a k-step hold g = 0 and a zero word (c = 0).
template <int NT>
QMOE_DEV void pf_bias(qmoe_f32x4 (&acc)[NT][2], uint32_t (&bsel)[NT][2], float g4) {
#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float c = fmaf(-128.f, bf16lo(bsel[j][b]), bf16hi(bsel[j][b]));
      acc[j][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(g4, c, acc[j][b], 0, 0, 0);
      bsel[j][b] = 0u;
    }
  }
}

// KB consecutive k-steps from ks0 of NT tiles (tile j at tb[j]) (with TAIL only those below
// nks; the loads past the end re-read the last k-step and are not used), all loads issued
// before any product.  ap[p]: the lane's row of plane p, offset to its 8-column piece
// (group g, half h at ap[p] + 64 g + 32 h; k-step ks reads group ks >> kshift).
template <int NP, int NT, int KB, bool TAIL>
QMOE_DEV void pf_batch(qmoe_f32x4 (&acc)[NT][2], uint32_t (&bsel)[NT][2],
                       const uint8_t *const (&tb)[NT], int ks0, int nks,
                       const uint16_t *const (&ap)[NP], int kshift) {
  const int lane = threadIdx.x % WAVE, lg = lane / 16;
  qmoe_u32x4 cv[KB][NT], xa[KB][NP][2];
  uint32_t sw[KB][NT];
#pragma unroll
  for (int u = 0; u < KB; ++u) {
    const int ks = TAIL ? min(ks0 + u, nks - 1) : ks0 + u;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint8_t *st = tb[j] + (size_t)ks * KSTEP_BYTES;
      cv[u][j] = *(const qmoe_u32x4 *)(st + 16 * lane);
      sw[u][j] = *(const uint32_t *)(st + 1024 + 4 * (lane % 32));
    }
    const int grp = ks >> kshift;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      xa[u][p][0] = *(const qmoe_u32x4 *)(ap[p] + GROUP * grp);
      xa[u][p][1] = *(const qmoe_u32x4 *)(ap[p] + GROUP * grp + 32);
    }
  }
#pragma unroll
  for (int u = 0; u < KB; ++u)
    if (!TAIL || ks0 + u < nks)
      pf_kstep<NP, NT>(acc, bsel, cv[u], xa[u], sw[u], ((ks0 + u) & 3) == lg);
}

// All nks k-steps of NT tiles, four at a time (KB divides 4): the products of each k-step,
// then the bias term of the four.  grow: the lane's row's group sums.
template <int NP, int NT, int KB>
QMOE_DEV void pf_tiles(qmoe_f32x4 (&acc)[NT][2], const uint8_t *const (&tb)[NT], int nks,
                       const uint16_t *const (&ap)[NP], const float *grow, int kshift) {
  static_assert(4 % KB == 0, "k-step batches tile the groups of four");
  const int lg = (threadIdx.x % WAVE) / 16;
  uint32_t bsel[NT][2];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    acc[j][0] = qmoe_f32x4{0.f, 0.f, 0.f, 0.f};
    acc[j][1] = qmoe_f32x4{0.f, 0.f, 0.f, 0.f};
    bsel[j][0] = bsel[j][1] = 0u;
  }
  for (int k4 = 0; k4 < nks; k4 += 4) {
    const int kq = k4 + lg;
    const float g4 = kq < nks ? grow[kq >> kshift] : 0.f;
    if (k4 + 4 <= nks) {
#pragma unroll
      for (int k0 = k4; k0 < k4 + 4; k0 += KB)
        pf_batch<NP, NT, KB, false>(acc, bsel, tb, k0, nks, ap, kshift);
    } else {
      for (int k0 = k4; k0 < nks; k0 += KB)
        pf_batch<NP, NT, KB, true>(acc, bsel, tb, k0, nks, ap, kshift);
    }
    pf_bias<NT>(acc, bsel, g4);
  }
}

// Workgroups (g < ng, b < nb) that share data per g: the shared expert's (weight group, token
// block) in both kernels below, whose token blocks re-read the group's weights, and the routed
// down's (slot, output tile group), whose tile groups re-read the slot's h rows.  Workgroups
// are dispatched round-robin over the 8 XCDs, each with its own L2, so the nb workgroups of
// one g get the block indices j = 8 (nb (g / 8) + b) + g % 8, which share one residue mod 8
// (one XCD, whose L2 then serves the re-reads) -- a bijection onto [0, pf_xcd_blocks) once ng
// is padded to a multiple of 8 (padding workgroups do nothing).
constexpr int PF_XCDS = 8;
inline __host__ __device__ int pf_xcd_blocks(int ng, int nb) {
  return (ng + PF_XCDS - 1) / PF_XCDS * PF_XCDS * nb;
}
QMOE_DEV void pf_xcd_block(int j, int nb, int &g, int &b) {
  const int q = j / PF_XCDS;
  g = j % PF_XCDS + PF_XCDS * (q / nb);
  b = q % nb;
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// grid: shared workgroups first (h group, block of PF_MT tokens), then routed (slot, h
// group); a workgroup of GU_WAVES waves owns the four tiles of one 64-column group of h, wave
// w the tiles 4 group + GU_NT w + j.  Tile j's gate rows 16 tile + [0, 16) are acc[j][0] and
// the matching up rows acc[j][1], so lane l holds gate and up of the same (row, h column
// 16 tile + l % 16).  A workgroup loops over its rows PF_MT at a time.  h = silu(gate) up goes
// to the hi/lo planes (routed rows in bucket order), and the group sums of hi + lo to gh_r /
// gh_s.
__global__ void __launch_bounds__(GU_WAVES * WAVE) gu_pf_kernel(FfnArgs a) {
  __shared__ float gpart[GU_WAVES][PF_MT];
  const int H = a.H, KG = H / GROUP, KS = KG << a.kshift;
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE, n = lane % 16, lg = lane / 16;
  const int grp_s = a.shared ? a.Is / GROUP : 0, ntb = (a.T + PF_MT - 1) / PF_MT;
  const int n_sh = grp_s ? pf_xcd_blocks(grp_s, ntb) : 0;
  int bid = blockIdx.x;
  SlotRows sr;
  int grp, m0, m1;
  if (bid < n_sh) {
    int tb;
    pf_xcd_block(bid, ntb, grp, tb);
    if (grp >= grp_s) return;
    slot_rows(a, 0, true, sr);
    m0 = tb * PF_MT;
    m1 = min(a.T, m0 + PF_MT);
  } else {
    bid -= n_sh;
    const int grp_r = a.I / GROUP;
    if (!slot_rows(a, bid / grp_r, false, sr)) return;
    grp = bid % grp_r;
    m0 = 0;
    m1 = sr.m;
  }
  const int I = sr.shared ? a.Is : a.I, KI = I / GROUP;
  const int tile0 = 4 * grp + GU_NT * wv;
  const uint8_t *tb[GU_NT];
#pragma unroll
  for (int j = 0; j < GU_NT; ++j) tb[j] = sr.blk + (size_t)(tile0 + j) * KS * KSTEP_BYTES;
  uint16_t *hhi = sr.shared ? a.hs_hi : a.hr_hi;
  uint16_t *hlo = sr.shared ? a.hs_lo : a.hr_lo;
  float *gh = sr.shared ? a.gh_s : a.gh_r;
  const int pos0 = sr.shared ? 0 : sr.beg;
  for (int p0 = m0; p0 < m1; p0 += PF_MT) {
    const int mt = min(PF_MT, m1 - p0);
    const int r = min(n, mt - 1);  // padding lanes repeat the last row
    const int tok = sr.shared ? p0 + r : flat_of(a, sr, p0 + r) / a.k;
    const uint16_t *const ap[1] = {a.x + (size_t)tok * H + 8 * lg};
    qmoe_f32x4 acc[GU_NT][2];
    pf_tiles<1, GU_NT, GU_KB>(acc, tb, KS, ap, a.gx + (size_t)tok * KG, a.kshift);
    float hs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < GU_NT; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * lg + i;
        if (m < mt) {
          const float h = silu(acc[j][0][i]) * acc[j][1][i];
          const uint32_t hi = f32_to_bf16_bits(h);
          const uint32_t lo = f32_to_bf16_bits(h - __uint_as_float(hi << 16));
          const size_t at = (size_t)(pos0 + p0 + m) * I + 16 * (tile0 + j) + n;
          hhi[at] = (uint16_t)hi;
          hlo[at] = (uint16_t)lo;
          hs[i] += __uint_as_float(hi << 16) + __uint_as_float(lo << 16);
        }
      }
    }
    // group sums: over the 16 lanes of each lane group, then over the waves (LDS permutes
    // here: a register form, quad DPP then the half-row and row mirrors, raised this kernel
    // from 113 to 131 VGPRs, one wave per SIMD less, and this runs once per row block,
    // outside the k-step loop)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hs[i] += __shfl_xor(hs[i], 1, WAVE);
      hs[i] += __shfl_xor(hs[i], 2, WAVE);
      hs[i] += __shfl_xor(hs[i], 4, WAVE);
      hs[i] += __shfl_xor(hs[i], 8, WAVE);
    }
    if (n == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) gpart[wv][4 * lg + i] = hs[i];
    }
    __syncthreads();
    if ((int)threadIdx.x < mt) {
      const int m = threadIdx.x;
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < GU_WAVES; ++w) t += gpart[w][m];
      gh[(size_t)(pos0 + p0 + m) * KI + grp] = t;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down projection
// grid: shared workgroups first (tile group, block of PF_MT tokens), then routed (slot, tile
// group); a tile group is D_WAVES * D_NT output tiles, wave w computing D_NT of them (32 rows
// of H each: acc[j][0] rows 0..15, acc[j][1] rows 16..31) over all of K, with the h hi and lo
// planes of PF_MT tokens as the activation rows.  Routed rows go to y by flat assignment id,
// shared rows to y_sh.
__global__ void __launch_bounds__(D_WAVES * WAVE) d_pf_kernel(FfnArgs a) {
  const int H = a.H, tiles = H / TILE_ROWS, tgroups = (tiles + D_WAVES * D_NT - 1) / (D_WAVES * D_NT);
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE, n = lane % 16, lg = lane / 16;
  const int ntb = (a.T + PF_MT - 1) / PF_MT;
  const int n_sh = a.shared ? pf_xcd_blocks(tgroups, ntb) : 0;
  int bid = blockIdx.x;
  SlotRows sr;
  int tg, m0, m1;
  if (bid < n_sh) {
    int tb;
    pf_xcd_block(bid, ntb, tg, tb);
    if (tg >= tgroups) return;
    slot_rows(a, 0, true, sr);
    m0 = tb * PF_MT;
    m1 = min(a.T, m0 + PF_MT);
  } else {
    int slot;
    pf_xcd_block(bid - n_sh, tgroups, slot, tg);
    if (slot >= a.n_slots || !slot_rows(a, slot, false, sr)) return;
    m0 = 0;
    m1 = sr.m;
  }
  const int tile0 = (D_WAVES * tg + wv) * D_NT;
  if (tile0 >= tiles) return;  // no barrier in this kernel
  const int K = sr.shared ? a.Is : a.I, KGd = K / GROUP, KSd = KGd << a.kshift;
  const uint8_t *dbase = sr.blk + block_geom(H, K, a.kshift).gu_bytes;
  const uint8_t *tb[D_NT];
#pragma unroll
  for (int j = 0; j < D_NT; ++j)  // tiles past the end re-read the last one (not stored)
    tb[j] = dbase + (size_t)min(tile0 + j, tiles - 1) * KSd * KSTEP_BYTES;
  const uint16_t *phi = sr.shared ? a.hs_hi : a.hr_hi;
  const uint16_t *plo = sr.shared ? a.hs_lo : a.hr_lo;
  const float *gh = sr.shared ? a.gh_s : a.gh_r;
  const int pos0 = sr.shared ? 0 : sr.beg;
  for (int p0 = m0; p0 < m1; p0 += PF_MT) {
    const int mt = min(PF_MT, m1 - p0);
    const size_t pos = (size_t)(pos0 + p0 + min(n, mt - 1));  // padding lanes repeat the last row
    const uint16_t *const ap[2] = {phi + pos * K + 8 * lg, plo + pos * K + 8 * lg};
    qmoe_f32x4 acc[D_NT][2];
    pf_tiles<2, D_NT, D_KB>(acc, tb, KSd, ap, gh + pos * KGd, a.kshift);
    int flat = 0;
    if (!sr.shared && lane < mt) flat = flat_of(a, sr, p0 + lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * lg + i;
      const int fm = __shfl(flat, m, WAVE);
      if (m < mt) {
        float *dst = sr.shared ? a.y_sh + (size_t)(p0 + m) * H : a.y + (size_t)fm * H;
#pragma unroll
        for (int j = 0; j < D_NT; ++j) {
          if (tile0 + j < tiles) {
            dst[TILE_ROWS * (tile0 + j) + n] = acc[j][0][i];
            dst[TILE_ROWS * (tile0 + j) + 16 + n] = acc[j][1][i];
          }
        }
      }
    }
  }
}

// Sums of every 64-element group of x [T, H] (n_groups = T H / 64), the gate/up bias term's
// operand, where no router pass has produced them.  The sum is the balanced pairwise tree
// over the 64 elements, the order the router pass uses, so both give the same bits.
__global__ void __launch_bounds__(256) gsum_kernel(const uint16_t *x, int n_groups, float *g) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_groups) return;
  const qmoe_u32x4 *p = (const qmoe_u32x4 *)(x + (size_t)i * GROUP);
  float v[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const qmoe_u32x4 w = p[j];
    v[4 * j + 0] = bf16lo(w.x) + bf16hi(w.x);
    v[4 * j + 1] = bf16lo(w.y) + bf16hi(w.y);
    v[4 * j + 2] = bf16lo(w.z) + bf16hi(w.z);
    v[4 * j + 3] = bf16lo(w.w) + bf16hi(w.w);
  }
#pragma unroll
  for (int w = 16; w >= 1; w /= 2) {
#pragma unroll
    for (int j = 0; j < w; ++j) v[j] = v[2 * j] + v[2 * j + 1];
  }
  g[i] = v[0];
}

// sum_j w[j] y[j * H + off .. + 4) over j = 0..k-1 in ascending order (fp32 FMAs); the loads of
// eight rows are in flight together (a loop of dependent round trips otherwise)
template <int B>
QMOE_DEV float4 routed_sum_b(const float *y, const float *w, int k, int H, size_t off) {
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += B) {
    float4 v[B];
    float wj[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int j = min(j0 + q, k - 1);   // rows past k re-read the last one (not used)
      wj[q] = w[j];
      v[q] = *(const float4 *)(y + (size_t)j * H + off);
    }
#pragma unroll
    for (int q = 0; q < B; ++q)
      if (j0 + q < k) {
        acc.x = fmaf(wj[q], v[q].x, acc.x);
        acc.y = fmaf(wj[q], v[q].y, acc.y);
        acc.z = fmaf(wj[q], v[q].z, acc.z);
        acc.w = fmaf(wj[q], v[q].w, acc.w);
      }
  }
  return acc;
}
// (up to 16 rows' loads in one batch, so that k <= 16 takes one round trip)
QMOE_DEV float4 routed_sum4(const float *y, const float *w, int k, int H, size_t off) {
  return k <= 8 ? routed_sum_b<8>(y, w, k, H, off) : routed_sum_b<16>(y, w, k, H, off);
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
    // the shared row and the residual loaded first, in flight with the routed rows
    const float4 vs = y_sh ? *(const float4 *)(y_sh + t * H + col) : float4{0.f, 0.f, 0.f, 0.f};
    const uint2 xb = *(const uint2 *)(x + t * H + col);
    float4 acc = routed_sum4(y + t * k * H, w + t * k, k, H, col);
    if (y_sh) {
      acc.x += vs.x; acc.y += vs.y; acc.z += vs.z; acc.w += vs.w;
    }
    acc.x += bf16lo(xb.x); acc.y += bf16hi(xb.x); acc.z += bf16lo(xb.y); acc.w += bf16hi(xb.y);
    const uint2 ob = {f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16),
                      f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16)};
    *(uint2 *)(out + t * H + col) = ob;
    if (out_f32) *(float4 *)(out_f32 + t * H + col) = acc;
  }
}

// cb2 with its post-combine steps (normalisation, residual, layer scalar), one workgroup per
// token row t:
//   m   = sum_j w[t,j] y[t*k+j] + y_sh[t]          fp32, j ascending, then the shared row
//   n   = gain * m / sqrt(mean(m^2) + RMS_EPS)      (gain null: n = m)
//   out = (x + n) * scalar                          (scalar null: 1)
// With neither step the arithmetic is combine_pf_kernel's.  H <= 4 * POST_THREADS * POST_V.
constexpr int POST_THREADS = 256, POST_V = 8;
__global__ void __launch_bounds__(POST_THREADS) combine_post_kernel(
    const uint16_t *x, const float *y, const float *w, const float *y_sh, const float *gain,
    const float *scalar, int H, int k, uint16_t *out, float *out_f32) {
  __shared__ float red[POST_THREADS / WAVE];
  const int t = blockIdx.x, tid = threadIdx.x, n4 = H / 4;
  float4 m[POST_V];
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < POST_V; ++v) {
    const int c = tid + POST_THREADS * v;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    if (c < n4) {
      acc = routed_sum4(y + (size_t)t * k * H, w + (size_t)t * k, k, H, (size_t)4 * c);
      if (y_sh) {
        const float4 s4 = *(const float4 *)(y_sh + (size_t)t * H + 4 * c);
        acc.x += s4.x; acc.y += s4.y; acc.z += s4.z; acc.w += s4.w;
      }
      ss = fmaf(acc.x, acc.x, ss);
      ss = fmaf(acc.y, acc.y, ss);
      ss = fmaf(acc.z, acc.z, ss);
      ss = fmaf(acc.w, acc.w, ss);
    }
    m[v] = acc;
  }
  float r = 1.f;
  if (gain) {
    ss = wave_sum(ss);
    if (tid % WAVE == 0) red[tid / WAVE] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < POST_THREADS / WAVE; ++i) tot += red[i];
    r = 1.f / sqrtf(tot / (float)H + RMS_EPS);
  }
  const float al = scalar ? *scalar : 1.f;
#pragma unroll
  for (int v = 0; v < POST_V; ++v) {
    const int c = tid + POST_THREADS * v;
    if (c >= n4) continue;
    float4 n = m[v];
    if (gain) {
      const float4 g = *(const float4 *)(gain + 4 * c);
      n.x = g.x * (n.x * r); n.y = g.y * (n.y * r); n.z = g.z * (n.z * r); n.w = g.w * (n.w * r);
    }
    const uint2 xb = *(const uint2 *)(x + (size_t)t * H + 4 * c);
    float4 o;
    o.x = (bf16lo(xb.x) + n.x) * al;
    o.y = (bf16hi(xb.x) + n.y) * al;
    o.z = (bf16lo(xb.y) + n.z) * al;
    o.w = (bf16hi(xb.y) + n.w) * al;
    const uint2 ob = {f32_to_bf16_bits(o.x) | (f32_to_bf16_bits(o.y) << 16),
                      f32_to_bf16_bits(o.z) | (f32_to_bf16_bits(o.w) << 16)};
    *(uint2 *)(out + (size_t)t * H + 4 * c) = ob;
    if (out_f32) *(float4 *)(out_f32 + (size_t)t * H + 4 * c) = o;
  }
}

}  // namespace qmoe
