// Grouped-GEMM kernels of the expert FFN on the gfx950 matrix cores (prefill chunks of the
// TurboFieldfare post, section "TurboFieldfare의 전문가 스트리밍 구조": up to 128 tokens per
// chunk, so each expert read serves every row routed to it).
//
// Operands are exact: the int4 codes become the bf16 values 128 + q (one AND-OR per two
// codes), activations are bf16 (x) or hi/lo bf16 planes (h).  Per k-step (one 64-input group
// with scale s and bias b of each weight row) and 32x32 output block:
//   t   = sum over the group of a * (128 + q)        four v_mfma_f32_32x32x16_bf16
//   acc += s * t                                      one FMA per accumulator (VALU)
//   acc += (b - 128 s) * sum over the group of a      one v_mfma_f32_32x32x2_f32, whose
//                                                     K = 2 entries are the two 32-column
//                                                     halves' activation sums
// so the result equals sum (s q + b) a with fp32 accumulation, as in the VALU path.
//
// Lane layout (v_mfma_f32_32x32x16_bf16): lane l supplies row (l % 32) of both operands for
// the 8-element sub-block (l / 32) of each 16-deep K block.  The store's k-step gives lane l
// the codes of weight row l % 32 for columns 32 (l / 32) + [0, 32), so word j of the lane's
// 16 bytes is K block j.  Activation rows (tokens) are M and weight rows are N, so every
// accumulator of a lane belongs to the lane's own weight row and uses its own scale.
// Accumulator r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//
// A workgroup (8 waves) owns whole weight tiles and loops over blocks of activation rows:
// the rows are staged in LDS (padded rows, with the sums of every 32 columns), the waves
// split the k-steps, and their partial blocks are added in LDS.
#pragma once
#include "common.h"
#include "store.h"

namespace qmoe {

typedef __bf16 qmoe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float qmoe_f32x16 __attribute__((ext_vector_type(16)));

constexpr int PF_W = 8;                 // waves per workgroup
constexpr int PF_THREADS = PF_W * WAVE;
constexpr int KBM = 6;                  // k-steps per load batch of a wave
constexpr int GU_MT = 10;               // token rows per gate/up pass
constexpr int GU_SH_PASSES = 3;         // passes per shared-expert gate/up workgroup
constexpr int D_MT = 16;                // token rows per down pass (hi + lo planes: 32 MFMA rows)
constexpr int D_TPW = 4;                // down tiles per workgroup (two waves per tile)
constexpr int D_SH_PASSES = 2;          // passes per shared-expert down workgroup
constexpr int PF_KMAX = 16;             // most k-steps a down workgroup stages (1024 columns)
constexpr uint32_t BF16_ONES = 0x3F803F80u;

QMOE_DEV int mfma_row(int lane, int r) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); }

// B operand: the 8 codes of word w as bf16 (128 + q), element order
QMOE_DEV qmoe_bf16x8 q4_operand(uint32_t w) {
  const qmoe_u32x4 v = {nib_pair(w, 0), nib_pair(w, 1), nib_pair(w, 2), nib_pair(w, 3)};
  return __builtin_bit_cast(qmoe_bf16x8, v);
}

// ---------------------------------------------------------------- LDS layouts
// Staged activations: rows of K bf16 with a stride of K + 8 (16 bytes of padding, so that
// the 32 rows read by a wave fall in different banks), then fp32 sums of every 32 columns.
inline __host__ __device__ int pf_stride(int K) { return K + 8; }
inline __host__ __device__ size_t pf_stage_bytes(int rows, int K) {
  return (size_t)rows * pf_stride(K) * 2 + (size_t)rows * (K / 32) * 4;
}
inline __host__ __device__ size_t gu_pf_lds(int H) {
  return pf_stage_bytes(GU_MT, H) + (size_t)PF_W * GU_MT * 32 * 4;
}
inline __host__ __device__ size_t d_pf_lds(int Kc) {
  return pf_stage_bytes(2 * D_MT, Kc) + (size_t)PF_W * D_MT * 32 * 4;
}

// Stage n rows (row r at src(r), K bf16 columns) into dst / sums.  Loads are issued eight per
// thread before any is stored.
template <class Src>
QMOE_DEV void pf_stage(Src src, int n, int K, uint16_t *dst, float *sums) {
  const int n8 = K / 8, total = n * n8, S = pf_stride(K);
  for (int base = 0; base < total; base += 8 * PF_THREADS) {
    qmoe_u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = base + (int)threadIdx.x + j * PF_THREADS;
      if (c < total) v[j] = *(const qmoe_u32x4 *)(src(c / n8) + 8 * (c % n8));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = base + (int)threadIdx.x + j * PF_THREADS;
      const int r = c / n8, cc = c % n8;
      float p = 0.f;
      if (c < total) {
        *(qmoe_u32x4 *)(dst + (size_t)r * S + 8 * cc) = v[j];
        p = bf16lo(v[j].x) + bf16hi(v[j].x) + bf16lo(v[j].y) + bf16hi(v[j].y) +
            bf16lo(v[j].z) + bf16hi(v[j].z) + bf16lo(v[j].w) + bf16hi(v[j].w);
      }
      // four consecutive threads hold one 32-column block (n8 is a multiple of 8)
      p += __shfl_xor(p, 1, WAVE);
      p += __shfl_xor(p, 2, WAVE);
      if (c < total && (cc & 3) == 0) sums[r * (K / 32) + cc / 4] = p;
    }
  }
}

// ---------------------------------------------------------------- one wave's k-steps
// k-steps [ks0, ks0 + nk) of the tile at tbase against staged row `arow` (LDS; nullptr for a
// padding row) whose 32-column sums are `asum`; columns of k-step ks start at ks * 64 - c0.
QMOE_DEV qmoe_f32x16 pf_tile_part(const uint8_t *tbase, int ks0, int nk, int c0,
                                  const uint16_t *arow, const float *asum) {
  const int lane = threadIdx.x % WAVE, rr = lane % 32, half = lane / 32;
  qmoe_f32x16 acc = {};
  for (int kc = 0; kc < nk; kc += KBM) {
    qmoe_u32x4 cv[KBM];
    uint32_t sb[KBM];
    load_batch<KBM>(tbase, ks0, kc, nk, lane, rr, cv, sb);
#pragma unroll
    for (int u = 0; u < KBM; ++u) {
      if (kc + u >= nk) break;
      const int col = (ks0 + kc + u) * GROUP - c0 + 32 * half;
      qmoe_u32x4 xa[4];
      float xs = 0.f;
      if (arow) {
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[j] = *(const qmoe_u32x4 *)(arow + col + 8 * j);
        xs = asum[col / 32];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[j] = qmoe_u32x4{0u, 0u, 0u, 0u};
      }
      qmoe_f32x16 t = {};
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(qmoe_bf16x8, xa[0]),
                                                  q4_operand(cv[u].x), t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(qmoe_bf16x8, xa[1]),
                                                  q4_operand(cv[u].y), t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(qmoe_bf16x8, xa[2]),
                                                  q4_operand(cv[u].z), t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(qmoe_bf16x8, xa[3]),
                                                  q4_operand(cv[u].w), t, 0, 0, 0);
      const float s = bf16lo(sb[u]), c = fmaf(-128.f, s, bf16hi(sb[u]));
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = fmaf(s, t[r], acc[r]);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(xs, c, acc, 0, 0, 0);
    }
  }
  return acc;
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// grid: shared workgroups first (tile, block of GU_SH_PASSES * GU_MT tokens), then routed
// (slot, tile); a routed workgroup loops over its bucket in blocks of GU_MT rows.
// h = silu(gate) * up goes to the hi/lo planes (routed rows in bucket order).
__global__ void __launch_bounds__(PF_THREADS) gu_pf_kernel(FfnArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int H = a.H, KS = H / GROUP;
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  uint16_t *xl = (uint16_t *)smem;
  float *xsum = (float *)(smem + (size_t)GU_MT * pf_stride(H) * 2);
  float *red = (float *)(smem + pf_stage_bytes(GU_MT, H));           // [PF_W][GU_MT][32]
  const int tiles_s = a.shared ? a.Is / 16 : 0;
  const int per_sh = GU_SH_PASSES * GU_MT;
  const int n_sh = tiles_s * ((a.T + per_sh - 1) / per_sh);
  int bid = blockIdx.x;
  SlotRows sr;
  int tile, m0, m1;
  if (bid < n_sh) {
    slot_rows(a, 0, true, sr);
    tile = bid % tiles_s;
    m0 = (bid / tiles_s) * per_sh;
    m1 = min(a.T, m0 + per_sh);
  } else {
    bid -= n_sh;
    const int tiles_r = a.I / 16;
    if (!slot_rows(a, bid / tiles_r, false, sr)) return;
    tile = bid % tiles_r;
    m0 = 0;
    m1 = sr.m;
  }
  const int I = sr.shared ? a.Is : a.I;
  const uint8_t *tbase = sr.blk + (size_t)tile * KS * KSTEP_BYTES;
  const int ks0 = (KS * wv) / PF_W, nk = (KS * (wv + 1)) / PF_W - ks0;
  for (int p0 = m0; p0 < m1; p0 += GU_MT) {
    const int mt = min(GU_MT, m1 - p0);
    pf_stage([&](int r) {
               const int t = sr.shared ? p0 + r : flat_of(a, sr, p0 + r) / a.k;
               return a.x + (size_t)t * H;
             }, mt, H, xl, xsum);
    __syncthreads();
    const int i = lane % 32;
    const bool live = i < mt;
    const qmoe_f32x16 acc = pf_tile_part(tbase, ks0, nk, 0, live ? xl + (size_t)i * pf_stride(H) : nullptr,
                                         xsum + i * (H / 32));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mfma_row(lane, r);
      if (m < mt) red[(wv * GU_MT + m) * 32 + lane % 32] = acc[r];
    }
    __syncthreads();
    for (int o = tid; o < mt * 16; o += PF_THREADS) {
      const int m = o / 16, n = o % 16;
      float g = 0.f, u = 0.f;
      for (int w = 0; w < PF_W; ++w) {
        g += red[(w * GU_MT + m) * 32 + n];
        u += red[(w * GU_MT + m) * 32 + 16 + n];
      }
      const float h = silu(g) * u;
      const uint32_t hi = f32_to_bf16_bits(h);
      const uint32_t lo = f32_to_bf16_bits(h - __uint_as_float(hi << 16));
      const size_t row = sr.shared ? (size_t)(p0 + m) : (size_t)(sr.beg + p0 + m);
      (sr.shared ? a.hs_hi : a.hr_hi)[row * I + 16 * tile + n] = (uint16_t)hi;
      (sr.shared ? a.hs_lo : a.hr_lo)[row * I + 16 * tile + n] = (uint16_t)lo;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down projection
// grid: shared workgroups first (K chunk c, tile group, block of D_SH_PASSES * D_MT tokens),
// then routed (slot, tile group).  Waves 2j and 2j+1 share tile D_TPW * group + j and split
// its k-steps.  The 32 MFMA rows of a pass are 16 tokens' h hi planes (rows 0..15) and lo
// planes (rows 16..31); a token's output is the sum of its two rows, accumulators r and r+8
// of the same lane.  Routed rows go to y (by flat assignment id), shared rows to the chunk's
// partial y_sh_part[c].
__global__ void __launch_bounds__(PF_THREADS) d_pf_kernel(FfnArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int H = a.H;
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int tiles_d = H / TILE_ROWS, groups = (tiles_d + D_TPW - 1) / D_TPW;
  const int per_sh = D_SH_PASSES * D_MT;
  const int mblk = (a.T + per_sh - 1) / per_sh;
  const int n_sh = a.shared ? a.n_sh_chunks * groups * mblk : 0;
  int bid = blockIdx.x;
  SlotRows sr;
  int g, m0, m1, kb0, nks, c = 0;
  if (bid < n_sh) {
    slot_rows(a, 0, true, sr);
    g = bid % groups;
    const int rest = bid / groups;
    c = rest % a.n_sh_chunks;
    m0 = (rest / a.n_sh_chunks) * per_sh;
    m1 = min(a.T, m0 + per_sh);
    const int KSs = a.Is / GROUP;
    kb0 = (KSs * c) / a.n_sh_chunks;
    nks = (KSs * (c + 1)) / a.n_sh_chunks - kb0;
  } else {
    bid -= n_sh;
    if (!slot_rows(a, bid / groups, false, sr)) return;
    g = bid % groups;
    m0 = 0;
    m1 = sr.m;
    kb0 = 0;
    nks = a.I / GROUP;
  }
  const int K = sr.shared ? a.Is : a.I;
  const int Kc = nks * GROUP, S = pf_stride(Kc);
  uint16_t *hl = (uint16_t *)smem;                                   // [2 * D_MT][S]
  float *hsum = (float *)(smem + (size_t)2 * D_MT * S * 2);          // [2 * D_MT][Kc/32]
  float *red = (float *)(smem + pf_stage_bytes(2 * D_MT, Kc));       // [PF_W][D_MT][32]
  const int tile = g * D_TPW + wv / 2, part = wv % 2;
  const bool tile_ok = tile < tiles_d;
  const BlockGeom geo = block_geom(H, K);
  const uint8_t *tbase = sr.blk + geo.gu_bytes + (size_t)min(tile, tiles_d - 1) * (K / GROUP) * KSTEP_BYTES;
  const int ks0 = kb0 + (nks * part) / 2, nk = tile_ok ? kb0 + (nks * (part + 1)) / 2 - ks0 : 0;
  const uint16_t *src_hi = sr.shared ? a.hs_hi : a.hr_hi;
  const uint16_t *src_lo = sr.shared ? a.hs_lo : a.hr_lo;
  for (int p0 = m0; p0 < m1; p0 += D_MT) {
    const int mt = min(D_MT, m1 - p0);
    pf_stage([&](int r) {
               const int i = r % mt;
               const size_t row = sr.shared ? (size_t)(p0 + i) : (size_t)(sr.beg + p0 + i);
               return (r < mt ? src_hi : src_lo) + row * K + (size_t)kb0 * GROUP;
             }, 2 * mt, Kc, hl, hsum);
    __syncthreads();
    // MFMA row m: plane m / 16, token m % 16; staged row index: plane * mt + token
    const int i = lane % 32, tok = i % 16, plane = i / 16;
    const bool live = tok < mt;
    const int srow = plane * mt + tok;
    const qmoe_f32x16 acc = pf_tile_part(tbase, ks0, nk, kb0 * GROUP,
                                         live ? hl + (size_t)srow * S : nullptr,
                                         hsum + srow * (Kc / 32));
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int m = mfma_row(lane, r);
      if (m < mt) red[(wv * D_MT + m) * 32 + lane % 32] = acc[r] + acc[r + 8];
    }
    __syncthreads();
    for (int o = tid; o < D_TPW * mt * 32; o += PF_THREADS) {
      const int j = o / (mt * 32), m = (o / 32) % mt, n = o % 32;
      const int tt = g * D_TPW + j;
      if (tt >= tiles_d) continue;
      const float yv = red[((2 * j) * D_MT + m) * 32 + n] + red[((2 * j + 1) * D_MT + m) * 32 + n];
      if (sr.shared)
        a.y_sh_part[((size_t)c * a.T + p0 + m) * H + TILE_ROWS * tt + n] = yv;
      else
        a.y[(size_t)flat_of(a, sr, p0 + m) * H + TILE_ROWS * tt + n] = yv;
    }
    __syncthreads();
  }
}

// out[t, :] = bf16( x[t, :] + sum_j w[t,j] y[t*k+j, :] + sum_c y_sh_part[c][t, :] ), fp32,
// j ascending then the shared chunks; four columns per thread.  Without `out` the shared
// chunks are only summed into y_sh (the standalone FFN entry point).
__global__ void __launch_bounds__(256) combine_pf_kernel(const uint16_t *x, const float *y,
                                                         const float *w, const float *y_sh_part,
                                                         int nsh, int T, int H, int k,
                                                         uint16_t *out, float *out_f32,
                                                         float *y_sh) {
  const size_t n4 = (size_t)T * H / 4;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < n4;
       o += (size_t)gridDim.x * blockDim.x) {
    const size_t t = (o * 4) / H, col = (o * 4) % H;
    float4 sh = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nsh; ++c) {
      const float4 v = *(const float4 *)(y_sh_part + ((size_t)c * T + t) * H + col);
      sh.x += v.x; sh.y += v.y; sh.z += v.z; sh.w += v.w;
    }
    if (!out) {
      *(float4 *)(y_sh + t * H + col) = sh;
      continue;
    }
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const float wj = w[t * k + j];
      const float4 v = *(const float4 *)(y + (t * k + j) * H + col);
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
      acc.z = fmaf(wj, v.z, acc.z);
      acc.w = fmaf(wj, v.w, acc.w);
    }
    acc.x += sh.x; acc.y += sh.y; acc.z += sh.z; acc.w += sh.w;
    const uint2 xb = *(const uint2 *)(x + t * H + col);
    acc.x += bf16lo(xb.x); acc.y += bf16hi(xb.x); acc.z += bf16lo(xb.y); acc.w += bf16hi(xb.y);
    const uint2 ob = {f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16),
                      f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16)};
    *(uint2 *)(out + t * H + col) = ob;
    if (out_f32) *(float4 *)(out_f32 + t * H + col) = acc;
  }
}

}  // namespace qmoe
