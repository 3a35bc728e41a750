// Expert FFN kernels over the packed store: SwiGLU gate/up projection and down projection
// with int4 codes decoded in registers (never written out), and the router-weighted combine
// with the shared expert and the residual (TurboFieldfare post, sections "TurboFieldfare의
// 전문가 스트리밍 구조" and "TurboFieldfare가 메모리를 아끼는 방식").
//
// Math of one k-step (64 inputs = one group with scale s and bias b) of one row:
//   sum_j (s q_j + b) x_j = s * sum_j (128 + q_j) x_j + (b - 128 s) * sum_j x_j
// The first sum comes from bf16 dot products of exact (128 + q) operands with exact bf16
// activations; the activation group sums are staged once per token.  Accumulation is fp32.
// The down projection's input h is fp32; it is carried as hi + lo bf16 parts
// (hi = bf16(h), lo = bf16(h - hi)), so its products keep ~16 significant bits.
#pragma once
#include "common.h"
#include "store.h"

namespace qmoe {

struct FfnArgs {
  const uint8_t *experts;     // routed blocks
  size_t stride;
  const uint8_t *shared;      // shared block or null
  int H, I, Is, k, T, n_experts;
  int kshift;                 // k-steps per group: 0 (4-bit experts) or 1 (8-bit, two planes)
  const uint16_t *x;          // [T, H] bf16
  const int32_t *offsets, *sorted, *active, *n_active;
  int n_slots;                // routed slots in the grid: active experts (no slot table) or
                              //   bucket blocks (slot table)
  uint16_t *hr_hi, *hr_lo;    // routed h [T*k, I] in bucket order
  uint16_t *hs_hi, *hs_lo;    // shared h [T, Is]
  float *y;                   // routed y [T*k, H] by flat id
  float *y_sh;                // shared y [T, H] or null
  const float *gx;            // sums of every 64-column group of x [T, H/64] (matrix-core path)
  float *gh_r, *gh_s;         // the same for h hi + lo: routed [T*k, I/64], shared [T, Is/64]
  const int32_t *slot_tab;    // [n_slots][4] block table {expert, first position, rows, first
                              //   flat id or -1} or null
  int n_sh_chunks;            // VALU down kernel: workgroups per tile for the shared block
};

// Resolve the rows handled by a workgroup of slot `slot` (routed) or the shared slot.
struct SlotRows {
  const uint8_t *blk;
  int m;       // number of rows
  int beg;     // first bucket position (routed) / 0 (shared)
  int first;   // flat assignment id of the first row (routed, from the slot table) or -1
  bool shared;
};

// Bucket data that would index outside the store or the assignment list makes the slot
// empty instead (the buffers are caller-provided in the standalone entry point).  With a
// slot table (layer path) one 16-byte load resolves the slot.
QMOE_DEV bool slot_rows(const FfnArgs &a, int slot, bool shared, SlotRows &r) {
  r.first = -1;
  if (shared) {
    r.blk = a.shared; r.m = a.T; r.beg = 0; r.shared = true;
    return true;
  }
  int e;
  if (a.slot_tab) {
    const qmoe_u32x4 ent = *(const qmoe_u32x4 *)(a.slot_tab + 4 * slot);
    e = (int)ent.x; r.beg = (int)ent.y; r.m = (int)ent.z; r.first = (int)ent.w;
    if (r.m <= 0) return false;
  } else {
    if (slot >= min(*a.n_active, a.n_experts)) return false;
    e = a.active[slot];
    if ((unsigned)e >= (unsigned)a.n_experts) return false;
    r.beg = a.offsets[e];
    r.m = a.offsets[e + 1] - r.beg;
  }
  if ((unsigned)e >= (unsigned)a.n_experts) return false;
  r.blk = a.experts + (size_t)e * a.stride;
  r.shared = false;
  if (r.first < 0 || r.first >= a.T * a.k) r.first = -1;
  return r.beg >= 0 && r.m > 0 && r.beg + r.m <= a.T * a.k;
}

// flat assignment id of row i of slot sr (bucket position sr.beg + i), kept inside [0, T*k)
QMOE_DEV int flat_of(const FfnArgs &a, const SlotRows &sr, int i) {
  if (i == 0 && sr.first >= 0) return sr.first;
  return min(max(a.sorted[sr.beg + i], 0), a.T * a.k - 1);
}

// ---------------------------------------------------------------- staging helpers
// Stage mb activation rows (bf16, row r read from src + rowsel(r) * K) into LDS, with the
// sum of every 32 consecutive elements (fp32) next to them.
template <int NT, class RowSel>
QMOE_DEV void stage_rows_bf16(const uint16_t *src, int K, int mb, RowSel rowsel, uint16_t *dst,
                              float *sums) {
  const int n8 = K / 8;
  for (int c = threadIdx.x; c < mb * n8; c += NT) {
    const int i = c / n8, cc = c % n8;
    const qmoe_u32x4 v = *(const qmoe_u32x4 *)(src + (size_t)rowsel(i) * K + 8 * cc);
    *(qmoe_u32x4 *)(dst + (size_t)i * K + 8 * cc) = v;
    float p = bf16lo(v.x) + bf16hi(v.x) + bf16lo(v.y) + bf16hi(v.y) + bf16lo(v.z) +
              bf16hi(v.z) + bf16lo(v.w) + bf16hi(v.w);
    p += xor1(p);
    p += xor2(p);
    if ((cc & 3) == 0) sums[i * (K / 32) + cc / 4] = p;
  }
}

// Same for h carried as hi/lo bf16 planes; the sums are of hi + lo.
template <int NT, class RowSel>
QMOE_DEV void stage_rows_hilo(const uint16_t *src_hi, const uint16_t *src_lo, int K, int mb,
                              RowSel rowsel, uint16_t *dst_hi, uint16_t *dst_lo, float *sums) {
  const int n8 = K / 8;
  for (int c = threadIdx.x; c < mb * n8; c += NT) {
    const int i = c / n8, cc = c % n8;
    const size_t row = (size_t)rowsel(i);
    const qmoe_u32x4 vh = *(const qmoe_u32x4 *)(src_hi + row * K + 8 * cc);
    const qmoe_u32x4 vl = *(const qmoe_u32x4 *)(src_lo + row * K + 8 * cc);
    *(qmoe_u32x4 *)(dst_hi + (size_t)i * K + 8 * cc) = vh;
    *(qmoe_u32x4 *)(dst_lo + (size_t)i * K + 8 * cc) = vl;
    float p = (bf16lo(vh.x) + bf16lo(vl.x)) + (bf16hi(vh.x) + bf16hi(vl.x)) +
              (bf16lo(vh.y) + bf16lo(vl.y)) + (bf16hi(vh.y) + bf16hi(vl.y)) +
              (bf16lo(vh.z) + bf16lo(vl.z)) + (bf16hi(vh.z) + bf16hi(vl.z)) +
              (bf16lo(vh.w) + bf16lo(vl.w)) + (bf16hi(vh.w) + bf16hi(vl.w));
    p += xor1(p);
    p += xor2(p);
    if ((cc & 3) == 0) sums[i * (K / 32) + cc / 4] = p;
  }
}

QMOE_DEV void lds_row16(const uint16_t *p, uint32_t v[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const qmoe_u32x4 t4 = *(const qmoe_u32x4 *)(p + 8 * q);
    v[4 * q] = t4.x; v[4 * q + 1] = t4.y; v[4 * q + 2] = t4.z; v[4 * q + 3] = t4.w;
  }
}

// Contribution of one k-step (32 codes of this lane, scale|bias word sb) to a row:
//   s * sum (128+q) x + (b - 128 s) * sum x
QMOE_DEV float kstep_bf16(const qmoe_u32x4 cv, uint32_t sb, const uint16_t *xrow, float xsum) {
  const uint32_t w4[4] = {cv.x, cv.y, cv.z, cv.w};
  uint32_t xv[16];
  lds_row16(xrow, xv);
  const float s = bf16lo(sb), b = bf16hi(sb);
  const float d = dot32_q4_bf16(w4, xv);
  return fmaf(s, d, fmaf(-128.f, s, b) * xsum);
}

QMOE_DEV float kstep_hilo(const qmoe_u32x4 cv, uint32_t sb, const uint16_t *hrow,
                          const uint16_t *lrow, float hsum) {
  const uint32_t w4[4] = {cv.x, cv.y, cv.z, cv.w};
  uint32_t xh[16], xl[16];
  lds_row16(hrow, xh);
  lds_row16(lrow, xl);
  const float s = bf16lo(sb), b = bf16hi(sb);
  const float d = dot32_q4_bf16(w4, xh) + dot32_q4_bf16(w4, xl);
  return fmaf(s, d, fmaf(-128.f, s, b) * hsum);
}

// Load k-steps ks0 + kc .. ks0 + kc + KB - 1 of a tile (clamped to the wave's last k-step,
// whose duplicates are loaded but not used): this lane's 16 code bytes and its row's
// scale|bias word, all loads issued before any is used.  The loads are non-temporal: these
// callers read every weight of a token step once, and the hint measured 0.6 us faster per
// one-token layer (the multi-token kernels, which re-read an expert per 16-row block, keep
// ordinary loads).
template <int KB>
QMOE_DEV void load_batch(const uint8_t *tbase, int ks0, int kc, int nk, int lane, int rr,
                         qmoe_u32x4 cv[KB], uint32_t sb[KB]) {
#pragma unroll
  for (int u = 0; u < KB; ++u) {
    const uint8_t *kb = tbase + (size_t)(ks0 + min(kc + u, nk - 1)) * KSTEP_BYTES;
    cv[u] = __builtin_nontemporal_load((const qmoe_u32x4 *)(kb + lane * 16));
    sb[u] = __builtin_nontemporal_load((const uint32_t *)(kb + 1024 + rr * 4));
  }
}

// ---------------------------------------------------------------- gate/up tile
// LDS: x [MB][H] bf16, xs [MB][H/32] fp32, red [W][MB][32] fp32
template <int W, int MB>
inline __host__ __device__ size_t gu_lds_bytes(int H) {
  return (size_t)MB * H * 2 + (size_t)MB * (H / 32) * 4 + (size_t)W * MB * 32 * 4;
}

// One tile (16 gate rows + the 16 matching up rows) for the rows of slot `sr`, split-K over
// W waves; each wave loads its k-steps in batches of KB (all loads of a batch in flight
// together, out-of-range entries re-read the last valid k-step and are not used).
template <int W, int MB, int KB>
QMOE_DEV void gu_tile(const FfnArgs &a, const SlotRows &sr, int tile, char *smem) {
  const int H = a.H;
  const int I = sr.shared ? a.Is : a.I;
  const int KS = (H / GROUP) << a.kshift;
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int rr = lane % 32, half = lane / 32;
  uint16_t *xl = (uint16_t *)smem;                              // [MB][H]
  float *xs = (float *)(smem + (size_t)MB * H * 2);              // [MB][H/32]
  float *red = xs + MB * (H / 32);                               // [W][MB][32]
  const uint8_t *tbase = sr.blk + (size_t)tile * KS * KSTEP_BYTES;
  const int ks0 = (KS * wv) / W, nk = (KS * (wv + 1)) / W - ks0;
  qmoe_u32x4 cv[KB];
  uint32_t sb[KB];
  // the first batch of weights is in flight while the activations are staged
  if (nk > 0) load_batch<KB>(tbase, ks0, 0, nk, lane, rr, cv, sb);
  for (int r0 = 0; r0 < sr.m; r0 += MB) {
    const int mb = min(MB, sr.m - r0);
    stage_rows_bf16<W * WAVE>(a.x, H, mb, [&](int i) {
      return sr.shared ? (r0 + i) : flat_of(a, sr, r0 + i) / a.k; }, xl, xs);
    __syncthreads();
    float acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = 0.f;
    for (int kc = 0; kc < nk; kc += KB) {
      if (kc > 0 || r0 > 0) load_batch<KB>(tbase, ks0, kc, nk, lane, rr, cv, sb);
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        if (kc + u < nk) {
          const int col = ((ks0 + kc + u) >> a.kshift) * GROUP + half * 32;
#pragma unroll
          for (int i = 0; i < MB; ++i)
            if (i < mb)
              acc[i] += kstep_bf16(cv[u], sb[u], xl + (size_t)i * H + col, xs[i * (H / 32) + col / 32]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const float tot = acc[i] + xor32(acc[i]);
      if (half == 0) red[(wv * MB + i) * 32 + rr] = tot;
    }
    __syncthreads();
    for (int o = tid; o < mb * 16; o += W * WAVE) {
      const int i = o / 16, r = o % 16;
      float g = 0.f, u = 0.f;
      for (int w = 0; w < W; ++w) {
        g += red[(w * MB + i) * 32 + r];
        u += red[(w * MB + i) * 32 + 16 + r];
      }
      const float h = silu(g) * u;
      const uint32_t hi = f32_to_bf16_bits(h);
      const uint32_t lo = f32_to_bf16_bits(h - __uint_as_float(hi << 16));
      const size_t row = sr.shared ? (size_t)(r0 + i) : (size_t)(sr.beg + r0 + i);
      uint16_t *dh = sr.shared ? a.hs_hi : a.hr_hi;
      uint16_t *dl = sr.shared ? a.hs_lo : a.hr_lo;
      dh[row * I + 16 * tile + r] = (uint16_t)hi;
      dl[row * I + 16 * tile + r] = (uint16_t)lo;
    }
    __syncthreads();
  }
}

// grid.x = n_slots * (I/16) routed tiles, then Is/16 shared tiles (if a.shared)
template <int W, int MB, int KB>
__global__ void __launch_bounds__(W * WAVE) gu_kernel(FfnArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int tiles_r = a.I / 16;
  const int n_routed = a.n_slots * tiles_r;
  int bid = blockIdx.x;
  SlotRows sr;
  int tile;
  if (bid < n_routed) {
    if (!slot_rows(a, bid / tiles_r, false, sr)) return;
    tile = bid % tiles_r;
  } else {
    slot_rows(a, 0, true, sr);
    tile = bid - n_routed;
  }
  gu_tile<W, MB, KB>(a, sr, tile, smem);
}

// ---------------------------------------------------------------- down tile (per slot)
// LDS: h hi [MB][Kc] bf16, h lo [MB][Kc] bf16, hsum [MB][Kc/32] fp32, red [W][MB][32] fp32
// where Kc = 64 * (k-steps of the workgroup)
template <int W, int MB>
inline __host__ __device__ size_t d_lds_bytes(int Kc) {
  return (size_t)MB * Kc * 4 + (size_t)MB * (Kc / 32) * 4 + (size_t)W * MB * 32 * 4;
}

// Groups [kb0, kb0 + nks) of one 32-row output tile of the down projection of slot `sr`
// (K = the block's width; a group is 1 << kshift k-steps).  Output rows go to dst (row of
// token r0+i = ysel(r0+i)).
template <int W, int MB, int KB, class YSel>
QMOE_DEV void d_tile(const FfnArgs &a, const SlotRows &sr, int tile, int kb0, int nks,
                     float *dst, YSel ysel, char *smem) {
  const int H = a.H;
  const int K = sr.shared ? a.Is : a.I;
  const int KS = (K / GROUP) << a.kshift, nkk = nks << a.kshift;
  const int Kc = nks * GROUP;
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int rr = lane % 32, half = lane / 32;
  uint16_t *hh = (uint16_t *)smem;                              // [MB][Kc]
  uint16_t *hl = hh + (size_t)MB * Kc;                          // [MB][Kc]
  float *hs = (float *)(hl + (size_t)MB * Kc);                  // [MB][Kc/32]
  float *red = hs + MB * (Kc / 32);                             // [W][MB][32]
  const BlockGeom geo = block_geom(H, K, a.kshift);
  const uint8_t *tbase =
      sr.blk + geo.gu_bytes + ((size_t)tile * KS + ((size_t)kb0 << a.kshift)) * KSTEP_BYTES;
  const int ks0 = (nkk * wv) / W, nk = (nkk * (wv + 1)) / W - ks0;
  const uint16_t *src_hi = (sr.shared ? a.hs_hi : a.hr_hi) + (size_t)kb0 * GROUP;
  const uint16_t *src_lo = (sr.shared ? a.hs_lo : a.hr_lo) + (size_t)kb0 * GROUP;
  qmoe_u32x4 cv[KB];
  uint32_t sb[KB];
  if (nk > 0) load_batch<KB>(tbase, ks0, 0, nk, lane, rr, cv, sb);
  for (int r0 = 0; r0 < sr.m; r0 += MB) {
    const int mb = min(MB, sr.m - r0);
    // h columns [kb0*64, kb0*64 + Kc) of the rows; source rows have stride K
    const int n8 = Kc / 8;
    for (int c = tid; c < mb * n8; c += W * WAVE) {
      const int i = c / n8, cc = c % n8;
      const size_t row = (size_t)(sr.beg + r0 + i);
      const qmoe_u32x4 vh = *(const qmoe_u32x4 *)(src_hi + row * K + 8 * cc);
      const qmoe_u32x4 vl = *(const qmoe_u32x4 *)(src_lo + row * K + 8 * cc);
      *(qmoe_u32x4 *)(hh + (size_t)i * Kc + 8 * cc) = vh;
      *(qmoe_u32x4 *)(hl + (size_t)i * Kc + 8 * cc) = vl;
      float p = (bf16lo(vh.x) + bf16lo(vl.x)) + (bf16hi(vh.x) + bf16hi(vl.x)) +
                (bf16lo(vh.y) + bf16lo(vl.y)) + (bf16hi(vh.y) + bf16hi(vl.y)) +
                (bf16lo(vh.z) + bf16lo(vl.z)) + (bf16hi(vh.z) + bf16hi(vl.z)) +
                (bf16lo(vh.w) + bf16lo(vl.w)) + (bf16hi(vh.w) + bf16hi(vl.w));
      p += xor1(p);
      p += xor2(p);
      if ((cc & 3) == 0) hs[i * (Kc / 32) + cc / 4] = p;
    }
    __syncthreads();
    float acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = 0.f;
    for (int kc = 0; kc < nk; kc += KB) {
      if (kc > 0 || r0 > 0) load_batch<KB>(tbase, ks0, kc, nk, lane, rr, cv, sb);
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        if (kc + u < nk) {
          const int col = ((ks0 + kc + u) >> a.kshift) * GROUP + half * 32;
#pragma unroll
          for (int i = 0; i < MB; ++i)
            if (i < mb)
              acc[i] += kstep_hilo(cv[u], sb[u], hh + (size_t)i * Kc + col,
                                   hl + (size_t)i * Kc + col, hs[i * (Kc / 32) + col / 32]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const float tot = acc[i] + xor32(acc[i]);
      if (half == 0) red[(wv * MB + i) * 32 + rr] = tot;
    }
    __syncthreads();
    for (int o = tid; o < mb * 32; o += W * WAVE) {
      const int i = o / 32, r = o % 32;
      float yv = 0.f;
      for (int w = 0; w < W; ++w) yv += red[(w * MB + i) * 32 + r];
      dst[(size_t)ysel(r0 + i) * H + 32 * tile + r] = yv;
    }
    __syncthreads();
  }
}

// grid = (H/32 tiles, n_slots routed slots + n_sh_chunks shared chunks if a.shared): routed
// rows go to a.y, the shared rows (one chunk) to a.y_sh.
template <int W, int MB, int KB>
__global__ void __launch_bounds__(W * WAVE) d_kernel(FfnArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int tile = blockIdx.x;
  const int slot = blockIdx.y;
  SlotRows sr;
  const bool shared = slot >= a.n_slots;
  if (!slot_rows(a, slot, shared, sr)) return;
  int kb0 = 0, nks = a.I / GROUP;
  float *dst = a.y;
  if (shared) {
    const int KSs = a.Is / GROUP, c = slot - a.n_slots, nc = a.n_sh_chunks;
    kb0 = (KSs * c) / nc;
    nks = (KSs * (c + 1)) / nc - kb0;
    dst = a.y_sh;
  }
  auto ysel = [&](int r) { return shared ? r : flat_of(a, sr, r); };
  d_tile<W, MB, KB>(a, sr, tile, kb0, nks, dst, ysel, smem);
}

// ---------------------------------------------------------------- standalone combine
// out[t, :] = bf16( sum_j w[t,j] y[t*k+j, :] + y_sh[t, :] + x[t, :] ), fp32, j ascending
__global__ void __launch_bounds__(256) combine_kernel(const uint16_t *x, const float *y,
                                                      const float *w, const float *y_sh,
                                                      int T, int H, int k, uint16_t *out,
                                                      float *out_f32) {
  const size_t n = (size_t)T * H;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < n;
       o += (size_t)gridDim.x * blockDim.x) {
    const size_t t = o / H, col = o % H;
    float acc = 0.f;
    for (int j0 = 0; j0 < k; j0 += 8) {   // eight rows' loads in flight, summed j ascending
      float v[8], wj[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = min(j0 + q, k - 1);
        wj[q] = w[t * k + j];
        v[q] = y[(t * k + j) * H + col];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j0 + q < k) acc = fmaf(wj[q], v[q], acc);
    }
    if (y_sh) acc += y_sh[o];
    acc += bf16_to_f32(x[o]);
    out[o] = (uint16_t)f32_to_bf16_bits(acc);
    if (out_f32) out_f32[o] = acc;
  }
}

__global__ void zero_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace qmoe

#include "mfma.h"
