// Router for calls of several tokens on the matrix cores, then top-k and bucketing.
//
// Same quantities as the router of router.h (TurboFieldfare post, section "TurboFieldfare의
// 전문가 스트리밍 구조", router listing; 8-bit affine projection of section "TurboFieldfare가
// 메모리를 아끼는 방식"): logit(t, e) = fac(t) * sum_h (s q + b)(e, h) * x(t, h) rscale(h) (+ bias e)
// with fac(t) = (1 / sqrt(H)) / sqrt(mean_h x(t, h)^2 + eps).  The projection of a block of 16
// tokens on 16 experts is a 16 x 16 product over the hidden axis, done with
// v_mfma_f32_16x16x4_f32 (fp32 operands, fp32 accumulation): A = x rscale (the activation the
// VALU router scales the same way), B = s q + b formed in fp32 as in the VALU router, one
// matrix-core step per 4 hidden columns.  Lane l of a step supplies A(row l % 16, k l / 16)
// and B(k l / 16, column l % 16); its accumulator i holds (row 4 (l / 16) + i, column
// l % 16).  The hidden columns are walked in an order that gives every lane 16 consecutive
// ones per 64-column group (lane group j takes columns 16 j + s at step s), the same order for
// A and B, so every lane reads 32 bytes of x, 16 bytes of codes and 64 bytes of router scales
// per group with vector loads.  Each wave takes one group, so a 16 x 16 tile is split over
// many workgroups (four groups each, added in LDS); their partial tiles and sums of x^2 go to
// the workspace.
//
// A second kernel adds the partial tiles of each token in split order, applies the norm
// factor and the bias, selects the top-k (one wave per token, router.h) and, in the layer
// path, buckets the assignments in its last workgroup.
#pragma once
#include "router.h"

namespace qmoe {

constexpr int RMF_WAVES = 4;
constexpr int RMF_THREADS = RMF_WAVES * WAVE;
constexpr int RMF_ROWS = 16;      // tokens per workgroup
constexpr int RMF_COLS = 16;      // experts per workgroup

// n_ks: the hidden groups are split over workgroups, RMF_WAVES groups (one per wave) each.
inline __host__ __device__ int rmf_splits(int H) { return (H / GROUP + RMF_WAVES - 1) / RMF_WAVES; }

// grid: ceil(T / 16) token blocks x ceil(E / 16) expert blocks x rmf_splits(H) splits.  Writes
// the split's partial products part[split][T][E] and, in expert block 0, its partial sums of
// x^2 ssq[split][T] and (if a.gsum) the sums of its groups of x by the balanced pairwise tree
// of gsum_kernel.  Plain stores: the next launch reads them.
__global__ void __launch_bounds__(RMF_THREADS) router_mf_kernel(RouterArgs a, float *part,
                                                                float *ssq) {
  __shared__ float tile[RMF_WAVES][4][WAVE];
  __shared__ float ssp[RMF_WAVES][RMF_ROWS];
  const int H = a.H, KG = H / GROUP, n_ks = rmf_splits(H);
  const int n_eb = (a.E + RMF_COLS - 1) / RMF_COLS;
  const int ks = blockIdx.x % n_ks, eb = (blockIdx.x / n_ks) % n_eb, tb = blockIdx.x / (n_ks * n_eb);
  const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
  const int r16 = lane % 16, j = lane / 16;
  const int t = min(tb * RMF_ROWS + r16, a.T - 1);    // A row: token (padding rows repeat)
  const int e = min(eb * RMF_COLS + r16, a.E - 1);    // B column: expert
  const int g = ks * RMF_WAVES + wv;                  // this wave's group
  qmoe_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  if (g < KG) {
    const uint16_t *xr = a.x + (size_t)t * H + GROUP * g + 16 * j;
    const qmoe_u32x4 xa = *(const qmoe_u32x4 *)xr;
    const qmoe_u32x4 xb = *(const qmoe_u32x4 *)(xr + 8);
    const qmoe_u32x4 qv = *(const qmoe_u32x4 *)(a.rq + (size_t)e * H + GROUP * g + 16 * j);
    float4 rs4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      rs4[c] = a.rscale ? *(const float4 *)(a.rscale + GROUP * g + 16 * j + 4 * c)
                        : float4{1.f, 1.f, 1.f, 1.f};
    const size_t so = (size_t)e * KG + g;
    const float s = bf16_to_f32(a.rs[so]), b = bf16_to_f32(a.rb[so]);
    const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
    const float rsv[16] = {rs4[0].x, rs4[0].y, rs4[0].z, rs4[0].w, rs4[1].x, rs4[1].y,
                           rs4[1].z, rs4[1].w, rs4[2].x, rs4[2].y, rs4[2].z, rs4[2].w,
                           rs4[3].x, rs4[3].y, rs4[3].z, rs4[3].w};
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const float xv = (st & 1) ? bf16hi(xw[st / 2]) : bf16lo(xw[st / 2]);
      ss = fmaf(xv, xv, ss);
      const float av = xv * rsv[st];
      const float bv = fmaf(s, (float)((qw[st / 4] >> (8 * (st % 4))) & 0xFFu), b);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
    }
  }
  // sums of x^2 per token row over the four lane groups of the row
  ss += xor16(ss);
  ss += xor32(ss);
  if (j == 0) ssp[wv][r16] = ss;
#pragma unroll
  for (int i = 0; i < 4; ++i) tile[wv][i][lane] = acc[i];
  __syncthreads();
  {
    // thread (i, l): tile entry (row 4 (l / 16) + i, column l % 16), the waves in order
    const int i = tid / WAVE, l = tid % WAVE;
    const int row = 4 * (l / 16) + i, col = l % 16;
    float v = 0.f;
    for (int w = 0; w < RMF_WAVES; ++w) v += tile[w][i][l];
    const int tt = tb * RMF_ROWS + row, ee = eb * RMF_COLS + col;
    if (tt < a.T && ee < a.E) part[((size_t)ks * a.T + tt) * a.E + ee] = v;
  }
  if (eb != 0) return;
  if (tid < RMF_ROWS && tb * RMF_ROWS + tid < a.T) {
    float v = 0.f;
    for (int w = 0; w < RMF_WAVES; ++w) v += ssp[w][tid];
    ssq[(size_t)ks * a.T + tb * RMF_ROWS + tid] = v;
  }
  if (a.gsum) {
    const int nrow = min(RMF_ROWS, a.T - tb * RMF_ROWS);
    const int ng = min(RMF_WAVES, KG - ks * RMF_WAVES);
    for (int p = tid; p < nrow * ng; p += RMF_THREADS) {
      const int rr = p / ng, gg = ks * RMF_WAVES + p % ng;
      const size_t tok = (size_t)tb * RMF_ROWS + rr;
      const qmoe_u32x4 *src = (const qmoe_u32x4 *)(a.x + tok * H + (size_t)GROUP * gg);
      float v[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const qmoe_u32x4 w4 = src[q];
        v[4 * q + 0] = bf16lo(w4.x) + bf16hi(w4.x);
        v[4 * q + 1] = bf16lo(w4.y) + bf16hi(w4.y);
        v[4 * q + 2] = bf16lo(w4.z) + bf16hi(w4.z);
        v[4 * q + 3] = bf16lo(w4.w) + bf16hi(w4.w);
      }
#pragma unroll
      for (int w = 16; w >= 1; w /= 2) {
#pragma unroll
        for (int q = 0; q < w; ++q) v[q] = v[2 * q] + v[2 * q + 1];
      }
      a.gsum[tok * KG + gg] = v[0];
    }
  }
}

// Logits of token t (lane l, chunk c: expert 64 c + l) from the partial tiles: the splits
// added in order, KB splits' loads in flight at once; then the top-k of the wave.
template <int NCH>
QMOE_DEV void rmf_token(const RouterArgs &a, const float *part, int t, float fac) {
  constexpr int KB = NCH >= 16 ? 4 : 8;
  const int lane = threadIdx.x % WAVE, E = a.E, n_ks = rmf_splits(a.H);
  float v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) v[c] = 0.f;
  for (int k0 = 0; k0 < n_ks; k0 += KB) {
    float pv[KB][NCH];
#pragma unroll
    for (int q = 0; q < KB; ++q)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int e = WAVE * c + lane;
        pv[q][c] = (k0 + q < n_ks && e < E) ? part[((size_t)(k0 + q) * a.T + t) * E + e] : 0.f;
      }
#pragma unroll
    for (int q = 0; q < KB; ++q)
#pragma unroll
      for (int c = 0; c < NCH; ++c) v[c] += pv[q][c];
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e = WAVE * c + lane;
    if (e < E) {
      v[c] *= fac;
      if (a.lbias) v[c] += a.lbias[e];
      a.logits[(size_t)t * E + e] = v[c];
    }
  }
  int myi;
  float myl;
  topk_run<NCH>([&](int c) { return WAVE * c + lane < E ? topk_ord(v[c]) : 0u; }, a.k, myi, myl);
  const float myw = topk_weight(myi, myl, a.k, a.pes);
  if (lane < a.k) {
    st_sys(a.topk_idx + (size_t)t * a.k + lane, myi);
    st_sys(a.topk_w + (size_t)t * a.k + lane, myw);
  }
}

// grid: ceil(T / 4) workgroups, one token per wave: the logits (norm factor from the summed
// x^2, the split products summed in split order, then the bias) are written to a.logits and
// selected from registers; with a.counts set, the last workgroup (counted in *a.cnt_all)
// buckets every assignment.
__global__ void __launch_bounds__(ROUTER_THREADS) router_topk_kernel(RouterArgs a,
                                                                     const float *part,
                                                                     const float *ssq) {
  extern __shared__ __align__(16) char smem[];
  const int wv = threadIdx.x / WAVE;
  const int t = blockIdx.x * ROUTER_WAVES + wv;
  const int n_ks = rmf_splits(a.H);
  if (t < a.T) {
    float tot = 0.f;
    for (int k0 = 0; k0 < n_ks; k0 += 16) {   // sixteen splits' loads in flight, added in order
      float pv[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) pv[q] = k0 + q < n_ks ? ssq[(size_t)(k0 + q) * a.T + t] : 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) tot += pv[q];
    }
    const float fac = a.inv_sqrt_h / sqrtf(tot / (float)a.H + RMS_EPS);
    const int nch = topk_chunks(a.E);
    if (nch <= 1) rmf_token<1>(a, part, t, fac);
    else if (nch <= 2) rmf_token<2>(a, part, t, fac);
    else if (nch <= 4) rmf_token<4>(a, part, t, fac);
    else if (nch <= 8) rmf_token<8>(a, part, t, fac);
    else rmf_token<TOPK_NCH>(a, part, t, fac);
  }
  if (a.counts == nullptr) return;
  if (!arrive_last(a.cnt_all, gridDim.x)) return;
  bucket_block<ROUTER_THREADS>([&](int f) { return ld_sys(a.topk_idx + f); }, a.T * a.k, a.E,
                               a.counts, a.offsets, a.sorted, a.active, a.n_active, a.slot_tab,
                               a.n_slots, (int *)smem);
}

}  // namespace qmoe
