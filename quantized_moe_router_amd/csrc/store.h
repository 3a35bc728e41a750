// Packed expert store: one fixed-stride block per expert (the Swiftlet article, section
// "같은 모델을 왜 이렇게 적은 메모리로 돌릴 수 있나": experts live in fixed-stride blocks so
// that one read fetches one expert).  Packing is a layout change only -- every code, scale
// and bias bit of the canonical MLX arrays is copied, nothing is dequantised (TurboFieldfare
// post, section "TurboFieldfare의 스트리밍 설치 방식").
//
// Block of an expert with width I (hidden H):
//   GU section: I/16 tiles; tile t holds gate rows 16t..16t+15 and up rows 16t..16t+15
//               (32 tile rows: rr < 16 gate, rr >= 16 up).
//   D  section: H/32 tiles; tile t holds down rows 32t..32t+31.
// A tile is a run of k-steps (64 input elements = one quantisation group each), 1152 B per
// k-step:  bytes [0, 1024): 64 chunks of 16 B, chunk c = (half c/32, tile row c%32) holding
//          the 32 codes of elements 64*ks + 32*half + [0, 32) of that row;
//          bytes [1024, 1152): 32 words, word rr = scale(rr, ks) | bias(rr, ks) << 16.
// Inside a chunk, 32-bit word d holds elements 8d..8d+7: element 8d+2i in nibble i and
// element 8d+2i+1 in nibble i+4 (i = 0..3), so that one AND-OR yields a bf16 pair aligned
// with an activation pair.  Wave lane l of a kernel reads chunk l of each k-step: one
// contiguous 1 KiB load per wave.
#pragma once
#include "common.h"

namespace qmoe {

struct BlockGeom {
  int H, I;
  int gu_tiles, gu_ks;   // I/16 tiles, H/64 k-steps each
  int d_tiles, d_ks;     // H/32 tiles, I/64 k-steps each
  size_t gu_bytes, d_bytes;
};

inline __host__ __device__ BlockGeom block_geom(int H, int I) {
  BlockGeom g;
  g.H = H;
  g.I = I;
  g.gu_tiles = I / 16;
  g.gu_ks = H / GROUP;
  g.d_tiles = H / TILE_ROWS;
  g.d_ks = I / GROUP;
  g.gu_bytes = (size_t)g.gu_tiles * g.gu_ks * KSTEP_BYTES;
  g.d_bytes = (size_t)g.d_tiles * g.d_ks * KSTEP_BYTES;
  return g;
}

inline size_t block_stride_bytes(int H, int I) {
  BlockGeom g = block_geom(H, I);
  size_t b = g.gu_bytes + g.d_bytes;
  return (b + 4095) & ~(size_t)4095;
}

// nibble slot (0..7) inside a packed word of the element at offset jj (0..7) in the word
QMOE_DEV int nibble_slot(int jj) { return (jj & 1) * 4 + (jj >> 1); }

struct CanonExpert {
  const uint8_t *gq, *uq, *dq;
  const uint16_t *gs, *gb, *us, *ub, *ds, *db;
};
struct CanonExpertOut {
  uint8_t *gq, *uq, *dq;
  uint16_t *gs, *gb, *us, *ub, *ds, *db;
};

// one thread per 16-byte chunk of the block (GU chunks first, then D chunks)
__global__ void pack_kernel(CanonExpert c, int H, int I, uint8_t *dst) {
  const BlockGeom g = block_geom(H, I);
  const long n_gu = (long)g.gu_tiles * g.gu_ks * 64;
  const long n_all = n_gu + (long)g.d_tiles * g.d_ks * 64;
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= n_all) return;
  const bool gu = id < n_gu;
  const long local = gu ? id : id - n_gu;
  const int chunk = (int)(local % 64);
  const long kst = local / 64;  // tile * ks_per_tile + ks
  const int ks_per = gu ? g.gu_ks : g.d_ks;
  const int tile = (int)(kst / ks_per);
  const int ks = (int)(kst % ks_per);
  const int rr = chunk % 32, half = chunk / 32;
  const uint8_t *q;
  const uint16_t *s, *b;
  int row, K;
  if (gu) {
    K = H;
    if (rr < 16) { q = c.gq; s = c.gs; b = c.gb; row = 16 * tile + rr; }
    else         { q = c.uq; s = c.us; b = c.ub; row = 16 * tile + rr - 16; }
  } else {
    K = I; q = c.dq; s = c.ds; b = c.db; row = 32 * tile + rr;
  }
  const int e0 = ks * GROUP + half * 32;
  const uint8_t *src = q + (size_t)row * (K / 2) + e0 / 2;  // 16 canonical bytes
  uint32_t w[4] = {0, 0, 0, 0};
  for (int j = 0; j < 32; ++j) {
    const uint32_t code = (src[j >> 1] >> ((j & 1) * 4)) & 0xFu;
    w[j >> 3] |= code << (4 * nibble_slot(j & 7));
  }
  uint8_t *base = dst + (gu ? 0 : g.gu_bytes) + (size_t)kst * KSTEP_BYTES;
  *(qmoe_u32x4 *)(base + chunk * 16) = qmoe_u32x4{w[0], w[1], w[2], w[3]};
  if (half == 0) {
    const size_t gi = (size_t)row * (K / GROUP) + ks;
    *(uint32_t *)(base + 1024 + rr * 4) = (uint32_t)s[gi] | ((uint32_t)b[gi] << 16);
  }
}

__global__ void unpack_kernel(const uint8_t *srcb, int H, int I, CanonExpertOut c) {
  const BlockGeom g = block_geom(H, I);
  const long n_gu = (long)g.gu_tiles * g.gu_ks * 64;
  const long n_all = n_gu + (long)g.d_tiles * g.d_ks * 64;
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= n_all) return;
  const bool gu = id < n_gu;
  const long local = gu ? id : id - n_gu;
  const int chunk = (int)(local % 64);
  const long kst = local / 64;
  const int ks_per = gu ? g.gu_ks : g.d_ks;
  const int tile = (int)(kst / ks_per);
  const int ks = (int)(kst % ks_per);
  const int rr = chunk % 32, half = chunk / 32;
  uint8_t *q;
  uint16_t *s, *b;
  int row, K;
  if (gu) {
    K = H;
    if (rr < 16) { q = c.gq; s = c.gs; b = c.gb; row = 16 * tile + rr; }
    else         { q = c.uq; s = c.us; b = c.ub; row = 16 * tile + rr - 16; }
  } else {
    K = I; q = c.dq; s = c.ds; b = c.db; row = 32 * tile + rr;
  }
  const uint8_t *base = srcb + (gu ? 0 : g.gu_bytes) + (size_t)kst * KSTEP_BYTES;
  const qmoe_u32x4 v = *(const qmoe_u32x4 *)(base + chunk * 16);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const int e0 = ks * GROUP + half * 32;
  uint8_t *dstq = q + (size_t)row * (K / 2) + e0 / 2;
  for (int m = 0; m < 16; ++m) {
    const int j0 = 2 * m, j1 = 2 * m + 1;
    const uint32_t c0 = (w[j0 >> 3] >> (4 * nibble_slot(j0 & 7))) & 0xFu;
    const uint32_t c1 = (w[j1 >> 3] >> (4 * nibble_slot(j1 & 7))) & 0xFu;
    dstq[m] = (uint8_t)(c0 | (c1 << 4));
  }
  if (half == 0) {
    const uint32_t sb = *(const uint32_t *)(base + 1024 + rr * 4);
    const size_t gi = (size_t)row * (K / GROUP) + ks;
    s[gi] = (uint16_t)(sb & 0xFFFFu);
    b[gi] = (uint16_t)(sb >> 16);
  }
}

}  // namespace qmoe
