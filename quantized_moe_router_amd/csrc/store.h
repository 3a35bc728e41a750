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
//
// 8-bit experts (MLX int8 group quantisation, the Swiftlet article, section "같은 모델을 왜
// 이렇게 적은 메모리로 돌릴 수 있나"): a code q = 16 qh + ql splits into two 4-bit codes, and
// s q + b = (16 s) qh + s ql + b, so each quantisation group becomes two consecutive k-steps
// of the layout above -- the high nibbles with scale 16 s (exact in bf16) and bias b, then the
// low nibbles with scale s and bias 0 -- that multiply the same 64 activations.  Every kernel
// runs on it unchanged except that k-step ks reads the activations of group ks >> kshift
// (kshift = 1 for 8-bit experts, 0 for 4-bit ones).  Packing stays exactly invertible.
#pragma once
#include "common.h"

namespace qmoe {

struct BlockGeom {
  int H, I;
  int gu_tiles, gu_ks;   // I/16 tiles, (H/64) << kshift k-steps each
  int d_tiles, d_ks;     // H/32 tiles, (I/64) << kshift k-steps each
  size_t gu_bytes, d_bytes;
};

inline __host__ __device__ BlockGeom block_geom(int H, int I, int kshift) {
  BlockGeom g;
  g.H = H;
  g.I = I;
  g.gu_tiles = I / 16;
  g.gu_ks = (H / GROUP) << kshift;
  g.d_tiles = H / TILE_ROWS;
  g.d_ks = (I / GROUP) << kshift;
  g.gu_bytes = (size_t)g.gu_tiles * g.gu_ks * KSTEP_BYTES;
  g.d_bytes = (size_t)g.d_tiles * g.d_ks * KSTEP_BYTES;
  return g;
}

inline size_t block_stride_bytes(int H, int I, int kshift) {
  BlockGeom g = block_geom(H, I, kshift);
  size_t b = g.gu_bytes + g.d_bytes;
  return (b + 4095) & ~(size_t)4095;
}

// nibble slot (0..7) inside a packed word of the element at offset jj (0..7) in the word
QMOE_HD int nibble_slot(int jj) { return (jj & 1) * 4 + (jj >> 1); }

struct CanonExpert {
  const uint8_t *gq, *uq, *dq;
  const uint16_t *gs, *gb, *us, *ub, *ds, *db;
};
struct CanonExpertOut {
  uint8_t *gq, *uq, *dq;
  uint16_t *gs, *gb, *us, *ub, *ds, *db;
};

// Where chunk `id` of a block (GU chunks first, then D chunks) comes from.
struct ChunkPos {
  bool gu;
  long kst;          // tile * k-steps per tile + ks
  int chunk, rr, half, row, K, ks, group, plane;
};
QMOE_HD bool chunk_pos(long id, int H, int I, int kshift, ChunkPos &c) {
  const BlockGeom g = block_geom(H, I, kshift);
  const long n_gu = (long)g.gu_tiles * g.gu_ks * 64;
  const long n_all = n_gu + (long)g.d_tiles * g.d_ks * 64;
  if (id < 0 || id >= n_all) return false;
  c.gu = id < n_gu;
  const long local = c.gu ? id : id - n_gu;
  c.chunk = (int)(local % 64);
  c.kst = local / 64;
  const int ks_per = c.gu ? g.gu_ks : g.d_ks;
  const int tile = (int)(c.kst / ks_per);
  c.ks = (int)(c.kst % ks_per);
  c.group = c.ks >> kshift;
  c.plane = kshift ? (c.ks & 1) : 0;   // 8-bit: 0 high nibbles, 1 low nibbles
  c.rr = c.chunk % 32;
  c.half = c.chunk / 32;
  if (c.gu) {
    c.K = H;
    c.row = 16 * tile + (c.rr & 15);
  } else {
    c.K = I;
    c.row = 32 * tile + c.rr;
  }
  return true;
}

// Element counts of the canonical arrays an index of the chunk map may touch (bounds of the
// debug build): codes of the matrix the chunk comes from (rows x K, in bytes), and its
// scale/bias arrays (rows x K/64).
QMOE_HD size_t canon_code_bytes(const ChunkPos &p, int H, int I, int kshift) {
  const size_t rows = p.gu ? I : H;
  return rows * (size_t)(kshift ? p.K : p.K / 2);
}
QMOE_HD size_t canon_group_count(const ChunkPos &p, int H, int I) {
  return (size_t)(p.gu ? I : H) * (p.K / GROUP);
}

// Packs chunk `id` of the block of one expert: 32 codes into 16 bytes, and for the first
// half-chunk of a tile row the k-step's scale|bias word.
QMOE_HD void pack_chunk(const CanonExpert &c, int H, int I, int kshift, uint8_t *dst, long id) {
  ChunkPos p;
  if (!chunk_pos(id, H, I, kshift, p)) return;
  const BlockGeom g = block_geom(H, I, kshift);
  const bool up = p.gu && p.rr >= 16;
  const uint8_t *q = p.gu ? (up ? c.uq : c.gq) : c.dq;
  const uint16_t *s = p.gu ? (up ? c.us : c.gs) : c.ds;
  const uint16_t *b = p.gu ? (up ? c.ub : c.gb) : c.db;
  const int e0 = p.group * GROUP + p.half * 32;
  const size_t n_codes = canon_code_bytes(p, H, I, kshift);
  uint32_t w[4] = {0, 0, 0, 0};
  for (int j = 0; j < 32; ++j) {
    uint32_t code;
    if (kshift) {
      const size_t at = (size_t)p.row * p.K + e0 + j;
      QMOE_BOUNDS(at < n_codes);
      const uint32_t q8 = q[at];
      code = p.plane ? (q8 & 0xFu) : (q8 >> 4);
    } else {
      const size_t at = (size_t)p.row * (p.K / 2) + e0 / 2 + (j >> 1);
      QMOE_BOUNDS(at < n_codes);
      code = (q[at] >> ((j & 1) * 4)) & 0xFu;
    }
    w[j >> 3] |= code << (4 * nibble_slot(j & 7));
  }
  const size_t off = (p.gu ? 0 : g.gu_bytes) + (size_t)p.kst * KSTEP_BYTES;
  QMOE_BOUNDS(off + p.chunk * 16 + 16 <= (p.gu ? g.gu_bytes : g.gu_bytes + g.d_bytes));
  uint8_t *base = dst + off;
  *(qmoe_u32x4 *)(base + p.chunk * 16) = qmoe_u32x4{w[0], w[1], w[2], w[3]};
  if (p.half == 0) {
    const size_t gi = (size_t)p.row * (p.K / GROUP) + p.group;
    QMOE_BOUNDS(gi < canon_group_count(p, H, I));
    uint32_t sw = s[gi], bw = b[gi];
    if (kshift && p.plane == 0) sw = f32_to_bf16_bits(bf16_to_f32((uint16_t)sw) * 16.f);  // exact
    if (kshift && p.plane == 1) bw = 0u;
    *(uint32_t *)(base + 1024 + p.rr * 4) = sw | (bw << 16);
  }
}

// Inverse of pack_chunk: chunk `id` back into the canonical arrays.
QMOE_HD void unpack_chunk(const uint8_t *srcb, int H, int I, int kshift, const CanonExpertOut &c,
                          long id) {
  ChunkPos p;
  if (!chunk_pos(id, H, I, kshift, p)) return;
  const BlockGeom g = block_geom(H, I, kshift);
  const bool up = p.gu && p.rr >= 16;
  uint8_t *q = p.gu ? (up ? c.uq : c.gq) : c.dq;
  uint16_t *s = p.gu ? (up ? c.us : c.gs) : c.ds;
  uint16_t *b = p.gu ? (up ? c.ub : c.gb) : c.db;
  const size_t off = (p.gu ? 0 : g.gu_bytes) + (size_t)p.kst * KSTEP_BYTES;
  QMOE_BOUNDS(off + p.chunk * 16 + 16 <= (p.gu ? g.gu_bytes : g.gu_bytes + g.d_bytes));
  const uint8_t *base = srcb + off;
  const qmoe_u32x4 v = *(const qmoe_u32x4 *)(base + p.chunk * 16);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const int e0 = p.group * GROUP + p.half * 32;
  const size_t n_codes = canon_code_bytes(p, H, I, kshift);
  if (kshift) {
    // the high-nibble k-step writes bits 7..4 of each code, the low one bits 3..0: both
    // k-steps of a group own the same bytes, so the high one writes the whole byte from both
    // (reading the low k-step's chunk, which is the next one)
    if (p.plane == 0) {
      QMOE_BOUNDS(off + KSTEP_BYTES + p.chunk * 16 + 16 <= g.gu_bytes + g.d_bytes);
      const qmoe_u32x4 v2 = *(const qmoe_u32x4 *)(base + KSTEP_BYTES + p.chunk * 16);
      const uint32_t w2[4] = {v2.x, v2.y, v2.z, v2.w};
      const size_t at = (size_t)p.row * p.K + e0;
      QMOE_BOUNDS(at + 32 <= n_codes);
      uint8_t *dq = q + at;
      for (int j = 0; j < 32; ++j)
        dq[j] = (uint8_t)((((w[j >> 3] >> (4 * nibble_slot(j & 7))) & 0xFu) << 4) |
                          ((w2[j >> 3] >> (4 * nibble_slot(j & 7))) & 0xFu));
    }
  } else {
    const size_t at = (size_t)p.row * (p.K / 2) + e0 / 2;
    QMOE_BOUNDS(at + 16 <= n_codes);
    uint8_t *dq = q + at;
    for (int m = 0; m < 16; ++m)
      dq[m] = (uint8_t)(((w[(2 * m) >> 3] >> (4 * nibble_slot((2 * m) & 7))) & 0xFu) |
                        (((w[(2 * m + 1) >> 3] >> (4 * nibble_slot((2 * m + 1) & 7))) & 0xFu) << 4));
  }
  if (p.half == 0) {
    const uint32_t sb = *(const uint32_t *)(base + 1024 + p.rr * 4);
    const size_t gi = (size_t)p.row * (p.K / GROUP) + p.group;
    QMOE_BOUNDS(gi < canon_group_count(p, H, I));
    if (!kshift) {
      s[gi] = (uint16_t)(sb & 0xFFFFu);
      b[gi] = (uint16_t)(sb >> 16);
    } else if (p.plane == 0) {
      b[gi] = (uint16_t)(sb >> 16);
    } else {
      s[gi] = (uint16_t)(sb & 0xFFFFu);
    }
  }
}

// one thread per 16-byte chunk of the block
__global__ void pack_kernel(CanonExpert c, int H, int I, int kshift, uint8_t *dst) {
  pack_chunk(c, H, I, kshift, dst, (long)blockIdx.x * blockDim.x + threadIdx.x);
}

__global__ void unpack_kernel(const uint8_t *srcb, int H, int I, int kshift, CanonExpertOut c) {
  unpack_chunk(srcb, H, I, kshift, c, (long)blockIdx.x * blockDim.x + threadIdx.x);
}

}  // namespace qmoe
