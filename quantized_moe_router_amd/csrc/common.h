// Device helpers shared by the qmoe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bounds.h"

#define QMOE_DEV __device__ __forceinline__
#define QMOE_HD __host__ __device__ __forceinline__

typedef __bf16 qmoe_bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t qmoe_u32x4 __attribute__((ext_vector_type(4)));

namespace qmoe {

constexpr int WAVE = 64;
constexpr int GROUP = 64;          // quantisation group (weights per scale/bias pair)
constexpr int KSTEP_BYTES = 1152;  // one k-step of a 32-row tile: 1024 B codes + 128 B scale|bias
constexpr int TILE_ROWS = 32;      // rows per store tile
constexpr int MAX_TOPK = 32;
constexpr int MAX_EXPERTS = 1024;
constexpr float RMS_EPS = 1e-6f;   // epsilon of every RMS norm of the layer
constexpr int CHUNK_TOKENS = 128;  // layer_forward processes at most this many tokens per pass

// ---------------------------------------------------------------- bf16 <-> fp32
QMOE_DEV float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
QMOE_DEV float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
QMOE_HD float bf16_to_f32(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
// round to nearest even (finite inputs)
QMOE_HD uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// D = a.lo*b.lo + a.hi*b.hi + c  (bf16 pairs, fp32 accumulate)
QMOE_DEV float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(qmoe_bf16x2, a),
                                         __builtin_bit_cast(qmoe_bf16x2, b), c, false);
}

// ---------------------------------------------------------------- int4 decode
// A packed 32-bit word of the store holds 8 codes of consecutive elements e0..e7 with
// element 2i in nibble i and element 2i+1 in nibble i+4 (i = 0..3).  OR-ing a nibble into
// the mantissa of bf16 128.0 (0x4300) gives the exact bf16 value 128 + q, so one AND-OR
// turns two codes into a bf16 pair (128+q_2i, 128+q_2i+1) aligned with the activation pair
// (x_2i, x_2i+1).  The dot products therefore sum (128 + q) * x; callers subtract
// 128 * sum(x) through the group bias term.
// The mask and the exponent pattern are handed over in VGPRs: a VOP3 instruction takes no
// literal operand on gfx950, and with both constants in registers the AND-OR is one
// v_and_or_b32 instead of a v_and_b32 and a v_or_b32 with literals.
constexpr uint32_t MAGIC2 = 0x43004300u;
QMOE_DEV uint32_t vreg_const(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}
QMOE_DEV uint32_t nib_pair(uint32_t w, int i) {
  return ((w >> (4 * i)) & vreg_const(0x000F000Fu)) | vreg_const(MAGIC2);
}

// sum over 32 elements of (128 + q_j) * x_j; w: 4 packed words, x: 16 bf16 pairs
QMOE_DEV float dot32_q4_bf16(const uint32_t w[4], const uint32_t x[16]) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    a0 = dot2bf(nib_pair(w[d], 0), x[4 * d + 0], a0);
    a1 = dot2bf(nib_pair(w[d], 1), x[4 * d + 1], a1);
    a0 = dot2bf(nib_pair(w[d], 2), x[4 * d + 2], a0);
    a1 = dot2bf(nib_pair(w[d], 3), x[4 * d + 3], a1);
  }
  return a0 + a1;
}

// ---------------------------------------------------------------- lane exchanges in registers
// Values of other lanes through lane swaps (v_permlane32_swap, v_permlane16_swap) and DPP
// inside 16-lane rows, instead of LDS permutes (each of which is a round trip through the LDS
// unit, and a reduction is a chain of them).
// xor32 / xor16: the value of lane l ^ 32 / l ^ 16.
QMOE_DEV float xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? p[0] : p[1]);
}
QMOE_DEV float xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 16) ? p[0] : p[1]);
}
template <int CTRL>
QMOE_DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
QMOE_DEV float xor1(float v) { return dpp<0xB1>(v); }   // quad_perm [1, 0, 3, 2]
QMOE_DEV float xor2(float v) { return dpp<0x4E>(v); }   // quad_perm [2, 3, 0, 1]

// Sum over the wave, as the xor butterfly 32, 16, 8, 4, 2, 1 adds them (the same bits in
// every lane): after the xor-32 and xor-16 steps the value repeats every 16 lanes, so the
// rotation of a row by 8 gives the xor-8 partner's value, and so on down to 1.
QMOE_DEV float wave_sum(float v) {
  v += xor32(v);
  v += xor16(v);
  v += dpp<0x128>(v);   // row_ror 8
  v += dpp<0x124>(v);   // row_ror 4
  v += dpp<0x122>(v);   // row_ror 2
  v += dpp<0x121>(v);   // row_ror 1
  return v;
}
QMOE_DEV float wave_max(float v) {
  v = fmaxf(v, xor32(v));
  v = fmaxf(v, xor16(v));
  v = fmaxf(v, dpp<0x128>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x122>(v));
  v = fmaxf(v, dpp<0x121>(v));
  return v;
}

QMOE_DEV float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- cross-workgroup hand-off
// Data that one workgroup hands to another inside the same launch is written with
// system-scope stores (written through past the per-XCD L2 caches) and read with
// system-scope loads.  A producer drains its stores (s_waitcnt 0) before it bumps a completion
// counter with a device-scope atomic; the consumer that sees the final count then reads the
// data.  This avoids a whole-L2 writeback/invalidate fence per workgroup, which costs tens of
// microseconds across a launch of several hundred workgroups on gfx950.
QMOE_DEV void st_sys(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); }
QMOE_DEV void st_sys(int32_t *p, int32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); }
QMOE_DEV float ld_sys(const float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); }
QMOE_DEV int32_t ld_sys(const int32_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); }
// Tagged words: a 32-bit value with a 32-bit tag (the launch epoch) in one 64-bit word, stored
// and loaded as single atomic accesses, so a reader that sees the tag it expects also sees
// the value written with it, without any counter or flag.
QMOE_DEV void st_tag(uint64_t *p, unsigned tag, float v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
QMOE_DEV uint64_t ld_tag(const uint64_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); }
QMOE_DEV bool tag_is(uint64_t v, unsigned tag) { return (uint32_t)(v >> 32) == tag; }
QMOE_DEV float tag_val(uint64_t v) { return __uint_as_float((uint32_t)v); }
QMOE_DEV void drain_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Every thread of the workgroup has issued its hand-off stores: drain them, count this
// workgroup in *cnt, and return true in the workgroup that completes the count (n arrivals).
// That workgroup resets the counter to zero for the next launch.
QMOE_DEV bool arrive_last(unsigned *cnt, unsigned n) {
  __shared__ int last_flag;
  drain_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (old == n - 1);
    if (old == n - 1) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return last_flag != 0;
}

}  // namespace qmoe
