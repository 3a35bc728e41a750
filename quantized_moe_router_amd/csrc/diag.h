// Diagnostic kernel: a plain streaming read, the achievable-bandwidth reference for the layer's
// weight streams.  It reads the first `bytes` bytes of each of n fixed-stride blocks (block
// ids[i] at base + ids[i] * stride) -- the same access shape as fetching n routed experts of the
// packed store -- and does nothing with the data but fold it into one word per wave, so that
// its time is the memory system's alone.
#pragma once
#include "common.h"

namespace qmoe {

constexpr int READ_MAX_BLOCKS = 64;
constexpr int READ_CHUNK = 16384;   // bytes per wave: 16 loads of 16 B per lane
constexpr int READ_INFLIGHT = 8;    // 16-byte loads a lane keeps in flight

struct ReadArgs {
  const uint8_t *base;
  size_t stride, bytes;
  int n;
  int32_t ids[READ_MAX_BLOCKS];
  uint32_t *sink;   // one word per wave
};

// Wave w reads chunk w % chunks_per_block of block w / chunks_per_block: 64 lanes x 16 B per
// load instruction (1 KiB contiguous), READ_INFLIGHT instructions in flight, non-temporal.
__global__ void __launch_bounds__(256) stream_read_kernel(ReadArgs a) {
  const int lane = threadIdx.x % WAVE;
  const size_t cpb = (a.bytes + READ_CHUNK - 1) / READ_CHUNK;
  const size_t gw = (size_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  const size_t bi = gw / cpb, c = gw % cpb;
  if (bi >= (size_t)a.n) return;
  const uint8_t *p = a.base + (size_t)a.ids[bi] * a.stride + c * READ_CHUNK;
  const size_t lim = min((size_t)READ_CHUNK, a.bytes - c * READ_CHUNK);
  uint32_t acc = 0u;
  for (size_t o = (size_t)lane * 16; o < lim; o += (size_t)WAVE * 16 * READ_INFLIGHT) {
    qmoe_u32x4 v[READ_INFLIGHT];
#pragma unroll
    for (int j = 0; j < READ_INFLIGHT; ++j) {
      const size_t off = o + (size_t)j * WAVE * 16;
      v[j] = off + 16 <= lim ? __builtin_nontemporal_load((const qmoe_u32x4 *)(p + off))
                             : qmoe_u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < READ_INFLIGHT; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (lane == 0) a.sink[gw] = acc;
}

inline size_t stream_read_waves(size_t bytes, int n) {
  return (size_t)n * ((bytes + READ_CHUNK - 1) / READ_CHUNK);
}

}  // namespace qmoe
