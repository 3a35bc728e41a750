// GPU side of the seeded synthetic input recipe (workloads/gen.py): Philox4x32-10 draws,
// Irwin-Hall(4) approximate normals and the MLX-affine int4 quantiser of the synthetic
// weights.  Every step is integer arithmetic or a single IEEE fp32 operation with round to
// nearest even (no contraction), so it reproduces the numpy implementation bit for bit.
// This is input generation only; it contains none of the layer's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;

__device__ __forceinline__ void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint32_t hi0 = __umulhi(M0, c[0]), lo0 = M0 * c[0];
    const uint32_t hi1 = __umulhi(M1, c[2]), lo1 = M1 * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

__device__ __forceinline__ int ih4(uint32_t a, uint32_t b) {
  return (int)((a & 0xFFFFu) + (a >> 16) + (b & 0xFFFFu) + (b >> 16)) - 131070;
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One thread per quantisation group (64 consecutive elements of a row) of `n_mat` matrices
// [rows, cols]; matrix m uses key (k0, tag0 + m * tag_step) and writes its codes/scales/biases
// at q + m * q_mat_stride etc.
__global__ void gen_int4_kernel(uint32_t k0, uint32_t tag0, uint32_t tag_step, int n_mat, int rows,
                                int cols, float c, float inv_qmax, uint8_t *q, uint16_t *s,
                                uint16_t *b) {
  const int gpr = cols / 64;
  const long n_groups = (long)n_mat * rows * gpr;
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= n_groups) return;
  const int m = (int)(id / ((long)rows * gpr));
  const long rem = id % ((long)rows * gpr);
  const int row = (int)(rem / gpr), g = (int)(rem % gpr);
  const uint32_t k1 = tag0 + (uint32_t)m * tag_step;
  const unsigned long long pair0 = ((unsigned long long)row * cols + (unsigned long long)g * 64) / 2;
  float w[64];
  float wmin = INFINITY, wmax = -INFINITY;
#pragma unroll 4
  for (int i = 0; i < 32; ++i) {
    const unsigned long long p = pair0 + i;
    uint32_t ctr[4] = {(uint32_t)p, (uint32_t)(p >> 32), 0u, 0u};
    philox10(ctr, k0, k1);
    const float a = __fmul_rn((float)ih4(ctr[0], ctr[1]), c);
    const float bb = __fmul_rn((float)ih4(ctr[2], ctr[3]), c);
    w[2 * i] = a;
    w[2 * i + 1] = bb;
    wmin = fminf(wmin, fminf(a, bb));
    wmax = fmaxf(wmax, fmaxf(a, bb));
  }
  const float s32 = __fmul_rn(__fsub_rn(wmax, wmin), inv_qmax);
  const uint32_t s16 = bf16_rne_bits(s32), b16 = bf16_rne_bits(wmin);
  const float sf = __uint_as_float(s16 << 16), bf = __uint_as_float(b16 << 16);
  const size_t mat_groups = (size_t)rows * gpr;
  uint8_t *qo = q + (size_t)m * rows * (cols / 2) + (size_t)row * (cols / 2) + g * 32;
  for (int j = 0; j < 64; j += 2) {
    uint32_t code[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float t = __fsub_rn(w[j + h], bf);
      uint32_t qq = 0;
      if (sf > 0.f) {
#pragma unroll
        for (int mm = 0; mm < 15; ++mm) {
          const float thr = __fmul_rn((float)mm + 0.5f, sf);
          qq += (t > thr) ? 1u : 0u;
          qq += (t == thr && (mm & 1)) ? 1u : 0u;
        }
      }
      code[h] = qq;
    }
    qo[j / 2] = (uint8_t)(code[0] | (code[1] << 4));
  }
  s[(size_t)m * mat_groups + (size_t)row * gpr + g] = (uint16_t)s16;
  b[(size_t)m * mat_groups + (size_t)row * gpr + g] = (uint16_t)b16;
}

// The 8-bit form of the same recipe: one thread per group, unpacked codes [rows, cols].  The
// code is the nearest integer to t / s with ties to even, found from fp32 floor(t / s) with
// exact corrections (q * s and (q + 0.5) * s are exact in fp32: at most 17 significant bits).
__global__ void gen_int8_kernel(uint32_t k0, uint32_t tag0, uint32_t tag_step, int n_mat, int rows,
                                int cols, float c, float inv_qmax, uint8_t *q, uint16_t *s,
                                uint16_t *b) {
  const int gpr = cols / 64;
  const long n_groups = (long)n_mat * rows * gpr;
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= n_groups) return;
  const int m = (int)(id / ((long)rows * gpr));
  const long rem = id % ((long)rows * gpr);
  const int row = (int)(rem / gpr), g = (int)(rem % gpr);
  const uint32_t k1 = tag0 + (uint32_t)m * tag_step;
  const unsigned long long pair0 = ((unsigned long long)row * cols + (unsigned long long)g * 64) / 2;
  float w[64];
  float wmin = INFINITY, wmax = -INFINITY;
#pragma unroll 4
  for (int i = 0; i < 32; ++i) {
    const unsigned long long p = pair0 + i;
    uint32_t ctr[4] = {(uint32_t)p, (uint32_t)(p >> 32), 0u, 0u};
    philox10(ctr, k0, k1);
    const float a = __fmul_rn((float)ih4(ctr[0], ctr[1]), c);
    const float bb = __fmul_rn((float)ih4(ctr[2], ctr[3]), c);
    w[2 * i] = a;
    w[2 * i + 1] = bb;
    wmin = fminf(wmin, fminf(a, bb));
    wmax = fmaxf(wmax, fmaxf(a, bb));
  }
  const float s32 = __fmul_rn(__fsub_rn(wmax, wmin), inv_qmax);
  const uint32_t s16 = bf16_rne_bits(s32), b16 = bf16_rne_bits(wmin);
  const float sf = __uint_as_float(s16 << 16), bf = __uint_as_float(b16 << 16);
  const size_t mat_groups = (size_t)rows * gpr;
  uint8_t *qo = q + (size_t)m * rows * cols + (size_t)row * cols + g * 64;
  for (int j = 0; j < 64; ++j) {
    const float t = __fsub_rn(w[j], bf);
    int qq = 0;
    if (sf > 0.f) {
      float f = floorf(__fdiv_rn(t, sf));
      if (t < __fmul_rn(f, sf)) f -= 1.f;
      if (t >= __fmul_rn(f + 1.f, sf)) f += 1.f;
      const float mid = __fmul_rn(f + 0.5f, sf);
      const int fi = (int)f;
      if (t > mid || (t == mid && (fi & 1))) f += 1.f;
      qq = (int)fminf(fmaxf(f, 0.f), 255.f);
    }
    qo[j] = (uint8_t)qq;
  }
  s[(size_t)m * mat_groups + (size_t)row * gpr + g] = (uint16_t)s16;
  b[(size_t)m * mat_groups + (size_t)row * gpr + g] = (uint16_t)b16;
}

}  // namespace

extern "C" {

// Draw n_mat int8 matrices [rows, cols] (codes unpacked: q holds n_mat * rows * cols bytes).
int qmoe_gen_int8(uint32_t k0, uint32_t tag0, uint32_t tag_step, int n_mat, int rows, int cols,
                  float c, float inv_qmax, uint8_t *q, uint16_t *s, uint16_t *b, void *stream) {
  if (n_mat <= 0 || rows <= 0 || cols <= 0 || cols % 64 || !q || !s || !b) return -1;
  const long n = (long)n_mat * rows * (cols / 64);
  hipLaunchKernelGGL(gen_int8_kernel, dim3((unsigned)((n + 127) / 128)), dim3(128), 0,
                     (hipStream_t)stream, k0, tag0, tag_step, n_mat, rows, cols, c, inv_qmax, q, s,
                     b);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Draw n_mat int4 matrices [rows, cols] for layer key k0 and tags tag0 + m * tag_step.
// q: n_mat * rows * cols/2 bytes; s, b: n_mat * rows * cols/64 bf16 (device pointers).
int qmoe_gen_int4(uint32_t k0, uint32_t tag0, uint32_t tag_step, int n_mat, int rows, int cols,
                  float c, float inv_qmax, uint8_t *q, uint16_t *s, uint16_t *b, void *stream) {
  if (n_mat <= 0 || rows <= 0 || cols <= 0 || cols % 64 || !q || !s || !b) return -1;
  const long n = (long)n_mat * rows * (cols / 64);
  hipLaunchKernelGGL(gen_int4_kernel, dim3((unsigned)((n + 127) / 128)), dim3(128), 0,
                     (hipStream_t)stream, k0, tag0, tag_step, n_mat, rows, cols, c, inv_qmax, q, s,
                     b);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}
