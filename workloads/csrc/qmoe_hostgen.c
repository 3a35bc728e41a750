/* Host (CPU) side of the seeded synthetic input recipe of workloads/gen.py, in plain C.
 *
 * The numpy functions normal_f32 and quantize_groups in gen.py define the recipe; this file
 * computes the same values (integer arithmetic, and IEEE fp32 / fp64 operations with round to
 * nearest even in the same order, built without contraction), only faster, so that the
 * oracle's inputs for full-size layers can be drawn on the CPU in seconds.  A CPU test checks
 * it bit for bit against the numpy functions.  It is input generation only and holds none of
 * the layer's arithmetic.
 *
 * Philox4x32-10: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers:
 * as easy as 1, 2, 3", SC'11, section 4.
 */
#include <math.h>
#include <stdint.h>

static const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;

static void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t p0 = (uint64_t)M0 * c[0], p1 = (uint64_t)M1 * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

/* Irwin-Hall sum of the four 16-bit halves of two words, centred (exact in int64) */
static int64_t ih4(uint32_t a, uint32_t b) {
  return (int64_t)(a & 0xFFFFu) + (a >> 16) + (b & 0xFFFFu) + (b >> 16) - 131070;
}

static uint16_t bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  return (uint16_t)(((uint64_t)v.u + 0x7FFFu + ((v.u >> 16) & 1u)) >> 16);
}

static float bf16_f32(uint16_t h) {
  union { float f; uint32_t u; } v;
  v.u = (uint32_t)h << 16;
  return v.f;
}

/* fp32 multiplier of the recipe: fp32(std / std_of_the_Irwin_Hall_sum) */
static float normal_scale(double std) {
  const double ih_std = sqrt((65536.0 * 65536.0 - 1.0) / 3.0);
  return (float)(std / ih_std);
}

/* n (even) approximately-N(0, std^2) fp32 values of tensor key (k0, k1), row-major: element
 * pair p = Philox counter (p mod 2^32, p div 2^32, 0, 0). */
int qmoe_host_normal(uint32_t k0, uint32_t k1, int64_t n, double std, float *out) {
  if (n < 0 || (n & 1) || !out) return -1;
  const float c = normal_scale(std);
  for (int64_t p = 0; p < n / 2; ++p) {
    uint32_t ctr[4] = {(uint32_t)p, (uint32_t)((uint64_t)p >> 32), 0u, 0u};
    philox10(ctr, k0, k1);
    out[2 * p] = (float)ih4(ctr[0], ctr[1]) * c;
    out[2 * p + 1] = (float)ih4(ctr[2], ctr[3]) * c;
  }
  return 0;
}

/* One quantisation group of 64 fp32 weights -> codes (unpacked), scale and bias bits. */
static void quantize_group(const float *w, int bits, uint8_t *q, uint16_t *s16o, uint16_t *b16o) {
  const int qmax = (1 << bits) - 1;
  float wmin = w[0], wmax = w[0];
  for (int i = 1; i < 64; ++i) {
    if (w[i] < wmin) wmin = w[i];
    if (w[i] > wmax) wmax = w[i];
  }
  const float rng = wmax - wmin;
  const float s32 = rng * (float)(1.0 / qmax);
  const uint16_t s16 = bf16_rne(s32), b16 = bf16_rne(wmin);
  const double sf = (double)bf16_f32(s16);
  const float bf = bf16_f32(b16);
  const double safe = sf > 0 ? sf : 1.0;
  for (int i = 0; i < 64; ++i) {
    const double t = (double)(float)(w[i] - bf);
    double qq = floor(t / safe);
    if (t < qq * safe) qq -= 1.0;
    if (t >= (qq + 1.0) * safe) qq += 1.0;
    const double mid = (qq + 0.5) * safe;
    const int odd = (int)(((long long)qq) & 1);   /* floor-mod 2 of an integer */
    if (t > mid || (t == mid && odd)) qq += 1.0;
    if (qq < 0) qq = 0;
    if (qq > qmax) qq = qmax;
    q[i] = sf > 0 ? (uint8_t)qq : 0;
  }
  *s16o = s16;
  *b16o = b16;
}

/* A quantised matrix [rows, cols] (cols a multiple of 64) drawn under key (k0, k1) with
 * weight std `std`: codes q (bits 4: packed [rows, cols/2], element 2m in the low nibble of
 * byte m; bits 8: [rows, cols]), bf16 scale and bias bits s, b [rows, cols/64]. */
int qmoe_host_matrix(uint32_t k0, uint32_t k1, int64_t rows, int64_t cols, double std, int bits,
                     uint8_t *q, uint16_t *s, uint16_t *b) {
  if (rows < 0 || cols <= 0 || cols % 64 || (bits != 4 && bits != 8) || !q || !s || !b) return -1;
  const float c = normal_scale(std);
  const int64_t gpr = cols / 64;
  float w[64];
  uint8_t codes[64];
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t g = 0; g < gpr; ++g) {
      const uint64_t pair0 = (uint64_t)(r * cols + g * 64) / 2;
      for (int i = 0; i < 32; ++i) {
        const uint64_t p = pair0 + (uint64_t)i;
        uint32_t ctr[4] = {(uint32_t)p, (uint32_t)(p >> 32), 0u, 0u};
        philox10(ctr, k0, k1);
        w[2 * i] = (float)ih4(ctr[0], ctr[1]) * c;
        w[2 * i + 1] = (float)ih4(ctr[2], ctr[3]) * c;
      }
      quantize_group(w, bits, codes, &s[r * gpr + g], &b[r * gpr + g]);
      if (bits == 8) {
        for (int i = 0; i < 64; ++i) q[r * cols + g * 64 + i] = codes[i];
      } else {
        for (int i = 0; i < 32; ++i)
          q[r * (cols / 2) + g * 32 + i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
      }
    }
  }
  return 0;
}
