/*
 * Seeded synthetic input generator (host C, OpenMP).
 *
 * This file only produces input tensors. It holds none of the sparse-attention
 * arithmetic: no scoring, selection, softmax or pooling. Both the fp64 oracle
 * and the HIP library consume the arrays it writes.
 *
 * Random stream: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11),
 * written here from that paper's definition. Counter = (block index lo, hi,
 * stream lo, hi), key = 64-bit seed. Every (tensor, sequence) pair gets its
 * own stream id, so any piece can be regenerated independently and the
 * output does not depend on the thread count.
 *
 * Normals: Box-Muller on two 24-bit uniforms, computed in fp64 and rounded to
 * fp32. Stored formats:
 *   bf16  round-to-nearest-even of the fp32 value (upper half of binary32),
 *   e4m3  OCP FP8 E4M3 ("e4m3fn": bias 7, max 448, no infinities) with one
 *         fp32 scale per row, scale = amax / 448 (1 for an all-zero row),
 *         code = RNE(x / scale), saturating at 448,
 *   mxfp4 OCP MX FP4 (E2M1 elements, one E8M0 scale per block of 32): block
 *         exponent X = floor(log2(amax)) - 2 (E2M1's largest exponent), clamped
 *         to [-127, 127] (-127 for an all-zero block), element = RNE(x / 2^X)
 *         on the E2M1 grid, saturating at 6; two elements per byte, the even
 *         one in the low nibble.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox4x32_10(const uint32_t ctr_in[4], uint32_t k0, uint32_t k1,
                                 uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* One Philox block -> four N(0,1) fp32 values. */
static inline void block_normals(uint64_t seed, uint64_t stream, uint64_t blk, float z[4]) {
  uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)stream,
                     (uint32_t)(stream >> 32)};
  uint32_t r[4];
  philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32), r);
  for (int p = 0; p < 2; ++p) {
    double u1 = ((double)(r[2 * p] >> 8) + 1.0) * (1.0 / 16777216.0); /* (0, 1] */
    double u2 = (double)(r[2 * p + 1] >> 8) * (1.0 / 16777216.0);     /* [0, 1) */
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586 * u2;
    z[2 * p] = (float)(rad * cos(th));
    z[2 * p + 1] = (float)(rad * sin(th));
  }
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Element i of stream (seed, stream) is component i%4 of block i/4. */
void synth_normal_f32(uint64_t seed, uint64_t stream, float* out, int64_t n) {
  int64_t nblk = (n + 3) / 4;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblk; ++b) {
    float z[4];
    block_normals(seed, stream, (uint64_t)b, z);
    for (int k = 0; k < 4; ++k) {
      int64_t i = b * 4 + k;
      if (i < n) out[i] = z[k];
    }
  }
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, uint16_t* out, int64_t n) {
  int64_t nblk = (n + 3) / 4;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblk; ++b) {
    float z[4];
    block_normals(seed, stream, (uint64_t)b, z);
    for (int k = 0; k < 4; ++k) {
      int64_t i = b * 4 + k;
      if (i < n) out[i] = f32_to_bf16_rne(z[k]);
    }
  }
}

/* Uniform [0, 1) fp32 with 24 random bits. */
void synth_uniform_f32(uint64_t seed, uint64_t stream, float* out, int64_t n) {
  int64_t nblk = (n + 3) / 4;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nblk; ++b) {
    uint32_t ctr[4] = {(uint32_t)b, (uint32_t)((uint64_t)b >> 32), (uint32_t)stream,
                       (uint32_t)(stream >> 32)};
    uint32_t r[4];
    philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32), r);
    for (int k = 0; k < 4; ++k) {
      int64_t i = b * 4 + k;
      if (i < n) out[i] = (float)(r[k] >> 8) * (1.0f / 16777216.0f);
    }
  }
}

/* Nearest OCP E4M3 code (ties to even) of a finite fp32 value, saturating at 448. */
static inline uint8_t e4m3_encode(float y) {
  uint8_t sign = 0;
  if (y < 0.0f || (y == 0.0f && signbit(y))) { sign = 0x80; y = -y; }
  if (!(y < 448.0f)) return (uint8_t)(sign | 0x7E);
  if (y == 0.0f) return sign;
  int e;
  frexpf(y, &e);      /* y = f * 2^e, f in [0.5, 1) -> floor(log2 y) = e - 1 */
  int E = e - 1;
  if (E < -6) {       /* subnormal range: quantum 2^-9, codes 0..8 */
    float m = nearbyintf(ldexpf(y, 9));
    return (uint8_t)(sign | (uint8_t)m); /* m == 8 is exactly the smallest normal 0x08 */
  }
  float m = nearbyintf(ldexpf(y, 3 - E)); /* in [8, 16] */
  if (m >= 16.0f) { m = 8.0f; E += 1; }
  int code = ((E + 7) << 3) | ((int)m - 8);
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

/* Row-wise e4m3 quantisation: x[rows][cols] fp32 -> codes[rows][cols], scale[rows]. */
void synth_quant_e4m3_rows(const float* x, int64_t rows, int64_t cols, uint8_t* codes,
                           float* scale) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * cols;
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
      float a = fabsf(xr[c]);
      if (a > amax) amax = a;
    }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    scale[r] = s;
    for (int64_t c = 0; c < cols; ++c) codes[r * cols + c] = e4m3_encode(xr[c] / s);
  }
}

/* Nearest FP4 E2M1 code (ties to the even code) of a finite fp32 value, saturating at 6. */
static inline uint8_t e2m1_encode(float y) {
  static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  uint8_t sign = 0;
  if (y < 0.0f || (y == 0.0f && signbit(y))) { sign = 8; y = -y; }
  if (!(y < 6.0f)) return (uint8_t)(sign | 7);
  int c = 0;
  while (c < 7 && mag[c + 1] <= y) ++c;          /* mag[c] <= y < mag[c+1] */
  const float lo = y - mag[c], hi = mag[c + 1] - y;
  if (hi < lo || (hi == lo && (c & 1))) ++c;       /* nearest; a tie goes to the even code */
  return (uint8_t)(sign | c);
}

/* One row of cols (a multiple of 32) fp32 values -> cols/2 packed E2M1 bytes and cols/32
   E8M0 block scales. */
static void mxfp4_row(const float* x, int64_t cols, uint8_t* codes, uint8_t* scales) {
  for (int64_t b = 0; b < cols / 32; ++b) {
    const float* xb = x + 32 * b;
    float amax = 0.0f;
    for (int k = 0; k < 32; ++k) {
      float a = fabsf(xb[k]);
      if (a > amax) amax = a;
    }
    int X = -127;
    if (amax > 0.0f) {
      int e;
      frexpf(amax, &e);                      /* floor(log2 amax) = e - 1 */
      X = e - 1 - 2;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    }
    scales[b] = (uint8_t)(X + 127);
    for (int k = 0; k < 32; k += 2) {
      uint8_t c0 = e2m1_encode(ldexpf(xb[k], -X));
      uint8_t c1 = e2m1_encode(ldexpf(xb[k + 1], -X));
      codes[16 * b + k / 2] = (uint8_t)(c0 | (c1 << 4));
    }
  }
}

/* Row-wise MXFP4 quantisation: x[rows][cols] fp32 -> codes[rows][cols/2], scales[rows][cols/32]. */
void synth_quant_mxfp4_rows(const float* x, int64_t rows, int64_t cols, uint8_t* codes,
                            uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    mxfp4_row(x + r * cols, cols, codes + r * (cols / 2), scales + r * (cols / 32));
}

/* Normal draws quantised straight to MXFP4 (same stream layout as synth_normal_e4m3_rows). */
void synth_normal_mxfp4_rows(uint64_t seed, uint64_t stream, int64_t rows, int64_t cols,
                             uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float buf[512];
    for (int64_t c = 0; c < cols; c += 4) {
      float z[4];
      block_normals(seed, stream, (uint64_t)((r * cols + c) / 4), z);
      for (int k = 0; k < 4; ++k) buf[c + k] = z[k];
    }
    mxfp4_row(buf, cols, codes + r * (cols / 2), scales + r * (cols / 32));
  }
}

/* Normal draws quantised straight to e4m3 without keeping the fp32 tensor:
 * rows of `cols` values from stream (seed, stream), row-major. */
void synth_normal_e4m3_rows(uint64_t seed, uint64_t stream, int64_t rows, int64_t cols,
                            uint8_t* codes, float* scale) {
  /* cols must be a multiple of 4 so that rows start on a Philox block. */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float buf[512];
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; c += 4) {
      float z[4];
      block_normals(seed, stream, (uint64_t)((r * cols + c) / 4), z);
      for (int k = 0; k < 4; ++k) {
        buf[c + k] = z[k];
        float a = fabsf(z[k]);
        if (a > amax) amax = a;
      }
    }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    scale[r] = s;
    for (int64_t c = 0; c < cols; ++c) codes[r * cols + c] = e4m3_encode(buf[c] / s);
  }
}
