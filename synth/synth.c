/*
 * Seeded, counter-based synthetic input generator.
 *
 * This module holds no arithmetic of the layer itself: it only turns
 * (seed, stream, index) triples into bytes, bf16 normals, fp32 normals and
 * uniforms, E8M0 exponent bytes, and FP8 E4M3 weight codes with their block
 * scales (how the synthetic checkpoint stores a block-scaled FP8 matrix).  Both the CPU oracle and the HIP path
 * read what it writes, so neither side ever produces the other's inputs.
 *
 * Every element is a pure function of (seed, stream, index), so any slice of
 * any tensor (for example one expert of a 896-expert layer) can be
 * regenerated on its own, in any order, by any number of threads.
 *
 * Mixing function: the SplitMix64 output function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).
 * Normals: the Box-Muller transform (Box and Muller, 1958), cosine branch only,
 * one 64-bit word per normal.  bf16: round-to-nearest-even of the fp32 value.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Base key of one stream: every tensor (or token batch) has its own stream id. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed * GOLDEN + 0x632BE59BD9B4E019ULL) ^ mix64(stream + GOLDEN));
}

/* The 64-bit random word of element `i` of a stream. */
static inline uint64_t word_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GOLDEN);
}

uint64_t synth_word(uint64_t seed, uint64_t stream, uint64_t i) {
  return word_at(stream_key(seed, stream), i);
}

/* Standard normal from one word: u1 in (0,1] from the top 24 bits, u2 in [0,1)
 * from the next 24 bits; z = sqrt(-2 ln u1) cos(2 pi u2), in double. */
static inline double normal_from_word(uint64_t w) {
  const double inv24 = 1.0 / 16777216.0;
  double u1 = ((double)(w >> 40) + 1.0) * inv24;
  double u2 = (double)((w >> 16) & 0xFFFFFFULL) * inv24;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* out[i] = bf16(RNE(float(mean + std * N(0,1)))) for indices start..start+n-1. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                       double mean, double std, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) {
    double z = normal_from_word(word_at(key, start + (uint64_t)i));
    out[i] = f32_to_bf16_rne((float)(mean + std * z));
  }
}

/* out[i] = float(mean + std * N(0,1)). */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                      double mean, double std, float* out) {
  uint64_t key = stream_key(seed, stream);
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) {
    double z = normal_from_word(word_at(key, start + (uint64_t)i));
    out[i] = (float)(mean + std * z);
  }
}

/* out[i] = float(lo + (hi - lo) * u), u = (top 24 bits + 0.5) / 2^24 in (0,1). */
void synth_uniform_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                       double lo, double hi, float* out) {
  uint64_t key = stream_key(seed, stream);
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) {
    uint64_t w = word_at(key, start + (uint64_t)i);
    double u = ((double)(w >> 40) + 0.5) / 16777216.0;
    out[i] = (float)(lo + (hi - lo) * u);
  }
}

/* Uniform random bytes: byte b of the stream is byte (b % 8) of word (b / 8).
 * Used for MXFP4 code bytes (two uniform 4-bit codes per byte). */
void synth_bytes(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, uint8_t* out) {
  uint64_t key = stream_key(seed, stream);
  uint64_t end = start + n;
  uint64_t w0 = start >> 3, w1 = (end + 7) >> 3;
  int64_t nw = (int64_t)(w1 - w0);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nw; ++j) {
    uint64_t wi = w0 + (uint64_t)j;
    uint64_t w = word_at(key, wi);
    uint64_t b0 = wi << 3;
    for (int q = 0; q < 8; ++q) {
      uint64_t b = b0 + (uint64_t)q;
      if (b >= start && b < end) out[b - start] = (uint8_t)(w >> (8 * q));
    }
  }
}

/* Bytes uniform over the integers lo..hi (inclusive), one word per byte.
 * Used for E8M0 scale bytes. */
void synth_uniform_int_u8(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                          uint32_t lo, uint32_t hi, uint8_t* out) {
  uint64_t key = stream_key(seed, stream);
  uint64_t span = (uint64_t)(hi - lo + 1);
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) {
    uint64_t w = word_at(key, start + (uint64_t)i);
    /* multiply-high of a 32-bit uniform by the span: bias below 2^-24 */
    uint64_t r = ((w >> 32) * span) >> 32;
    out[i] = (uint8_t)(lo + r);
  }
}

/* E4M3 code (OCP 8-bit floating point, E4M3 variant: bias 7, 3 mantissa bits, subnormals
 * below 2^-6, largest finite 448) of an fp32 value with |y| <= 448, rounded to the nearest
 * representable value, ties to the even mantissa. */
static inline uint8_t e4m3_code(float y) {
  uint32_t u;
  memcpy(&u, &y, 4);
  const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a < 0x3C800000u) {                    /* below 2^-6: multiples of 2^-9 (code 8 = 2^-6) */
    float m = rintf(fabsf(y) * 512.0f);
    return (uint8_t)(sign | (uint8_t)m);
  }
  /* keep 3 of the 23 mantissa bits, rounding to nearest even (a carry moves the exponent) */
  const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) & 0xFFF00000u;
  const int e = (int)(r >> 23) - 127;
  return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | ((r >> 20) & 7u)));
}

/* Approximately standard normal from one word: the sum of its four 16-bit uniforms,
 * centred and scaled to unit variance (Irwin-Hall, n = 4; range +-2 sqrt 3).  No
 * transcendental, for the multi-gigabyte FP8 expert sets. */
static inline float irwin_hall4(uint64_t w) {
  const float inv16 = 1.0f / 65536.0f;
  float sum = 0.f;
  for (int k = 0; k < 4; ++k) sum += ((float)((w >> (16 * k)) & 0xFFFFu) + 0.5f) * inv16;
  return (sum - 2.0f) * 1.7320508075688772f;
}

/* A matrix of FP8 E4M3 weights with one fp32 scale per 128 x 128 block (the K2 block
 * card's expert format as the synthetic layers store it): w = std * irwin_hall4 of the
 * word of element r * cols + c (stream index start + r * cols + c); per block
 * scale = max |w| / 448 in fp32, code = E4M3 of the fp32 quotient w / scale.
 * codes: rows * cols bytes, row-major; scales: ceil(rows/128) * ceil(cols/128) floats. */
void synth_fp8_block128(uint64_t seed, uint64_t stream, uint64_t start, int64_t rows, int64_t cols,
                        double std, uint8_t* codes, float* scales) {
  uint64_t key = stream_key(seed, stream);
  const int64_t br = (rows + 127) / 128, bc = (cols + 127) / 128;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < br * bc; ++b) {
    const int64_t r0 = (b / bc) * 128, c0 = (b % bc) * 128;
    const int64_t r1 = r0 + 128 < rows ? r0 + 128 : rows, c1 = c0 + 128 < cols ? c0 + 128 : cols;
    float wb[128 * 128];
    float amax = 0.f;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) {
        float w = (float)std * irwin_hall4(word_at(key, start + (uint64_t)(r * cols + c)));
        wb[(r - r0) * 128 + (c - c0)] = w;
        float aw = fabsf(w);
        if (aw > amax) amax = aw;
      }
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    scales[b] = s;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) {
        float y = wb[(r - r0) * 128 + (c - c0)] / s;
        if (y > 448.0f) y = 448.0f;
        if (y < -448.0f) y = -448.0f;
        codes[r * cols + c] = e4m3_code(y);
      }
  }
}
