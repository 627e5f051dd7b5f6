/*
 * Seeded synthetic inputs for the LatentMoE layer workloads.
 *
 * This is test and benchmark infrastructure shared by the CPU oracle and the
 * GPU path: it draws the token batch x and the weight matrices, nothing else.
 * It holds none of the layer's arithmetic.
 *
 * Random stream: SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: output i of stream `key` is mix(key + (i + 1) * GAMMA).
 * Every tensor has its own key derived from (seed, tensor id, sub id), so any
 * expert's matrices can be regenerated alone, in any order, on any thread.
 *
 * Normals: Box-Muller (Box and Muller, 1958) on the two 24-bit halves of one
 * 64-bit output, in float, so element 2i and 2i+1 of a tensor come from
 * output i.
 *
 * Weights are drawn ~N(0, std^2) in fp32 and stored as MXFP4 (OCP Microscaling
 * v1.0 reading used throughout this repository): per block of 32 consecutive
 * values along K, shared exponent floor(log2(amax)) - 2, clamped to
 * [-127, 127] and stored as the E8M0 byte (exp + 127), or byte 0 for an
 * all-zero block; each element is v / 2^exp rounded to nearest-even on the
 * E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}, saturating at 6, sign kept (also
 * for zero). Codes are packed two per byte, element 2i in the low nibble.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t k3gen_key(uint64_t seed, uint32_t tensor, uint32_t sub) {
  uint64_t k = mix64(seed + GAMMA);
  k = mix64(k ^ ((uint64_t)tensor * 0xD1B54A32D192ED03ULL) ^ GAMMA);
  k = mix64(k ^ ((uint64_t)sub * 0xABC98388FB8FAC03ULL) ^ (GAMMA << 1));
  return k;
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static inline void normal_pair(uint64_t key, uint64_t i, float* a, float* b) {
  uint64_t r = draw(key, i);
  float u1 = (float)((r >> 40) + 1) * 0x1p-24f;        /* (0, 1] */
  float u2 = (float)((r >> 16) & 0xFFFFFFu) * 0x1p-24f; /* [0, 1) */
  float rad = sqrtf(-2.0f * logf(u1));
  float ang = 6.28318530717958647692f * u2;
  float sn, cs;
  sincosf(ang, &sn, &cs);
  *a = rad * cs;
  *b = rad * sn;
}

/* Raw 64-bit outputs 0..n-1 of a stream. */
void k3gen_u64(uint64_t seed, uint32_t tensor, uint32_t sub, int64_t n, uint64_t* out) {
  uint64_t key = k3gen_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = draw(key, (uint64_t)i);
}

/* n (even) normals scaled by stddev. */
void k3gen_normal(uint64_t seed, uint32_t tensor, uint32_t sub, int64_t n, float stddev, float* out) {
  uint64_t key = k3gen_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < n / 2; ++p) {
    float a, b;
    normal_pair(key, (uint64_t)p, &a, &b);
    out[2 * p] = a * stddev;
    out[2 * p + 1] = b * stddev;
  }
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* n (even) normals scaled by stddev, rounded to bf16 (returned as raw bits). */
void k3gen_bf16(uint64_t seed, uint32_t tensor, uint32_t sub, int64_t n, float stddev, uint16_t* out) {
  uint64_t key = k3gen_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < n / 2; ++p) {
    float a, b;
    normal_pair(key, (uint64_t)p, &a, &b);
    out[2 * p] = f32_to_bf16_rne(a * stddev);
    out[2 * p + 1] = f32_to_bf16_rne(b * stddev);
  }
}

/* E2M1 code (sign in bit 3) of v, with v already divided by the block scale. */
static inline uint8_t e2m1_code(float v) {
  float a = fabsf(v);
  uint8_t c = (uint8_t)((a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
                        (a > 5.0f));
  return (uint8_t)(c | (signbit(v) ? 8u : 0u));
}

/* 2^e for e in [-127, 127], built from its bit pattern (exact). */
static inline float pow2f(int e) {
  uint32_t u = e >= -126 ? (uint32_t)(e + 127) << 23 : 0x00400000u;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* One row of K fp32 values -> K/2 code bytes and K/32 scale bytes. */
static void quantize_row_fp4(const float* w, int64_t K, uint8_t* codes, uint8_t* scales) {
  for (int64_t b = 0; b < K / 32; ++b) {
    const float* v = w + 32 * b;
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    if (amax == 0.0f) {
      scales[b] = 0;
      for (int i = 0; i < 16; ++i)
        codes[16 * b + i] = (uint8_t)((signbit(v[2 * i]) ? 8u : 0u) | ((signbit(v[2 * i + 1]) ? 8u : 0u) << 4));
      continue;
    }
    int ex;
    frexpf(amax, &ex); /* amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1 */
    int shared = ex - 1 - 2;
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
    scales[b] = (uint8_t)(shared + 127);
    float inv = pow2f(-shared);
    for (int i = 0; i < 16; ++i) {
      uint8_t lo = e2m1_code(v[2 * i] * inv);
      uint8_t hi = e2m1_code(v[2 * i + 1] * inv);
      codes[16 * b + i] = (uint8_t)(lo | (hi << 4));
    }
  }
}

/*
 * `count` matrices [N, K] ~ N(0, stddev^2), matrix c drawn from stream
 * (seed, tensor, sub0 + c), stored back to back as MXFP4:
 * codes [count, N, K/2], scales [count, N, K/32]. K must be a multiple of 32.
 */
void k3gen_mxfp4_many(uint64_t seed, uint32_t tensor, uint32_t sub0, int32_t count, int64_t N, int64_t K,
                      float stddev, uint8_t* codes, uint8_t* scales) {
  int64_t rows = (int64_t)count * N;
#pragma omp parallel
  {
    float buf[8192];
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
      int64_t c = r / N, n = r % N;
      uint64_t key = k3gen_key(seed, tensor, sub0 + (uint32_t)c);
      uint64_t pair0 = (uint64_t)(n * K) / 2;
      for (int64_t k0 = 0; k0 < K; k0 += 8192) {
        int64_t len = K - k0 < 8192 ? K - k0 : 8192;
        for (int64_t p = 0; p < len / 2; ++p) {
          float a, b;
          normal_pair(key, pair0 + (uint64_t)(k0 / 2 + p), &a, &b);
          buf[2 * p] = a * stddev;
          buf[2 * p + 1] = b * stddev;
        }
        quantize_row_fp4(buf, len, codes + r * (K / 2) + k0 / 2, scales + r * (K / 32) + k0 / 32);
      }
    }
  }
}
