/*
 * Seeded synthetic inputs for the MoE-layer workloads.
 *
 * This is input preparation only: it draws the random tensors (activations,
 * router weights, expert weights) and quantises the expert weights into the
 * storage formats the layer consumes.  It holds none of the layer's forward
 * arithmetic (no dequantisation, no matrix products, no routing): both the
 * CPU oracle and the GPU path receive what this file writes and nothing else.
 *
 * Random numbers: a counter-based generator.  Every value is a pure function
 * of (seed, stream, element index), so the bytes do not depend on the number
 * of threads or on the order in which blocks are filled.  The bit mixer is
 * the SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) applied to key + (i+1)*gamma,
 * i.e. the i-th output of a SplitMix64 stream started at `key`.  Normals come
 * from the Box-Muller transform in single precision, one pair per two
 * consecutive counters (24 random bits per uniform).
 *
 * Quantisers (the input recipe of the workloads):
 *  - OCP E4M3FN ("fp8 e4m3", bias 7, largest finite 448, no infinities) with
 *    one f32 scale per 128x128 block of the [rows x cols] matrix,
 *    scale = amax/448, code = RNE(w/scale) saturated to +-448.  This is the
 *    weight format of the LongCat FP8 checkpoint described on the dragon.c
 *    page (section "Precision": routed experts in e4m3 with 128x128 blockwise
 *    f32 scales).
 *  - OCP E2M1 ("fp4") codes, two per byte, element 2i in the low nibble, with
 *    one UE8M0 (power-of-two) scale byte per 32 contiguous input elements of
 *    a row, exponent = ceil(log2(amax/6)).  Sizes follow the DeepSeek-V4.1-
 *    Flash post on the dev.to page (section "Bytes per token decide
 *    everything": 17.93 MiB per expert in FP4 with scales).
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of one random stream: (seed, stream id) -> 64-bit key. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GAMMA) ^ mix64(stream * GAMMA + 0x632BE59BD9B4E019ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t ctr) { return mix64(key + (ctr + 1) * GAMMA); }

/* Uniform in the open interval (0, 1), 53 random bits. */
static inline double unif01(uint64_t z) { return ((double)(z >> 11) + 0.5) * 0x1.0p-53; }

/* Standard normal for element index i of a stream: pair m = i/2 gives
 * (r cos a, r sin a); even i takes the cosine, odd i the sine. */
/* Uniform in the open interval (0, 1) as a float, 24 random bits. */
static inline float unif01f(uint64_t z) { return ((float)(z >> 40) + 0.5f) * 0x1.0p-24f; }

/* Standard normal pair m (Box-Muller in single precision): elements 2m and
 * 2m+1 of a stream are r*cos(a) and r*sin(a). */
static inline void normal_pair(uint64_t key, uint64_t m, float* z0, float* z1) {
  float u1 = unif01f(draw(key, 2 * m));
  float u2 = unif01f(draw(key, 2 * m + 1));
  float r = sqrtf(-2.0f * logf(u1));
  float sn, cs;
  sincosf(6.28318530717958647692f * u2, &sn, &cs);
  *z0 = r * cs;
  *z1 = r * sn;
}

static inline float normal_at(uint64_t key, uint64_t i) {
  float z0, z1;
  normal_pair(key, i >> 1, &z0, &z1);
  return (i & 1) ? z1 : z0;
}

/* Fill out[j] = f32(stddev * N_(start+j)). */
static void fill_normal_f32(uint64_t key, uint64_t start, int64_t n, double stddev, float* out) {
  int64_t j = 0;
  if ((start & 1) && n > 0) {
    out[0] = (float)(stddev * normal_at(key, start));
    j = 1;
  }
  for (; j + 1 < n; j += 2) {
    float z0, z1;
    normal_pair(key, (start + (uint64_t)j) >> 1, &z0, &z1);
    out[j] = (float)(stddev * z0);
    out[j + 1] = (float)(stddev * z1);
  }
  if (j < n) out[j] = (float)(stddev * normal_at(key, start + (uint64_t)j));
}

/* f32 -> bf16 bits, round to nearest even (finite inputs; NaN -> quiet NaN). */
static inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline uint32_t f32_bits(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  return u;
}

/* f32 -> OCP E4M3FN code, round to nearest even, saturating to +-448.
 * Normal range: round the 23-bit significand to 3 bits on the bit pattern
 * (a carry moves into the exponent), then rebias 127 -> 7. */
static inline uint8_t enc_e4m3(float v) {
  uint32_t u = f32_bits(v);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80);
  float a = fabsf(v);
  if (!(a < 448.0f)) return sign | 0x7E;           /* saturate (NaN never produced) */
  if (a < 0x1.0p-6f) return sign | (uint8_t)rintf(a * 512.0f); /* quantum 2^-9; 8 -> 0x08 */
  uint32_t m = u & 0x7FFFFFFFu;
  m += 0x7FFFFu + ((m >> 20) & 1u);
  uint32_t code = (m >> 20) - (120u << 3);         /* (exp - 127 + 7) << 3 | mant */
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

/* f32 -> OCP E2M1 code (4 bits), round to nearest even, saturating to +-6. */
static inline uint8_t enc_e2m1(float v) {
  uint32_t u = f32_bits(v);
  uint8_t sign = (uint8_t)((u >> 28) & 0x8);
  float a = fabsf(v);
  if (!(a < 6.0f)) return sign | 0x7;
  if (a < 1.0f) return sign | (uint8_t)rintf(a * 2.0f); /* quantum 0.5; 2 -> 1.0 (code 2) */
  uint32_t m = u & 0x7FFFFFFFu;
  m += 0x1FFFFFu + ((m >> 22) & 1u);
  uint32_t code = (m >> 22) - (126u << 1);         /* (exp - 127 + 1) << 1 | mant */
  if (code > 7) code = 7;
  return sign | (uint8_t)code;
}

/* UE8M0 byte for a group whose absolute maximum is amax:
 * 2^(byte-127) = 2^ceil(log2(amax/6)), the quotient taken in f32; byte 0 for an
 * all-zero group. */
static inline uint8_t ue8m0_for_amax(float amax) {
  if (amax == 0.0f) return 0;
  float v = amax / 6.0f;
  int ex;
  float fr = frexpf(v, &ex);            /* v = fr * 2^ex, fr in [0.5, 1) */
  int E = (fr == 0.5f) ? ex - 1 : ex;   /* exact ceil(log2 v) */
  int b = E + 127;
  if (b < 0) b = 0;
  if (b > 254) b = 254;
  return (uint8_t)b;
}

/* ---------------------------------------------------------------- exports */

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) { return stream_key(seed, stream); }

/* out[j] = f32(stddev * N(seed, stream, start + j)), j < n. */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double stddev,
                      float* out) {
  uint64_t key = stream_key(seed, stream);
  const int64_t CH = 1 << 16;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < (n + CH - 1) / CH; ++c) {
    int64_t b = c * CH, len = n - b < CH ? n - b : CH;
    fill_normal_f32(key, start + (uint64_t)b, len, stddev, out + b);
  }
}

/* out[j] = bf16_rne(f32(N(seed, stream, start + j))), j < n. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
  const int64_t CH = 1 << 14;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < (n + CH - 1) / CH; ++c) {
    float buf[1 << 14];
    int64_t b = c * CH, len = n - b < CH ? n - b : CH;
    fill_normal_f32(key, start + (uint64_t)b, len, 1.0, buf);
    for (int64_t j = 0; j < len; ++j) out[b + j] = f32_to_bf16_rne(buf[j]);
  }
}

/* out[j] = uniform(0,1) in double for counters start + j. */
void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double* out) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t j = 0; j < n; ++j) out[j] = unif01(draw(key, start + (uint64_t)j));
}

/* Elementwise codecs, exported so that tests can pin them. */
void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = f32_to_bf16_rne(in[j]);
}
void synth_enc_e4m3(const float* in, int64_t n, uint8_t* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = enc_e4m3(in[j]);
}
void synth_enc_e2m1(const float* in, int64_t n, uint8_t* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = enc_e2m1(in[j]);
}
void synth_ue8m0(const float* amax, int64_t n, uint8_t* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = ue8m0_for_amax(amax[j]);
}

/* Quantise one [N x K] f32 matrix to e4m3 codes [N][K] with f32 scales
 * [N/128][K/128] (N, K multiples of 128). */
void synth_quant_e4m3_b128(const float* w, int64_t N, int64_t K, uint8_t* q, float* s) {
  int64_t nb = N / 128, kb = K / 128;
  for (int64_t bn = 0; bn < nb; ++bn)
    for (int64_t bk = 0; bk < kb; ++bk) {
      float amax = 0.0f;
      for (int64_t r = 0; r < 128; ++r)
        for (int64_t c = 0; c < 128; ++c) {
          float a = fabsf(w[(bn * 128 + r) * K + bk * 128 + c]);
          if (a > amax) amax = a;
        }
      float scale = amax / 448.0f;
      s[bn * kb + bk] = scale;
      for (int64_t r = 0; r < 128; ++r)
        for (int64_t c = 0; c < 128; ++c) {
          int64_t i = (bn * 128 + r) * K + bk * 128 + c;
          q[i] = (amax == 0.0f) ? 0 : enc_e4m3(w[i] / scale);
        }
    }
}

/* Quantise one [N x K] f32 matrix to packed e2m1 codes [N][K/2] with UE8M0
 * scales [N][K/32] (K multiple of 32). */
void synth_quant_e2m1_g32(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* s) {
  int64_t G = K / 32;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < G; ++g) {
      const float* src = w + n * K + g * 32;
      float amax = 0.0f;
      for (int c = 0; c < 32; ++c) {
        float a = fabsf(src[c]);
        if (a > amax) amax = a;
      }
      uint8_t b = ue8m0_for_amax(amax);
      s[n * G + g] = b;
      int sh = 127 - (int)b; /* scale the group by 2^-(b-127) */
      uint8_t* dst = q + n * (K / 2) + g * 16;
      if (sh >= -126) {      /* 2^sh is a normal float: the product is correctly rounded */
        uint32_t pb = (uint32_t)(sh + 127) << 23;
        float pw;
        memcpy(&pw, &pb, 4);
        for (int c = 0; c < 32; c += 2) {
          uint8_t lo = (amax == 0.0f) ? 0 : enc_e2m1(src[c] * pw);
          uint8_t hi = (amax == 0.0f) ? 0 : enc_e2m1(src[c + 1] * pw);
          dst[c / 2] = (uint8_t)(lo | (hi << 4));
        }
      } else {
        for (int c = 0; c < 32; c += 2) {
          uint8_t lo = enc_e2m1(ldexpf(src[c], sh));
          uint8_t hi = enc_e2m1(ldexpf(src[c + 1], sh));
          dst[c / 2] = (uint8_t)(lo | (hi << 4));
        }
      }
    }
}

/* Quantise one [N x K] f32 matrix to packed e2m1 codes [N][K/2] with one
 * E4M3 scale byte per 16 consecutive inputs [N][K/16] (K multiple of 16): the
 * group's scale is amax/6, stored as its E4M3 code (round to nearest even);
 * the codes are the e2m1 codes of w / (amax/6), so a value that the rounded
 * scale pushes past 6 saturates. */
void synth_quant_nvfp4_g16(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* s) {
  int64_t G = K / 16;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < G; ++g) {
      const float* src = w + n * K + g * 16;
      float amax = 0.0f;
      for (int c = 0; c < 16; ++c) {
        float a = fabsf(src[c]);
        if (a > amax) amax = a;
      }
      const float scale = amax / 6.0f;
      s[n * G + g] = enc_e4m3(scale);
      uint8_t* dst = q + n * (K / 2) + g * 8;
      for (int c = 0; c < 16; c += 2) {
        uint8_t lo = (amax == 0.0f) ? 0 : enc_e2m1(src[c] / scale);
        uint8_t hi = (amax == 0.0f) ? 0 : enc_e2m1(src[c + 1] / scale);
        dst[c / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
}

/* Draw and quantise the [N x K] matrix of experts e0..e0+ne-1, each from
 * its own stream (stream_base + e), entries ~ N(0, stddev^2) in f32.
 * fmt 0: e4m3 / 128x128 f32 scales; fmt 1: e2m1 / UE8M0 per 32;
 * fmt 2: e2m1 / E4M3 per 16.
 * q: codes of the ne experts, contiguous, expert-major; s: their scales.
 * Work is split over (expert, row band); every band is a pure function
 * of its counters, so the output does not depend on the thread count. */
void synth_expert_matrices(uint64_t seed, uint64_t stream_base, int64_t e0, int64_t ne, int64_t N,
                           int64_t K, double stddev, int fmt, uint8_t* q, void* s) {
  const int64_t R = fmt == 0 ? 128 : 32; /* rows per band: one scale-block row for e4m3 */
  int64_t bands = N / R;
  int64_t q_per_e = fmt == 0 ? N * K : N * K / 2;
  int64_t s_per_e = fmt == 0 ? (N / 128) * (K / 128) : (fmt == 1 ? N * (K / 32) : N * (K / 16));
#pragma omp parallel
  {
    float* buf = (float*)malloc(sizeof(float) * (size_t)R * (size_t)K);
#pragma omp for schedule(dynamic, 1)
    for (int64_t job = 0; job < ne * bands; ++job) {
      int64_t e = job / bands, b = job % bands;
      uint64_t key = stream_key(seed, stream_base + (uint64_t)(e0 + e));
      fill_normal_f32(key, (uint64_t)(b * R * K), R * K, stddev, buf);
      if (fmt == 0) {
        synth_quant_e4m3_b128(buf, R, K, q + e * q_per_e + b * R * K,
                              (float*)s + e * s_per_e + b * (K / 128));
      } else if (fmt == 1) {
        synth_quant_e2m1_g32(buf, R, K, q + e * q_per_e + b * R * (K / 2),
                             (uint8_t*)s + e * s_per_e + b * R * (K / 32));
      } else {
        synth_quant_nvfp4_g16(buf, R, K, q + e * q_per_e + b * R * (K / 2),
                              (uint8_t*)s + e * s_per_e + b * R * (K / 16));
      }
    }
    free(buf);
  }
}
