/*
 * Seeded synthetic inputs: weights, prompts and KV contents for the decode workloads.
 *
 * This module produces DATA only.  It holds none of the decode arithmetic; the CPU
 * oracle and the GPU library each consume its output through their own code.
 *
 * Generator definition (counter based, so every element is independent of order and
 * thread count):
 *   key(seed, tensor)   = mix64(seed * 0x9E3779B97F4A7C15 ^ mix64(tensor + 0x632BE59BD9B4E019))
 *   word(key, i)        = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
 *   unit(w)             = ((w >> 11) + 0.5) * 2^-53            in (0, 1)
 *   mix64               = the SplitMix64 output finaliser (Steele, Lea, Flood 2014)
 * Normals use the Box-Muller transform in double precision: element pair j takes
 * u1 = unit(word(key, 2j)), u2 = unit(word(key, 2j+1)), r = sqrt(-2 ln u1),
 * element 2j = r cos(2 pi u2), element 2j+1 = r sin(2 pi u2); then times std and
 * rounded to nearest-even into the storage format.
 * Uniform integers in [0, n): word(key, i) mod n (bias below 2^-40 for n < 2^24).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t sg_key(uint64_t seed, uint64_t tensor) {
  return mix64(seed * 0x9E3779B97F4A7C15ull ^ mix64(tensor + 0x632BE59BD9B4E019ull));
}

static inline uint64_t sg_word(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ull); }

static inline double sg_unit(uint64_t w) { return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

/* Storage encoders of the generator's own (round to nearest even, IEEE binary16 / bfloat16). */
static uint16_t sg_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static uint16_t sg_to_f16(double v) {
  /* exact RNE from double: scale into the binary16 grid */
  uint16_t sign = 0;
  if (signbit(v)) { sign = 0x8000; v = -v; }
  if (isnan(v)) return 0x7e00;
  if (v >= 65520.0) return sign | 0x7c00;
  int e;
  double m = frexp(v, &e); /* v = m * 2^e, m in [0.5,1) */
  if (v == 0.0) return sign;
  int exp16 = e - 1 + 15; /* biased exponent if normal */
  double q;
  if (exp16 <= 0) {
    q = nearbyint(ldexp(v, 24)); /* subnormal unit 2^-24 */
    return sign | (uint16_t)q;    /* q may reach 1024 = smallest normal, encoded correctly */
  }
  q = nearbyint(ldexp(m, 11)); /* 11 significant bits, in [1024, 2048] */
  if (q == 2048.0) { q = 1024.0; exp16 += 1; }
  if (exp16 >= 31) return sign | 0x7c00;
  return sign | (uint16_t)(exp16 << 10) | (uint16_t)((int)q - 1024);
}

static double sg_normal(uint64_t key, uint64_t i) {
  uint64_t j = i >> 1;
  double u1 = sg_unit(sg_word(key, 2 * j));
  double u2 = sg_unit(sg_word(key, 2 * j + 1));
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* out[i] = N(mean, std) rounded into fmt: 0 = binary16, 1 = bfloat16, 2 = float32 (bit pattern) */
void sg_normal_fill(uint64_t seed, uint64_t tensor, uint64_t n, double mean, double std, int fmt, void* out) {
  uint64_t key = sg_key(seed, tensor);
  if (fmt == 2) {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) o[i] = (float)(mean + std * sg_normal(key, (uint64_t)i));
    return;
  }
  uint16_t* o = (uint16_t*)out;
  if (fmt == 0) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) o[i] = sg_to_f16(mean + std * sg_normal(key, (uint64_t)i));
  } else {
    /* bf16: round the double to float first only when that is exact to RNE; use a direct path */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
      double v = mean + std * sg_normal(key, (uint64_t)i);
      /* RNE of a double into bf16 (8 significant bits) */
      if (v == 0.0) { o[i] = signbit(v) ? 0x8000 : 0; continue; }
      int e;
      double m = frexp(fabs(v), &e);
      double q = nearbyint(ldexp(m, 8)); /* [128, 256] */
      double r = ldexp(q, e - 8);
      float f = (float)(v < 0 ? -r : r); /* exact: r has 8 significant bits */
      o[i] = sg_to_bf16(f);
    }
  }
}

/* Uniform integers in [0, n) */
void sg_uniform_int(uint64_t seed, uint64_t tensor, uint64_t count, uint32_t n, int32_t* out) {
  uint64_t key = sg_key(seed, tensor);
  for (uint64_t i = 0; i < count; ++i) out[i] = (int32_t)(sg_word(key, i) % n);
}

/* ---- OCP FP8 E4M3FN encoding used to prepare block-quantised weights (data preparation) ---- */
static double sg_e4m3_value(int c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* nearest-even, saturating to +-448; the input is finite */
static uint8_t sg_to_e4m3(double v) {
  uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7e;
  /* search the 127 non-negative finite codes (monotone) */
  int lo = 0, hi = 0x7e;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (sg_e4m3_value(mid) <= a) lo = mid; else hi = mid;
  }
  double vl = sg_e4m3_value(lo), vh = sg_e4m3_value(hi);
  int code;
  if (a - vl < vh - a) code = lo;
  else if (a - vl > vh - a) code = hi;
  else code = (lo & 1) ? hi : lo;
  if (a < vl) code = lo; /* a == 0 case */
  return sign | (uint8_t)code;
}

static float sg_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Quantise a bf16 matrix [rows][cols] into E4M3 codes with one fp32 scale per 128x128 block:
 * S = amax(block)/448 (1 when the block is all zero), q = RNE_sat(w / S).
 * scales is [ceil(rows/128)][ceil(cols/128)]. */
void sg_quant_e4m3_block(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* q, float* scales) {
  int64_t br = (rows + 127) / 128, bc = (cols + 127) / 128;
#pragma omp parallel for schedule(dynamic)
  for (int64_t b = 0; b < br * bc; ++b) {
    int64_t bi = b / bc, bj = b % bc;
    int64_t r0 = bi * 128, r1 = r0 + 128 < rows ? r0 + 128 : rows;
    int64_t c0 = bj * 128, c1 = c0 + 128 < cols ? c0 + 128 : cols;
    float amax = 0.f;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) {
        float a = fabsf(sg_bf16_value(w[r * cols + c]));
        if (a > amax) amax = a;
      }
    float s = amax > 0.f ? amax / 448.0f : 1.0f;
    scales[bi * bc + bj] = s;
    for (int64_t r = r0; r < r1; ++r)
      for (int64_t c = c0; c < c1; ++c) q[r * cols + c] = sg_to_e4m3((double)sg_bf16_value(w[r * cols + c]) / (double)s);
  }
}

/* Quantise float values with a given scale (used for synthetic FP8 KV contents). */
void sg_quant_e4m3_scaled(const float* v, int64_t n, float s, uint8_t* q) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) q[i] = sg_to_e4m3((double)v[i] / (double)s);
}

/* Symmetric weight-only integer quantisation of a bf16 matrix, per row and per group of 128
 * columns: s = bf16(max |w| / qmax) (1 for an all-zero group), q = clamp(round-half-even(w / s),
 * -qmax, qmax) with qmax = 127 (bits 8) or 7 (bits 4).  int8 codes are one signed byte each
 * ([rows][cols]); int4 codes are two per byte, the even column in the low nibble
 * ([rows][cols / 2], cols even).  Scales are bf16 bits [rows][ceil(cols / 128)]. */
void sg_quant_int_group(const uint16_t* w, int64_t rows, int64_t cols, int bits, uint8_t* q, uint16_t* scales) {
  const int64_t ng = (cols + 127) / 128;
  const double qmax = bits == 8 ? 127.0 : 7.0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < rows; ++r) {
    if (bits == 4)
      for (int64_t c = 0; c < cols / 2; ++c) q[r * (cols / 2) + c] = 0;
    for (int64_t g = 0; g < ng; ++g) {
      const int64_t c0 = g * 128, c1 = c0 + 128 < cols ? c0 + 128 : cols;
      float amax = 0.f;
      for (int64_t c = c0; c < c1; ++c) {
        const float a = fabsf(sg_bf16_value(w[r * cols + c]));
        if (a > amax) amax = a;
      }
      const uint16_t sb = amax > 0.f ? sg_to_bf16(amax / (float)qmax) : (uint16_t)0x3F80;
      scales[r * ng + g] = sb;
      const double s = (double)sg_bf16_value(sb);
      for (int64_t c = c0; c < c1; ++c) {
        double v = nearbyint((double)sg_bf16_value(w[r * cols + c]) / s);
        if (v > qmax) v = qmax;
        if (v < -qmax) v = -qmax;
        const int iv = (int)v;
        if (bits == 8) {
          q[r * cols + c] = (uint8_t)(int8_t)iv;
        } else {
          q[r * (cols / 2) + c / 2] |= (uint8_t)((iv & 15) << (4 * (c & 1)));
        }
      }
    }
  }
}
