// CPU oracle for batch-1 greedy decode of a dense Llama-style decoder.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
// CPU-baseline leg may load this library.  It shares no code, header or table with the
// GPU library: every codec and every operation below is written out here from its plain
// definition, in the order the decode step defines it, with fp32 activations and fp32
// accumulation in ascending index order.
//
// What it follows (pages: "AutoMegaKernel: A Statically-Checked Agent Harness for
// Self-Retargeting Megakernel Synthesis", Method / Layer 1, names the step's
// instructions GEMV, attention and RMSNorm for HF Llama-family decoders; "Netra Kernel"
// summary, details section, names GQA attention over an FP8 KV cache and FP8 E4M3
// block-scale weights; the AutoMegaKernel explainer's results name weight-only int8 (W8A16)
// and int4 variants of the same kernels; the rest of the step is the standard Llama decoder):
//   x = E[tok]; per layer: xn = rmsnorm(x, g1); q,k,v = W xn; rotate-half RoPE on q,k;
//   append k,v to the cache (rounded to the cache format); grouped-query softmax
//   attention over cache positions 0..p; x += Wo o; xn = rmsnorm(x, g2);
//   x += Wd (silu(Wg xn) * (Wu xn)); finally logits = Wlm rmsnorm(x, gf), token = argmax
//   with the lowest index winning ties.
// Every function is pinned by the oracle tests (closed forms, invariants, brute force).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

enum Fmt { F16 = 0, BF16 = 1, E4M3 = 2, I8 = 3, I4 = 4 };

// ---------------------------------------------------------------------------------------------
// Storage codecs (IEEE binary16, bfloat16 = upper half of binary32, OCP FP8 E4M3FN)
// ---------------------------------------------------------------------------------------------
inline float bits_f32(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
inline uint32_t f32_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

float dec_f16(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = std::ldexp((double)m, -24);          // subnormal: m * 2^-24
  else v = std::ldexp(1.0 + m / 1024.0, e - 15);
  return (float)(s ? -v : v);
}

uint16_t enc_f16(float f) {
  const uint32_t u = f32_bits(f);
  const uint16_t sign = (u >> 16) & 0x8000;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7e00;                // NaN
  if (a >= 0x477ff000u) return sign | 0x7c00;               // >= 65520 rounds to infinity
  if (a >= 0x38800000u) {                                   // binary16 normal range
    uint32_t h = (((a >> 23) - 112u) << 10) | ((a & 0x7fffffu) >> 13);
    const uint32_t rem = a & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;
    return sign | (uint16_t)h;
  }
  if (a <= 0x33000000u) return sign;                        // <= 2^-25 rounds to zero
  const uint32_t e32 = a >> 23, m = (a & 0x7fffffu) | 0x800000u;
  const uint32_t shift = 126u - e32;                        // value in units of 2^-24
  uint32_t h = m >> shift;
  const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1u);
  if (rem > half || (rem == half && (h & 1u))) h += 1;
  return sign | (uint16_t)h;
}

float dec_bf16(uint16_t b) { return bits_f32((uint32_t)b << 16); }

uint16_t enc_bf16(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float dec_e4m3(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? std::ldexp((double)m, -9) : std::ldexp(1.0 + m / 8.0, e - 7);
  return (float)(s ? -v : v);
}

// nearest-even, saturating to +-448 (the format has no infinity)
uint8_t enc_e4m3(float f) {
  if (std::isnan(f)) return 0x7f;
  const uint8_t sign = std::signbit(f) ? 0x80 : 0;
  const double a = std::fabs((double)f);
  if (a >= 448.0) return sign | 0x7e;
  if (a < std::ldexp(1.0, -6)) {                            // subnormal grid: units of 2^-9
    const double q = std::nearbyint(std::ldexp(a, 9));       // 8 means 2^-6, which is code 8
    return sign | (uint8_t)q;
  }
  int e = (int)std::floor(std::log2(a));
  if (std::ldexp(1.0, e) > a) e -= 1;                       // guard log2 rounding
  if (std::ldexp(1.0, e + 1) <= a) e += 1;
  double q = std::nearbyint(std::ldexp(a, 3 - e));          // in [8, 16]
  if (q == 16.0) { q = 8.0; e += 1; }
  const int code = ((e + 7) << 3) | ((int)q - 8);
  return sign | (uint8_t)(code > 0x7e ? 0x7e : code);
}

// Every binary16 and E4M3 code decoded once by the definitions above: whole-model runs decode
// billions of weights, and a table look-up returns the same value as the definition.
struct DecodeTables {
  std::vector<float> f16, e4m3;
  DecodeTables() : f16(65536), e4m3(256) {
    for (uint32_t c = 0; c < 65536; ++c) f16[c] = dec_f16((uint16_t)c);
    for (uint32_t c = 0; c < 256; ++c) e4m3[c] = dec_e4m3((uint8_t)c);
  }
};
const DecodeTables& tables() {
  static const DecodeTables t;
  return t;
}

inline float dec(int fmt, const void* p, size_t i) {
  if (fmt == F16) return tables().f16[((const uint16_t*)p)[i]];
  if (fmt == BF16) return dec_bf16(((const uint16_t*)p)[i]);
  return tables().e4m3[((const uint8_t*)p)[i]];
}

inline size_t fmt_size(int fmt) { return fmt == E4M3 ? 1 : 2; }

// ---------------------------------------------------------------------------------------------
// Operations
// ---------------------------------------------------------------------------------------------

// RMSNorm: y_i = (x_i * r) * g_i with r = 1 / sqrt(mean(x^2) + eps); the sum runs in index order.
void rmsnorm(const float* x, const float* g, int n, float eps, float* y) {
  float ss = 0.f;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  const float r = 1.0f / std::sqrt(ss / (float)n + eps);
  for (int i = 0; i < n; ++i) y[i] = (x[i] * r) * g[i];
}

// Weight-only integer formats (W8A16 and W4A16): the code q(n,k) is a two's-complement
// integer, one signed byte per element (int8) or two per byte with the even column in the low
// nibble (int4, cols even); every row has one bf16 scale per group of 128 columns.
inline int int_code(int fmt, const void* W, int cols, int n, int k) {
  const size_t i = (size_t)n * cols + k;
  if (fmt == I8) return ((const int8_t*)W)[i];
  const uint8_t b = ((const uint8_t*)W)[i / 2];
  const int nib = (k & 1) ? (b >> 4) : (b & 15);
  return nib >= 8 ? nib - 16 : nib;
}

inline bool is_int(int fmt) { return fmt == I8 || fmt == I4; }

// Dequantised weight element: w(n,k) = dec(W[n][k]) (16-bit), dec(q[n][k]) * S[n/128][k/128]
// (fp8, fp32 block scales), or q(n,k) * s[n][k/128] (int8 / int4, bf16 group scales).
inline float weight(int fmt, const void* W, const void* S, int cols, int n, int k) {
  const int nb = (cols + 127) / 128;
  if (is_int(fmt)) return (float)int_code(fmt, W, cols, n, k) * dec_bf16(((const uint16_t*)S)[(size_t)n * nb + k / 128]);
  const float w = dec(fmt, W, (size_t)n * cols + k);
  if (fmt != E4M3) return w;
  return w * ((const float*)S)[(size_t)(n / 128) * nb + k / 128];
}

// Y[t][n] = sum_k w(n,k) * X[t][k] for B tokens, k ascending, fp32 (one sum per (t, n)).
// The integer weight formats take their activation operand in binary16 (the "A16" of W8A16):
// every element of X is first rounded to the nearest binary16 value.
void matmul_tokens(int fmt, const void* W, const void* S, int rows, int cols, const float* Xin, int B, float* Y) {
  std::vector<float> Xh;
  const float* X = Xin;
  if (is_int(fmt)) {
    Xh.resize((size_t)cols * B);
    for (size_t i = 0; i < Xh.size(); ++i) Xh[i] = dec_f16(enc_f16(Xin[i]));
    X = Xh.data();
  }
  std::vector<float> XT((size_t)cols * B);
  for (int t = 0; t < B; ++t)
    for (int k = 0; k < cols; ++k) XT[(size_t)k * B + t] = X[(size_t)t * cols + k];
#pragma omp parallel
  {
    std::vector<float> wrow(cols), acc(B);
#pragma omp for schedule(static)
    for (int n = 0; n < rows; ++n) {
      for (int k = 0; k < cols; ++k) wrow[k] = weight(fmt, W, S, cols, n, k);
      if (B == 1) {  // one token (decode): the same sum, in a register
        float a = 0.f;
        for (int k = 0; k < cols; ++k) a = a + wrow[k] * X[k];
        Y[n] = a;
        continue;
      }
      for (int t = 0; t < B; ++t) acc[t] = 0.f;
      for (int k = 0; k < cols; ++k) {
        const float w = wrow[k];
        const float* xk = &XT[(size_t)k * B];
        for (int t = 0; t < B; ++t) acc[t] = acc[t] + w * xk[t];
      }
      for (int t = 0; t < B; ++t) Y[(size_t)t * rows + n] = acc[t];
    }
  }
}

// Rotate-half RoPE on one head vector u[hd] at position p: for i < hd/2 the pair
// (u_i, u_{i+hd/2}) turns by phi = p * theta^(-2i/hd) (angle in double, cos/sin rounded to fp32).
void rope(float* u, int hd, int p, double theta) {
  const int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    const double phi = (double)p * std::pow(theta, -2.0 * i / (double)hd);
    const float c = (float)std::cos(phi), s = (float)std::sin(phi);
    const float a = u[i], b = u[i + half];
    u[i] = a * c - b * s;
    u[i + half] = b * c + a * s;
  }
}

// Softmax attention of one query head over T cached positions of one KV head.
// K, V: [T][hd] in the cache format (fp8 values are code * scale).
void attend(const float* q, const void* K, const void* V, int fmt, float ks, float vs, int T, int hd, float* out) {
  std::vector<float> s(T > 0 ? T : 1);
  const float root = std::sqrt((float)hd);
  for (int t = 0; t < T; ++t) {
    float d = 0.f;
    for (int i = 0; i < hd; ++i) {
      float kv = dec(fmt, K, (size_t)t * hd + i);
      if (fmt == E4M3) kv = kv * ks;
      d += q[i] * kv;
    }
    s[t] = d / root;
  }
  float m = -INFINITY;
  for (int t = 0; t < T; ++t) m = s[t] > m ? s[t] : m;
  float Z = 0.f;
  for (int t = 0; t < T; ++t) { s[t] = std::exp(s[t] - m); Z += s[t]; }
  for (int i = 0; i < hd; ++i) {
    float acc = 0.f;
    for (int t = 0; t < T; ++t) {
      float vv = dec(fmt, V, (size_t)t * hd + i);
      if (fmt == E4M3) vv = vv * vs;
      acc += s[t] * vv;
    }
    out[i] = acc / Z;
  }
}

inline float silu(float z) { return z / (1.0f + std::exp(-z)); }

// Greedy choice: the largest value, lowest index on ties; -1 if any value is NaN.
int argmax(const float* v, int n) {
  int best = -1;
  for (int i = 0; i < n; ++i) {
    if (std::isnan(v[i])) return -1;
    if (best < 0 || v[i] > v[best]) best = i;
  }
  return best;
}

}  // namespace

// =============================================================================================
// C ABI
// =============================================================================================
extern "C" {

struct orc_config {
  int L, H, nq, nkv, hd, F, V;
  float eps;
  double theta;
  int wfmt;     // format of the linear weights (0 f16, 1 bf16, 2 e4m3 with 128x128 block scales,
                // 3 int8 / 4 int4 with bf16 scales per row and 128-column group)
  int efmt;     // format of the embedding and norm gains (0 f16, 1 bf16)
  int kvfmt;    // format of the KV cache (0 f16, 1 bf16, 2 e4m3 with per (layer, kv head, K|V) scale)
  int max_seq;
};

// Per layer the 9 tensors wq wk wv wo w_gate w_up w_down attn_norm ffn_norm (canonical [out][in]),
// and for fp8 / int8 / int4 the 7 scale arrays of the linear tensors.
struct orc_weights {
  const void* embed;
  const void* final_norm;
  const void* lm_head;
  const void* lm_head_scale;
  const void* const* layer;        // L * 9
  const void* const* layer_scale;  // L * 7, or NULL
};

struct orc_model {
  orc_config c;
  const void* embed;
  std::vector<float> final_norm;
  const void* lm_head;
  const void* lm_head_scale;
  std::vector<const void*> layer;
  std::vector<const void*> layer_scale;
  std::vector<std::vector<float>> gains;  // per layer: attn_norm, ffn_norm as fp32
  std::vector<uint8_t> kcache, vcache;    // [L][nkv][max_seq][hd] in the cache format
  std::vector<float> kv_scale;            // [L][nkv][2]
  std::vector<float> kv_amax;             // [L][nkv][2]: largest |k|, |v| appended since the last reset
  int pos;
};

// ---- codecs over arrays ----
void orc_decode(int fmt, const void* src, int64_t n, float* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = dec(fmt, src, (size_t)i);
}

void orc_encode(int fmt, const float* src, int64_t n, void* dst) {
  for (int64_t i = 0; i < n; ++i) {
    if (fmt == F16) ((uint16_t*)dst)[i] = enc_f16(src[i]);
    else if (fmt == BF16) ((uint16_t*)dst)[i] = enc_bf16(src[i]);
    else ((uint8_t*)dst)[i] = enc_e4m3(src[i]);
  }
}

// ---- single operations ----
void orc_rmsnorm(const float* x, const float* g, int n, float eps, float* y) { rmsnorm(x, g, n, eps, y); }

void orc_gemv(int fmt, const void* W, const void* S, int rows, int cols, const float* x, float* y) {
  matmul_tokens(fmt, W, S, rows, cols, x, 1, y);
}

// Dequantised weight matrix (any weight format): out[n][k] = w(n,k).
void orc_weight_matrix(int fmt, const void* W, const void* S, int rows, int cols, float* out) {
  for (int n = 0; n < rows; ++n)
    for (int k = 0; k < cols; ++k) out[(size_t)n * cols + k] = weight(fmt, W, S, cols, n, k);
}

void orc_matmul_tokens(int fmt, const void* W, const void* S, int rows, int cols, const float* X, int B, float* Y) {
  matmul_tokens(fmt, W, S, rows, cols, X, B, Y);
}

void orc_rope(float* u, int hd, int p, double theta) { rope(u, hd, p, theta); }

void orc_attend(const float* q, const void* K, const void* V, int fmt, float ks, float vs, int T, int hd, float* out) {
  attend(q, K, V, fmt, ks, vs, T, hd, out);
}

float orc_silu(float z) { return silu(z); }

int orc_argmax(const float* v, int n) { return argmax(v, n); }

// ---- model ----
orc_model* orc_create(const orc_config* c, const orc_weights* w) {
  if (c->hd % 2 || c->nq % c->nkv) return nullptr;
  if (c->wfmt == I4 && (c->H % 2 || c->F % 2)) return nullptr;  // int4 rows hold whole bytes
  orc_model* m = new orc_model();
  m->c = *c;
  m->embed = w->embed;
  m->lm_head = w->lm_head;
  m->lm_head_scale = w->lm_head_scale;
  m->final_norm.resize(c->H);
  orc_decode(c->efmt, w->final_norm, c->H, m->final_norm.data());
  m->layer.assign(w->layer, w->layer + (size_t)c->L * 9);
  if (w->layer_scale) m->layer_scale.assign(w->layer_scale, w->layer_scale + (size_t)c->L * 7);
  else m->layer_scale.assign((size_t)c->L * 7, nullptr);
  m->gains.resize((size_t)c->L * 2);
  for (int l = 0; l < c->L; ++l)
    for (int j = 0; j < 2; ++j) {
      m->gains[l * 2 + j].resize(c->H);
      orc_decode(c->efmt, m->layer[l * 9 + 7 + j], c->H, m->gains[l * 2 + j].data());
    }
  const size_t kvn = (size_t)c->L * c->nkv * c->max_seq * c->hd * fmt_size(c->kvfmt);
  m->kcache.assign(kvn, 0);
  m->vcache.assign(kvn, 0);
  m->kv_scale.assign((size_t)c->L * c->nkv * 2, 1.0f);
  m->kv_amax.assign((size_t)c->L * c->nkv * 2, 0.0f);
  m->pos = 0;
  return m;
}

void orc_destroy(orc_model* m) { delete m; }

int orc_get_pos(const orc_model* m) { return m->pos; }

void orc_set_kv_scales(orc_model* m, const float* s) {
  std::memcpy(m->kv_scale.data(), s, m->kv_scale.size() * sizeof(float));
}

// Largest |k| (after RoPE) and |v| per (layer, kv head) over the rows appended since the last reset,
// before rounding to the cache format: out [L][nkv][2].
void orc_kv_amax(const orc_model* m, float* out) {
  std::memcpy(out, m->kv_amax.data(), m->kv_amax.size() * sizeof(float));
}

void orc_reset_kv_amax(orc_model* m) { std::fill(m->kv_amax.begin(), m->kv_amax.end(), 0.0f); }

// Static FP8 KV scales from those maxima: the largest value maps to the largest E4M3 magnitude,
// S = amax / 448 in fp32 (1 where nothing but zeros was appended).
void orc_kv_scales_from_amax(const orc_model* m, float* out) {
  for (size_t i = 0; i < m->kv_amax.size(); ++i) out[i] = m->kv_amax[i] > 0.0f ? m->kv_amax[i] / 448.0f : 1.0f;
}

static inline size_t kv_index(const orc_config& c, int l, int g, int p) {
  return (((size_t)l * c.nkv + g) * c.max_seq + p) * c.hd;
}

// Canonical KV contents [L][nkv][P][hd] in the cache format; sets pos = P.
int orc_load_kv(orc_model* m, const void* k, const void* v, int P) {
  const orc_config& c = m->c;
  if (P < 0 || P > c.max_seq) return -1;
  const size_t es = fmt_size(c.kvfmt), row = (size_t)P * c.hd * es;
  for (int l = 0; l < c.L; ++l)
    for (int g = 0; g < c.nkv; ++g) {
      const size_t src = ((size_t)l * c.nkv + g) * row;
      std::memcpy(&m->kcache[kv_index(c, l, g, 0) * es], (const uint8_t*)k + src, row);
      std::memcpy(&m->vcache[kv_index(c, l, g, 0) * es], (const uint8_t*)v + src, row);
    }
  m->pos = P;
  return 0;
}

int orc_read_kv(const orc_model* m, void* k, void* v, int P) {
  const orc_config& c = m->c;
  if (P < 0 || P > c.max_seq) return -1;
  const size_t es = fmt_size(c.kvfmt), row = (size_t)P * c.hd * es;
  for (int l = 0; l < c.L; ++l)
    for (int g = 0; g < c.nkv; ++g) {
      const size_t dst = ((size_t)l * c.nkv + g) * row;
      std::memcpy((uint8_t*)k + dst, &m->kcache[kv_index(c, l, g, 0) * es], row);
      std::memcpy((uint8_t*)v + dst, &m->vcache[kv_index(c, l, g, 0) * es], row);
    }
  return 0;
}

// Run B consecutive tokens at positions pos..pos+B-1 through the decoder (causal attention
// over the cache).  logits (if not NULL) receives the logits of the LAST token.  Returns the
// argmax of those logits when they are computed, else 0.
// Teacher-forced rounding (B == 1 only): with force_k / force_v (cache-format codes [L][nkv][hd])
// the row appended at this position is the given one, not this step's own rounding of k and v,
// which goes to own_k / own_v (if not NULL) instead; the rest of the step then reads the forced
// row, as a teacher-forced step reads a given token.
static int forward_tokens(orc_model* m, const int32_t* toks, int B, float* logits, const uint8_t* force_k = nullptr,
                          const uint8_t* force_v = nullptr, uint8_t* own_k = nullptr, uint8_t* own_v = nullptr) {
  const orc_config& c = m->c;
  const int H = c.H, hd = c.hd, qd = c.nq * hd, kvd = c.nkv * hd, grp = c.nq / c.nkv;
  const int p0 = m->pos;
  std::vector<float> x((size_t)B * H), xn((size_t)B * H), q((size_t)B * qd), k((size_t)B * kvd),
      v((size_t)B * kvd), o((size_t)B * qd), y((size_t)B * H), gt((size_t)B * c.F), up((size_t)B * c.F),
      h((size_t)B * c.F);
  for (int t = 0; t < B; ++t)
    for (int i = 0; i < H; ++i) x[(size_t)t * H + i] = dec(c.efmt, m->embed, (size_t)toks[t] * H + i);
  const size_t es = fmt_size(c.kvfmt);
  for (int l = 0; l < c.L; ++l) {
    const void* const* W = &m->layer[(size_t)l * 9];
    const void* const* S = &m->layer_scale[(size_t)l * 7];
    for (int t = 0; t < B; ++t) rmsnorm(&x[(size_t)t * H], m->gains[l * 2].data(), H, c.eps, &xn[(size_t)t * H]);
    matmul_tokens(c.wfmt, W[0], S[0], qd, H, xn.data(), B, q.data());
    matmul_tokens(c.wfmt, W[1], S[1], kvd, H, xn.data(), B, k.data());
    matmul_tokens(c.wfmt, W[2], S[2], kvd, H, xn.data(), B, v.data());
    for (int t = 0; t < B; ++t) {
      const int p = p0 + t;
      for (int j = 0; j < c.nq; ++j) rope(&q[(size_t)t * qd + j * hd], hd, p, c.theta);
      for (int g = 0; g < c.nkv; ++g) {
        float* kg = &k[(size_t)t * kvd + g * hd];
        float* vg = &v[(size_t)t * kvd + g * hd];
        rope(kg, hd, p, c.theta);
        uint8_t* kdst = &m->kcache[kv_index(c, l, g, p) * es];
        uint8_t* vdst = &m->vcache[kv_index(c, l, g, p) * es];
        float* amax = &m->kv_amax[((size_t)l * c.nkv + g) * 2];
        for (int i = 0; i < hd; ++i) {
          amax[0] = std::fabs(kg[i]) > amax[0] ? std::fabs(kg[i]) : amax[0];
          amax[1] = std::fabs(vg[i]) > amax[1] ? std::fabs(vg[i]) : amax[1];
        }
        if (c.kvfmt == E4M3) {
          const float ks = m->kv_scale[((size_t)l * c.nkv + g) * 2], vs = m->kv_scale[((size_t)l * c.nkv + g) * 2 + 1];
          for (int i = 0; i < hd; ++i) {
            kdst[i] = enc_e4m3(kg[i] / ks);
            vdst[i] = enc_e4m3(vg[i] / vs);
          }
        } else {
          orc_encode(c.kvfmt, kg, hd, kdst);
          orc_encode(c.kvfmt, vg, hd, vdst);
        }
        const size_t row = ((size_t)l * c.nkv + g) * hd * es;  // this (layer, kv head) row in [L][nkv][hd]
        if (own_k) std::memcpy(own_k + row, kdst, hd * es);
        if (own_v) std::memcpy(own_v + row, vdst, hd * es);
        if (force_k) std::memcpy(kdst, force_k + row, hd * es);
        if (force_v) std::memcpy(vdst, force_v + row, hd * es);
      }
    }
#pragma omp parallel for schedule(dynamic) collapse(2)
    for (int t = 0; t < B; ++t)
      for (int j = 0; j < c.nq; ++j) {
        const int g = j / grp, T = p0 + t + 1;
        const float ks = m->kv_scale[((size_t)l * c.nkv + g) * 2], vs = m->kv_scale[((size_t)l * c.nkv + g) * 2 + 1];
        attend(&q[(size_t)t * qd + j * hd], &m->kcache[kv_index(c, l, g, 0) * es], &m->vcache[kv_index(c, l, g, 0) * es],
               c.kvfmt, ks, vs, T, hd, &o[(size_t)t * qd + j * hd]);
      }
    matmul_tokens(c.wfmt, W[3], S[3], H, qd, o.data(), B, y.data());
    for (size_t i = 0; i < x.size(); ++i) x[i] = x[i] + y[i];
    for (int t = 0; t < B; ++t) rmsnorm(&x[(size_t)t * H], m->gains[l * 2 + 1].data(), H, c.eps, &xn[(size_t)t * H]);
    matmul_tokens(c.wfmt, W[4], S[4], c.F, H, xn.data(), B, gt.data());
    matmul_tokens(c.wfmt, W[5], S[5], c.F, H, xn.data(), B, up.data());
    for (size_t i = 0; i < h.size(); ++i) h[i] = silu(gt[i]) * up[i];
    matmul_tokens(c.wfmt, W[6], S[6], H, c.F, h.data(), B, y.data());
    for (size_t i = 0; i < x.size(); ++i) x[i] = x[i] + y[i];
  }
  m->pos = p0 + B;
  if (!logits) return 0;
  std::vector<float> xf(H);
  rmsnorm(&x[(size_t)(B - 1) * H], m->final_norm.data(), H, c.eps, xf.data());
  matmul_tokens(c.wfmt, m->lm_head, m->lm_head_scale, c.V, H, xf.data(), 1, logits);
  return argmax(logits, c.V);
}

// Prefill positions 0..P-1 (token blocks of `block` positions; the result does not depend on
// the block size).  Returns argmax(logits[P-1]) and writes those logits if asked.
int orc_prefill(orc_model* m, const int32_t* toks, int P, int block, float* logits) {
  const orc_config& c = m->c;
  if (P <= 0 || P > c.max_seq) return -2;
  if (block <= 0) block = 64;
  m->pos = 0;
  std::vector<float> lg(c.V);
  int tok = 0;
  for (int s = 0; s < P; s += block) {
    const int B = P - s < block ? P - s : block;
    const bool last = s + B == P;
    tok = forward_tokens(m, toks + s, B, last ? lg.data() : nullptr);
  }
  if (logits) std::memcpy(logits, lg.data(), sizeof(float) * c.V);
  return tok;
}

// One decode step with teacher-forced rounding of the appended KV row (see forward_tokens):
// force_k / force_v [L][nkv][hd] codes are appended; own_k / own_v receive this step's own codes.
int orc_step_forced(orc_model* m, int32_t tok, const void* force_k, const void* force_v, void* own_k, void* own_v,
                    float* logits) {
  const orc_config& c = m->c;
  if (m->pos >= c.max_seq) return -2;
  std::vector<float> lg(c.V);
  const int next = forward_tokens(m, &tok, 1, lg.data(), (const uint8_t*)force_k, (const uint8_t*)force_v,
                                  (uint8_t*)own_k, (uint8_t*)own_v);
  if (logits) std::memcpy(logits, lg.data(), sizeof(float) * c.V);
  return next;
}

// One decode step: token `tok` at position pos; pos += 1.  Returns the greedy next token.
int orc_step(orc_model* m, int32_t tok, float* logits) {
  const orc_config& c = m->c;
  if (m->pos >= c.max_seq) return -2;
  std::vector<float> lg(c.V);
  const int next = forward_tokens(m, &tok, 1, lg.data());
  if (logits) std::memcpy(logits, lg.data(), sizeof(float) * c.V);
  return next;
}

}  // extern "C"

#include <omp.h>
extern "C" int orc_num_threads(void) { return omp_get_max_threads(); }
extern "C" void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
