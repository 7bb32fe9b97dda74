/*
 * mbgen.c — seeded synthetic inputs for hot-expert replication and token
 * dispatch/combine: routing decisions (top-K expert ids and gate weights) and
 * token / expert-output rows.
 *
 * This file is shared input plumbing. It holds none of the planning, dispatch
 * or combine arithmetic; both the GPU library and the CPU oracle consume what
 * it writes, and neither is linked against it.
 *
 * Random numbers are counter based: value i of a stream is a pure function of
 * (seed, stream tag, i), so any subset of rows can be regenerated on its own
 * and the result does not depend on the number of threads.
 *
 *  - Mixer: the splitmix64 finaliser (Steele, Lea & Flood, "Fast Splittable
 *    Pseudorandom Number Generators", OOPSLA 2014), applied to
 *    key + (i + 1) * 0x9E3779B97F4A7C15.
 *  - Uniform (0,1): the top 53 bits of the mixed word, offset by half a step.
 *  - Normal: Box–Muller (1958) on uniforms 2j and 2j+1, cosine branch for
 *    even i and sine branch for odd i, in double precision.
 *  - Gumbel(0,1): -ln(-ln u).
 *
 * Routing model. Expert popularity is Zipf: the expert of popularity rank j
 * (1-based) has p_j proportional to j^-s, and popularity ranks are mapped to
 * expert ids by a seeded Fisher–Yates permutation. Token t's logit for
 * expert e is noise[t][e] + beta * ln p(e), with noise either N(0,1) or
 * Gumbel(0,1) (Gumbel noise with beta = 1 is Plackett–Luce sampling from p).
 * The K experts with the largest logits are selected (distinct by
 * construction; equal logits rank the lower expert id first) and listed in
 * descending logit order. Gate weights are the softmax over the K selected
 * logits, computed in double and stored as float.
 *
 * Row formats: fp32, bf16 (round to nearest even from the fp32 value) and
 * OCP fp8 e4m3fn with one fp32 scale per 128-element block
 * (scale = amax / 448, element = RNE(x / scale) with saturation at +-448).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MBGEN_GOLDEN 0x9E3779B97F4A7C15ULL

/* Stream tags: one independent counter stream per kind of input. */
enum {
  MBGEN_TAG_PERM = 1,
  MBGEN_TAG_NOISE = 2,
  MBGEN_TAG_X = 3,
  MBGEN_TAG_YEXP = 4,
};

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tag) {
  return mix64(mix64(seed + MBGEN_GOLDEN) ^ (tag * 0xD1B54A32D192ED03ULL));
}

static inline uint64_t ctr64(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1ULL) * MBGEN_GOLDEN);
}

static inline double u01(uint64_t v) {
  return ((double)(v >> 11) + 0.5) * 0x1.0p-53;
}

/* Normal number i of the stream. */
static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t j = i >> 1;
  double u1 = u01(ctr64(key, 2 * j));
  double u2 = u01(ctr64(key, 2 * j + 1));
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

static inline double gumbel_at(uint64_t key, uint64_t i) {
  return -log(-log(u01(ctr64(key, i))));
}

int mbgen_version(void) { return 1; }

uint64_t mbgen_u64(uint64_t seed, uint32_t tag, uint64_t i) {
  return ctr64(stream_key(seed, tag), i);
}

double mbgen_uniform(uint64_t seed, uint32_t tag, uint64_t i) {
  return u01(ctr64(stream_key(seed, tag), i));
}

double mbgen_normal(uint64_t seed, uint32_t tag, uint64_t i) {
  return normal_at(stream_key(seed, tag), i);
}

/* perm[j] = expert id of popularity rank j (0-based), seeded Fisher–Yates. */
void mbgen_permutation(uint64_t seed, int32_t n, int32_t* perm) {
  uint64_t key = stream_key(seed, MBGEN_TAG_PERM);
  for (int32_t i = 0; i < n; ++i) perm[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)(ctr64(key, (uint64_t)i) % (uint64_t)(i + 1));
    int32_t tmp = perm[i];
    perm[i] = perm[j];
    perm[j] = tmp;
  }
}

/* ln p(e) for every expert e under Zipf(s) popularity mapped by perm. */
void mbgen_log_popularity(uint64_t seed, int32_t n_experts, double zipf_s,
                          double* lnp) {
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_experts);
  mbgen_permutation(seed, n_experts, perm);
  double z = 0.0;
  for (int32_t j = 1; j <= n_experts; ++j) z += pow((double)j, -zipf_s);
  double lnz = log(z);
  for (int32_t j = 1; j <= n_experts; ++j)
    lnp[perm[j - 1]] = -zipf_s * log((double)j) - lnz;
  free(perm);
}

/*
 * Routing decisions for n_tokens tokens: ids[t*K + k], w[t*K + k].
 * noise_kind: 0 = N(0,1), 1 = Gumbel(0,1). The popularity permutation comes
 * from pop_seed and the per-token noise from noise_seed. Returns 0, or -1
 * on bad sizes.
 */
int mbgen_routing_ex(int32_t n_tokens, int32_t n_experts, int32_t top_k,
                     int32_t noise_kind, double zipf_s, double beta,
                     uint64_t pop_seed, uint64_t noise_seed, int32_t* ids, float* w) {
  if (n_tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts ||
      top_k > 256 || (noise_kind != 0 && noise_kind != 1))
    return -1;
  double* lnp = (double*)malloc(sizeof(double) * (size_t)n_experts);
  mbgen_log_popularity(pop_seed, n_experts, zipf_s, lnp);
  const uint64_t key = stream_key(noise_seed, MBGEN_TAG_NOISE);
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < n_tokens; ++t) {
    double best_l[256];
    int32_t best_e[256];
    int32_t nb = 0;
    for (int32_t e = 0; e < n_experts; ++e) {
      uint64_t i = (uint64_t)t * (uint64_t)n_experts + (uint64_t)e;
      double l = (noise_kind == 0 ? normal_at(key, i) : gumbel_at(key, i)) +
                 beta * lnp[e];
      /* Insert after every kept entry that is >= l: equal logits keep the
       * lower expert id (seen first) ahead. */
      int32_t p = nb;
      while (p > 0 && l > best_l[p - 1]) --p;
      if (p >= top_k) continue;
      int32_t last = nb < top_k ? nb : top_k - 1;
      for (int32_t q = last; q > p; --q) {
        best_l[q] = best_l[q - 1];
        best_e[q] = best_e[q - 1];
      }
      best_l[p] = l;
      best_e[p] = e;
      if (nb < top_k) ++nb;
    }
    double mx = best_l[0], den = 0.0;
    for (int32_t k = 0; k < top_k; ++k) den += exp(best_l[k] - mx);
    for (int32_t k = 0; k < top_k; ++k) {
      ids[(size_t)t * top_k + k] = best_e[k];
      w[(size_t)t * top_k + k] = (float)(exp(best_l[k] - mx) / den);
    }
  }
  free(lnp);
  return 0;
}

/* One seed for both the popularity permutation and the noise. */
int mbgen_routing(int32_t n_tokens, int32_t n_experts, int32_t top_k,
                  int32_t noise_kind, double zipf_s, double beta,
                  uint64_t seed, int32_t* ids, float* w) {
  return mbgen_routing_ex(n_tokens, n_experts, top_k, noise_kind, zipf_s, beta, seed, seed,
                          ids, w);
}

/* ---- row formats ------------------------------------------------------ */

static inline uint32_t f32_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

uint16_t mbgen_f32_to_bf16(float f) {
  uint32_t b = f32_bits(f);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu))
    return (uint16_t)((b >> 16) | 0x0040u); /* quiet NaN */
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

float mbgen_bf16_to_f32(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

/* OCP fp8 e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, 0x7F / 0xFF are NaN, largest finite 448. RNE, saturating. */
uint8_t mbgen_f32_to_e4m3(float f) {
  uint8_t sign = (uint8_t)((f32_bits(f) >> 24) & 0x80u);
  if (isnan(f)) return (uint8_t)(sign | 0x7Fu);
  double a = fabs((double)f);
  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
  if (a < 0x1p-6) {
    /* subnormal quantum 2^-9; a result of 8 quanta is the smallest normal,
     * whose code (exponent 1, mantissa 0) is also 8 */
    double m = rint(a * 512.0);
    return (uint8_t)(sign | (uint8_t)m);
  }
  int ex;
  double fr = frexp(a, &ex); /* a = fr * 2^ex, fr in [0.5, 1) */
  int biased = ex - 1 + 7;
  double man = rint((2.0 * fr - 1.0) * 8.0);
  if (man >= 8.0) {
    man = 0.0;
    ++biased;
  }
  int code = (biased << 3) | (int)man;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | (uint8_t)code);
}

float mbgen_e4m3_to_f32(uint8_t v) {
  int s = v & 0x80, e = (v >> 3) & 0xF, m = v & 7;
  double r;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    r = ldexp((double)m, -9);
  else
    r = ldexp(1.0 + m / 8.0, e - 7);
  return (float)(s ? -r : r);
}

/*
 * Rows of N(0,1) values: element (r, i) of the row block is normal number
 * (row0 + r) * H + i of stream (seed, tag). Row indices may be given
 * explicitly (rows != NULL, n entries) or as the range [row0, row0 + n).
 */
static inline int64_t row_index(const int64_t* rows, int64_t row0, int64_t r) {
  return rows ? rows[r] : row0 + r;
}

void mbgen_rows_f32(uint64_t seed, uint32_t tag, const int64_t* rows,
                    int64_t row0, int64_t n, int32_t hidden, float* out) {
  const uint64_t key = stream_key(seed, tag);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    uint64_t base = (uint64_t)row_index(rows, row0, r) * (uint64_t)hidden;
    float* o = out + r * (int64_t)hidden;
    for (int32_t i = 0; i < hidden; ++i) o[i] = (float)normal_at(key, base + i);
  }
}

void mbgen_rows_bf16(uint64_t seed, uint32_t tag, const int64_t* rows,
                     int64_t row0, int64_t n, int32_t hidden, uint16_t* out) {
  const uint64_t key = stream_key(seed, tag);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    uint64_t base = (uint64_t)row_index(rows, row0, r) * (uint64_t)hidden;
    uint16_t* o = out + r * (int64_t)hidden;
    for (int32_t i = 0; i < hidden; ++i)
      o[i] = mbgen_f32_to_bf16((float)normal_at(key, base + i));
  }
}

/* fp8 rows plus one fp32 scale per 128-element block (hidden % 128 == 0).
 * If deq != NULL it also receives the bf16 (RNE) of q * scale. */
int mbgen_rows_fp8(uint64_t seed, uint32_t tag, const int64_t* rows,
                   int64_t row0, int64_t n, int32_t hidden, uint8_t* q,
                   float* scale, uint16_t* deq) {
  if (hidden % 128) return -1;
  const uint64_t key = stream_key(seed, tag);
  const int32_t nb = hidden / 128;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    uint64_t base = (uint64_t)row_index(rows, row0, r) * (uint64_t)hidden;
    float v[128];
    for (int32_t b = 0; b < nb; ++b) {
      float amax = 0.0f;
      for (int32_t i = 0; i < 128; ++i) {
        v[i] = (float)normal_at(key, base + (uint64_t)(b * 128 + i));
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
      }
      float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      scale[r * nb + b] = sc;
      for (int32_t i = 0; i < 128; ++i) {
        uint8_t c = mbgen_f32_to_e4m3(v[i] / sc);
        q[r * (int64_t)hidden + b * 128 + i] = c;
        if (deq)
          deq[r * (int64_t)hidden + b * 128 + i] =
              mbgen_f32_to_bf16(mbgen_e4m3_to_f32(c) * sc);
      }
    }
  }
  return 0;
}
