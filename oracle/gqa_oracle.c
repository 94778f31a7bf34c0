/*
 * Plain fp64 CPU oracle for one grouped-query-attention decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the GPU library.
 *
 * What it computes, and where that is defined:
 *
 *   "Grouped-Query Attention (GQA) and Multi-Query Attention (MQA):
 *    Mathematical Foundations, Arithmetic Intensity, and KV-Cache Scaling
 *    Mechanics", section 2, subsection "Grouped-Query Attention (GQA)":
 *    query head i uses the key/value head of its group g(i), with
 *    g(i) = floor((i-1)/R) + 1 in 1-based numbering, R = H_Q / H_KV, and
 *        Head_i = softmax(Q_i K_g(i)^T / sqrt(d_k) + M) V_g(i).
 *   Same page, subsection "Multi-Head Attention (MHA)": M is the causal mask.
 *
 * Readings taken where the page leaves a step open (all are the plainest
 * reading the rest of the page supports):
 *   - Decode step: the single query is the newest position, so the causal
 *     mask admits exactly the cached positions t in [0, seq_len).  Positions
 *     at or beyond seq_len are never read.
 *   - The 1/sqrt(d_k) factor is an explicit `scale` argument (a float the
 *     caller passes; the workloads use 1/sqrt(d)).
 *   - seq_len == 0 (softmax over an empty set) returns a zero vector.
 *   - The max score is subtracted inside the exponent; this changes nothing
 *     in exact arithmetic and only keeps exp() in range.
 *   - bf16 inputs are widened by their definition (the 16 stored bits are the
 *     upper half of an IEEE binary32), which is exact.
 *
 * Lower-precision caches (oracle_gqa_decode_fp8): the same page's KV
 * footprint formula (section 1, "KV Cache Memory Footprint") carries the
 * bytes per element as a factor of its own (2 for FP16/BF16), and
 * "Grouped-Query Attention Shares Keys Without Sharing Every Query" keeps it
 * as "bytes per element".  The pages give no format or dequantisation rule;
 * read as one byte per element in the OCP 8-bit floating-point format E4M3
 * (sign, 4 exponent bits of bias 7, 3 mantissa bits; subnormals; no
 * infinities; S.1111.111 is NaN; largest finite 448), and a cached key
 * (value) equal to k_scale (v_scale) times its E4M3 value, one scale per
 * array.  The attention then runs on those values as above.
 *
 * Also: the rotary position embedding of section 4 of the same page
 * ("Rotary Position Embeddings (RoPE) Interaction"), for the step that
 * appends the new token's keys and values to the cache (oracle_rope).
 *
 * Parity status: every function here is pinned by CPU tests against
 * closed forms, invariants, a library routine and the printed tables of the
 * pages (see the oracle tests); none is "parity unpinned".
 *
 * Build: gcc -O2 -fno-fast-math -fopenmp -shared -fPIC gqa_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2, ORACLE_E4M3 = 3 };

/* The value of one OCP E4M3 byte, from the format's definition: sign bit,
 * exponent field e (bias 7), mantissa field m; e = 0 is subnormal
 * (m/8 * 2^(1-7)), e = 15 with m = 7 is NaN, anything else is normal
 * ((1 + m/8) * 2^(e-7)). */
static double e4m3_value(uint8_t x) {
  const int sign = x >> 7, e = (x >> 3) & 0xF, m = x & 0x7;
  if (e == 0xF && m == 0x7) return NAN;
  const double mag = e == 0 ? ldexp((double)m / 8.0, 1 - 7) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Widen element `idx` of an array of the given type to double. */
static double load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == ORACLE_F64) return ((const double*)base)[idx];
  if (dtype == ORACLE_E4M3) return e4m3_value(((const uint8_t*)base)[idx]);
  if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
  /* bf16: the stored half-word is the high half of a binary32. */
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Group of query head i (0-based), for R = H_Q / H_KV query heads per group.
 * Written as the page's 1-based g(i) = floor((i-1)/R) + 1, then moved back to
 * 0-based numbering. */
int64_t oracle_group_of(int64_t i, int64_t R) {
  int64_t i1 = i + 1;
  int64_t g1 = (i1 - 1) / R + 1;
  return g1 - 1;
}

/* Row index (in units of d elements) of token t of KV head h of sequence b.
 * Sequence b owns tokens [kv_offsets[b], kv_offsets[b+1]) of capacity per KV
 * head; its H_KV heads are stored one after another, each `cap` rows long.
 * The dense layout [B][H_KV][T_max][d] is kv_offsets[b] = b * T_max. */
static int64_t kv_row(const int64_t* kv_offsets, int64_t H_kv, int64_t b, int64_t h, int64_t t) {
  int64_t cap = kv_offsets[b + 1] - kv_offsets[b];
  return kv_offsets[b] * H_kv + h * cap + t;
}

/* Where the cache rows of a call live: the dense/packed layout of kv_row(),
 * or a paged one -- a pool of pages of `page` tokens, page p holding rows
 * (p * H_kv + h) * page + j for its token j of KV head h, and sequence b's
 * token t in page block_table[b * max_pages + t / page]. */
typedef struct {
  const int64_t* kv_offsets; /* dense/packed: [B+1]; NULL when paged */
  const int32_t* block_table;
  int64_t max_pages, page;
  int64_t H_kv;
} cache_layout;

static int64_t cache_row(const cache_layout* L, int64_t b, int64_t h, int64_t t) {
  if (L->block_table) {
    int64_t p = L->block_table[b * L->max_pages + t / L->page];
    return (p * L->H_kv + h) * L->page + t % L->page;
  }
  return kv_row(L->kv_offsets, L->H_kv, b, h, t);
}

static int64_t cache_capacity(const cache_layout* L, int64_t b) {
  return L->block_table ? L->max_pages * L->page : L->kv_offsets[b + 1] - L->kv_offsets[b];
}

/* A cached key or value array: element idx stands for scale * (its stored
 * value); scale is 1 for full-precision caches. */
typedef struct {
  const void* data;
  int dtype;
  double scale;
} kv_array;

static double kv_elem(const kv_array* a, int64_t idx) { return a->scale * load_elem(a->data, idx, a->dtype); }

/*
 * Attention weights and output of one query head.
 *   q, q_off : query array (elements of type dtype) and the element offset
 *              of Q_i's d elements
 *   K, V  : whole cache arrays, addressed through cache_row()
 *   w     : optional, receives the n softmax weights (may be NULL)
 *   out   : receives the d outputs
 *   s     : scratch of at least the sequence's capacity
 * Returns 0, or -1 when n is negative or exceeds the sequence's capacity.
 */
static int head_forward(const void* q, int64_t q_off, int dtype, const kv_array* K, const kv_array* V, int64_t d,
                        const cache_layout* L, int64_t b, int64_t g, int64_t n, double scale,
                        double* s /* scratch, n */, double* w, double* out) {
  int64_t cap = cache_capacity(L, b);
  if (n < 0 || n > cap) return -1;
  for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
  if (n == 0) return 0;

  /* Scores: s_t = scale * (Q_i . K_g,t), the masked-in positions only. */
  for (int64_t t = 0; t < n; ++t) {
    int64_t row = cache_row(L, b, g, t) * d;
    double acc = 0.0;
    for (int64_t c = 0; c < d; ++c) acc += load_elem(q, q_off + c, dtype) * kv_elem(K, row + c);
    s[t] = scale * acc;
  }
  /* softmax over t in [0, n). */
  double m = s[0];
  for (int64_t t = 1; t < n; ++t) if (s[t] > m) m = s[t];
  double z = 0.0;
  for (int64_t t = 0; t < n; ++t) z += exp(s[t] - m);
  /* Weighted sum of the group's value rows. */
  for (int64_t t = 0; t < n; ++t) {
    double wt = exp(s[t] - m) / z;
    if (w) w[t] = wt;
    int64_t row = cache_row(L, b, g, t) * d;
    for (int64_t c = 0; c < d; ++c) out[c] += wt * kv_elem(V, row + c);
  }
  return 0;
}

static int check_dims(int64_t B, int64_t H_q, int64_t H_kv, int64_t d, int dtype) {
  if (B < 0 || H_q <= 0 || H_kv <= 0 || d <= 0) return -1;
  if (H_q % H_kv != 0) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
  return 0;
}

/*
 * GQA decode outputs for a list of query heads.
 *   q          : [B][H_q][d]
 *   k, v       : cache, layout given by kv_offsets (see kv_row)
 *   kv_offsets : [B+1] token offsets (capacity prefix sums)
 *   seq_lens   : [B] valid cached tokens per sequence
 *   head_ids   : n_heads entries b*H_q + i, or NULL for all B*H_q heads in order
 *   out        : [n_heads][d] fp64
 * Returns 0 on success, -1 on invalid arguments (nothing is written then for
 * the offending head).
 */
static int decode_heads(int64_t B, int64_t H_q, int64_t H_kv, int64_t d, int dtype, const void* q, const kv_array* K,
                        const kv_array* V, const cache_layout* L, const int32_t* seq_lens, double scale,
                        int64_t n_heads, const int64_t* head_ids, double* out) {
  if (check_dims(B, H_q, H_kv, d, dtype)) return -1;
  if (!head_ids) n_heads = B * H_q;
  int64_t R = H_q / H_kv;
  int64_t max_cap = 0;
  for (int64_t b = 0; b < B; ++b) {
    int64_t cap = cache_capacity(L, b);
    if (cap < 0) return -1;
    if (cap > max_cap) max_cap = cap;
  }
  for (int64_t j = 0; j < n_heads; ++j) {
    int64_t id = head_ids ? head_ids[j] : j;
    if (id < 0 || id >= B * H_q) return -1;
  }
  int status = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_cap > 0 ? max_cap : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t j = 0; j < n_heads; ++j) {
      int64_t id = head_ids ? head_ids[j] : j;
      int64_t b = id / H_q, i = id % H_q;
      int64_t g = oracle_group_of(i, R);
      int rc = s ? head_forward(q, (b * H_q + i) * d, dtype, K, V, d, L, b, g,
                                (int64_t)seq_lens[b], scale, s, NULL, out + j * d)
                 : -1;
      if (rc) {
#pragma omp atomic write
        status = rc;
      }
    }
    free(s);
  }
  return status;
}

int oracle_gqa_decode(int64_t B, int64_t H_q, int64_t H_kv, int64_t d, int dtype,
                      const void* q, const void* k, const void* v,
                      const int64_t* kv_offsets, const int32_t* seq_lens, double scale,
                      int64_t n_heads, const int64_t* head_ids, double* out) {
  cache_layout L = {kv_offsets, NULL, 0, 0, H_kv};
  const kv_array K = {k, dtype, 1.0}, V = {v, dtype, 1.0};
  return decode_heads(B, H_q, H_kv, d, dtype, q, &K, &V, &L, seq_lens, scale, n_heads, head_ids, out);
}

/*
 * The same outputs for a cache of one-byte OCP E4M3 elements (see the file
 * header): k8, v8 in the dense/packed layout of kv_row(), each key element
 * standing for k_scale times its E4M3 value and each value element for
 * v_scale times its own.  q (and the outputs) as for oracle_gqa_decode.
 * Returns -1 also for a non-finite scale.
 */
int oracle_gqa_decode_fp8(int64_t B, int64_t H_q, int64_t H_kv, int64_t d, int dtype,
                          const void* q, const void* k8, const void* v8,
                          const int64_t* kv_offsets, const int32_t* seq_lens, double scale,
                          double k_scale, double v_scale, int64_t n_heads, const int64_t* head_ids, double* out) {
  if (!isfinite(k_scale) || !isfinite(v_scale)) return -1;
  cache_layout L = {kv_offsets, NULL, 0, 0, H_kv};
  const kv_array K = {k8, ORACLE_E4M3, k_scale}, V = {v8, ORACLE_E4M3, v_scale};
  return decode_heads(B, H_q, H_kv, d, dtype, q, &K, &V, &L, seq_lens, scale, n_heads, head_ids, out);
}

/* The E4M3 cache of oracle_gqa_decode_fp8 held in pages of a pool, as in
 * oracle_gqa_decode_paged. */
int oracle_gqa_decode_paged_fp8(int64_t B, int64_t H_q, int64_t H_kv, int64_t d, int dtype,
                                const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, int64_t max_pages, int64_t page,
                                const int32_t* seq_lens, double scale, double k_scale, double v_scale,
                                int64_t n_heads, const int64_t* head_ids, double* out) {
  if (!block_table || max_pages < 0 || page <= 0) return -1;
  if (!isfinite(k_scale) || !isfinite(v_scale)) return -1;
  cache_layout L = {NULL, block_table, max_pages, page, H_kv};
  const kv_array K = {k_pool, ORACLE_E4M3, k_scale}, V = {v_pool, ORACLE_E4M3, v_scale};
  return decode_heads(B, H_q, H_kv, d, dtype, q, &K, &V, &L, seq_lens, scale, n_heads, head_ids, out);
}

/* The OCP E4M3 byte of x: the nearest E4M3 value, ties to the even
 * mantissa, saturating at +-448 (a cached element stays finite; infinities
 * saturate too); NaN gives the NaN code 0x7F.  Written from the format's
 * definition: below 2^-6 the grid is m * 2^-9 (m = 0 .. 8, where m = 8 is the
 * smallest normal), above it (1 + m/8) * 2^e with e in [-6, 8]. */
static uint8_t e4m3_code(double x) {
  if (isnan(x)) return 0x7F;
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  const double a = fabs(x);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) return sign | (uint8_t)nearbyint(ldexp(a, 9));   /* m * 2^-9, m <= 8 */
  int e = (int)floor(log2(a));
  if (ldexp(1.0, e) > a) e -= 1;          /* guard the floor of log2 against rounding */
  if (ldexp(1.0, e + 1) <= a) e += 1;
  int m = (int)nearbyint((ldexp(a, -e) - 1.0) * 8.0);
  if (m == 8) {
    m = 0;
    e += 1;
  }
  return sign | (uint8_t)(((e + 7) << 3) | m);
}

/* The E4M3 bytes of n doubles (the encoder the quantising append follows). */
int oracle_e4m3_encode(int64_t n, const double* x, uint8_t* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = e4m3_code(x[j]);
  return 0;
}

/* The values of n OCP E4M3 bytes (the decoder the fp8 attention uses). */
int oracle_e4m3_decode(int64_t n, const uint8_t* codes, double* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = e4m3_value(codes[j]);
  return 0;
}

/*
 * The same outputs with the cache in pages: k_pool, v_pool hold pages of
 * `page` tokens (page p, KV head h, token j at row (p * H_kv + h) * page + j),
 * and sequence b's token t is in page block_table[b * max_pages + t / page]
 * (capacity max_pages * page tokens).  Page ids must be valid for the pool.
 */
int oracle_gqa_decode_paged(int64_t B, int64_t H_q, int64_t H_kv, int64_t d, int dtype,
                            const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, int64_t max_pages, int64_t page,
                            const int32_t* seq_lens, double scale, int64_t n_heads, const int64_t* head_ids,
                            double* out) {
  if (!block_table || max_pages < 0 || page <= 0) return -1;
  cache_layout L = {NULL, block_table, max_pages, page, H_kv};
  const kv_array K = {k_pool, dtype, 1.0}, V = {v_pool, dtype, 1.0};
  return decode_heads(B, H_q, H_kv, d, dtype, q, &K, &V, &L, seq_lens, scale, n_heads, head_ids, out);
}

/* Softmax weights of one query head (b, i): w[0..seq_lens[b]) and its output. */
int oracle_gqa_head_weights(int64_t B, int64_t H_q, int64_t H_kv, int64_t d, int dtype,
                            const void* q, const void* k, const void* v,
                            const int64_t* kv_offsets, const int32_t* seq_lens, double scale,
                            int64_t b, int64_t i, double* w, double* out) {
  if (check_dims(B, H_q, H_kv, d, dtype)) return -1;
  if (b < 0 || b >= B || i < 0 || i >= H_q) return -1;
  int64_t n = seq_lens[b];
  int64_t cap = kv_offsets[b + 1] - kv_offsets[b];
  if (n < 0 || n > cap) return -1;
  double* s = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
  if (!s) return -1;
  cache_layout L = {kv_offsets, NULL, 0, 0, H_kv};
  const kv_array K = {k, dtype, 1.0}, V = {v, dtype, 1.0};
  int rc = head_forward(q, (b * H_q + i) * d, dtype, &K, &V, d, &L, b,
                        oracle_group_of(i, H_q / H_kv), n, scale, s, w, out);
  free(s);
  return rc;
}

/*
 * Rotary position embedding of n vectors of d elements (d even):
 * "Grouped-Query Attention (GQA) and Multi-Query Attention (MQA): ...",
 * section 4, "Rotary Position Embeddings (RoPE) Interaction".  R_{Theta,m}
 * is block diagonal with one 2x2 rotation R_{theta_j,m} per pair of
 * consecutive elements, so elements 2j and 2j+1 (0-based) turn by the angle
 * m * theta_j.  The page leaves theta_j and the orientation open; read as
 * theta_j = base^(-2j/d) for j = 0 .. d/2-1 (base a parameter) and
 * R = [[cos, -sin], [sin, cos]] acting on the pair as a column vector.
 *   x   : n*d elements of the given dtype (vector v at x[v*d])
 *   pos : n positions m, one per vector
 *   out : n*d doubles
 * Returns 0, or -1 for an odd or non-positive d, or a non-positive base.
 */
int oracle_rope(int64_t n, int64_t d, int dtype, const void* x, const int64_t* pos, double base, double* out) {
  if (d <= 0 || d % 2 != 0 || !(base > 0.0)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t v = 0; v < n; ++v) {
    for (int64_t j = 0; j < d / 2; ++j) {
      const double theta = pow(base, -2.0 * (double)j / (double)d);
      const double a = (double)pos[v] * theta;
      const double c = cos(a), s = sin(a);
      const double x0 = load_elem(x, v * d + 2 * j, dtype), x1 = load_elem(x, v * d + 2 * j + 1, dtype);
      out[v * d + 2 * j] = x0 * c - x1 * s;
      out[v * d + 2 * j + 1] = x0 * s + x1 * c;
    }
  }
  return 0;
}

/* Threads the oracle's parallel loops use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
