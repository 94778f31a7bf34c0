// Shared device-side pieces of the GQA decode kernels (gfx950).
//
// Work decomposition.  A "unit" is one (layer, sequence b, KV head g); its
// G = H_q / H_kv query heads (i = g*G .. g*G+G-1, the contiguous grouping of
// "Grouped-Query Attention (GQA) and Multi-Query Attention (MQA): ...",
// section 2, g(i)) all read that one K/V head.  A unit's valid tokens
// [0, n_b) are cut into chunks of `chunk` tokens; one workgroup handles one
// (unit, chunk) and reads every K/V byte of its chunk exactly once, for all G
// heads.  Each workgroup ends with a running-softmax state per head: the
// maximum m of its scores (base-2 domain), the sum l of 2^(s - m) and the
// un-normalised sum O of 2^(s - m) * V.  A unit with one chunk writes
// O / l straight to the output.  Otherwise every chunk stores its state in the
// workspace and a second, small kernel launched behind the first on the same
// stream (the kernel boundary makes the states visible) combines them in
// chunk order, which keeps the result deterministic:
//   M = max_k m_k,  out = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k.
//
// The matrix-core path splits the work differently ("token split", below):
// all valid tokens of all units, in (layer, sequence, KV head, token) order,
// form one stream that is cut into equal spans, one per workgroup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxGroup = 64;    // largest G = H_q / H_kv supported
constexpr int kMaxBatch = 4096;  // sequences per call on the token-split path (prefix sums live in LDS)

struct Problem {
  const void* q;              // [L][B][H_q][D]
  const void* k;              // cache, dense or packed
  const void* v;
  void* out;                  // [L][B][H_q][D]
  const int64_t* kv_offsets;  // [B+1] or nullptr (dense)
  const int32_t* seq_lens;    // [B]
  float* ws_ml;               // partial states (m, l): chunk path [units][n_chunks][G][2],
                              //   token-split path [spans][2][G][2]
  float* ws_o;                // partial O: [units][n_chunks][G][D] or [spans][2][G][D]
  int64_t* ws_desc;           // token-split path: [spans][4] merge descriptors
  int32_t* ws_cnt;            // token-split path, fused merge: [spans] arrival counters (zero between calls)
  int32_t fused;              // token-split path: 1 = the last piece of a split unit to finish merges it
  int32_t B, H_q, H_kv, G, T_max, L;
  int32_t T_cap;              // planned bound on valid tokens (seq_len_hint, else T_max)
  int32_t chunk, n_chunks;    // chunk path: tokens per chunk, chunks of the longest sequence
  int32_t groups;             // token-split path: decode workgroups launched
  int32_t span;               // token-split path: positions per span (one per workgroup and layer; 0: balanced)
  int32_t dyn_chunks;         // token-split path, layer batches: chunks of the last layer claimed at run time (0: none)
  int32_t* ws_ticket;         // their arrival ticket (a counter of the workspace, zero between calls)
  int32_t out_bf16;
  float scale_log2;           // scale * log2(e): scores are kept in base 2
  const int32_t* block_table; // paged cache: [B][max_pages] page ids, or nullptr
  int32_t max_pages, page;    // paged cache: table entries per sequence, tokens per page (a multiple of 16)
  float out_mul;              // factor of every normalised output (the value scale of an E4M3 cache, else 1)
  // Decode with the append of the new token (one layer; plain, packed or
  // paged cache of bf16 or E4M3 elements): sequence b's token at position
  // m = max(seq_lens[b], 0) is turned
  // by the rotary embedding and written to cache row m (when m < capacity),
  // and the attention covers it.
  const void* k_new;          // [B][H_kv][D] keys before the rotation
  const void* v_new;          // [B][H_kv][D]
  void* q_out;                // [B][H_q][D] turned queries
  int32_t* new_seq_lens;      // [B] or nullptr
  double rope_base;
  // The fused append into an E4M3 cache: the new key (value) is stored as the
  // code of key / k_scale (value / v_scale).
  float k_scale, v_scale;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even float -> bfloat16 bits (IEEE definition; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// The OCP E4M3 byte of y, from the format's definition: |y| >= 448
// saturates; below 2^-6 the grid is m * 2^-9 (m = 0 .. 8, m = 8 being the
// smallest normal); above, three mantissa bits rounded to nearest even, a
// carry moving into the exponent; NaN is 0x7F.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7Fu;                 // NaN
  if (a >= 0x43e00000u) return sign | 0x7Eu;         // |y| >= 448 (and infinities)
  if (a < 0x3c800000u) return sign | (uint32_t)rintf(__uint_as_float(a) * 512.f);   // |y| < 2^-6
  const uint32_t e = (a >> 23) - 127u + 7u;          // biased E4M3 exponent, 1 .. 15
  const uint32_t m = a & 0x7fffffu;
  const uint32_t rem = m & 0xfffffu;
  const uint32_t q = (m >> 20) + ((rem > 0x80000u || (rem == 0x80000u && ((m >> 20) & 1u))) ? 1u : 0u);
  return sign | ((e << 3) + q);
}

// Rotary embedding ("Grouped-Query Attention (GQA) and Multi-Query
// Attention (MQA): ...", section 4): the cosine and sine of pair j's angle
// m * base^(-2j/D) (computed in double precision, as m * theta_j reaches
// 1e5 radians, then rounded to float), and the turn of the pair (x0, x1) by
// it.  The turn is written with explicit fused multiply-adds so that every
// kernel that uses it rounds alike.
__device__ __forceinline__ void rope_angle(double base, int64_t m, int j, int D, float& c, float& s) {
  const double a = (double)m * pow(base, -2.0 * (double)j / (double)D);
  double sd, cd;
  sincos(a, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}
__device__ __forceinline__ void rope_turn(float x0, float x1, float c, float s, float& y0, float& y1) {
  y0 = fmaf(x0, c, -(x1 * s));
  y1 = fmaf(x0, s, x1 * c);
}

struct UnitInfo {
  int64_t row0;   // first cache row (units of D elements) of this unit
  int32_t n;      // valid tokens
  int32_t l, b, g;
};

// Locate unit u = (l*B + b)*H_kv + g.  Dense: rows ((l*B+b)*H_kv+g)*T_max.
// Packed: l*off[B]*H_kv + off[b]*H_kv + g*cap_b with cap_b = off[b+1]-off[b].
__device__ __forceinline__ UnitInfo unit_info(const Problem& p, int unit) {
  UnitInfo ui;
  ui.g = unit % p.H_kv;
  int lb = unit / p.H_kv;
  ui.b = lb % p.B;
  ui.l = lb / p.B;
  int64_t cap;
  if (p.kv_offsets) {
    int64_t o0 = p.kv_offsets[ui.b], o1 = p.kv_offsets[ui.b + 1];
    cap = o1 - o0;
    ui.row0 = (int64_t)ui.l * p.kv_offsets[p.B] * p.H_kv + o0 * p.H_kv + (int64_t)ui.g * cap;
  } else {
    cap = p.T_max;
    ui.row0 = (int64_t)unit * p.T_max;
  }
  // Valid tokens, clamped into [0, min(capacity, planned bound)]: the split
  // plan (and the workspace sized from it) covers at most T_cap tokens.
  int64_t n = p.seq_lens[ui.b];
  if (cap > p.T_cap) cap = p.T_cap;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  ui.n = (int32_t)n;
  return ui;
}

__device__ __forceinline__ int chunks_of(int n, int chunk) { return n <= 0 ? 1 : (n + chunk - 1) / chunk; }

__device__ __forceinline__ int64_t out_row0(const Problem& p, const UnitInfo& ui) {
  return (int64_t)(ui.l * p.B + ui.b) * p.H_q + (int64_t)ui.g * p.G;
}

// Final store of one output element (row = global query-head row, c = column).
__device__ __forceinline__ void store_out(const Problem& p, int64_t row, int c, int D, float val) {
  if (p.out_bf16)
    reinterpret_cast<uint16_t*>(p.out)[row * D + c] = (uint16_t)f32_to_bf16_rne(val);
  else
    reinterpret_cast<float*>(p.out)[row * D + c] = val;
}

// Combine the chunk states of every unit that needed more than one chunk.
// One workgroup of 256 threads per (unit, 256/D heads); thread -> (head, column).
template <int D>
__global__ __launch_bounds__(256) void gqa_merge_chunks(Problem p) {
  constexpr int HPB = 256 / D;   // heads per workgroup
  const int groups = (p.G + HPB - 1) / HPB;
  const int unit = blockIdx.x / groups;
  const int h = (blockIdx.x % groups) * HPB + threadIdx.x / D;
  const int c = threadIdx.x % D;
  const UnitInfo ui = unit_info(p, unit);
  const int nck = chunks_of(ui.n, p.chunk);
  if (nck == 1 || h >= p.G) return;   // single-chunk units were finished by the decode kernel
  const float* ml = p.ws_ml + (int64_t)unit * p.n_chunks * p.G * 2 + 2 * h;
  const float* o = p.ws_o + ((int64_t)unit * p.n_chunks * p.G + h) * D + c;
  const int64_t sml = (int64_t)p.G * 2, so = (int64_t)p.G * D;
  // One pass in chunk order, rescaling the running sums whenever the maximum
  // grows; the loads of a chunk do not depend on earlier chunks, so they can
  // all be in flight together.
  float M = -INFINITY, num = 0.f, den = 0.f;
#pragma unroll 4
  for (int k = 0; k < nck; ++k) {
    const float mk = ml[k * sml], lk = ml[k * sml + 1], ok = o[k * so];
    const float Mn = fmaxf(M, mk);
    const float a = exp2f(M - Mn), f = exp2f(mk - Mn);   // M = -inf on the first chunk: a = 0
    num = num * a + f * ok;
    den = den * a + f * lk;
    M = Mn;
  }
  store_out(p, out_row0(p, ui) + h, c, D, den > 0.f ? num / den : 0.f);
}

// ---------------------------------------------------------------------------
// Token split.  Sequence b contributes n_b valid tokens to each of its H_kv
// units per layer; with P the exclusive prefix sums of n_b, the stream
// position of token t of unit (l, b, g) is
//     l * H_kv * P[B]  +  H_kv * P[b]  +  g * n_b  +  t.
// Each layer's positions are cut into spans of `span` positions, numbered
// v = l * groups + w ("virtual spans"): span v covers
//     [l * per_layer + w * span, min(l * per_layer + (w + 1) * span, (l + 1) * per_layer)),
// and workgroup w takes spans w, groups + w, 2 groups + w, ... in turn, one
// layer after the other, so that at any time the workgroups stream the same
// layer.  A layer batch (L >= 2) under the balanced split instead cuts its
// last layer into `dyn` chunks of `dspan` positions (spans
// v = (L - 1) * groups + c), which the workgroups claim one at a time from an
// arrival ticket once their static spans are done: workgroups that streamed
// faster take more of the last layer, and all end close together.  Every
// unit that lies inside one span is finished there; only the first and the
// last unit piece of a span can be partial (state slots 2v and 2v + 1; a
// piece covering a whole span uses slot 2v).  A unit never crosses a layer,
// so the spans holding its pieces are consecutive.  A span's pieces depend
// only on its bounds, whichever workgroup streams it.

// Exclusive prefix sums of the units' stream lengths into sm_P[0..B] (all
// threads of the workgroup take part; B <= kMaxBatch).  A unit's stream
// length is its valid token count; for a paged cache (PAGED) it is rounded up
// to a multiple of 16, so that every 16-token tile of a unit starts at a
// multiple of 16 and lies in one page, and the clamped counts go to
// sm_N[0..B).  sm_wave holds NT/64 ints.
// APPEND: sm_M[b] receives the new token's position m and the length counts
// it when the cache has room (m < capacity).
template <int NT, bool PAGED, bool APPEND = false>
__device__ __forceinline__ void build_prefix(const Problem& p, int32_t* sm_P, int32_t* sm_N, int32_t* sm_wave,
                                             int32_t* sm_M = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = p.B;
  const int E = (B + NT - 1) / NT;   // entries per thread, contiguous
  const int b0 = tid * E;
  int local = 0;
  for (int b = b0; b < b0 + E && b < B; ++b) {
    int64_t cap = p.kv_offsets ? p.kv_offsets[b + 1] - p.kv_offsets[b] : (int64_t)p.T_max;
    int64_t n = p.seq_lens[b];
    if constexpr (APPEND) {
      n = n < 0 ? 0 : n;
      sm_M[b] = (int32_t)n;
      n = n < cap ? n + 1 : cap;
    }
    if (cap > p.T_cap) cap = p.T_cap;
    n = n < 0 ? 0 : (n > cap ? cap : n);
    if constexpr (PAGED) {
      sm_N[b] = (int32_t)n;
      n = (n + 15) / 16 * 16;
    }
    sm_P[b] = (int32_t)n;
    local += (int32_t)n;
  }
  int v = local;   // inclusive scan of the per-thread totals within the wavefront
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) sm_wave[wave] = v;
  __syncthreads();
  int run = v - local;
  for (int w = 0; w < wave; ++w) run += sm_wave[w];
  for (int b = b0; b < b0 + E && b < B; ++b) {
    const int n = sm_P[b];
    sm_P[b] = run;
    run += n;
  }
  if (b0 < B && b0 + E >= B) sm_P[B] = run;   // the thread holding the last entry writes the total
  __syncthreads();
}

// Values every lane of a wavefront holds alike (read back from LDS, so the
// compiler cannot tell) moved to scalar registers.
__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// CLAIMS: the kernel instance of layer batches whose last layer is claimed
// in chunks (the other instances compile none of that).
template <bool CLAIMS>
struct TokenSpaceT {
  int64_t per_layer;   // H_kv * P[B]
  int64_t total;       // L * per_layer
  int64_t span;        // positions per static span of a layer, a multiple of 16
  int64_t groups;      // static spans per layer (the workgroups launched)
  int64_t sl;          // layers cut into static spans: L, or L - 1 with a claimed last layer
  int64_t dyn;         // CLAIMS: chunks of the claimed last layer (0: none)
  int64_t dspan;       // CLAIMS: positions per chunk of the claimed last layer, a multiple of 16

  // first position of span v, one past its last (a chunk past the layer's
  // last position is empty), and the span holding position x
  __device__ __forceinline__ int64_t start(int64_t v) const {
    if constexpr (CLAIMS) {
      if (v >= sl * groups) return sl * per_layer + (v - sl * groups) * dspan;
    }
    const int64_t l = v / groups;
    return l * per_layer + (v - l * groups) * span;
  }
  __device__ __forceinline__ int64_t end(int64_t v) const {
    if constexpr (CLAIMS) {
      if (v >= sl * groups) return min(start(v) + dspan, (sl + 1) * per_layer);
    }
    const int64_t l = v / groups;
    return min(start(v) + span, (l + 1) * per_layer);
  }
  __device__ __forceinline__ int64_t span_of(int64_t x) const {
    const int64_t l = x / per_layer;
    if constexpr (CLAIMS) {
      if (l >= sl) return sl * groups + (x - sl * per_layer) / dspan;
    }
    return l * groups + (x - l * per_layer) / span;
  }
};

template <bool CLAIMS>
__device__ __forceinline__ TokenSpaceT<CLAIMS> token_space(const Problem& p, const int32_t* sm_P) {
  TokenSpaceT<CLAIMS> ts;
  ts.per_layer = (int64_t)p.H_kv * uniform(sm_P[p.B]);
  ts.total = ts.per_layer * p.L;
  ts.groups = p.groups;
  if (p.span > 0) {
    ts.span = p.span;
  } else {
    const int64_t s = (ts.per_layer + p.groups - 1) / p.groups;
    ts.span = (s + 15) / 16 * 16;
    if (ts.span == 0) ts.span = 16;
  }
  ts.dyn = CLAIMS ? p.dyn_chunks : 0;
  ts.sl = ts.dyn > 0 ? p.L - 1 : p.L;
  ts.dspan = 16;
  if (ts.dyn > 0) {
    const int64_t s = (ts.per_layer + ts.dyn - 1) / ts.dyn;
    ts.dspan = s > 16 ? (s + 15) / 16 * 16 : 16;
  }
  return ts;
}

struct Piece {
  UnitInfo ui;     // row0, n (valid tokens), l, b, g of the unit holding the position
  int64_t start;   // stream position of the unit's token 0
  int t;           // token of the unit at the located position
  int npad;        // stream positions of the unit (n, rounded up to 16 for a paged cache)
};

// The piece of unit (l, b, g) that starts at its token t, at stream
// position start + t.
template <bool PAGED>
__device__ __forceinline__ Piece fill_piece(const Problem& p, const int32_t* sm_P, const int32_t* sm_N, int l, int b,
                                            int g, int t, int64_t start) {
  Piece pc;
  const int v = uniform(sm_P[b + 1]) - uniform(sm_P[b]);   // stream positions of each unit of sequence b
  pc.t = t;
  pc.start = start;
  pc.npad = v;
  pc.ui.l = l;
  pc.ui.b = b;
  pc.ui.g = g;
  if constexpr (PAGED) {
    pc.ui.n = uniform(sm_N[b]);
    pc.ui.row0 = (int64_t)g * p.page;   // KV head g's rows of a page (the page comes per tile)
    return pc;
  }
  pc.ui.n = v;
  if (p.kv_offsets) {
    const int64_t o0 = p.kv_offsets[b], cap = p.kv_offsets[b + 1] - o0;
    pc.ui.row0 = (int64_t)l * p.kv_offsets[p.B] * p.H_kv + o0 * p.H_kv + (int64_t)g * cap;
  } else {
    pc.ui.row0 = ((int64_t)(l * p.B + b) * p.H_kv + g) * p.T_max;
  }
  return pc;
}

// The unit holding stream position x (0 <= x < total): a binary search over
// the prefix sums.
template <bool PAGED, typename TS>
__device__ __forceinline__ Piece locate(const Problem& p, const int32_t* sm_P, const int32_t* sm_N, const TS& ts,
                                        int64_t x) {
  const int l = (int)(x / ts.per_layer);
  const int64_t r = x - (int64_t)l * ts.per_layer;
  int lo = 0, hi = p.B - 1;   // largest b with H_kv * P[b] <= r (such b holds tokens)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)p.H_kv * uniform(sm_P[mid]) <= r) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int32_t pb = uniform(sm_P[b]);
  const int v = uniform(sm_P[b + 1]) - pb;
  const int64_t r2 = r - (int64_t)p.H_kv * pb;
  const int g = (int)(r2 / v);
  const int t = (int)(r2 - (int64_t)g * v);
  return fill_piece<PAGED>(p, sm_P, sm_N, l, b, g, t, x - t);
}

// The unit after pc's in the stream, from its token 0 (the caller knows one
// exists): the next KV head of the same sequence, else the next sequence
// with tokens, else the first such sequence of the next layer.  No division
// and no search: a piece boundary costs a few LDS reads.
template <bool PAGED>
__device__ __forceinline__ Piece next_unit(const Problem& p, const int32_t* sm_P, const int32_t* sm_N,
                                           const Piece& pc) {
  int l = pc.ui.l, b = pc.ui.b, g = pc.ui.g + 1;
  if (g == p.H_kv) {
    g = 0;
    for (int k = 0; k < p.L * p.B; ++k) {   // sequences without tokens hold no stream positions
      if (++b == p.B) {
        b = 0;
        ++l;
      }
      if (uniform(sm_P[b + 1]) != uniform(sm_P[b])) break;
    }
  }
  return fill_piece<PAGED>(p, sm_P, sm_N, l, b, g, 0, pc.start + pc.npad);
}

// Zero the outputs of sequences with no valid token (every layer), spread
// over the workgroups of a launch.
template <int D, int NT>
__device__ __forceinline__ void zero_empty_sequences(const Problem& p, const int32_t* sm_P, int wg, int n_wg) {
  for (int lb = wg; lb < p.L * p.B; lb += n_wg) {
    const int b = lb % p.B;
    if (sm_P[b + 1] != sm_P[b]) continue;
    const int64_t row = (int64_t)lb * p.H_q;
    for (int e = threadIdx.x; e < p.H_q * D; e += NT) store_out(p, row + e / D, e % D, D, 0.f);
  }
}

// The fused append's outputs that no decode piece writes (one layer):
// new_seq_lens (workgroup 0; the length grows by the appended token, a full
// cache keeps the length given), and the turned queries of sequences without
// any token to attend to (spread over the workgroups).
template <int D, int NT>
__device__ __forceinline__ void append_side_outputs(const Problem& p, const int32_t* sm_P, const int32_t* sm_M,
                                                    int wg, int n_wg) {
  if (wg == 0 && p.new_seq_lens) {
    for (int b = threadIdx.x; b < p.B; b += NT) {
      const int64_t cap = p.kv_offsets ? p.kv_offsets[b + 1] - p.kv_offsets[b] : (int64_t)p.T_max;
      const int32_t m = sm_M[b];
      p.new_seq_lens[b] = m < cap ? m + 1 : p.seq_lens[b];
    }
  }
  for (int b = wg; b < p.B; b += n_wg) {
    if (sm_P[b + 1] != sm_P[b]) continue;
    const int64_t row = (int64_t)b * p.H_q;
    for (int e = threadIdx.x; e < p.H_q * (D / 2); e += NT) {
      const int h = e / (D / 2), j = e % (D / 2);
      float c, s, y0, y1;
      rope_angle(p.rope_base, sm_M[b], j, D, c, s);
      const uint16_t* qi = static_cast<const uint16_t*>(p.q) + (row + h) * D + 2 * j;
      rope_turn(bf16_to_f32(qi[0]), bf16_to_f32(qi[1]), c, s, y0, y1);
      uint16_t* qo = static_cast<uint16_t*>(p.q_out) + (row + h) * D + 2 * j;
      qo[0] = (uint16_t)f32_to_bf16_rne(y0);
      qo[1] = (uint16_t)f32_to_bf16_rne(y1);
    }
  }
}

// Agent-coherent accesses to one state slot of the workspace: buffer
// instructions with the sc1 cache policy (stores write through the XCD's L2
// to memory, loads miss in it), the policy agent-scope atomic accesses get on
// gfx950.  The fused merge moves partial states between workgroups through
// these: they are coherent across the XCDs' separate L2 caches without the L2
// write-back and invalidate that an agent-scope release/acquire fence would
// cost.  The buffer descriptor covers the slot only (offsets are 32-bit;
// accesses beyond it would be dropped by the hardware range check).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kPolicySc1 = 16;                 // cache-policy operand of the buffer builtins: sc1
constexpr int kRsrcWord3 = 0x00020000;         // raw 32-bit buffer, no swizzle, no stride
__device__ __forceinline__ Rsrc slot_rsrc(const float* base, int floats) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, floats * 4, kRsrcWord3);
}
__device__ __forceinline__ void store4_coherent(Rsrc r, int idx, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, idx * 4, 0, kPolicySc1);
}
__device__ __forceinline__ void store2_coherent(Rsrc r, int idx, float a, float b) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{a, b}), r, idx * 4, 0, kPolicySc1);
}
__device__ __forceinline__ f32x4 load4_coherent(Rsrc r, int idx) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, idx * 4, 0, kPolicySc1));
}
__device__ __forceinline__ f32x2 load2_coherent(Rsrc r, int idx) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, idx * 4, 0, kPolicySc1));
}

// Partial merge state of output columns c .. c+3 of one head: the running
// maximum M, the denominator sum_k 2^(m_k - M) l_k and the numerator
// sum_k 2^(m_k - M) O_k.  Empty: M = -inf, den = 0, num = 0.
struct MergeAcc {
  float M, den;
  f32x4 num;
};
// Two partial states combined (commutative: a + b and b + a round alike, so
// both lanes of a butterfly obtain the same bits).
__device__ __forceinline__ MergeAcc merge_combine(const MergeAcc& x, const MergeAcc& y) {
  MergeAcc r;
  r.M = fmaxf(x.M, y.M);
  const float a = x.M == -INFINITY ? 0.f : exp2f(x.M - r.M);
  const float b = y.M == -INFINITY ? 0.f : exp2f(y.M - r.M);
  r.den = x.den * a + y.den * b;
  r.num = x.num * a + y.num * b;
  return r;
}
// The normalised output of a complete state (0 when no token contributed).
__device__ __forceinline__ f32x4 merge_finish(const Problem& p, const MergeAcc& s) {
  const float inv = s.den > 0.f ? p.out_mul / s.den : 0.f;
  return s.num * inv;
}

// Merge state of output columns c .. c+3 (c a multiple of 4) of head hd of a
// split unit over the pieces of spans w_first, w_first + stride, ... up to
// w_last (span w0's piece is in slot first_slot, span w's in slot 2w), in
// that order:
//   M = max_k m_k,  out = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k,
// with a running maximum.  The loads of kMergeBatch pieces are issued
// together (indices past the last piece are clamped to an in-bounds piece and
// their values unused).  COHERENT: the pieces were published with the sc1
// stores above.
constexpr int kMergeBatch = 8;
template <bool COHERENT>
__device__ __forceinline__ MergeAcc merge_pieces(const Problem& p, int64_t w0, int64_t w_first, int64_t w_last,
                                                 int stride, int64_t first_slot, int hd, int c, int D) {
  const int G = p.G;
  MergeAcc acc{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int64_t wb = w_first; wb <= w_last; wb += (int64_t)kMergeBatch * stride) {
    f32x2 ml[kMergeBatch];
    f32x4 ok[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int64_t w = min(wb + (int64_t)u * stride, w_last);
      const int64_t slot = w == w0 ? first_slot : 2 * w;
      if (COHERENT) {
        ml[u] = load2_coherent(slot_rsrc(p.ws_ml + slot * G * 2, G * 2), 2 * hd);
        ok[u] = load4_coherent(slot_rsrc(p.ws_o + slot * G * D, G * D), hd * D + c);
      } else {
        ml[u] = *reinterpret_cast<const f32x2*>(p.ws_ml + (slot * G + hd) * 2);
        ok[u] = *reinterpret_cast<const f32x4*>(p.ws_o + (slot * G + hd) * D + c);
      }
    }
    // A clamped index is a no-op (a = 1, f = 0) taken by selects, not a
    // branch: a branch would let the compiler sink each load to its use.
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const bool real = wb + (int64_t)u * stride <= w_last;
      const float Mn = real ? fmaxf(acc.M, ml[u][0]) : acc.M;
      const float a = real ? exp2f(acc.M - Mn) : 1.f;   // M = -inf on the first piece: a = 0
      const float f = real ? exp2f(ml[u][0] - Mn) : 0.f;
      acc.num = acc.num * a + f * ok[u];
      acc.den = acc.den * a + f * ml[u][1];
      acc.M = Mn;
    }
  }
  return acc;
}

// Final store of four consecutive output columns.
__device__ __forceinline__ void store_out4(const Problem& p, int64_t row, int c, int D, f32x4 v) {
  if (p.out_bf16) {
    const uint32_t w0 = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
    const uint32_t w1 = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + row * D + c) = u32x2{w0, w1};
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + row * D + c) = v;
  }
}

// Fused merge of a split unit, run by every thread of the workgroup that just
// published one piece of it with the sc1 stores (from wavefront 0).  Thread 0
// waits until those stores have completed, then counts the piece in the
// unit's arrival counter (indexed by w0, the span holding the unit's first
// token; agent-scope atomic).  The workgroup that brings the count to
// the number of pieces reads every piece back with sc1 loads, in piece
// order (deterministic), writes the output and resets the counter to zero
// for the next call.  Pieces: w0's slot first_slot, then slot 2w of every
// later span w <= w_last.
template <int D, int NT>
__device__ __forceinline__ void fused_merge(const Problem& p, int64_t w0, int64_t w_last, int64_t first_slot, int64_t orow,
                            int* sm_flag) {
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);   // the publishing stores (this wavefront's) have completed
    const int prev = __hip_atomic_fetch_add(p.ws_cnt + w0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sm_flag = prev == (int)(w_last - w0);
  }
  __syncthreads();
  const bool last = *sm_flag;
  __syncthreads();   // sm_flag is reused by the next piece
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const int G = p.G;
  // four columns per thread
  const int nq = G * D / 4;
  for (int q = threadIdx.x; q < nq; q += NT)
    store_out4(p, orow + 4 * q / D, 4 * q % D, D,
               merge_finish(p, merge_pieces<true>(p, w0, w0, w_last, 1, first_slot, 4 * q / D, 4 * q % D, D)));
  if (threadIdx.x == 0) __hip_atomic_store(p.ws_cnt + w0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge descriptor of span m for the merge kernel, written by the decode
// workgroup that streams span m (threads 0..3):
//   {w0, w_last, output row of the unit's first head, first piece slot}
// when span m starts inside a unit that began in an earlier span (w0 < m is
// the span holding the unit's first token, w_last the one holding its last),
// else w0 = -1.  The spans w0+1 .. w_last of such a unit share its merge.
__device__ __forceinline__ void write_merge_desc(const Problem& p, int64_t m, int64_t w0, int64_t w_last,
                                                 int64_t orow, int64_t first_slot) {
  const int i = threadIdx.x;
  if (i < 4) p.ws_desc[4 * m + i] = i == 0 ? w0 : (i == 1 ? w_last : (i == 2 ? orow : first_slot));
}

// Merge of the token-split path: one workgroup of 256 threads per span m
// (every span of every layer).  The H = w_last - w0 spans w0+1 .. w_last of
// a split unit share its merge: helper h = m - w0 - 1 combines a contiguous
// block of the unit's output quads (four columns of one head), one quad per
// thread.
template <int D>
__global__ __launch_bounds__(256) void gqa_merge_spans(Problem p) {
  constexpr int NT = 256;
  const int m = blockIdx.x;
  const int64_t* dsc = p.ws_desc + 4 * (int64_t)m;
  const int64_t w0 = uniform(dsc[0]);
  if (w0 < 0) return;
  const int64_t w_last = uniform(dsc[1]), orow = uniform(dsc[2]), first_slot = uniform(dsc[3]);
  const int nq = p.G * D / 4;
  const int H = (int)(w_last - w0), h = (int)(m - w0 - 1);
  const int per = (nq + H - 1) / H;
  const int q0 = h * per, q1 = min(nq, (h + 1) * per);
  // S lanes (adjacent, a power of two up to 16) share each group of four
  // columns: lane k of the S merges pieces w0 + k, w0 + k + S, ..., then a
  // butterfly over the S lanes combines their states, so a unit of many
  // pieces needs few dependent load rounds per lane.
  int S = 1;
  while (S < 16 && 2 * S * (q1 - q0) <= NT) S *= 2;
  const int sub = (int)threadIdx.x % S;
  const int groups = NT / S;
  for (int qb = q0; qb < q1; qb += groups) {   // uniform trip count: every lane reaches the shuffles
    const int q = min(qb + (int)threadIdx.x / S, q1 - 1);
    MergeAcc acc = merge_pieces<false>(p, w0, w0 + sub, w_last, S, first_slot, 4 * q / D, 4 * q % D, D);
    for (int o = 1; o < S; o *= 2) {
      MergeAcc y;
      y.M = __shfl_xor(acc.M, o);
      y.den = __shfl_xor(acc.den, o);
#pragma unroll
      for (int e = 0; e < 4; ++e) y.num[e] = __shfl_xor(acc.num[e], o);
      acc = merge_combine(acc, y);
    }
    if (sub == 0 && qb + (int)threadIdx.x / S < q1) store_out4(p, orow + 4 * q / D, 4 * q % D, D, merge_finish(p, acc));
  }
}

}  // namespace gqa
