// Matrix-core GQA decode kernel for bf16 queries, D = 64 or 128,
// G <= 16*HB*HG; caches of bf16 elements (dense, packed or paged) or of
// one-byte E4M3 elements (dense or paged), which are widened to bf16 exactly
// before the products.
//
// Work split ("token split", see common.h): the valid tokens of each layer's
// units form one stream cut into equal spans, one per workgroup (one per CU),
// so every workgroup streams the same number of bytes whatever the sequence
// lengths; in a layer batch a workgroup takes its span of each layer in turn
// (and, when the batch's last layer is claimed, chunks of that layer from a
// ticket once its spans are done).  A workgroup walks a span unit piece by
// unit piece.  Its
// wavefronts each serve HB blocks of 16 heads (one block for up to 16 heads,
// two beyond) and are laid out as (head group, tile lane): up to 32 heads all
// four wavefronts are tile lanes of one group, 33..64 heads use two groups
// of two lanes.  For each piece, lane l
// streams the 16-token tiles l, l+NL, l+2NL, ... straight from HBM into
// registers (the lanes sweep adjacent memory together), and every K/V byte
// leaves HBM once for all G query heads of the group.  Each wavefront holds
// two batches of TPW tiles in registers: it computes one while the next one
// (of the same piece, or the first batch of the span's next piece) is
// loading, so the stream does not stop at piece boundaries, where the
// wavefronts combine their softmax states.
//
// Scores: S^T[token][head] = K Q^T on v_mfma_f32_16x16x32_bf16, with
//   A = 16 key rows x 32 columns (lane (m = lane%16, q4 = lane/16) holds 8
//       consecutive bf16 of row m: one 16-byte load), B = the group's queries
//       (16 heads per block).
// The result leaves lane (q4, n) holding the scores of head n for tokens
// 4*q4 .. 4*q4+3: exactly the B operand the P.V product needs from that lane,
// so the softmax weights never move between lanes.
//
// P.V: O^T[col][head] += V^T P^T, A = V^T.  Lane (m, q4) holds rows
// 4*q4 .. 4*q4+3 of the tile, D/16 consecutive columns each (16 lanes cover a
// row, so each load instruction reads 4 complete rows); column r of that run
// becomes the A operand of column block r after a half-word repack (block r
// holds columns D/16*m + r).
//
// Softmax weights enter the bf16 product as a two-term split p = hi + lo
// (hi = bf16(p), lo = bf16(p - hi)), so their rounding error stays near
// 2^-17 of p instead of 2^-9; the normaliser l sums the fp32 p.  Both terms
// go through one v_mfma_f32_16x16x32_bf16: its 32-long reduction runs over
// the 16 tokens twice, the lane's four tokens with their hi weights and then
// the same four with their lo weights (A repeats the lane's V values), so the
// split costs no second product.  The running
// maximum is only moved (and O, l rescaled) on tiles where it grows for some
// head of the wavefront; otherwise the rescale factor would be exactly 1.
#pragma once

#include <type_traits>

#include "common.h"

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int D>
struct VRow;   // the per-lane slice of one V row: D/16 bf16
template <>
struct VRow<128> {
  typedef u32x4 type;
};
template <>
struct VRow<64> {
  typedef u32x2 type;
};

// D(16x16) += A(16x32) B(32x16), bf16 inputs, fp32 accumulate.
__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Two weights as packed bf16 pairs hi = bf16(p), lo = bf16(p - hi).
__device__ __forceinline__ void split_weights(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(p0, p1);
  lo = pack_bf16x2(p0 - __uint_as_float(hi << 16), p1 - __uint_as_float(hi & 0xffff0000u));
}

// How far (in base-2 exponent) a score may exceed the running reference
// before O and l are rescaled to a new one.
constexpr float kRescaleSlack = 8.f;

// 2^x on the hardware instruction alone (v_exp_f32, 1 ulp).  Results below
// 2^-126 come out as 0 instead of subnormals: a softmax weight that small,
// next to the weight 1 of the running maximum, is below every rounding of
// the sums it enters.  2^-inf = 0.
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of x over the four lanes m, m + 16, m + 32, m + 48 (the lanes of
// one row index m in the wavefront's four 16-lane rows), in every one of
// them.  Two lane swaps on the vector ALU: rows 0/1 and 2/3, then the two
// halves.  Each swap of a value with itself leaves the row's partner value
// in one result and its own in the other.
__device__ __forceinline__ float max_over_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum of x over the same four lanes, in every one of them (rows 0 + 1 and
// 2 + 3 first, then the two halves: every lane adds in the same order).
__device__ __forceinline__ float sum_over_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Low (hi = false) or high halves of two words, packed: {x0.half, x1.half}.
template <bool HI>
__device__ __forceinline__ uint32_t pack_halves(uint32_t x0, uint32_t x1) {
  return __builtin_amdgcn_perm(x1, x0, HI ? 0x07060302u : 0x05040100u);
}

template <int D>
struct Tile16 {
  static constexpr int KS = D / 32;
  u32x4 k[KS];                   // A operands of the score product (row m16)
  typename VRow<D>::type v[4];   // V rows 4*q4 + i, columns D/16*m16 ..
};

// A tile of one-byte E4M3 elements as loaded: lane (q4, m16) holds bytes
// 64*h + 16*q4 .. +15 of K row m16 for h < D/64 (the A operands of every
// score step, see load_q: each load instruction reads 64 contiguous bytes of
// 16 rows) and bytes D/16*m16 .. of V rows 4*q4 + i.
template <int D>
struct Tile16F8 {
  u32x4 k[D / 64];
  typename std::conditional<D == 128, u32x2, uint32_t>::type v[4];
};

// Two E4M3 bytes (the low or the high half-word of w) to two bf16.  Every
// E4M3 value is a bf16 value, so the conversion (scale 1) is exact.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4{e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0), e4m3x2_to_bf16x2<false>(w1),
               e4m3x2_to_bf16x2<true>(w1)};
}
// An E4M3 tile with its keys widened to bf16 (the score product's A
// operands); the values stay bytes until they become P.V operands.
template <int D>
struct Tile16K8 {
  u32x4 k[D / 32];
  typename std::conditional<D == 128, u32x2, uint32_t>::type v[4];
};
template <int D>
__device__ __forceinline__ Tile16K8<D> widen(const Tile16F8<D>& t) {
  Tile16K8<D> w;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) w.k[s] = e4m3x8_to_bf16x8(t.k[s / 2][2 * (s % 2)], t.k[s / 2][2 * (s % 2) + 1]);
#pragma unroll
  for (int i = 0; i < 4; ++i) w.v[i] = t.v[i];
  return w;
}

// A operand of P.V column block r (the lane's V rows 4*q4 .. 4*q4+3 at column
// D/16*m + r, as two bf16 pairs).  bf16 tiles: a half-word repack of two row
// slices per pair.  E4M3 tiles: one byte permutation gathers rows (0, 1) (or
// (2, 3)) of columns r and r + 1 (r even) and one conversion widens the pair
// of column r or of column r + 1, so the permutation serves two blocks.
template <int D>
__device__ __forceinline__ u32x2 v_operand(const Tile16<D>& T, int r) {
  const int w = r >> 1;
  if (r & 1) return u32x2{pack_halves<true>(T.v[0][w], T.v[1][w]), pack_halves<true>(T.v[2][w], T.v[3][w])};
  return u32x2{pack_halves<false>(T.v[0][w], T.v[1][w]), pack_halves<false>(T.v[2][w], T.v[3][w])};
}
template <int D>
__device__ __forceinline__ u32x2 v_operand(const Tile16K8<D>& T, int r) {
  const int k = r & 3;   // byte of the row word holding column r
  const uint32_t sel = (k & 2) ? 0x07030602u : 0x05010400u;   // {x0.b, x1.b, x0.b+1, x1.b+1}, b = k & ~1
  uint32_t x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (D == 128)
      x[i] = T.v[i][r >> 2];
    else
      x[i] = T.v[i];
  }
  const uint32_t p01 = __builtin_amdgcn_perm(x[1], x[0], sel), p23 = __builtin_amdgcn_perm(x[3], x[2], sel);
  if (k & 1) return u32x2{e4m3x2_to_bf16x2<true>(p01), e4m3x2_to_bf16x2<true>(p23)};
  return u32x2{e4m3x2_to_bf16x2<false>(p01), e4m3x2_to_bf16x2<false>(p23)};
}

// Heads: each wavefront serves HB blocks of 16 query heads; the wavefronts
// form HG groups (wavefront w is in group w % HG and streams tile lane w / HG
// of the NW / HG lanes), so the workgroup covers 16 * HB * HG heads.  With
// HG > 1 a tile is read once per group; the repeats are served by the caches.
// PAGED: the cache is held in pages of a pool (p.block_table); every tile
// then lies in one page, whose id is fetched one batch ahead of the tile's
// loads so that the loads never wait for the table.
// KV8: cache elements are one-byte E4M3 values (bf16 queries).  Tiles move
// as bytes and are widened to bf16, exactly, just before the products; the
// key scale is folded into p.scale_log2 and the value scale into p.out_mul.
// APPEND (cache of bf16 or E4M3 elements: plain, packed or paged): the
// decode step fused with the append of each sequence's new token.  The
// token's position m comes from seq_lens[b]; the queries are turned by the
// rotary embedding in registers when a piece becomes current (and written
// to q_out by the unit's first piece), and the attention covers the new
// token: the piece that ends a grown unit turns the new key, its tile
// holding row m takes the turned key and the value instead of the cache's
// row, and wavefront 0 writes them to cache row m.  With KV8 the new row is
// what the quantising append stores: the key turned in fp32 and divided by
// k_scale, the value divided by v_scale, each encoded to E4M3 bytes; the
// tile takes those bytes before it is widened.
template <int D, int HB, int HG, int NW, int TPW, bool PAGED, bool KV8, bool APPEND = false, bool CLAIMS = false>
__global__ __launch_bounds__(NW * 64) void gqa_decode_mfma(Problem p) {
  static_assert(NW % HG == 0, "head groups must divide the wavefronts");
  // CLAIMS: the instance for layer batches whose last layer is claimed in
  // chunks (layer batches are neither paged nor fused with the append; two
  // head blocks would spill with the claim's code)
  static_assert(!CLAIMS || (!PAGED && !APPEND && HB == 1), "claimed chunks: one head block, plain layout");
  constexpr int NT = NW * 64, TILE = 16, KS = D / 32, VW = D / 16;
  constexpr int NL = NW / HG;             // tile lanes
  constexpr int HP = HB * 16;             // heads per wavefront
  constexpr int SLOT = HB * VW * 4 * 64;  // floats of one wavefront's O in lane order
  typedef typename VRow<D>::type vrow_t;
  typedef typename std::conditional<KV8, uint8_t, uint16_t>::type kv_t;   // one cache element
  typedef typename std::conditional<KV8, Tile16F8<D>, Tile16<D>>::type tile_t;

  __shared__ float sm_slot[(NL > 1 ? HG * (NL - 1) : 1) * SLOT];
  __shared__ float sm_wm[NW][HP], sm_wl[NW][HP];
  __shared__ int32_t sm_P[kMaxBatch + 1];
  __shared__ int32_t sm_N[PAGED ? kMaxBatch : 1];
  __shared__ int32_t sm_wave[NW];
  __shared__ int sm_flag;
  __shared__ int32_t sm_claim;
  __shared__ int32_t sm_M[APPEND ? kMaxBatch : 1];        // APPEND: new token positions
  __shared__ float sm_cs[APPEND ? NW : 1][2][2][D / 2];  // APPEND: each wavefront's cosines and sines, two tables
  // APPEND: each wavefront's turned new key and new value, one row each per
  // table (bf16 elements, or E4M3 bytes in the first half of each row)
  __shared__ __align__(16) uint16_t sm_kvn[APPEND ? NW : 1][2][2][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);   // wavefront index, in a scalar register (everything derived from it is too)
  const int hg = wave % HG, tl = wave / HG;
  const int m16 = lane & 15, q4 = lane >> 4;
  const int G = p.G;
  const int head0 = hg * HP + m16;      // this lane's query head of block 0 (block hb: head0 + 16 hb)
  const float sl2 = p.scale_log2;

  build_prefix<NT, PAGED, APPEND>(p, sm_P, sm_N, sm_wave, sm_M);
  const TokenSpaceT<CLAIMS> ts = token_space<CLAIMS>(p, sm_P);
  zero_empty_sequences<D, NT>(p, sm_P, blockIdx.x, gridDim.x);
  if constexpr (APPEND) append_side_outputs<D, NT>(p, sm_P, sm_M, blockIdx.x, gridDim.x);
  // This workgroup streams spans v = blockIdx.x, + groups, + 2 groups, ...
  // (its span of each static layer in turn), then chunks of a claimed last
  // layer until none is left; [s0, s1) is the current span.
  //
  // The next chunk of the claimed layer, or -1: thread 0 takes a ticket and
  // LDS hands it to the workgroup (every wavefront claims at the same point
  // of the workgroup's span sequence, so the barriers match).  Each
  // workgroup's last claim is the one that finds the chunks gone, so the
  // call makes dyn + groups claims; the last of them sets the ticket back to
  // zero for the next call.  A chunk past the layer's last position gets its
  // empty merge descriptor here.
  auto claim = [&]() __attribute__((always_inline)) -> int64_t {
    if constexpr (!CLAIMS) return -1;
    for (;;) {
      if (tid == 0) {
        const int32_t c = __hip_atomic_fetch_add(p.ws_ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int64_t)c == ts.dyn + ts.groups - 1)
          __hip_atomic_store(p.ws_ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_claim = c;
      }
      __syncthreads();
      const int64_t c = uniform(sm_claim);
      __syncthreads();   // sm_claim is rewritten by the next claim
      if (c >= ts.dyn) return -1;
      const int64_t vc = ts.sl * ts.groups + c;
      if (ts.start(vc) < ts.end(vc)) return vc;
      if (!p.fused) write_merge_desc(p, vc, -1, -1, 0, 0);
    }
  };
  // The span after v in this workgroup's sequence, or -1.
  auto following_span = [&](int64_t vv) __attribute__((always_inline)) -> int64_t {
    if (vv + ts.groups < ts.sl * ts.groups) return vv + ts.groups;   // its span of the next static layer
    return CLAIMS && ts.dyn > 0 ? claim() : -1;
  };
  int64_t v = blockIdx.x;
  if constexpr (CLAIMS) {
    if (v * ts.span >= ts.per_layer) {
      // this workgroup's static span of every layer is empty (uniform)
      if (!p.fused)
        for (int64_t m = v; m < ts.sl * ts.groups; m += ts.groups) write_merge_desc(p, m, -1, -1, 0, 0);
      v = ts.dyn > 0 ? claim() : -1;
      if (v < 0) return;
    }
  }
  int64_t s0 = ts.start(v), s1 = ts.end(v);
  if constexpr (!CLAIMS) {
    if (s0 >= s1) {   // w * span >= per_layer: this workgroup's span of every layer is empty (uniform)
      if (!p.fused)
        for (int64_t m = v; m < (int64_t)p.L * ts.groups; m += ts.groups) write_merge_desc(p, m, -1, -1, 0, 0);
      return;
    }
  }

  // Per-lane element offsets inside a tile (relative to the tile's first row).
  // E4M3 keys: the lane holds columns 64h + 16q4 .. +15 (step s of the score
  // product takes columns 64(s/2) + 16q4 + 8(s%2) .. +7 of K and of q alike).
  const uint32_t koff = KV8 ? (uint32_t)(m16 * D + 16 * q4) : (uint32_t)(m16 * D + 8 * q4);
  const uint32_t voff = (uint32_t)(4 * q4 * D + VW * m16);
  const uint32_t koff_b = koff * (uint32_t)sizeof(kv_t), voff_b = voff * (uint32_t)sizeof(kv_t);   // in bytes

  // One piece: the part [c0, c1) of a unit that lies in this span.
  struct Ctx {
    const kv_t* kg;          // dense/packed: the unit's row 0; paged: the pool shifted to KV head g
    const kv_t* vg;
    const int32_t* pages;    // paged: the sequence's block-table row
    int64_t x;        // stream position of token c0
    int64_t next;     // stream position after the piece (past the unit's padding when it ends the unit)
    int64_t start;    // stream position of the unit's token 0
    int64_t orow;     // output row of the unit's first head
    int64_t w0, w_last;      // a split unit: the spans holding its first and its last token
    int64_t slot;            // state slot of a split piece: 2v for the span's first piece, else 2v + 1
    int64_t first_slot;      // a split unit: the slot of its piece in span w0
    int c0, c1, ntiles;
    bool whole;
    Piece at;         // the unit and the piece's first token
    // APPEND: the new token's position and its index in the unit when this
    // piece holds it (else -1)
    int32_t m, mnew;
    int tab;          // the wavefront's angle table of the piece (tables alternate by piece)
  };
  int tab_next = 0;
  // The piece of the span that starts at stream position x, located as pc.
  auto open_at = [&](const Piece& pc, int64_t x) __attribute__((always_inline)) {
    Ctx c;
    c.at = pc;
    c.x = x;
    c.start = pc.start;
    c.c0 = pc.t;
    c.c1 = (int)min((int64_t)pc.ui.n, pc.t + (s1 - x));
    if constexpr (PAGED) c.next = c.c1 == pc.ui.n ? pc.start + pc.npad : x + (c.c1 - c.c0);
    if constexpr (PAGED) c.pages = p.block_table + (int64_t)pc.ui.b * p.max_pages;
    c.ntiles = (c.c1 - c.c0 + TILE - 1) / TILE;
    c.whole = c.c0 == 0 && c.c1 == pc.ui.n;
    c.slot = 2 * v + (x == s0 ? 0 : 1);
    // a split unit's merge only: the spans holding its first and last token,
    // and its first piece, w0's last one unless the unit starts w0's span
    c.w0 = c.w_last = c.first_slot = 0;
    if (!c.whole) {
      c.w0 = ts.span_of(pc.start);
      c.w_last = ts.span_of(pc.start + pc.ui.n - 1);
      c.first_slot = 2 * c.w0 + (pc.start != ts.start(c.w0) ? 1 : 0);
    }
    c.kg = reinterpret_cast<const kv_t*>(p.k) + pc.ui.row0 * D;
    c.vg = reinterpret_cast<const kv_t*>(p.v) + pc.ui.row0 * D;
    c.orow = out_row0(p, pc.ui);
    if constexpr (APPEND) {
      c.m = uniform(sm_M[pc.ui.b]);
      // the piece holds the new token when it reaches the end of a unit that
      // grew by it (the unit then has m + 1 tokens)
      c.mnew = (c.c1 == pc.ui.n && pc.ui.n == c.m + 1) ? c.m : -1;
      c.tab = tab_next;   // the piece's angle table (filled by fill_angles)
      tab_next ^= 1;
    }
    return c;
  };
  auto open_piece = [&](int64_t x) __attribute__((always_inline)) {
    return open_at(locate<PAGED>(p, sm_P, sm_N, ts, x), x);
  };
  // The first piece of span v (s0 and s1 set to its bounds); its merge
  // descriptor goes out with it.
  auto open_span = [&]() __attribute__((always_inline)) {
    s0 = ts.start(v);
    s1 = ts.end(v);
    const Ctx c = open_piece(s0);
    if (!p.fused) write_merge_desc(p, v, c.c0 > 0 ? c.w0 : -1, c.w_last, c.orow, c.first_slot);
    return c;
  };
  // B operands of the score product: query head head0 + 16 hb, columns 32s + 8q4 .. +7.
  auto load_q = [&](u32x4 (&qf)[HB][KS], const Ctx& c) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = head0 + 16 * hb;
      const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q) + (c.orow + h) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int col = KV8 ? 64 * (s >> 1) + 16 * q4 + 8 * (s & 1) : 32 * s + 8 * q4;   // the columns K's step s holds
        qf[hb][s] = (h < G) ? *reinterpret_cast<const u32x4*>(qg + col) : u32x4{0, 0, 0, 0};
      }
    }
  };
  // A tile's 16 rows are consecutive in memory, from row tr of kg/vg: row t0
  // of the unit, or, in a paged cache, row t0 % page of the page holding
  // token t0 (tiles start at multiples of 16 there and never cross a page).
  auto load_tile = [&](tile_t& T, const Ctx& c, int t0, int64_t tr) __attribute__((always_inline)) {
    if constexpr (KV8) {
      typedef typename std::remove_reference<decltype(T.v[0])>::type vraw_t;
      if (t0 + TILE <= c.c1) {
        // full tile: a wave-uniform base, the lane's 32-bit offset, immediates
        const char* kt = reinterpret_cast<const char*>(c.kg + tr * D) + koff_b;
        const char* vt = reinterpret_cast<const char*>(c.vg + tr * D) + voff_b;
#pragma unroll
        for (int s = 0; s < D / 64; ++s)
          T.k[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + 64 * s));
#pragma unroll
        for (int i = 0; i < 4; ++i) T.v[i] = __builtin_nontemporal_load(reinterpret_cast<const vraw_t*>(vt + i * D));
      } else {
        // ragged tail: rows past the piece are clamped to its last valid row
        // (in bounds), their weights forced to 0 below
        const int last = c.c1 - 1;
        const kv_t* kb = PAGED ? c.kg + (tr - t0) * D : c.kg;
        const kv_t* vb = PAGED ? c.vg + (tr - t0) * D : c.vg;
        const kv_t* kt = kb + (int64_t)min(t0 + m16, last) * D + 16 * q4;
#pragma unroll
        for (int s = 0; s < D / 64; ++s)
          T.k[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + 64 * s));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          T.v[i] = __builtin_nontemporal_load(
              reinterpret_cast<const vraw_t*>(vb + (int64_t)min(t0 + 4 * q4 + i, last) * D + VW * m16));
      }
    } else if (t0 + TILE <= c.c1) {
      // full tile: a wave-uniform base, the lane's 32-bit offset, immediates
      const char* kt = reinterpret_cast<const char*>(c.kg + tr * D) + koff_b;
      const char* vt = reinterpret_cast<const char*>(c.vg + tr * D) + voff_b;
#pragma unroll
      for (int s = 0; s < KS; ++s) T.k[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + 64 * s));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        T.v[i] = __builtin_nontemporal_load(reinterpret_cast<const vrow_t*>(vt + i * D * 2));
    } else {
      // ragged tail: rows past the piece are clamped to its last valid row
      // (in bounds and finite); their weights are forced to 0 below
      // (tr - t0: the offset of the tile's page from the unit's row 0)
      const int last = c.c1 - 1;
      const uint16_t* kb = PAGED ? c.kg + (tr - t0) * D : c.kg;
      const uint16_t* vb = PAGED ? c.vg + (tr - t0) * D : c.vg;
      const uint16_t* kt = kb + (int64_t)min(t0 + m16, last) * D + 8 * q4;
#pragma unroll
      for (int s = 0; s < KS; ++s) T.k[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + 32 * s));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        T.v[i] = __builtin_nontemporal_load(
            reinterpret_cast<const vrow_t*>(vb + (int64_t)min(t0 + 4 * q4 + i, last) * D + VW * m16));
    }
  };
  // The TPW tiles j, j+NL, ... of a batch.  Every load is issued (an index past
  // the piece's last tile is clamped to it: in bounds, its compute skipped), so
  // the number of loads in flight is the same on every path; a conditional
  // load would make the compiler wait for all of them before any compute.
  auto tile_t0 = [&](const Ctx& c, int j, int u) __attribute__((always_inline)) {
    return c.c0 + min(j + NL * u, c.ntiles - 1) * TILE;
  };
  // Paged: page ids of the tiles of batch j (clamped like the loads).  The
  // table is read through the constant address space (it is not written
  // while the kernel runs): a wave-uniform load there is a scalar load,
  // counted apart from the tile loads, so waiting for an id never waits for
  // the tiles issued before it.
  auto fetch_pages = [&](int32_t (&pid)[TPW], const Ctx& c, int j) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      typedef const __attribute__((address_space(4))) int32_t* table_ptr;
      const table_ptr row = (table_ptr)c.pages;
#pragma unroll
      for (int u = 0; u < TPW; ++u) pid[u] = row[tile_t0(c, j, u) / p.page];
    }
  };
  const int64_t page_rows = (int64_t)p.H_kv * p.page;   // pool rows per page
  auto load_batch = [&](tile_t (&T)[TPW], const Ctx& c, int j, const int32_t (&pid)[TPW])
                        __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t0 = tile_t0(c, j, u);
      if constexpr (PAGED)
        load_tile(T[u], c, t0, (int64_t)pid[u] * page_rows + t0 % p.page);
      else
        load_tile(T[u], c, t0, t0);
    }
  };

  u32x4 qf[HB][KS];
  float m_run[HB], l_run[HB];
  f32x4 oacc[VW][HB];
  auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      m_run[hb] = -INFINITY;
      l_run[hb] = 0.f;
#pragma unroll
      for (int r = 0; r < VW; ++r) oacc[r][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // The reference m_run moves only when some head's maximum (mx, over the
  // head's lanes) passes it by more than kRescaleSlack (wave-uniform test):
  // until then the weights 2^(x - m_run) stay below 2^kRescaleSlack, which
  // fp32 sums and the two-term bf16 split carry at full relative precision,
  // and O and l need no rescaling.  Every state keeps the m_run its weights
  // were taken against, so merges combine them exactly as before.
  auto rebase = [&](int hb, float mx) __attribute__((always_inline)) {
    if (__any(mx > m_run[hb] + kRescaleSlack)) {
      const float m_new = fmaxf(m_run[hb], mx);
      const float alpha = exp2_raw(m_run[hb] - m_new);   // 0 on the first tile, 1 where nothing grew
      m_run[hb] = m_new;
      l_run[hb] *= alpha;
#pragma unroll
      for (int r = 0; r < VW; ++r) oacc[r][hb] *= alpha;
    }
  };
  // Scores of one tile for head block hb, in base 2, with tokens at or past
  // c1 masked.
  auto tile_scores = [&](float (&x)[4], const f32x4& sc, int t0, int c1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = sc[i] * sl2;
    if (t0 + TILE > c1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + 4 * q4 + i >= c1) x[i] = -INFINITY;
    }
  };

  // T: a Tile16 (bf16 cache) or a Tile16K8 (E4M3 cache, keys widened).
  auto compute_core = [&](const auto& T, int t0, int c1) __attribute__((always_inline)) {
    u32x2 phi[HB], plo[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) sc = mfma_k32(T.k[s], qf[hb][s], sc);
      float x[4];
      tile_scores(x, sc, t0, c1);
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = max_over_rows(mx);
      rebase(hb, mx);
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = exp2_raw(x[i] - m_run[hb]);
        l_run[hb] += pv[i];
      }
      uint32_t h01, h23, l01, l23;
      split_weights(pv[0], pv[1], h01, l01);
      split_weights(pv[2], pv[3], h23, l23);
      phi[hb] = u32x2{h01, h23};
      plo[hb] = u32x2{l01, l23};
    }
#pragma unroll
    for (int r = 0; r < VW; ++r) {
      const u32x2 va = v_operand<D>(T, r);
      const u32x4 vv = u32x4{va[0], va[1], va[0], va[1]};
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        oacc[r][hb] = mfma_k32(vv, u32x4{phi[hb][0], phi[hb][1], plo[hb][0], plo[hb][1]}, oacc[r][hb]);
    }
  };
  // APPEND: the tile that holds the new token (row m of the unit, in
  // registers from the cache's stale row) takes the turned key and the value
  // from LDS in the lanes holding that row (the tail's clamped rows too); an
  // E4M3 tile takes the new row's bytes before it is widened.
  auto compute_tile = [&](const tile_t& T, const Ctx& c, int t0, auto may_hold_new) __attribute__((always_inline)) {
    if constexpr (APPEND && decltype(may_hold_new)::value) {
      // one product either way: only the substitution is conditional
      tile_t U = T;
      if (c.mnew >= t0 && c.mnew < t0 + TILE) {   // wave-uniform
        const int mn = c.mnew, last = c.c1 - 1;
        if constexpr (KV8) {
          typedef typename std::remove_reference<decltype(U.v[0])>::type vraw_t;
          const uint8_t* kn = reinterpret_cast<const uint8_t*>(&sm_kvn[wave][c.tab][0][0]);
          const uint8_t* vn = reinterpret_cast<const uint8_t*>(&sm_kvn[wave][c.tab][1][0]);
          if (min(t0 + m16, last) == mn) {
#pragma unroll
            for (int h = 0; h < D / 64; ++h) U.k[h] = *reinterpret_cast<const u32x4*>(kn + 64 * h + 16 * q4);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (min(t0 + 4 * q4 + i, last) == mn) U.v[i] = *reinterpret_cast<const vraw_t*>(vn + VW * m16);
        } else {
          const uint16_t* kn = &sm_kvn[wave][c.tab][0][0];
          const uint16_t* vn = &sm_kvn[wave][c.tab][1][0];
          if (min(t0 + m16, last) == mn) {
#pragma unroll
            for (int s = 0; s < KS; ++s) U.k[s] = *reinterpret_cast<const u32x4*>(kn + 32 * s + 8 * q4);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (min(t0 + 4 * q4 + i, last) == mn) U.v[i] = *reinterpret_cast<const vrow_t*>(vn + VW * m16);
        }
      }
      if constexpr (KV8)
        compute_core(widen(U), t0, c.c1);
      else
        compute_core(U, t0, c.c1);
    } else if constexpr (KV8) {
      compute_core(widen(T), t0, c.c1);
    } else {
      compute_core(T, t0, c.c1);
    }
  };
  // APPEND: the queries (and the new key) of a piece are turned once its
  // first batch and the batch after it have been issued (the first compute
  // of the piece; see ensure_turned), so that loads stay in flight meanwhile,
  // with the angle table the piece's opening filled.  Score step s of a lane
  // covers the 8 columns qcol(s) .. +7 (see load_q), that is the 4 pairs
  // qcol(s)/2 .. +3.  The unit's first piece writes the turned queries of
  // its heads to q_out.
  auto qcol = [&](int s) __attribute__((always_inline)) {
    return KV8 ? 64 * (s >> 1) + 16 * q4 + 8 * (s & 1) : 32 * s + 8 * q4;
  };
  auto turn_words = [&](const u32x4& w, const float (&cc)[4], const float (&ss)[4]) __attribute__((always_inline)) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float y0, y1;
      rope_turn(bf16_to_f32(w[k] & 0xffffu), bf16_to_f32(w[k] >> 16), cc[k], ss[k], y0, y1);
      r[k] = f32_to_bf16_rne(y0) | (f32_to_bf16_rne(y1) << 16);
    }
    return r;
  };
  // APPEND: the new row of the piece that ends a grown unit, one element
  // pair per lane: lane jp < D/2 holds key and value elements 2jp, 2jp+1 (two
  // bf16 each).  Loaded when the piece is opened, with its queries, and used
  // by turn_piece.
  const int jp = lane & (D / 2 - 1);
  uint32_t kn_pair = 0, vn_pair = 0;
  auto load_new_row = [&](const Ctx& c) __attribute__((always_inline)) {
    if constexpr (APPEND) {
      if (c.mnew >= 0) {   // wave-uniform
        const int64_t nrow = ((int64_t)c.at.ui.b * p.H_kv + c.at.ui.g) * (D / 2);   // in pairs
        kn_pair = reinterpret_cast<const uint32_t*>(p.k_new)[nrow + jp];
        vn_pair = reinterpret_cast<const uint32_t*>(p.v_new)[nrow + jp];
      }
    }
  };
  auto turn_piece = [&](Ctx& c) __attribute__((always_inline)) {
    if constexpr (APPEND) {
      const float* tab = &sm_cs[wave][c.tab][0][0];
      // the cosines and sines of the lane's pairs of score step s
      auto angles = [&](int s, float (&cc)[4], float (&ss)[4]) __attribute__((always_inline)) {
        const int j0 = qcol(s) / 2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          cc[k] = tab[j0 + k];
          ss[k] = tab[D / 2 + j0 + k];
        }
      };
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        float cc[4], ss[4];
        angles(s, cc, ss);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) qf[hb][s] = turn_words(qf[hb][s], cc, ss);
      }
      // Only the piece that ends a grown unit needs the new row (loaded with
      // the piece's queries): lane jp turns key pair jp, and the row goes to
      // the wavefront's slot for the tile that holds it (the substitution in
      // compute_tile reads it back in its own lane layout) and, from
      // wavefront 0, to cache row m (no other workgroup reads that row, and
      // this piece's tile holding it takes the slot's copy whatever it
      // loaded).
      if (c.mnew >= 0) {   // wave-uniform
        // cache row m: the unit's row m, or row m % page of the page the
        // sequence's table names for it (within the pool shifted to head g)
        int64_t crow = c.mnew;
        if constexpr (PAGED) crow = (int64_t)c.pages[c.mnew / p.page] * p.H_kv * p.page + c.mnew % p.page;
        float k0, k1;
        rope_turn(bf16_to_f32(kn_pair & 0xffffu), bf16_to_f32(kn_pair >> 16), tab[jp], tab[D / 2 + jp], k0, k1);
        if (lane < D / 2) {
          if constexpr (KV8) {
            // the quantising append's arithmetic: the turned fp32 key and the
            // value divided by their scales, each to its E4M3 code
            const uint32_t kc = e4m3_encode(k0 / p.k_scale) | (e4m3_encode(k1 / p.k_scale) << 8);
            const uint32_t vc = e4m3_encode(bf16_to_f32(vn_pair & 0xffffu) / p.v_scale) |
                                (e4m3_encode(bf16_to_f32(vn_pair >> 16) / p.v_scale) << 8);
            reinterpret_cast<uint16_t*>(&sm_kvn[wave][c.tab][0][0])[jp] = (uint16_t)kc;
            reinterpret_cast<uint16_t*>(&sm_kvn[wave][c.tab][1][0])[jp] = (uint16_t)vc;
            if (wave == 0) {
              reinterpret_cast<uint16_t*>(const_cast<kv_t*>(c.kg) + crow * D)[jp] = (uint16_t)kc;
              reinterpret_cast<uint16_t*>(const_cast<kv_t*>(c.vg) + crow * D)[jp] = (uint16_t)vc;
            }
          } else {
            const uint32_t kt = f32_to_bf16_rne(k0) | (f32_to_bf16_rne(k1) << 16);
            reinterpret_cast<uint32_t*>(&sm_kvn[wave][c.tab][0][0])[jp] = kt;
            reinterpret_cast<uint32_t*>(&sm_kvn[wave][c.tab][1][0])[jp] = vn_pair;   // the value row as it is
            if (wave == 0) {
              reinterpret_cast<uint32_t*>(const_cast<kv_t*>(c.kg) + crow * D)[jp] = kt;
              reinterpret_cast<uint32_t*>(const_cast<kv_t*>(c.vg) + crow * D)[jp] = vn_pair;
            }
          }
        }
      }
      if (c.c0 == 0 && tl == 0) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const int h = head0 + 16 * hb;
          if (h >= G) continue;
          uint16_t* qo = reinterpret_cast<uint16_t*>(p.q_out) + (c.orow + h) * D;
#pragma unroll
          for (int s = 0; s < KS; ++s) *reinterpret_cast<u32x4*>(qo + qcol(s)) = qf[hb][s];
        }
      }
    }
  };
  // APPEND: lane j < D/2 computes pair j's cosine and sine for the piece's
  // position into the wavefront's table of the piece (the previous piece may
  // still read the other one).  Called right after the piece's first loads
  // are issued, so that this arithmetic overlaps their latency.
  auto fill_angles = [&](const Ctx& c) __attribute__((always_inline)) {
    if constexpr (APPEND) {
      float* tab = &sm_cs[wave][c.tab][0][0];
      if (lane < D / 2) rope_angle(p.rope_base, c.m, lane, D, tab[lane], tab[D / 2 + lane]);
    }
  };
  // may_hold_new: std::true_type unless the batch is known not to hold the
  // piece's last tile (the only one that can hold an appended token)
  auto compute_batch = [&](const tile_t (&T)[TPW], const Ctx& c, int j,
                           auto may_hold_new) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (j + NL * u < c.ntiles) compute_tile(T[u], c, c.c0 + (j + NL * u) * TILE, may_hold_new);
    }
  };

  // End of a piece: combine the states of the wavefronts of each head group,
  // then the first wavefront of each group stores its heads: the normalised
  // output (whole unit) or the piece's state (split unit).
  auto end_piece = [&](const Ctx& c) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const float lt = sum_over_rows(l_run[hb]);
      if (q4 == 0) {
        sm_wm[wave][hb * 16 + m16] = m_run[hb];
        sm_wl[wave][hb * 16 + m16] = lt;
      }
    }
    __syncthreads();
    float Mh[HB], Lh[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int e = hb * 16 + m16;
      float M = sm_wm[hg][e];
#pragma unroll
      for (int k = 1; k < NL; ++k) M = fmaxf(M, sm_wm[hg + HG * k][e]);
      float L = 0.f;
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        const float mk = sm_wm[hg + HG * k][e];
        if (mk != -INFINITY) L += exp2f(mk - M) * sm_wl[hg + HG * k][e];
      }
      Mh[hb] = M;
      Lh[hb] = L;
      const float f = (m_run[hb] == -INFINITY) ? 0.f : exp2f(m_run[hb] - M);
#pragma unroll
      for (int r = 0; r < VW; ++r) oacc[r][hb] *= f;
    }
    // One round: every tile lane of a head group but the first leaves its O
    // in an LDS slot of its own, and the first adds them in lane order.  The
    // other lanes go straight on to the next piece; the slots are rewritten
    // only after the next piece's first barrier, which the first lane reaches
    // after its reads.
    if constexpr (NL > 1) {
      if (tl > 0) {
        float* dst = sm_slot + (hg * (NL - 1) + (tl - 1)) * SLOT + lane;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int r = 0; r < VW; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[((hb * VW + r) * 4 + i) * 64] = oacc[r][hb][i];
      }
      __syncthreads();
      if (tl == 0) {
#pragma unroll
        for (int k = 0; k < NL - 1; ++k) {
          const float* src = sm_slot + (hg * (NL - 1) + k) * SLOT + lane;
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int r = 0; r < VW; ++r)
#pragma unroll
              for (int i = 0; i < 4; ++i) oacc[r][hb][i] += src[((hb * VW + r) * 4 + i) * 64];
        }
      }
    }

    // Lane (q4, m16) holds head head0 + 16 hb of each block, columns D/16*(4*q4+i) + r.
    if (tl == 0) {
      const int64_t slot = c.slot;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int h = head0 + 16 * hb;
        if (h >= G) continue;
        if (c.whole) {
          const float inv = Lh[hb] > 0.f ? p.out_mul / Lh[hb] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = VW * (4 * q4 + i);
            if (p.out_bf16) {
              uint32_t wds[VW / 2];
#pragma unroll
              for (int r = 0; r < VW; r += 2)
                wds[r / 2] = f32_to_bf16_rne(oacc[r][hb][i] * inv) | (f32_to_bf16_rne(oacc[r + 1][hb][i] * inv) << 16);
              uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + (c.orow + h) * D + col;
              if constexpr (VW == 8)
                *reinterpret_cast<u32x4*>(dst) = u32x4{wds[0], wds[1], wds[2], wds[3]};
              else
                *reinterpret_cast<u32x2*>(dst) = u32x2{wds[0], wds[1]};
            } else {
              float* dst = reinterpret_cast<float*>(p.out) + (c.orow + h) * D + col;
#pragma unroll
              for (int r = 0; r < VW; r += 4)
                *reinterpret_cast<f32x4*>(dst + r) =
                    f32x4{oacc[r][hb][i] * inv, oacc[r + 1][hb][i] * inv, oacc[r + 2][hb][i] * inv,
                          oacc[r + 3][hb][i] * inv};
            }
          }
        } else if (p.fused) {
          // 16-byte stores that write through to memory, so that a workgroup
          // on another XCD reads them back (see fused_merge)
          const Rsrc ro = slot_rsrc(p.ws_o + slot * G * D, G * D);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = VW * (4 * q4 + i);
#pragma unroll
            for (int r = 0; r < VW; r += 4)
              store4_coherent(ro, h * D + col + r,
                              f32x4{oacc[r][hb][i], oacc[r + 1][hb][i], oacc[r + 2][hb][i], oacc[r + 3][hb][i]});
          }
          if (q4 == 0) store2_coherent(slot_rsrc(p.ws_ml + slot * G * 2, G * 2), 2 * h, Mh[hb], Lh[hb]);
        } else {
          float* wo = p.ws_o + (slot * G + h) * D;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = VW * (4 * q4 + i);
#pragma unroll
            for (int r = 0; r < VW; r += 4)
              *reinterpret_cast<f32x4*>(wo + col + r) =
                  f32x4{oacc[r][hb][i], oacc[r + 1][hb][i], oacc[r + 2][hb][i], oacc[r + 3][hb][i]};
          }
          if (q4 == 0) {
            p.ws_ml[(slot * G + h) * 2] = Mh[hb];
            p.ws_ml[(slot * G + h) * 2 + 1] = Lh[hb];
          }
        }
      }
    }
    if (!c.whole && p.fused) {
      if constexpr (HG > 1) {
        // every storing wavefront's stores complete before thread 0 counts the piece
        if (tl == 0 && hg > 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();
      }
      fused_merge<D, NT>(p, c.w0, c.w_last, c.first_slot, c.orow, &sm_flag);
    }
  };

  // ---- main loop ------------------------------------------------------------
  // Two tile buffers in turn: while one batch is computed the next one (of the
  // same piece, or the first batch of the next piece: of the span, or of the
  // workgroup's span of the next layer) is already loading, so the end of a
  // piece (the combine across wavefronts and the stores) overlaps the next
  // piece's first loads.
  Ctx pc = open_span();
  int j = tl;
  int32_t pid[TPW];   // paged: page ids of the next batch to load
  fetch_pages(pid, pc, j);
  load_q(qf, pc);
  load_new_row(pc);
  reset_state();
  tile_t TA[TPW], TB[TPW];
  load_batch(TA, pc, j, pid);
  fetch_pages(pid, pc, j + NL * TPW);
  fill_angles(pc);
  // APPEND: whether the current piece's queries and new row are still to
  // be turned.  A piece of several batches (for this wavefront) is turned
  // right before its first compute, which a step (not the steady-state loop)
  // makes after issuing the next batch, so that a batch stays in flight
  // while the turn waits for the queries; the first piece, and a piece of
  // one batch, are turned when opened.
  bool turn_pending = APPEND;
  auto ensure_turned = [&]() __attribute__((always_inline)) {
    if constexpr (APPEND) {
      if (turn_pending) {   // wave-uniform
        turn_piece(pc);
        turn_pending = false;
      }
    }
  };
  ensure_turned();   // the first piece's queries and new row were issued before its first batch
  // One step with `cur` loaded: false if it is the workgroup's last batch
  // (left for the caller), else load the next batch into `nxt` and compute
  // `cur`.
  auto step = [&](const tile_t (&cur)[TPW], tile_t (&nxt)[TPW]) __attribute__((always_inline)) -> bool {
    const bool piece_done = j + NL * TPW >= pc.ntiles;
    const int64_t xn = PAGED ? pc.next : pc.x + (pc.c1 - pc.c0);
    const bool span_done = xn >= s1;
    int64_t vn = v + ts.groups;   // without claims: the workgroup's span of the next layer
    if constexpr (CLAIMS) {
      if (piece_done && span_done) {
        vn = following_span(v);
        if (vn < 0) return false;
      }
    } else {
      if (piece_done && span_done && vn >= (int64_t)p.L * ts.groups) return false;
    }
    if (piece_done) {
      // the piece ran to its unit's end (the next one starts the next unit)
      // or to its span's (the next one starts the workgroup's next span)
      auto to_span = [&]() __attribute__((always_inline)) {
        v = vn;
        return open_span();
      };
      const Ctx pn = span_done ? to_span() : open_at(next_unit<PAGED>(p, sm_P, sm_N, pc.at), xn);
      fetch_pages(pid, pn, tl);
      load_batch(nxt, pn, tl, pid);
      fetch_pages(pid, pn, tl + NL * TPW);
      compute_batch(cur, pc, j, std::true_type{});
      load_q(qf, pn);   // the next piece's queries (and new row): their latency overlaps end_piece
      load_new_row(pn);
      end_piece(pc);
      reset_state();
      pc = pn;
      fill_angles(pc);
      turn_pending = APPEND;
      // a piece of one batch for this wavefront (or none): its only compute is
      // its last, made by the step that ends it, so it is turned now
      if (tl + NL * TPW >= pc.ntiles) ensure_turned();
      j = tl;
    } else {
      load_batch(nxt, pc, j + NL * TPW, pid);
      fetch_pages(pid, pc, j + 2 * NL * TPW);
      ensure_turned();
      compute_batch(cur, pc, j, std::true_type{});
      j += NL * TPW;
    }
    return true;
  };
  for (;;) {
    // Steady state: while the piece has two more batches, neither step ends
    // it, and this loop carries only the running softmax state.  Its tiles
    // all lie below j + 2 NL TPW <= ntiles - 1, so none is the piece's last.
    // A piece whose queries are not turned yet first goes through a step.
    while (!turn_pending && j + 2 * NL * TPW < pc.ntiles) {
      load_batch(TB, pc, j + NL * TPW, pid);
      fetch_pages(pid, pc, j + 2 * NL * TPW);
      compute_batch(TA, pc, j, std::false_type{});
      load_batch(TA, pc, j + 2 * NL * TPW, pid);
      fetch_pages(pid, pc, j + 3 * NL * TPW);
      compute_batch(TB, pc, j + NL * TPW, std::false_type{});
      j += 2 * NL * TPW;
    }
    if (!step(TA, TB)) {
      compute_batch(TA, pc, j, std::true_type{});
      break;
    }
    if (!step(TB, TA)) {
      compute_batch(TB, pc, j, std::true_type{});
      break;
    }
  }
  end_piece(pc);
}

}  // namespace gqa
