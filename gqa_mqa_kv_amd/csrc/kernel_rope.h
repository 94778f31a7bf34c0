// Append the new token of every sequence to the KV cache, with rotary
// position embedding ("Grouped-Query Attention (GQA) and Multi-Query
// Attention (MQA): ...", section 4, "Rotary Position Embeddings (RoPE)
// Interaction"): the token of sequence b is at position m = seq_lens[b];
// every query head and, once per KV head, the key are turned by R_{Theta,m},
// a 2x2 rotation of each pair of consecutive elements (2j, 2j+1) by the
// angle m * theta_j, theta_j = base^(-2j/d).
//
// One workgroup of 256 threads per sequence.  The d/2 angles are computed
// once, in double precision (m * theta_j reaches 1e5 radians), and shared
// through LDS as single-precision cosine and sine; each thread then turns
// element pairs of the queries and keys.
//
// KV8: the cache holds one-byte OCP E4M3 elements; the rotated key and the
// value are stored as the codes of key / k_scale and value / v_scale (nearest
// E4M3 value, ties to the even mantissa, saturating at +-448, NaN to 0x7F).
#pragma once

#include "common.h"

namespace gqa {

struct RopeProblem {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  void* q_out;
  const int64_t* kv_offsets;   // [B+1] or nullptr (dense [B][H_kv][T_max][D])
  const int32_t* block_table;  // paged pool [num_pages][H_kv][page][D]: [B][max_pages] page ids, or nullptr
  int32_t max_pages, page;
  const int32_t* seq_lens;     // [B]
  int32_t* new_seq_lens;       // [B] or nullptr (may equal seq_lens)
  int32_t B, H_q, H_kv, T_max;
  double base;
  float k_scale, v_scale;      // KV8: what a key / value code is multiplied by
};

// e4m3_encode (common.h) turns a value into its E4M3 byte.

template <typename T>
struct RopeElem;
template <>
struct RopeElem<float> {
  static __device__ __forceinline__ float get(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  static __device__ __forceinline__ void put(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
};
template <>
struct RopeElem<uint16_t> {
  static __device__ __forceinline__ float get(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void put(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16_rne(v);
  }
};

template <typename T, int D, bool KV8>
__global__ __launch_bounds__(256) void gqa_append_rope(RopeProblem p) {
  constexpr int NT = 256, P = D / 2;
  __shared__ float sm_cos[P], sm_sin[P];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int64_t cap = p.kv_offsets ? p.kv_offsets[b + 1] - p.kv_offsets[b] : (int64_t)p.T_max;
  const int32_t len = p.seq_lens[b];
  const int64_t m = len < 0 ? 0 : len;     // the new token's position
  const bool append = m < cap;             // a full cache is left as it is
  for (int j = tid; j < P; j += NT) rope_angle(p.base, m, j, D, sm_cos[j], sm_sin[j]);
  __syncthreads();

  // rows of this token: q and out [B][H_q][D], k_new/v_new [B][H_kv][D]
  const int64_t qrow = (int64_t)b * p.H_q, krow = (int64_t)b * p.H_kv;
  int64_t crow0 = 0, cstride = 0;   // cache row of KV head g: crow0 + g * cstride
  if (p.block_table) {
    if (append) {   // the page holding position m (read only when m < capacity <= max_pages * page)
      const int64_t pid = p.block_table[(int64_t)b * p.max_pages + m / p.page];
      crow0 = pid * p.H_kv * p.page + m % p.page;
      cstride = p.page;
    }
  } else if (p.kv_offsets) {
    crow0 = p.kv_offsets[b] * p.H_kv + m;
    cstride = cap;
  } else {
    crow0 = (int64_t)b * p.H_kv * p.T_max + m;
    cstride = p.T_max;
  }
  const int nq = p.H_q * P, nk = p.H_kv * P;
  for (int e = tid; e < nq + nk; e += NT) {
    const int j = e % P;
    const float c = sm_cos[j], s = sm_sin[j];
    if (e < nq) {
      const int64_t i0 = (qrow + e / P) * D + 2 * j;
      const float x0 = RopeElem<T>::get(p.q, i0), x1 = RopeElem<T>::get(p.q, i0 + 1);
      float y0, y1;
      rope_turn(x0, x1, c, s, y0, y1);
      RopeElem<T>::put(p.q_out, i0, y0);
      RopeElem<T>::put(p.q_out, i0 + 1, y1);
    } else if (append) {
      const int g = (e - nq) / P;
      const int64_t i0 = (krow + g) * D + 2 * j, o0 = (crow0 + g * cstride) * D + 2 * j;
      const float x0 = RopeElem<T>::get(p.k_new, i0), x1 = RopeElem<T>::get(p.k_new, i0 + 1);
      float k0, k1;
      rope_turn(x0, x1, c, s, k0, k1);
      if constexpr (KV8) {
        uint8_t* kc = static_cast<uint8_t*>(p.k_cache);
        uint8_t* vc = static_cast<uint8_t*>(p.v_cache);
        kc[o0] = (uint8_t)e4m3_encode(k0 / p.k_scale);
        kc[o0 + 1] = (uint8_t)e4m3_encode(k1 / p.k_scale);
        vc[o0] = (uint8_t)e4m3_encode(RopeElem<T>::get(p.v_new, i0) / p.v_scale);
        vc[o0 + 1] = (uint8_t)e4m3_encode(RopeElem<T>::get(p.v_new, i0 + 1) / p.v_scale);
      } else {
        RopeElem<T>::put(p.k_cache, o0, k0);
        RopeElem<T>::put(p.k_cache, o0 + 1, k1);
        // the value row is stored as it is
        RopeElem<T>::put(p.v_cache, o0, RopeElem<T>::get(p.v_new, i0));
        RopeElem<T>::put(p.v_cache, o0 + 1, RopeElem<T>::get(p.v_new, i0 + 1));
      }
    }
  }
  if (p.new_seq_lens) {
    __syncthreads();   // every thread has read seq_lens[b] (new_seq_lens may be the same array)
    if (tid == 0) p.new_seq_lens[b] = append ? (int32_t)(m + 1) : len;
  }
}

}  // namespace gqa
