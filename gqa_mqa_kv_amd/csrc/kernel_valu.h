// Vector-ALU GQA decode kernel: any G <= 64, fp32 or bf16 storage, D = 64/128.
//
// One workgroup of 256 threads per (unit, chunk).  Tiles of 64 tokens of K and
// V are staged through LDS (converted to fp32); scores for all G heads of the
// group are computed from that single copy, the running softmax is updated
// one wavefront per head, and P.V is accumulated in fp32 registers, thread t
// owning output elements (head, column) = t, t+256, ...
#pragma once

#include "common.h"

namespace gqa {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float get(const float* p, int64_t i) { return p[i]; }
};
template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void gqa_decode_valu(Problem p) {
  constexpr int NT = 256, TT = 64, NW = NT / 64;
  constexpr int OMAX = kMaxGroup * D / NT;   // output elements per thread at G = 64
  constexpr int KP = D + 1;                  // padded LDS row (conflict-free column walks)
  __shared__ float q_s[kMaxGroup][D];
  __shared__ float k_s[TT][KP];
  __shared__ float v_s[TT][KP];
  __shared__ float s_s[kMaxGroup][TT + 1];
  __shared__ float m_s[kMaxGroup], l_s[kMaxGroup], a_s[kMaxGroup];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = blockIdx.x / p.n_chunks, chunk = blockIdx.x % p.n_chunks;
  const UnitInfo ui = unit_info(p, unit);
  const int c0 = chunk * p.chunk;
  if (c0 >= (ui.n > 0 ? ui.n : 1)) return;   // beyond this sequence: nothing to do
  const int c1 = min(ui.n, c0 + p.chunk);
  const int G = p.G;

  const T* qg = reinterpret_cast<const T*>(p.q) + ((int64_t)(ui.l * p.B + ui.b) * p.H_q + (int64_t)ui.g * G) * D;
  const T* kg = reinterpret_cast<const T*>(p.k) + ui.row0 * D;
  const T* vg = reinterpret_cast<const T*>(p.v) + ui.row0 * D;

  for (int e = tid; e < G * D; e += NT) q_s[e / D][e % D] = Elem<T>::get(qg, e);
  for (int h = tid; h < G; h += NT) {
    m_s[h] = -INFINITY;
    l_s[h] = 0.f;
  }
  float o[OMAX];
#pragma unroll
  for (int r = 0; r < OMAX; ++r) o[r] = 0.f;
  __syncthreads();

  // Tile t+1's K/V elements are loaded into registers while tile t is
  // computed; thread tid owns elements e = tid + NT * r of a tile (row e / D,
  // column e % D).  Rows past the chunk load a clamped (valid) row, stored
  // as 0.
  constexpr int EPT = TT * D / NT;
  float kr[EPT], vr[EPT];
  auto load_regs = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int e = tid + NT * r, t = min(t0 + e / D, c1 - 1);
      kr[r] = Elem<T>::get(kg, (int64_t)t * D + e % D);
      vr[r] = Elem<T>::get(vg, (int64_t)t * D + e % D);
    }
  };
  if (c1 > c0) load_regs(c0);   // an empty sequence has no row to load
  for (int t0 = c0; t0 < c1; t0 += TT) {
    const int nt = min(TT, c1 - t0);
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int e = tid + NT * r, t = e / D, c = e % D;
      k_s[t][c] = t < nt ? kr[r] : 0.f;
      v_s[t][c] = t < nt ? vr[r] : 0.f;
    }
    load_regs(min(t0 + TT, c1 - 1));   // the next tile (the last one again at the end: in bounds, unused)
    __syncthreads();
    // scores, base 2: s = (q . k) * scale * log2(e)
    for (int e = tid; e < G * TT; e += NT) {
      int h = e / TT, t = e % TT;
      float acc = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) acc = fmaf(q_s[h][c], k_s[t][c], acc);
      s_s[h][t] = acc * p.scale_log2;
    }
    __syncthreads();
    // running softmax, one wavefront per head
    for (int h = wave; h < G; h += NW) {
      float s = (lane < nt) ? s_s[h][lane] : -INFINITY;
      float mx = s;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      float m_old = m_s[h];
      float m_new = fmaxf(m_old, mx);
      float pr = (lane < nt) ? exp2f(s - m_new) : 0.f;
      float sum = pr;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      if (lane < TT) s_s[h][lane] = pr;
      if (lane == 0) {
        float alpha = exp2f(m_old - m_new);   // m_old = -inf on the first tile -> 0
        l_s[h] = l_s[h] * alpha + sum;
        m_s[h] = m_new;
        a_s[h] = alpha;
      }
    }
    __syncthreads();
    // O = alpha * O + P V
#pragma unroll
    for (int r = 0; r < OMAX; ++r) {
      int e = tid + r * NT;
      if (e < G * D) {
        int h = e / D, c = e % D;
        float acc = o[r] * a_s[h];
        for (int t = 0; t < nt; ++t) acc = fmaf(s_s[h][t], v_s[t][c], acc);
        o[r] = acc;
      }
    }
    __syncthreads();
  }
  // Store the result: the normalised output when this unit has one chunk,
  // else this chunk's state (O, m, l) for the merge kernel.
  const int nck = chunks_of(ui.n, p.chunk);
  const int64_t orow = out_row0(p, ui);
  const int64_t slot = (int64_t)unit * p.n_chunks + chunk;
#pragma unroll
  for (int r = 0; r < OMAX; ++r) {
    int e = tid + r * NT;
    if (e < G * D) {
      int h = e / D, c = e % D;
      if (nck == 1)
        store_out(p, orow + h, c, D, l_s[h] > 0.f ? o[r] / l_s[h] : 0.f);
      else
        p.ws_o[slot * G * D + e] = o[r];
    }
  }
  if (nck > 1)
    for (int h = tid; h < G; h += NT) {
      p.ws_ml[(slot * G + h) * 2] = m_s[h];
      p.ws_ml[(slot * G + h) * 2 + 1] = l_s[h];
    }
}

}  // namespace gqa
