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
// workspace and the states are combined in chunk order, which keeps the
// result deterministic, either by the unit's last workgroup to finish (fused
// merge, below) or by a second small kernel launched behind the first on the
// same stream (the kernel boundary then makes the states visible):
//   M = max_k m_k,  out = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

constexpr int kMaxGroup = 64;   // largest G = H_q / H_kv supported

struct Problem {
  const void* q;              // [L][B][H_q][D]
  const void* k;              // cache, dense or packed
  const void* v;
  void* out;                  // [L][B][H_q][D]
  const int64_t* kv_offsets;  // [B+1] or nullptr (dense)
  const int32_t* seq_lens;    // [B]
  float* ws_ml;               // [units][n_chunks][G][2]   (m, l)
  float* ws_o;                // [units][n_chunks][G][D]
  int32_t* ws_cnt;            // [units] arrival counters of the fused merge (zero between calls)
  int32_t fused_merge;        // 1: the last-arriving workgroup of a unit merges; 0: separate kernel
  int32_t B, H_q, H_kv, G, T_max, L;
  int32_t T_cap;              // planned bound on valid tokens (seq_len_hint, else T_max)
  int32_t chunk, n_chunks;
  int32_t out_bf16;
  float scale_log2;           // scale * log2(e): scores are kept in base 2
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even float -> bfloat16 bits (IEEE definition; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
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

// Agent-coherent 32-bit accesses (global_load/store with sc1 on gfx950): the
// chunk states of the fused merge travel through these, so they bypass the
// per-XCD L2s that are not coherent with each other for ordinary accesses.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Fused merge, called by every thread of a workgroup that has published its
// chunk state with store_coherent (thread 0 of the publishing wavefront
// passes publisher = true).  Publishing order: the state's agent-coherent
// stores complete (s_waitcnt), then the unit's arrival counter is bumped with
// an agent-scope atomic.  The workgroup that brings the count to nck reads
// every chunk state back with agent-coherent loads, in chunk order, writes
// the output, and returns the counter to zero for the next call.
template <int D, int NT>
__device__ void fused_merge(const Problem& p, int unit, const UnitInfo& ui, int nck, bool publisher, int* sm_flag) {
  if (publisher) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);   // this wavefront's coherent stores have completed
    const int prev = __hip_atomic_fetch_add(p.ws_cnt + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sm_flag = (prev == nck - 1);
  }
  __syncthreads();
  if (!*sm_flag) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const int G = p.G;
  const float* ml = p.ws_ml + (int64_t)unit * p.n_chunks * G * 2;
  const float* o = p.ws_o + (int64_t)unit * p.n_chunks * G * D;
  const int64_t orow = out_row0(p, ui);
  for (int e = threadIdx.x; e < G * D; e += NT) {
    const int h = e / D, c = e % D;
    float M = -INFINITY, num = 0.f, den = 0.f;
#pragma unroll 4
    for (int k = 0; k < nck; ++k) {
      const float mk = load_coherent(ml + ((int64_t)k * G + h) * 2);
      const float lk = load_coherent(ml + ((int64_t)k * G + h) * 2 + 1);
      const float ok = load_coherent(o + ((int64_t)k * G + h) * D + c);
      const float Mn = fmaxf(M, mk);
      const float a = exp2f(M - Mn), f = exp2f(mk - Mn);
      num = num * a + f * ok;
      den = den * a + f * lk;
      M = Mn;
    }
    store_out(p, orow + h, c, D, den > 0.f ? num / den : 0.f);
  }
  if (threadIdx.x == 0) __hip_atomic_store(p.ws_cnt + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

}  // namespace gqa
