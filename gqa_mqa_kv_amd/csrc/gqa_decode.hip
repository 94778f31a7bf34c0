// Host side of the C ABI declared in include/gqa_decode.h: argument checks,
// the split-KV planner and kernel dispatch.  Everything here runs on the host
// and never reads device memory or synchronises.
#include "gqa_decode.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "kernel_mfma.h"
#include "kernel_rope.h"
#include "kernel_valu.h"

namespace {

// Vector-ALU path: sequences are cut into chunks of a planned size.
constexpr int kTargetWorkgroups = 256;    // one per CU on a 256-CU part
constexpr int kMinChunk = 256;            // at least one 32-token tile per wavefront
constexpr int kMaxChunk = 8192;           // bounds the longest workgroup (tail of ragged batches)

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (queried once per device, under
// std::call_once, so any thread may ask; 256, the MI355X count, when no
// device answers, e.g. in a build environment).
constexpr int kMaxCuDevices = 64;
struct CuCount {
  std::once_flag once;
  int n = 256;
};
CuCount g_cu[kMaxCuDevices];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxCuDevices) {
    (void)hipGetLastError();
    return 256;
  }
  CuCount& c = g_cu[dev];
  std::call_once(c.once, [&] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      c.n = n;
    else
      (void)hipGetLastError();
  });
  return c.n;
}

// The kernel family a call launches: the cache's element type and layout,
// and whether the append of the new token is fused in.
struct KernelKind {
  bool kv8 = false, paged = false, append = false;
  bool claims = false;   // a layer batch whose last layer is claimed in chunks
};

int max_waves(int hb);
int max_tiles(int hb, bool kv8);
int default_tiles(int hb, bool kv8);
int resident_groups_per_cu(const gqa_dims* d, const KernelKind& kind, int waves, int tiles);

bool use_mfma(const gqa_dims* d) {
  if (d->path == GQA_PATH_MFMA) return true;
  return d->path == GQA_PATH_AUTO && d->dtype == GQA_DTYPE_BF16 && d->batch <= gqa::kMaxBatch;
}

gqa_status check_dims(const gqa_dims* d, int32_t L) {
  if (!d) return GQA_ERR_INVALID_ARG;
  if (L < 1 || d->batch < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->max_seq_len < 1)
    return GQA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return GQA_ERR_INVALID_ARG;
  if (d->dtype != GQA_DTYPE_F32 && d->dtype != GQA_DTYPE_BF16) return GQA_ERR_INVALID_ARG;
  if (d->out_dtype != GQA_DTYPE_F32 && d->out_dtype != GQA_DTYPE_BF16) return GQA_ERR_INVALID_ARG;
  if (d->seq_len_hint < 0 || d->seq_len_hint > d->max_seq_len) return GQA_ERR_INVALID_ARG;
  if (d->chunk_tokens < 0 || d->chunk_tokens % 64 != 0) return GQA_ERR_INVALID_ARG;
  if (d->path != GQA_PATH_AUTO && d->path != GQA_PATH_VALU && d->path != GQA_PATH_MFMA) return GQA_ERR_INVALID_ARG;
  if (d->workgroup_waves != 0 && d->workgroup_waves != 4 && d->workgroup_waves != 8 && d->workgroup_waves != 16)
    return GQA_ERR_INVALID_ARG;
  if (d->tiles_in_flight < 0 || d->tiles_in_flight == 3 || d->tiles_in_flight > 4) return GQA_ERR_INVALID_ARG;
  if (d->merge != GQA_MERGE_AUTO && d->merge != GQA_MERGE_FUSED && d->merge != GQA_MERGE_KERNEL)
    return GQA_ERR_INVALID_ARG;
  if (d->workgroups_per_cu < 0 || d->workgroups_per_cu > 4) return GQA_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return GQA_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads > gqa::kMaxGroup) return GQA_ERR_UNSUPPORTED;
  if (d->path == GQA_PATH_MFMA && (d->dtype != GQA_DTYPE_BF16 || d->batch > gqa::kMaxBatch))
    return GQA_ERR_UNSUPPORTED;
  const int64_t T = d->seq_len_hint > 0 ? d->seq_len_hint : d->max_seq_len;
  if ((int64_t)d->batch * T > INT32_MAX) return GQA_ERR_UNSUPPORTED;   // prefix sums are 32-bit
  const int64_t units = (int64_t)L * d->batch * d->num_kv_heads;
  if (units > INT32_MAX) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

// Fused merge: arrival counters live at the start of the workspace in a
// region of fixed size for every dims, so that calls of any shape can share
// a workspace (each leaves every counter it used at zero; nothing else is
// stored there while the counters are in use).
constexpr int64_t kCounterSlots = 1 << 18;
constexpr size_t kCounterBytes = (size_t)kCounterSlots * 4;
constexpr int64_t kFusedMaxPieces = 8;
// A layer batch under the balanced split hands out its last layer in this
// many chunks per workgroup, claimed at run time (the ticket is the last
// counter of the region).
constexpr int64_t kDynChunksPerGroup = 8;
constexpr int64_t kTicketSlot = kCounterSlots - 1;
// The matrix-core instances that can claim chunks (the kernel's CLAIMS): one
// head block, neither paged nor fused with the append.
bool claims_last_layer(int hb, const KernelKind& kind) { return hb == 1 && !kind.paged && !kind.append; }

struct Plan {
  bool mfma, fused;
  int32_t waves, tiles;
  int32_t chunk, n_chunks;   // vector path
  int32_t groups, span;      // matrix-core path (span 0: balanced over the groups)
  int64_t dyn;               // matrix-core layer batch: chunks of the last layer claimed at run time
  int64_t nspans;            // matrix-core path: spans of the call (static ones and chunks)
  int64_t units;
  size_t ws_bytes, cnt_bytes, desc_bytes, ml_bytes;
};

// kind: the kernel the call launches (its tile default and, for more than
// one workgroup per CU, its occupancy).
Plan make_plan(const gqa_dims* d, int32_t L, const KernelKind& kind = KernelKind{}) {
  const bool kv8 = kind.kv8;
  Plan p;
  p.mfma = use_mfma(d);
  p.units = (int64_t)L * d->batch * d->num_kv_heads;
  const int64_t T = d->seq_len_hint > 0 ? d->seq_len_hint : d->max_seq_len;
  const int64_t G = d->num_q_heads / d->num_kv_heads;
  const int hb = (int)((G + 15) / 16);
  p.waves = 4;
  p.tiles = 1;
  p.chunk = p.n_chunks = p.groups = p.span = 0;
  p.dyn = p.nspans = 0;
  int64_t slots;
  if (p.mfma) {
    p.waves = d->workgroup_waves ? d->workgroup_waves : 4;
    if (p.waves > max_waves(hb)) p.waves = max_waves(hb);
    p.tiles = d->tiles_in_flight ? d->tiles_in_flight : default_tiles(hb, kv8);
    if (p.tiles > max_tiles(hb, kv8)) p.tiles = max_tiles(hb, kv8);
    // Token split: each layer's valid tokens (at most B * H_kv * T) are
    // shared evenly by the workgroups, by default one per CU, and every
    // workgroup takes its share of one layer after the other: co-resident
    // workgroups (and wavefronts beyond four per CU) are served unevenly by
    // the memory system, and with equal static shares the slowest one sets
    // the time.  A forced chunk_tokens sets the span instead.
    // stream positions of a layer, at most: a paged cache counts each unit's
    // length rounded up to 16 (plain caches use the same bound, so one
    // workspace size serves both)
    const int64_t upper = (int64_t)d->batch * d->num_kv_heads * ((T + 15) / 16 * 16);
    if (d->chunk_tokens > 0) {
      p.span = d->chunk_tokens;
      p.groups = (int32_t)std::min<int64_t>(std::max<int64_t>(ceil_div(upper, p.span), 1), INT32_MAX / 2 / L);
    } else {
      // every workgroup must be resident at once (equal spans: a second
      // dispatch round would double the time)
      const int want = d->workgroups_per_cu ? d->workgroups_per_cu : 1;
      const int64_t per_cu =
          want == 1 ? 1 : std::max(1, std::min(want, resident_groups_per_cu(d, kind, p.waves, p.tiles)));
      p.groups = (int32_t)std::max<int64_t>(1, std::min<int64_t>(cu_count() * per_cu, ceil_div(upper, 16)));
    }
    // a layer batch under the balanced split: the last layer in chunks that
    // the workgroups claim once their static spans are done, so that the
    // ones that streamed faster take more of it
    if (L >= 2 && d->chunk_tokens <= 0 && claims_last_layer(hb, kind)) p.dyn = kDynChunksPerGroup * p.groups;
    p.nspans = (int64_t)(p.dyn > 0 ? L - 1 : L) * p.groups + p.dyn;
    slots = 2 * p.nspans;   // two per span
  } else {
    int64_t c;
    if (d->chunk_tokens > 0) {
      c = d->chunk_tokens;
    } else {
      const int64_t per_unit = p.units > 0 ? ceil_div(kTargetWorkgroups, p.units) : 1;
      c = ceil_div(ceil_div(T, per_unit), kMinChunk) * kMinChunk;
      if (c < kMinChunk) c = kMinChunk;
      if (c > kMaxChunk) c = kMaxChunk;
    }
    p.chunk = (int32_t)c;
    p.n_chunks = (int32_t)ceil_div(T, c);
    while (p.units * p.n_chunks > INT32_MAX) {   // only for absurd shapes with a forced tiny chunk
      p.chunk *= 2;
      p.n_chunks = (int32_t)ceil_div(T, p.chunk);
    }
    slots = p.n_chunks > 1 ? p.units * p.n_chunks : 0;
  }
  // Fused merge while a unit spans few workgroups (one workgroup then reads
  // all of its pieces at the end); with many pieces per unit the separate
  // merge kernel spreads the merge over every workgroup the unit touches.
  p.fused = false;
  if (p.mfma && p.nspans <= kTicketSlot) {
    const int64_t span_est =
        p.span > 0 ? p.span
                   : std::max<int64_t>(16, ceil_div((int64_t)d->batch * d->num_kv_heads * T,
                                                    p.dyn > 0 ? p.dyn : (int64_t)p.groups));
    const int64_t pieces = ceil_div(T, span_est) + 1;
    p.fused = d->merge == GQA_MERGE_FUSED || (d->merge == GQA_MERGE_AUTO && pieces <= kFusedMaxPieces);
  }
  if (slots == 0 || p.units == 0) {
    p.ws_bytes = p.cnt_bytes = p.ml_bytes = p.desc_bytes = 0;
  } else {
    p.cnt_bytes = kCounterBytes;   // reserved on every path: nothing but counters is ever stored there
    p.desc_bytes = p.mfma ? (size_t)ceil_div(4 * 8 * p.nspans, 256) * 256 : 0;
    p.ml_bytes = (size_t)ceil_div(slots * G * 2 * 4, 256) * 256;
    p.ws_bytes = p.cnt_bytes + p.desc_bytes + p.ml_bytes + (size_t)(slots * G * d->head_dim * 4);
  }
  return p;
}

typedef void (*kernel_fn)(gqa::Problem);

// Kernel variants per head-block count hb = ceil(G/16).  A wavefront serves
// one block of 16 heads (G <= 16) or two (G <= 64); beyond 32 heads the four
// wavefronts form two head groups.  Each wavefront holds two tile batches in
// registers (the one it computes and the next one, loading), which leaves
// room for one wavefront per SIMD; two tiles per batch fit up to G = 32 (the
// two-block variant then holds 502 of its 512 registers).
int max_waves(int) { return 4; }
// One-byte tiles hold half the registers and half the bytes of bf16 ones,
// so the one-block E4M3 variant loads two per batch by default (measured:
// 10-20 % faster than one on every workload; four, on request, gain 3 % on
// very long units and lose 10 % on the 8B and ragged 70B layers).
int max_tiles(int hb, bool kv8) { return hb == 1 ? (kv8 ? 4 : 2) : hb == 2 ? 2 : 1; }
int default_tiles(int hb, bool kv8) { return kv8 && hb == 1 ? 2 : 1; }

template <int D, bool PAGED = false, bool KV8 = false>
kernel_fn mfma_kernel(int hb, int, int tiles) {
  switch (hb) {
    case 1:
      if (KV8 && tiles == 4) return gqa::gqa_decode_mfma<D, 1, 1, 4, KV8 ? 4 : 2, PAGED, KV8>;
      return tiles == 2 ? gqa::gqa_decode_mfma<D, 1, 1, 4, 2, PAGED, KV8>
                        : gqa::gqa_decode_mfma<D, 1, 1, 4, 1, PAGED, KV8>;
    case 2:
      return tiles == 2 ? gqa::gqa_decode_mfma<D, 2, 1, 4, 2, PAGED, KV8> : gqa::gqa_decode_mfma<D, 2, 1, 4, 1, PAGED, KV8>;
    default: return gqa::gqa_decode_mfma<D, 2, 2, 4, 1, PAGED, KV8>;
  }
}

// A layer batch whose last layer the workgroups claim in chunks (one head
// block, plain or packed layout).
template <int D, bool KV8 = false>
kernel_fn mfma_claims_kernel(int tiles) {
  if (KV8 && tiles == 4) return gqa::gqa_decode_mfma<D, 1, 1, 4, KV8 ? 4 : 2, false, KV8, false, true>;
  return tiles == 2 ? gqa::gqa_decode_mfma<D, 1, 1, 4, 2, false, KV8, false, true>
                    : gqa::gqa_decode_mfma<D, 1, 1, 4, 1, false, KV8, false, true>;
}

// The decode fused with the append (cache of bf16 or E4M3 elements: plain,
// packed or paged): up to two tiles per batch for one head block (a request
// of four runs as two), one otherwise.
template <int D, bool PAGED = false, bool KV8 = false>
kernel_fn mfma_append_kernel(int hb, int tiles) {
  switch (hb) {
    case 1:
      return tiles >= 2 ? gqa::gqa_decode_mfma<D, 1, 1, 4, 2, PAGED, KV8, true>
                        : gqa::gqa_decode_mfma<D, 1, 1, 4, 1, PAGED, KV8, true>;
    case 2: return gqa::gqa_decode_mfma<D, 2, 1, 4, 1, PAGED, KV8, true>;
    default: return gqa::gqa_decode_mfma<D, 2, 2, 4, 1, PAGED, KV8, true>;
  }
}

// Where the cache of a call lives and what its elements are.
struct CacheArgs {
  const int64_t* kv_offsets = nullptr;   // packed layout, else dense
  const int32_t* block_table = nullptr;  // paged layout (one layer; page a multiple of 16)
  int32_t max_pages = 0, page = 0;
  bool e4m3 = false;                     // one-byte OCP E4M3 elements
  float k_scale = 1.f, v_scale = 1.f;    // E4M3: what each key / value element is multiplied by
  // the decode fused with the append of each sequence's new token
  const void* k_new = nullptr;           // non-null: fused append
  const void* v_new = nullptr;
  void* q_out = nullptr;
  int32_t* new_seq_lens = nullptr;
  double rope_base = 0.0;
};

KernelKind kind_of(const CacheArgs& ca) {
  KernelKind k;
  k.kv8 = ca.e4m3;
  k.paged = ca.block_table != nullptr;
  k.append = ca.k_new != nullptr;
  return k;
}

// The matrix-core kernel of a kind (waves and tiles as planned).
kernel_fn mfma_kernel_of(const gqa_dims* d, const KernelKind& kind, int waves, int tiles) {
  const int G = d->num_q_heads / d->num_kv_heads;
  const int hb = (G + 15) / 16;
  const bool d128 = d->head_dim == 128;
  if (kind.claims)
    return kind.kv8 ? (d128 ? mfma_claims_kernel<128, true>(tiles) : mfma_claims_kernel<64, true>(tiles))
                    : (d128 ? mfma_claims_kernel<128>(tiles) : mfma_claims_kernel<64>(tiles));
  if (kind.append && kind.paged && kind.kv8)
    return d128 ? mfma_append_kernel<128, true, true>(hb, tiles) : mfma_append_kernel<64, true, true>(hb, tiles);
  if (kind.append && kind.kv8)
    return d128 ? mfma_append_kernel<128, false, true>(hb, tiles) : mfma_append_kernel<64, false, true>(hb, tiles);
  if (kind.append && kind.paged)
    return d128 ? mfma_append_kernel<128, true>(hb, tiles) : mfma_append_kernel<64, true>(hb, tiles);
  if (kind.append) return d128 ? mfma_append_kernel<128>(hb, tiles) : mfma_append_kernel<64>(hb, tiles);
  if (kind.kv8 && kind.paged)
    return d128 ? mfma_kernel<128, true, true>(hb, waves, tiles) : mfma_kernel<64, true, true>(hb, waves, tiles);
  if (kind.kv8)
    return d128 ? mfma_kernel<128, false, true>(hb, waves, tiles) : mfma_kernel<64, false, true>(hb, waves, tiles);
  if (kind.paged) return d128 ? mfma_kernel<128, true>(hb, waves, tiles) : mfma_kernel<64, true>(hb, waves, tiles);
  return d128 ? mfma_kernel<128>(hb, waves, tiles) : mfma_kernel<64>(hb, waves, tiles);
}

kernel_fn pick_kernel(const gqa_dims* d, const Plan& plan, const CacheArgs& ca) {
  if (plan.mfma) {
    KernelKind k = kind_of(ca);
    k.claims = plan.dyn > 0;
    return mfma_kernel_of(d, k, plan.waves, plan.tiles);
  }
  if (d->dtype == GQA_DTYPE_F32)
    return d->head_dim == 128 ? gqa::gqa_decode_valu<float, 128> : gqa::gqa_decode_valu<float, 64>;
  return d->head_dim == 128 ? gqa::gqa_decode_valu<uint16_t, 128> : gqa::gqa_decode_valu<uint16_t, 64>;
}

// Workgroups of the matrix-core kernel a call of this kind launches that fit
// on one CU together (HIP occupancy query; 1 when no device answers).
int resident_groups_per_cu(const gqa_dims* d, const KernelKind& kind, int waves, int tiles) {
  const kernel_fn k = mfma_kernel_of(d, kind, waves, tiles);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k), 64 * waves, 0) !=
          hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    return 1;
  }
  return n;
}

// Every argument check of a decode launch, on the host; fills the plan.
// *nothing_to_do is set for an empty batch (valid, nothing is enqueued).
gqa_status check_launch(int32_t L, const void* q, const void* k, const void* v, const CacheArgs& ca,
                        const int32_t* seq_lens, float scale, const void* out, const gqa_dims* d, const void* ws,
                        size_t ws_bytes, Plan* plan, bool* nothing_to_do) {
  *nothing_to_do = false;
  gqa_status st = check_dims(d, L);
  if (st != GQA_OK) return st;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (d->batch == 0) {
    *nothing_to_do = true;
    return GQA_OK;
  }
  if (!q || !k || !v || !seq_lens || !out) return GQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(seq_lens, 4))
    return GQA_ERR_INVALID_ARG;
  if (ca.kv_offsets && !aligned(ca.kv_offsets, 8)) return GQA_ERR_INVALID_ARG;
  *plan = make_plan(d, L, kind_of(ca));
  if (plan->ws_bytes > 0 && (!ws || ws_bytes < plan->ws_bytes || !aligned(ws, 256))) return GQA_ERR_WORKSPACE;
  return GQA_OK;
}

gqa_status launch(int32_t L, const void* q, const void* k, const void* v, const CacheArgs& ca,
                  const int32_t* seq_lens, float scale, void* out, const gqa_dims* d, void* ws, size_t ws_bytes,
                  void* stream) {
  Plan plan;
  bool nothing;
  gqa_status st = check_launch(L, q, k, v, ca, seq_lens, scale, out, d, ws, ws_bytes, &plan, &nothing);
  if (st != GQA_OK || nothing) return st;

  gqa::Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.kv_offsets = ca.kv_offsets;
  p.block_table = ca.block_table;
  p.max_pages = ca.max_pages;
  p.page = ca.page;
  p.seq_lens = seq_lens;
  char* w = static_cast<char*>(ws);
  p.ws_cnt = plan.ws_bytes ? reinterpret_cast<int32_t*>(w) : nullptr;
  w += plan.cnt_bytes;
  p.ws_desc = plan.ws_bytes ? reinterpret_cast<int64_t*>(w) : nullptr;
  w += plan.desc_bytes;
  p.ws_ml = plan.ws_bytes ? reinterpret_cast<float*>(w) : nullptr;
  w += plan.ml_bytes;
  p.ws_o = plan.ws_bytes ? reinterpret_cast<float*>(w) : nullptr;
  p.fused = plan.fused;
  p.B = d->batch;
  p.H_q = d->num_q_heads;
  p.H_kv = d->num_kv_heads;
  p.G = d->num_q_heads / d->num_kv_heads;
  p.T_max = d->max_seq_len;
  p.T_cap = d->seq_len_hint > 0 ? d->seq_len_hint : d->max_seq_len;
  p.L = L;
  p.chunk = plan.chunk;
  p.n_chunks = plan.n_chunks;
  p.groups = plan.groups;
  p.span = plan.span;
  p.dyn_chunks = (int32_t)plan.dyn;
  p.ws_ticket = plan.dyn > 0 ? p.ws_cnt + kTicketSlot : nullptr;
  p.out_bf16 = d->out_dtype == GQA_DTYPE_BF16;
  // Scores are kept in base 2.  An E4M3 cache folds its key scale into the
  // score factor (one rounding of the exact product) and its value scale
  // into the normalisation of every output.
  p.scale_log2 = ca.e4m3 ? (float)((double)scale * (double)ca.k_scale * 1.4426950408889634)
                         : scale * 1.4426950408889634f;
  p.out_mul = ca.e4m3 ? ca.v_scale : 1.f;
  p.k_new = ca.k_new;
  p.v_new = ca.v_new;
  p.q_out = ca.q_out;
  p.new_seq_lens = ca.new_seq_lens;
  p.rope_base = ca.rope_base;
  p.k_scale = ca.k_scale;
  p.v_scale = ca.v_scale;

  hipStream_t s = static_cast<hipStream_t>(stream);
  void* args[] = {&p};
  const int64_t grid = plan.mfma ? plan.groups : plan.units * plan.n_chunks;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(pick_kernel(d, plan, ca)), dim3((unsigned)grid),
                                 dim3(64 * plan.waves), args, 0, s);
  if (e != hipSuccess) return GQA_ERR_LAUNCH;
  // The merge runs as a second kernel: the kernel boundary orders every
  // partial state before it is read.
  if (plan.mfma && !plan.fused) {
    const void* mk = d->head_dim == 128 ? reinterpret_cast<const void*>(gqa::gqa_merge_spans<128>)
                                        : reinterpret_cast<const void*>(gqa::gqa_merge_spans<64>);
    e = hipLaunchKernel(mk, dim3((unsigned)plan.nspans), dim3(256), args, 0, s);   // one per span
  } else if (plan.n_chunks > 1) {
    const int hpb = 256 / d->head_dim;
    const int64_t mgrid = plan.units * ((p.G + hpb - 1) / hpb);
    if (mgrid > INT32_MAX) return GQA_ERR_UNSUPPORTED;
    const void* mk = d->head_dim == 128 ? reinterpret_cast<const void*>(gqa::gqa_merge_chunks<128>)
                                        : reinterpret_cast<const void*>(gqa::gqa_merge_chunks<64>);
    e = hipLaunchKernel(mk, dim3((unsigned)mgrid), dim3(256), args, 0, s);
  }
  return e == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t gqa_decode_workspace_bytes(const gqa_dims* dims, int32_t num_layers) {
  if (check_dims(dims, num_layers) != GQA_OK) return 0;
  // the most any entry point taking these dims can need: the kernels of the
  // cache kinds differ in their tile default and occupancy
  size_t most = 0;
  for (int v = 0; v < 8; ++v) {
    KernelKind k;
    k.kv8 = v & 1;
    k.paged = v & 2;
    k.append = v & 4;
    most = std::max(most, make_plan(dims, num_layers, k).ws_bytes);
  }
  return most;
}

gqa_status gqa_decode_plan(const gqa_dims* dims, int32_t num_layers, int32_t* chunk_tokens, int32_t* num_chunks) {
  gqa_status st = check_dims(dims, num_layers);
  if (st != GQA_OK) return st;
  if (!chunk_tokens || !num_chunks) return GQA_ERR_INVALID_ARG;
  const Plan p = make_plan(dims, num_layers);
  *chunk_tokens = p.mfma ? p.span : p.chunk;
  *num_chunks = p.mfma ? p.groups : p.n_chunks;
  return GQA_OK;
}

gqa_status gqa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, float scale,
                      void* out, const gqa_dims* dims, void* workspace, size_t workspace_bytes, void* stream) {
  return launch(1, q, k_cache, v_cache, CacheArgs{}, seq_lens, scale, out, dims, workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_layers(int32_t num_layers, const void* q, const void* k_cache, const void* v_cache,
                             const int64_t* kv_offsets, const int32_t* seq_lens, float scale, void* out,
                             const gqa_dims* dims, void* workspace, size_t workspace_bytes, void* stream) {
  CacheArgs ca;
  ca.kv_offsets = kv_offsets;
  return launch(num_layers, q, k_cache, v_cache, ca, seq_lens, scale, out, dims, workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                            int32_t max_pages, int32_t page_size, const int32_t* seq_lens, float scale, void* out,
                            const gqa_dims* dims, void* workspace, size_t workspace_bytes, void* stream) {
  gqa_status st = check_dims(dims, 1);
  if (st != GQA_OK) return st;
  if (page_size <= 0 || page_size % 16 != 0 || max_pages <= 0) return GQA_ERR_INVALID_ARG;
  if ((int64_t)max_pages * page_size < dims->max_seq_len) return GQA_ERR_INVALID_ARG;
  if (!use_mfma(dims)) return GQA_ERR_UNSUPPORTED;   // the matrix-core kernel only (bf16)
  if (dims->batch == 0) return GQA_OK;
  if (!block_table || !aligned(block_table, 4)) return GQA_ERR_INVALID_ARG;
  CacheArgs ca;
  ca.block_table = block_table;
  ca.max_pages = max_pages;
  ca.page = page_size;
  return launch(1, q, k_pool, v_pool, ca, seq_lens, scale, out, dims, workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                                int32_t max_pages, int32_t page_size, const int32_t* seq_lens, float scale,
                                float k_scale, float v_scale, void* out, const gqa_dims* dims, void* workspace,
                                size_t workspace_bytes, void* stream) {
  gqa_status st = check_dims(dims, 1);
  if (st != GQA_OK) return st;
  if (page_size <= 0 || page_size % 16 != 0 || max_pages <= 0) return GQA_ERR_INVALID_ARG;
  if ((int64_t)max_pages * page_size < dims->max_seq_len) return GQA_ERR_INVALID_ARG;
  if (dims->dtype != GQA_DTYPE_BF16 || !use_mfma(dims)) return GQA_ERR_UNSUPPORTED;   // matrix-core kernel only
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale)) return GQA_ERR_INVALID_ARG;
  if (dims->batch == 0) return GQA_OK;
  if (!block_table || !aligned(block_table, 4)) return GQA_ERR_INVALID_ARG;
  CacheArgs ca;
  ca.block_table = block_table;
  ca.max_pages = max_pages;
  ca.page = page_size;
  ca.e4m3 = true;
  ca.k_scale = k_scale;
  ca.v_scale = v_scale;
  return launch(1, q, k_pool, v_pool, ca, seq_lens, scale, out, dims, workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_fp8(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, float scale,
                          float k_scale, float v_scale, void* out, const gqa_dims* dims, void* workspace,
                          size_t workspace_bytes, void* stream) {
  gqa_status st = check_dims(dims, 1);
  if (st != GQA_OK) return st;
  if (dims->dtype != GQA_DTYPE_BF16 || !use_mfma(dims)) return GQA_ERR_UNSUPPORTED;   // matrix-core kernel only
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale)) return GQA_ERR_INVALID_ARG;
  CacheArgs ca;
  ca.e4m3 = true;
  ca.k_scale = k_scale;
  ca.v_scale = v_scale;
  return launch(1, q, k_cache, v_cache, ca, seq_lens, scale, out, dims, workspace, workspace_bytes, stream);
}

// e4m3: the caches hold one-byte E4M3 codes of key / k_scale and value / v_scale.
gqa_status gqa_decode_layers_fp8(int32_t num_layers, const void* q, const void* k_cache, const void* v_cache,
                                 const int64_t* kv_offsets, const int32_t* seq_lens, float scale, float k_scale,
                                 float v_scale, void* out, const gqa_dims* dims, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  gqa_status st = check_dims(dims, num_layers);
  if (st != GQA_OK) return st;
  if (dims->dtype != GQA_DTYPE_BF16 || !use_mfma(dims)) return GQA_ERR_UNSUPPORTED;   // matrix-core kernel only
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale)) return GQA_ERR_INVALID_ARG;
  CacheArgs ca;
  ca.kv_offsets = kv_offsets;
  ca.e4m3 = true;
  ca.k_scale = k_scale;
  ca.v_scale = v_scale;
  return launch(num_layers, q, k_cache, v_cache, ca, seq_lens, scale, out, dims, workspace, workspace_bytes, stream);
}

namespace {
gqa_status append_launch(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                         const int64_t* kv_offsets, const int32_t* block_table, int32_t max_pages, int32_t page,
                         const int32_t* seq_lens, int32_t* new_seq_lens, float rope_base, void* q_out,
                         const gqa_dims* dims, void* stream, bool e4m3 = false, float k_scale = 1.f,
                         float v_scale = 1.f) {
  gqa_status st = check_dims(dims, 1);
  if (st != GQA_OK) return st;
  if (!std::isfinite(rope_base) || !(rope_base > 0.f)) return GQA_ERR_INVALID_ARG;
  if (e4m3 && (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale) || !(v_scale > 0.f)))
    return GQA_ERR_INVALID_ARG;
  if (dims->batch == 0) return GQA_OK;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !seq_lens || !q_out) return GQA_ERR_INVALID_ARG;
  const uintptr_t e = dims->dtype == GQA_DTYPE_F32 ? 4 : 2;
  const uintptr_t ec = e4m3 ? 1 : e;   // cache element size
  if (!aligned(q, e) || !aligned(k_new, e) || !aligned(v_new, e) || !aligned(k_cache, ec) || !aligned(v_cache, ec) ||
      !aligned(q_out, e) || !aligned(seq_lens, 4) || (new_seq_lens && !aligned(new_seq_lens, 4)) ||
      (kv_offsets && !aligned(kv_offsets, 8)) || (block_table && !aligned(block_table, 4)))
    return GQA_ERR_INVALID_ARG;
  gqa::RopeProblem p;
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.q_out = q_out;
  p.kv_offsets = kv_offsets;
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.page = page;
  p.seq_lens = seq_lens;
  p.new_seq_lens = new_seq_lens;
  p.B = dims->batch;
  p.H_q = dims->num_q_heads;
  p.H_kv = dims->num_kv_heads;
  p.T_max = dims->max_seq_len;
  p.base = (double)rope_base;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  typedef void (*rope_fn)(gqa::RopeProblem);
  rope_fn k;
  const bool d128 = dims->head_dim == 128;
  if (e4m3) {
    if (dims->dtype == GQA_DTYPE_F32)
      k = d128 ? gqa::gqa_append_rope<float, 128, true> : gqa::gqa_append_rope<float, 64, true>;
    else
      k = d128 ? gqa::gqa_append_rope<uint16_t, 128, true> : gqa::gqa_append_rope<uint16_t, 64, true>;
  } else if (dims->dtype == GQA_DTYPE_F32) {
    k = d128 ? gqa::gqa_append_rope<float, 128, false> : gqa::gqa_append_rope<float, 64, false>;
  } else {
    k = d128 ? gqa::gqa_append_rope<uint16_t, 128, false> : gqa::gqa_append_rope<uint16_t, 64, false>;
  }
  void* args[] = {&p};
  if (hipLaunchKernel(reinterpret_cast<const void*>(k), dim3((unsigned)dims->batch), dim3(256), args, 0,
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return GQA_ERR_LAUNCH;
  return GQA_OK;
}
}  // namespace

namespace {
// The fused append and decode on a plain or packed cache (block_table null)
// or on a paged pool.
// e4m3: the cache holds one-byte E4M3 codes of key / k_scale and
// value / v_scale, and the new row is quantised so.
gqa_status decode_append_launch(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                const int64_t* kv_offsets, const int32_t* block_table, int32_t max_pages,
                                int32_t page, const int32_t* seq_lens, int32_t* new_seq_lens, float rope_base,
                                float scale, void* q_out, void* out, const gqa_dims* dims, void* workspace,
                                size_t workspace_bytes, void* stream, bool e4m3 = false, float k_scale = 1.f,
                                float v_scale = 1.f) {
  gqa_status st = check_dims(dims, 1);
  if (st != GQA_OK) return st;
  if (dims->dtype != GQA_DTYPE_BF16 || !use_mfma(dims)) return GQA_ERR_UNSUPPORTED;   // matrix-core kernel only
  if (dims->seq_len_hint != 0) return GQA_ERR_INVALID_ARG;   // the lengths grow inside the call
  if (!std::isfinite(rope_base) || !(rope_base > 0.f)) return GQA_ERR_INVALID_ARG;
  if (e4m3 && (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale) || !(v_scale > 0.f)))
    return GQA_ERR_INVALID_ARG;
  if (dims->batch == 0) return GQA_OK;
  if (!k_new || !v_new || !q_out) return GQA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(q_out, 16)) return GQA_ERR_INVALID_ARG;
  // every workgroup reads q and seq_lens while others write q_out and new_seq_lens
  if (q_out == q || static_cast<const void*>(new_seq_lens) == static_cast<const void*>(seq_lens))
    return GQA_ERR_INVALID_ARG;
  if (new_seq_lens && !aligned(new_seq_lens, 4)) return GQA_ERR_INVALID_ARG;
  CacheArgs cb;
  cb.kv_offsets = kv_offsets;
  cb.block_table = block_table;
  cb.max_pages = max_pages;
  cb.page = page;
  cb.e4m3 = e4m3;
  cb.k_scale = k_scale;
  cb.v_scale = v_scale;
  const int64_t G = dims->num_q_heads / dims->num_kv_heads;
  if (G > 16 && new_seq_lens) {
    // Two head blocks: there the fused kernel needs more registers than a
    // SIMD holds and spills at every piece end, and the append kernel followed
    // by the decode of the grown cache is faster, with the same results (both
    // turn, round and substitute alike).  Every argument of both launches is
    // checked before the first is enqueued.
    Plan plan;
    bool nothing;
    st = check_launch(1, q_out, k_cache, v_cache, cb, new_seq_lens, scale, out, dims, workspace, workspace_bytes,
                      &plan, &nothing);
    if (st != GQA_OK) return st;
    st = append_launch(q, k_new, v_new, k_cache, v_cache, kv_offsets, block_table, max_pages, page, seq_lens,
                       new_seq_lens, rope_base, q_out, dims, stream, e4m3, k_scale, v_scale);
    if (st != GQA_OK) return st;
    return launch(1, q_out, k_cache, v_cache, cb, new_seq_lens, scale, out, dims, workspace, workspace_bytes, stream);
  }
  CacheArgs ca = cb;
  ca.k_new = k_new;
  ca.v_new = v_new;
  ca.q_out = q_out;
  ca.new_seq_lens = new_seq_lens;
  ca.rope_base = (double)rope_base;
  return launch(1, q, k_cache, v_cache, ca, seq_lens, scale, out, dims, workspace, workspace_bytes, stream);
}
}  // namespace

gqa_status gqa_decode_append_rope(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                  const int64_t* kv_offsets, const int32_t* seq_lens, int32_t* new_seq_lens,
                                  float rope_base, float scale, void* q_out, void* out, const gqa_dims* dims,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return decode_append_launch(q, k_new, v_new, k_cache, v_cache, kv_offsets, nullptr, 0, 0, seq_lens, new_seq_lens,
                              rope_base, scale, q_out, out, dims, workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_append_rope_paged(const void* q, const void* k_new, const void* v_new, void* k_pool,
                                        void* v_pool, const int32_t* block_table, int32_t max_pages,
                                        int32_t page_size, const int32_t* seq_lens, int32_t* new_seq_lens,
                                        float rope_base, float scale, void* q_out, void* out, const gqa_dims* dims,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  if (page_size <= 0 || page_size % 16 != 0 || max_pages <= 0) return GQA_ERR_INVALID_ARG;
  if (dims && (int64_t)max_pages * page_size < dims->max_seq_len) return GQA_ERR_INVALID_ARG;
  if (!block_table || !aligned(block_table, 4)) return GQA_ERR_INVALID_ARG;
  return decode_append_launch(q, k_new, v_new, k_pool, v_pool, nullptr, block_table, max_pages, page_size, seq_lens,
                              new_seq_lens, rope_base, scale, q_out, out, dims, workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_append_rope_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, const int64_t* kv_offsets, const int32_t* seq_lens,
                                      int32_t* new_seq_lens, float rope_base, float scale, float k_scale,
                                      float v_scale, void* q_out, void* out, const gqa_dims* dims, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return decode_append_launch(q, k_new, v_new, k_cache, v_cache, kv_offsets, nullptr, 0, 0, seq_lens, new_seq_lens,
                              rope_base, scale, q_out, out, dims, workspace, workspace_bytes, stream, true, k_scale,
                              v_scale);
}

gqa_status gqa_decode_append_rope_paged_fp8(const void* q, const void* k_new, const void* v_new, void* k_pool,
                                            void* v_pool, const int32_t* block_table, int32_t max_pages,
                                            int32_t page_size, const int32_t* seq_lens, int32_t* new_seq_lens,
                                            float rope_base, float scale, float k_scale, float v_scale, void* q_out,
                                            void* out, const gqa_dims* dims, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  if (page_size <= 0 || page_size % 16 != 0 || max_pages <= 0) return GQA_ERR_INVALID_ARG;
  if (dims && (int64_t)max_pages * page_size < dims->max_seq_len) return GQA_ERR_INVALID_ARG;
  if (!block_table || !aligned(block_table, 4)) return GQA_ERR_INVALID_ARG;
  return decode_append_launch(q, k_new, v_new, k_pool, v_pool, nullptr, block_table, max_pages, page_size, seq_lens,
                              new_seq_lens, rope_base, scale, q_out, out, dims, workspace, workspace_bytes, stream,
                              true, k_scale, v_scale);
}

gqa_status gqa_append_rope(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int64_t* kv_offsets, const int32_t* seq_lens, int32_t* new_seq_lens,
                           float rope_base, void* q_out, const gqa_dims* dims, void* stream) {
  return append_launch(q, k_new, v_new, k_cache, v_cache, kv_offsets, nullptr, 0, 0, seq_lens, new_seq_lens, rope_base,
                       q_out, dims, stream);
}

gqa_status gqa_append_rope_paged(const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                 const int32_t* block_table, int32_t max_pages, int32_t page_size,
                                 const int32_t* seq_lens, int32_t* new_seq_lens, float rope_base, void* q_out,
                                 const gqa_dims* dims, void* stream) {
  if (page_size <= 0 || page_size % 16 != 0 || max_pages <= 0) return GQA_ERR_INVALID_ARG;
  if (dims && (int64_t)max_pages * page_size < dims->max_seq_len) return GQA_ERR_INVALID_ARG;
  if (dims && dims->batch > 0 && !block_table) return GQA_ERR_INVALID_ARG;
  return append_launch(q, k_new, v_new, k_pool, v_pool, nullptr, block_table, max_pages, page_size, seq_lens,
                       new_seq_lens, rope_base, q_out, dims, stream);
}

gqa_status gqa_append_rope_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               const int64_t* kv_offsets, const int32_t* seq_lens, int32_t* new_seq_lens,
                               float rope_base, float k_scale, float v_scale, void* q_out, const gqa_dims* dims,
                               void* stream) {
  return append_launch(q, k_new, v_new, k_cache, v_cache, kv_offsets, nullptr, 0, 0, seq_lens, new_seq_lens, rope_base,
                       q_out, dims, stream, true, k_scale, v_scale);
}

gqa_status gqa_append_rope_paged_fp8(const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                     const int32_t* block_table, int32_t max_pages, int32_t page_size,
                                     const int32_t* seq_lens, int32_t* new_seq_lens, float rope_base, float k_scale,
                                     float v_scale, void* q_out, const gqa_dims* dims, void* stream) {
  if (page_size <= 0 || page_size % 16 != 0 || max_pages <= 0) return GQA_ERR_INVALID_ARG;
  if (dims && (int64_t)max_pages * page_size < dims->max_seq_len) return GQA_ERR_INVALID_ARG;
  if (dims && dims->batch > 0 && !block_table) return GQA_ERR_INVALID_ARG;
  return append_launch(q, k_new, v_new, k_pool, v_pool, nullptr, block_table, max_pages, page_size, seq_lens,
                       new_seq_lens, rope_base, q_out, dims, stream, true, k_scale, v_scale);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// gqa_decode_noalloc: the partial states of gqa_decode in a static device
// buffer instead of a caller workspace, for callers that cannot allocate.
// In host code `scratch` names a host-side stand-in of the array, not its
// device address: the address of each device's copy is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// pointer is ever passed to a kernel.
namespace {

static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;   // device address of this device's copy of `scratch`
};
ScratchSlot g_scratch[kMaxDevices];

__global__ __launch_bounds__(256) void zero_words(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// The device address of `scratch` on the device `stream` runs on (the
// current device), or nullptr when the runtime cannot give it.
void* scratch_ptr(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return;   // slot.ptr stays null: every call on this device reports GQA_ERR_LAUNCH
    }
    // The arrival counters must start at zero.  The array is zero when the
    // code object is loaded; clear the counter region once more on the
    // caller's stream, except inside a graph capture, where the clear would
    // only run at replay.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) {
      void* args[] = {&p, nullptr};
      int64_t n = (int64_t)(kCounterBytes / 4);
      args[1] = &n;
      if (hipLaunchKernel(reinterpret_cast<const void*>(zero_words), dim3(256), dim3(256), args, 0, stream) !=
          hipSuccess) {
        (void)hipGetLastError();
        return;
      }
    }
    slot.ptr = p;
  });
  return slot.ptr;
}

}  // namespace

extern "C" {

gqa_status gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                              float scale, void* out, const gqa_dims* dims, void* stream) {
  gqa_status st = check_dims(dims, 1);
  if (st != GQA_OK) return st;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (dims->batch == 0) return GQA_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !out) return GQA_ERR_INVALID_ARG;
  if (make_plan(dims, 1).ws_bytes > GQA_NOALLOC_SCRATCH_BYTES) return GQA_ERR_SCRATCH;
  void* ws = scratch_ptr(static_cast<hipStream_t>(stream));
  if (!ws) return GQA_ERR_LAUNCH;
  return launch(1, q, k_cache, v_cache, CacheArgs{}, seq_lens, scale, out, dims, ws, GQA_NOALLOC_SCRATCH_BYTES,
                stream);
}

const char* gqa_status_string(gqa_status s) {
  switch (s) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARG: return "GQA_ERR_INVALID_ARG: invalid argument";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: unsupported shape, dtype or path";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or too small";
    case GQA_ERR_LAUNCH: return "GQA_ERR_LAUNCH: kernel launch failed";
    case GQA_ERR_SCRATCH: return "GQA_ERR_SCRATCH: the call needs more scratch than the static buffer holds";
  }
  return "unknown gqa_status";
}

}  // extern "C"
