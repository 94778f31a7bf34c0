/*
 * gqa_decode.h -- C ABI of an MI355X (gfx950) library for one decode step of
 * grouped-query attention.
 *
 * The operation ("Grouped-Query Attention (GQA) and Multi-Query Attention
 * (MQA): Mathematical Foundations, Arithmetic Intensity, and KV-Cache Scaling
 * Mechanics", section 2, subsection "Grouped-Query Attention (GQA)"):
 * H_q query heads are split into H_kv contiguous groups of G = H_q / H_kv;
 * query head i reads key/value head g = i / G (0-based form of the page's
 * g(i) = floor((i-1)/R) + 1), and
 *
 *     out[b, i, :] = softmax_t( scale * q[b, i, :] . K[b, g, t, :] ) V[b, g, t, :]
 *
 * over the cached positions t in [0, seq_lens[b]).  At decode time the single
 * new query is the last position, so the page's causal mask M admits exactly
 * those positions.  G = 1 is multi-head attention ("Multi-Head Attention
 * (MHA)" subsection); H_kv = 1 is multi-query attention ("Multi-Query
 * Attention (MQA)" subsection).  seq_lens[b] == 0 yields a zero output row.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every tensor pointer is a device pointer owned by the caller; the
 *   library allocates nothing, keeps no pointer after the call returns and
 *   has no mutable global state (apart from the static buffer that
 *   gqa_decode_noalloc uses in place of a workspace).  All tensors are dense
 *   and row-major.
 *   q, out    : [B][H_q][d]           (per layer, see gqa_decode_layers)
 *   k_cache,
 *   v_cache   : [B][H_kv][T_max][d]   (dense layout)
 *   seq_lens  : [B] int32, device memory; never read by the host.  Values are
 *               clamped on the device into [0, min(capacity of the sequence,
 *               seq_len_hint if set, max_seq_len)].
 *   q, k_cache, v_cache and out must be 16-byte aligned; out must not
 *   overlap any input.
 * Types.  q, k_cache and v_cache share dims->dtype (fp32 or bf16), except
 *   in the *_fp8 decode calls, whose caches hold one-byte E4M3 elements; out has
 *   dims->out_dtype.  Products, softmax and sums are accumulated in fp32; a
 *   bf16 output is rounded to nearest-even.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls
 *   only enqueue work and return; inputs must stay unchanged, and out is
 *   valid, once the stream reaches the call.  No host synchronisation.
 * Work split.  The matrix-core path divides each layer's valid tokens, in
 *   (sequence, KV head, token) order, evenly among its workgroups (one per
 *   CU by default), whatever the sequence lengths; each workgroup takes its
 *   share of layer 0, then of layer 1, and so on.  The vector path cuts
 *   each sequence into chunks of a planned size.  Pieces of a (layer,
 *   sequence, KV head) computed by different workgroups leave partial
 *   softmax states in the workspace that are combined in a fixed order
 *   (results are deterministic), either inside the decode kernel by the
 *   last workgroup to finish a piece of it, or by a second kernel on the same
 *   stream (see gqa_merge).
 * Workspace.  Those partial states live in a caller-provided device
 *   workspace of at least gqa_decode_workspace_bytes() bytes, 256-byte
 *   aligned (may be NULL when that size is 0).  Its first 1 MiB holds
 *   arrival counters and nothing else, for every dims and path:
 *   zero-fill a workspace once before its first use; every call that
 *   completes leaves the counters at zero again, so calls of any shape
 *   ordered on one stream may share a workspace without clearing it.  Calls
 *   that may overlap in time need separate workspaces.
 * Errors.  Every entry point returns a gqa_status and never throws.  Argument
 *   errors are detected on the host before anything is enqueued.  Faults
 *   inside a kernel surface at the next synchronisation, as usual in HIP.
 * Threads.  Entry points are reentrant and may be called from any thread.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_dtype {
  GQA_DTYPE_F32 = 0,   /* IEEE binary32 */
  GQA_DTYPE_BF16 = 1   /* bfloat16: the upper 16 bits of a binary32 */
} gqa_dtype;

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment, H_q % H_kv != 0 */
  GQA_ERR_UNSUPPORTED = 2,  /* head_dim not 64/128, G > 64, dtype/path pairing, more than
                               4096 sequences on the matrix-core path */
  GQA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  GQA_ERR_LAUNCH = 4,       /* the HIP runtime refused the launch */
  GQA_ERR_SCRATCH = 5       /* gqa_decode_noalloc only: the call needs more partial-state
                               memory than the library's static buffer holds */
} gqa_status;

/* Which kernel family runs the step.  AUTO picks the matrix-core kernel for
 * bf16 inputs (up to 4096 sequences) and the vector-ALU kernel otherwise. */
typedef enum gqa_path {
  GQA_PATH_AUTO = 0,
  GQA_PATH_VALU = 1,   /* vector ALU, any supported dtype */
  GQA_PATH_MFMA = 2    /* matrix cores (v_mfma_f32_16x16x32_bf16), bf16 inputs only */
} gqa_path;

/* How the partial states of a (layer, sequence, KV head) split between
 * workgroups are combined on the matrix-core path.  FUSED: the workgroup that
 * finishes the last piece merges them inside the decode kernel (one kernel
 * per call).  KERNEL: a second kernel merges them, spread over every
 * workgroup the split touched.  AUTO: FUSED while a sequence can span at
 * most about 8 workgroups, else KERNEL.  The vector path always uses a second
 * kernel. */
typedef enum gqa_merge {
  GQA_MERGE_AUTO = 0,
  GQA_MERGE_FUSED = 1,
  GQA_MERGE_KERNEL = 2
} gqa_merge;

typedef struct gqa_dims {
  int32_t batch;         /* B >= 0 (B == 0 is a no-op) */
  int32_t num_q_heads;   /* H_q >= 1 */
  int32_t num_kv_heads;  /* H_kv >= 1, divides H_q; G = H_q / H_kv <= 64 */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t max_seq_len;   /* T_max >= 1: rows per (sequence, KV head) of the dense
                            cache; for a packed cache, an upper bound on every
                            sequence's capacity */
  int32_t dtype;         /* gqa_dtype of q, k_cache, v_cache */
  int32_t out_dtype;     /* gqa_dtype of out */
  int32_t seq_len_hint;  /* 0, or an upper bound (<= max_seq_len) on every
                            seq_lens[b]; the split is planned over it and
                            larger values are clamped to it on the device */
  int32_t chunk_tokens;  /* 0: the planner splits the work; otherwise a positive
                            multiple of 64: tokens per workgroup and layer
                            (matrix-core path) or per chunk of a sequence
                            (vector path) */
  int32_t path;          /* gqa_path */
  int32_t workgroup_waves; /* 0, 4, 8 or 16 (others are invalid): wavefronts
                              per workgroup of the matrix-core kernel.  Every
                              value runs as 4: each wavefront keeps two tile
                              batches in registers, which leaves room for one
                              wavefront per SIMD */
  int32_t tiles_in_flight; /* 0: default; else 1, 2 or 4: 16-token tiles per
                              load batch of each wavefront of the matrix-core
                              kernel.  A wavefront computes one batch while
                              the next one loads.  bf16 caches: default 1,
                              at most 2 for G <= 32, else 1.  E4M3 caches
                              (gqa_decode_fp8): default 2 and at most 4
                              for G <= 16; default 1 and at most 2 for
                              G <= 32; else 1.  Larger requests run at the
                              variant's limit. */
  int32_t merge;           /* gqa_merge */
  int32_t workgroups_per_cu; /* 0: default (1); else matrix-core workgroups
                                launched per compute unit when the split is
                                balanced (no chunk_tokens): 1 to 4, reduced to
                                what the kernel's registers and LDS let reside
                                on one CU together */
} gqa_dims;

/*
 * Bytes of workspace a call with these dims and `num_layers` layers needs
 * (0 when no partial state can arise): the most that any entry point taking
 * these dims (plain, packed, paged, E4M3, fused append) can need, since their
 * kernels differ in tile default and occupancy.  Depends on its arguments,
 * on the CU count of the current device (taken as 256 when no device
 * answers) and, with workgroups_per_cu > 1, on the kernels' occupancy;
 * touches no device memory.  Returns 0 for invalid dims as well; the decode
 * call then reports the error.
 */
size_t gqa_decode_workspace_bytes(const gqa_dims* dims, int32_t num_layers);

/*
 * The work split planned for these dims (as gqa_decode and gqa_decode_layers
 * plan it; with workgroups_per_cu > 1 the other entry points may plan fewer
 * workgroups, by their kernels' occupancy).  Matrix-core path: *chunk_tokens is
 * the forced tokens per workgroup and layer (0 when each layer's valid
 * tokens are shared evenly at run time) and *num_chunks the number of
 * workgroups (each takes its share of every layer in turn).  Vector path: tokens
 * per chunk and the chunk count of the longest possible sequence.  Returns
 * GQA_OK or GQA_ERR_INVALID_ARG / GQA_ERR_UNSUPPORTED (outputs untouched
 * then).  Host only (it may ask the HIP runtime for the CU count).
 */
gqa_status gqa_decode_plan(const gqa_dims* dims, int32_t num_layers, int32_t* chunk_tokens,
                           int32_t* num_chunks);

/*
 * One decode step of one layer (dense cache [B][H_kv][T_max][d]).
 * scale multiplies q.K (the page's 1/sqrt(d_k); passed explicitly).
 */
gqa_status gqa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                      float scale, void* out, const gqa_dims* dims, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * One decode step of `num_layers` independent layers in a single launch.
 * Layers share seq_lens; each has its own queries, cache and output:
 *   q, out     : [L][B][H_q][d]
 *   kv_offsets : NULL for the dense cache [L][B][H_kv][T_max][d]; otherwise a
 *                device array of B+1 int64 token offsets (non-decreasing,
 *                kv_offsets[0] == 0) describing the packed cache: element
 *                (l, b, h, t, c) sits at
 *                  l*S + (kv_offsets[b]*H_kv + h*cap_b + t)*d + c,
 *                cap_b = kv_offsets[b+1] - kv_offsets[b] (<= max_seq_len),
 *                S = kv_offsets[B]*H_kv*d.  This stores only each sequence's
 *                own capacity (the logical cache size of "Grouped-Query
 *                Attention Shares Keys Without Sharing Every Query", without
 *                padding to T_max).  The dense layout is kv_offsets[b] = b*T_max.
 * The result equals num_layers separate gqa_decode calls: each layer is
 * split among the workgroups as a one-layer call with these dims splits it,
 * and every workgroup takes its share of each layer in turn.  Under the
 * balanced split (chunk_tokens 0) with G <= 16, the last layer is instead
 * cut into eight chunks per workgroup that the workgroups claim at run time
 * once their shares of the other layers are done, so that the workgroups
 * that streamed faster take more of it.  Results are deterministic (a
 * chunk's result does not depend on which workgroup computes it, and
 * partial results are merged in a fixed order); with the same merge
 * (dims->merge FUSED or KERNEL) every layer but such a claimed last one is
 * bitwise the one-layer call's.  The workspace grows with num_layers (two
 * partial-state slots per workgroup and layer, and per claimed chunk).
 */
gqa_status gqa_decode_layers(int32_t num_layers, const void* q, const void* k_cache, const void* v_cache,
                             const int64_t* kv_offsets, const int32_t* seq_lens, float scale, void* out,
                             const gqa_dims* dims, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step of one layer over a cache of one-byte elements.  The KV
 * footprint formula of "Grouped-Query Attention (GQA) and Multi-Query
 * Attention (MQA): ...", section 1 ("KV Cache Memory Footprint"), counts the
 * bytes per element as a factor of its own (two for FP16/BF16); this call
 * halves it.  The pages name no format: each element is an OCP E4M3 byte
 * (sign, 4 exponent bits of bias 7, 3 mantissa bits, subnormals, no
 * infinities, S.1111.111 NaN, largest finite 448), and the cached key (value)
 * it stands for is k_scale (v_scale) times its E4M3 value.
 *   k_cache, v_cache : [B][H_kv][T_max][d] bytes, 16-byte aligned
 *   k_scale, v_scale : finite; one scale per array (GQA_ERR_INVALID_ARG
 *                      otherwise)
 *   q, out           : bf16 queries [B][H_q][d], out as for gqa_decode
 *                      (dims->dtype must be GQA_DTYPE_BF16)
 * The attention is the one above on those values, accumulated in fp32; the
 * E4M3 values are widened to bf16, which is exact.  Matrix-core path only
 * (otherwise GQA_ERR_UNSUPPORTED); seq_lens, scale, workspace
 * (gqa_decode_workspace_bytes(dims, 1)), stream and the errors as for
 * gqa_decode.
 */
gqa_status gqa_decode_fp8(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, float scale,
                          float k_scale, float v_scale, void* out, const gqa_dims* dims, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * gqa_decode_layers over caches of one-byte E4M3 elements: the dense
 * [L][B][H_kv][T_max][d] or packed (kv_offsets) layouts of gqa_decode_layers,
 * counted in bytes, with the element format and scales of gqa_decode_fp8.
 * One k_scale and one v_scale hold for every layer of the call (layers with
 * scales of their own are separate calls).  q, out: [L][B][H_q][d], q bf16.
 * Matrix-core path only (GQA_ERR_UNSUPPORTED otherwise); workspace
 * gqa_decode_workspace_bytes(dims, num_layers).  The result equals
 * num_layers separate gqa_decode_fp8 calls on the layers' caches.
 */
gqa_status gqa_decode_layers_fp8(int32_t num_layers, const void* q, const void* k_cache, const void* v_cache,
                                 const int64_t* kv_offsets, const int32_t* seq_lens, float scale, float k_scale,
                                 float v_scale, void* out, const gqa_dims* dims, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * gqa_decode_fp8 with the cache held in pages of a pool: the pools are one
 * byte per element, in the layout of gqa_decode_paged ([num_pages][H_kv]
 * [page_size][d], 16-byte aligned), read through block_table as there, each
 * element standing for k_scale or v_scale times its E4M3 value as in
 * gqa_decode_fp8.  Every argument rule and error of those two calls applies.
 */
gqa_status gqa_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                                int32_t max_pages, int32_t page_size, const int32_t* seq_lens, float scale,
                                float k_scale, float v_scale, void* out, const gqa_dims* dims, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * One decode step of one layer whose cache is held in pages of a pool.
 * "Grouped-Query Attention Shares Keys Without Sharing Every Query" counts
 * paging among the allocations a serving system adds on top of the logical
 * cache size; the attention is the one defined above, only the place of each
 * cached row changes:
 *   k_pool, v_pool : pages of page_size tokens, [num_pages][H_kv][page_size][d]
 *                    (page p, KV head h, token j of the page at row
 *                    (p * H_kv + h) * page_size + j)
 *   block_table    : [B][max_pages] int32 page ids (device): token t of
 *                    sequence b is in page block_table[b][t / page_size]
 *   page_size      : a positive multiple of 16
 *   max_pages      : entries per sequence; max_pages * page_size >=
 *                    dims->max_seq_len, the capacity each sequence's lengths
 *                    are clamped to.
 * The pools are 16-byte aligned and the table 4-byte aligned
 * (GQA_ERR_INVALID_ARG otherwise).  Only the table entries of valid tokens
 * are read; they must name pages of the pool, and sequences may share pages.
 * bf16 caches on the matrix-core path only (otherwise
 * GQA_ERR_UNSUPPORTED); the workspace is gqa_decode_workspace_bytes(dims, 1).
 * q, out, seq_lens, scale, stream and the errors as for gqa_decode.
 */
gqa_status gqa_decode_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                            int32_t max_pages, int32_t page_size, const int32_t* seq_lens, float scale, void* out,
                            const gqa_dims* dims, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The step before a decode step: append each sequence's new token to the
 * cache of one layer, with rotary position embedding ("Grouped-Query
 * Attention (GQA) and Multi-Query Attention (MQA): ...", section 4, "Rotary
 * Position Embeddings (RoPE) Interaction": the rotation R_{Theta,m} turns each
 * pair of consecutive elements (2j, 2j+1) of a head by m * theta_j).  The
 * page leaves theta_j open; here theta_j = rope_base^(-2j/d), j < d/2, and a
 * pair (x0, x1) becomes (x0 cos - x1 sin, x0 sin + x1 cos).
 * The new token of sequence b is at position m = max(seq_lens[b], 0) (the
 * cache holds tokens 0 .. m-1).  Every one of its H_q query heads is turned
 * by R_{Theta,m} into q_out; its key is turned once per KV head (the G query
 * heads of a group share it) and written, with its value, to cache row m of
 * that KV head; new_seq_lens[b] = m + 1.  A sequence whose cache is full
 * (m >= capacity) is not appended: its cache is untouched and its length is
 * copied unchanged (its queries are still turned, at position m).
 *   q, q_out      : [B][H_q][d], dims->dtype (q_out may equal q)
 *   k_new, v_new  : [B][H_kv][d], dims->dtype
 *   k_cache, v_cache : dense [B][H_kv][T_max][d] when kv_offsets is NULL,
 *                  else the packed layout of gqa_decode_layers (one layer)
 *   seq_lens      : [B] int32, tokens already cached (device)
 *   new_seq_lens  : [B] int32 or NULL (device; may equal seq_lens)
 *   rope_base     : finite and > 0
 * Pointers need the alignment of their element type (4 bytes for fp32,
 * 2 for bf16, 4 for seq_lens, 8 for kv_offsets).  dims->dtype, head_dim,
 * batch, num_q_heads, num_kv_heads and max_seq_len are used; the other fields
 * are validated as for gqa_decode but have no effect.  Rotation in fp32 with angles in double precision;
 * bf16 results are rounded to nearest-even.  Enqueues one kernel on `stream`.
 * Errors as for gqa_decode (GQA_ERR_INVALID_ARG for a bad rope_base).
 */
gqa_status gqa_append_rope(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int64_t* kv_offsets, const int32_t* seq_lens, int32_t* new_seq_lens,
                           float rope_base, void* q_out, const gqa_dims* dims, void* stream);

/*
 * gqa_append_rope followed by gqa_decode (bf16, matrix-core path), in one
 * launch up to G = 16 query heads per KV head: sequence b's new token at position m = max(seq_lens[b], 0) is
 * turned and appended exactly as gqa_append_rope does (cache row m of every
 * KV head when m < capacity, q_out, new_seq_lens), and out is the attention
 * of the turned queries over the cache including that token, as gqa_decode
 * computes it on the updated cache and lengths.  Results equal the two calls
 * in sequence, bit for bit.
 *   q, k_new, v_new, k_cache, v_cache, kv_offsets, rope_base : as for
 *                  gqa_append_rope (q, k_new, v_new and q_out 16-byte
 *                  aligned); the cache is plain or packed, one layer
 *   q_out        : [B][H_q][d], required, and must not be q (workgroups
 *                  read q while others write q_out)
 *   new_seq_lens : [B] or NULL, and must not be seq_lens (same reason)
 *   scale, out, dims, workspace, stream : as for gqa_decode;
 *                  dims->seq_len_hint must be 0 (GQA_ERR_INVALID_ARG)
 * For callers that run a decode step right after the append: the append's
 * launch (and its read of q) disappears into the decode kernel.  For G > 16
 * with new_seq_lens given, the call enqueues the append kernel and then the
 * decode of the grown cache (the fused kernel spills registers there and is
 * slower); with new_seq_lens NULL it is one kernel at every G.  The results
 * are the same either way.
 */
gqa_status gqa_decode_append_rope(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                  const int64_t* kv_offsets, const int32_t* seq_lens, int32_t* new_seq_lens,
                                  float rope_base, float scale, void* q_out, void* out, const gqa_dims* dims,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same fused step on a cache held in pages of a pool: gqa_append_rope_paged
 * followed by gqa_decode_paged, bit for bit (one launch up to G = 16, or with
 * new_seq_lens NULL; else the two kernels).  The new token of sequence b goes
 * to row m % page_size of page block_table[b][m / page_size] of each KV head,
 * m = max(seq_lens[b], 0), when m < dims->max_seq_len; that table entry must
 * name a page of the pool (the caller allocates it first).  k_pool, v_pool,
 * block_table, max_pages, page_size: as for gqa_decode_paged; everything else
 * as for gqa_decode_append_rope.  The table is only read.
 */
gqa_status gqa_decode_append_rope_paged(const void* q, const void* k_new, const void* v_new, void* k_pool,
                                        void* v_pool, const int32_t* block_table, int32_t max_pages,
                                        int32_t page_size, const int32_t* seq_lens, int32_t* new_seq_lens,
                                        float rope_base, float scale, void* q_out, void* out, const gqa_dims* dims,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_append_rope_fp8 followed by gqa_decode_fp8, and gqa_append_rope_paged_fp8
 * followed by gqa_decode_paged_fp8: the fused step of gqa_decode_append_rope
 * and gqa_decode_append_rope_paged on caches of one-byte OCP E4M3 elements
 * ("Grouped-Query Attention (GQA) and Multi-Query Attention (MQA): ...",
 * section 4, "Rotary Position Embeddings (RoPE) Interaction", with the
 * bytes-per-element factor of section 1 halved).  The new key is turned in
 * fp32 and stored as the code of key / k_scale, the value as the code of
 * value / v_scale (nearest E4M3 value, ties to even, saturating at +-448),
 * exactly as the quantising append stores them; the attention reads every
 * element, the new ones included, as k_scale (v_scale) times its E4M3 value,
 * as gqa_decode_fp8 does.  Results (out, q_out, the cache bytes, the lengths)
 * equal the two calls in sequence, bit for bit.
 *   q, k_new, v_new, q_out : bf16 (dims->dtype), 16-byte aligned
 *   k_cache, v_cache / k_pool, v_pool : E4M3 bytes in the layouts of
 *                  gqa_decode_fp8 / gqa_decode_paged_fp8, 16-byte aligned
 *   k_scale, v_scale : finite and > 0 (GQA_ERR_INVALID_ARG otherwise)
 * One launch up to G = 16 query heads per KV head, or with new_seq_lens
 * NULL; else the append kernel and the decode.  Every other argument rule
 * and error as for gqa_decode_append_rope (dense or packed caches) and
 * gqa_decode_append_rope_paged (paged pools).
 */
gqa_status gqa_decode_append_rope_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, const int64_t* kv_offsets, const int32_t* seq_lens,
                                      int32_t* new_seq_lens, float rope_base, float scale, float k_scale,
                                      float v_scale, void* q_out, void* out, const gqa_dims* dims, void* workspace,
                                      size_t workspace_bytes, void* stream);
gqa_status gqa_decode_append_rope_paged_fp8(const void* q, const void* k_new, const void* v_new, void* k_pool,
                                            void* v_pool, const int32_t* block_table, int32_t max_pages,
                                            int32_t page_size, const int32_t* seq_lens, int32_t* new_seq_lens,
                                            float rope_base, float scale, float k_scale, float v_scale, void* q_out,
                                            void* out, const gqa_dims* dims, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * The same step for a cache held in pages of a pool (the layout of
 * gqa_decode_paged): the rotated key and the value of sequence b's new token
 * go to row m % page_size of page block_table[b][m / page_size] of each KV
 * head, m = max(seq_lens[b], 0).  The capacity of a sequence is
 * dims->max_seq_len (<= max_pages * page_size); a full sequence is not
 * appended.  The table entry of position m must name a page of the pool when
 * m < dims->max_seq_len (the caller allocates the page first); it is the only
 * entry read.  page_size: a positive multiple of 16; block_table 4-byte
 * aligned.  Everything else, and the errors, as for gqa_append_rope.
 */
gqa_status gqa_append_rope_paged(const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                 const int32_t* block_table, int32_t max_pages, int32_t page_size,
                                 const int32_t* seq_lens, int32_t* new_seq_lens, float rope_base, void* q_out,
                                 const gqa_dims* dims, void* stream);

/*
 * The append step for caches of one-byte OCP E4M3 elements (the caches of
 * gqa_decode_fp8 and gqa_decode_paged_fp8).  The pages give no rule for
 * turning a value into such a byte; here the rotated key is stored as the
 * code of key / k_scale and the value as the code of value / v_scale: the
 * nearest E4M3 value, ties to the even mantissa, saturating at +-448 (a cached
 * element stays finite), NaN to 0x7F.  The division and the rotation run in
 * fp32.  k_scale and v_scale: finite and > 0 (GQA_ERR_INVALID_ARG otherwise).
 * q, k_new, v_new and q_out are fp32 or bf16 (dims->dtype); the caches need
 * no alignment.  Everything else as for gqa_append_rope (dense or packed
 * caches) and gqa_append_rope_paged (paged pools).
 */
gqa_status gqa_append_rope_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               const int64_t* kv_offsets, const int32_t* seq_lens, int32_t* new_seq_lens,
                               float rope_base, float k_scale, float v_scale, void* q_out, const gqa_dims* dims,
                               void* stream);
gqa_status gqa_append_rope_paged_fp8(const void* q, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                     const int32_t* block_table, int32_t max_pages, int32_t page_size,
                                     const int32_t* seq_lens, int32_t* new_seq_lens, float rope_base, float k_scale,
                                     float v_scale, void* q_out, const gqa_dims* dims, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * gqa_decode with its partial states kept in a static device buffer of the
 * library instead of a caller workspace: GQA_NOALLOC_SCRATCH_BYTES on each
 * GPU the call runs on, held from the first call on that GPU until the
 * process ends.  The call allocates and frees nothing.
 *   Limit: a call whose plan needs more than GQA_NOALLOC_SCRATCH_BYTES of
 *   partial states (gqa_decode_workspace_bytes(dims, 1) bounds what it
 *   needs) returns GQA_ERR_SCRATCH before enqueueing anything.  32 MiB holds
 *   every split up to G = 64 at one workgroup per CU on a 256-CU part.
 *   Sharing: every call on one GPU uses that GPU's one buffer, and it keeps
 *   the last call's contents.  Calls ordered on one stream may follow each
 *   other freely (each completed call leaves the arrival counters at zero);
 *   calls that may overlap in time on one GPU (other streams, other host
 *   threads) race and must not be issued.
 *   First call on a device: the buffer's device address is looked up, and
 *   its counter region is zero-filled by a kernel on `stream` (skipped while
 *   the stream is capturing a graph; the buffer is zero when the library is
 *   loaded).  `stream` runs on the current device (NULL: its default stream).
 * q, k_cache, v_cache, seq_lens, scale, out, dims, stream and every other
 * error as for gqa_decode; the results equal gqa_decode's bit for bit.
 */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
gqa_status gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                              float scale, void* out, const gqa_dims* dims, void* stream);

/* Static, human-readable name of a status code. */
const char* gqa_status_string(gqa_status status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
