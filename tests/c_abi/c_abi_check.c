/*
 * The library's C boundary used from plain C, with no Python and no torch:
 * device memory and a stream from the HIP runtime, inputs from a seeded
 * counter-based generator written here, and every output compared, element
 * by element, with the fp64 C oracle (test infrastructure, linked by this
 * test only).  Bar: max |gpu - oracle| <= 2e-3 for bf16 inputs with fp32
 * accumulation and fp32 output.
 *
 * Calls: first, four host threads at once, each with a stream, a workspace
 * and a shape of its own, make the process's first calls of the library
 * (gqa_decode_workspace_bytes and gqa_decode, three times each: the library
 * promises calls from any thread); then gqa_decode_workspace_bytes,
 * gqa_decode_plan, gqa_decode (a ragged batch whose units split over
 * several workgroups), gqa_decode_layers (the
 * packed layout, three layers in one launch), gqa_decode_noalloc (twice, the
 * second call smaller), and argument errors reported before anything is
 * enqueued (a short workspace, a null pointer, an unsupported head size).
 * Exit status 0 when every check holds; each check prints one line.
 *
 * The computation checked is the grouped-query attention of "Grouped-Query
 * Attention (GQA) and Multi-Query Attention (MQA): Mathematical Foundations,
 * Arithmetic Intensity, and KV-Cache Scaling Mechanics", section 2
 * (query head i reads KV head i / G, G = H_q / H_kv).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gqa_decode.h"

/* the oracle's entry point (oracle/gqa_oracle.c) */
int oracle_gqa_decode(int64_t B, int64_t H_q, int64_t H_kv, int64_t d, int dtype, const void* q, const void* k,
                      const void* v, const int64_t* kv_offsets, const int32_t* seq_lens, double scale,
                      int64_t n_heads, const int64_t* head_ids, double* out);

static int failures = 0;

#define HIP_OK(call)                                                               \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(2);                                                                     \
    }                                                                              \
  } while (0)

static void check(int ok, const char* what) {
  printf("%s: %s\n", ok ? "ok  " : "FAIL", what);
  fflush(stdout);
  if (!ok) ++failures;
}

/* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", 2014), one output per counter value. */
static uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

/* A bf16 value in [-1, 1): the top 16 bits of a float drawn uniformly from
 * that interval (the library and the oracle both read these bits). */
static uint16_t draw_bf16(uint64_t seed, uint64_t i) {
  const uint64_t r = splitmix64(seed * 0x100000001B3ull + i);
  const float f = (float)((double)(r >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0);
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static void fill(uint16_t* x, size_t n, uint64_t seed) {
  for (size_t i = 0; i < n; ++i) x[i] = draw_bf16(seed, i);
}

/* Device memory of `bytes` (at least 16), holding a copy of h unless h is NULL. */
static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
  if (h && bytes) HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

static gqa_dims make_dims(int B, int H_q, int H_kv, int d, int T_max) {
  gqa_dims dm;
  memset(&dm, 0, sizeof dm);
  dm.batch = B;
  dm.num_q_heads = H_q;
  dm.num_kv_heads = H_kv;
  dm.head_dim = d;
  dm.max_seq_len = T_max;
  dm.dtype = GQA_DTYPE_BF16;
  dm.out_dtype = GQA_DTYPE_F32;
  dm.path = GQA_PATH_AUTO;
  dm.merge = GQA_MERGE_AUTO;
  return dm;
}

/* max |gpu - oracle| over n outputs; any non-finite gpu output counts as inf */
static double max_err(const float* gpu, const double* ref, size_t n) {
  double e = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double g = (double)gpu[i];
    if (!isfinite(g)) return INFINITY;
    const double a = fabs(g - ref[i]);
    if (a > e) e = a;
  }
  return e;
}

/* One layer, dense cache [B][H_kv][T_max][d]: gqa_decode (or, noalloc != 0,
 * gqa_decode_noalloc) against the oracle. */
static void dense_case(int B, int H_q, int H_kv, int d, int T_max, const int32_t* lens, uint64_t seed,
                       hipStream_t s, int noalloc, const char* label) {
  const size_t nq = (size_t)B * H_q * d, nkv = (size_t)B * H_kv * T_max * d;
  uint16_t* q = (uint16_t*)malloc(nq * 2);
  uint16_t* k = (uint16_t*)malloc(nkv * 2);
  uint16_t* v = (uint16_t*)malloc(nkv * 2);
  fill(q, nq, seed);
  fill(k, nkv, seed + 1);
  fill(v, nkv, seed + 2);
  const float scale = 1.0f / sqrtf((float)d);
  gqa_dims dm = make_dims(B, H_q, H_kv, d, T_max);

  void *dq = to_device(q, nq * 2), *dk = to_device(k, nkv * 2), *dv = to_device(v, nkv * 2);
  void* dl = to_device(lens, (size_t)B * 4);
  void* dout = to_device(NULL, nq * 4);
  gqa_status st;
  if (noalloc) {
    st = gqa_decode_noalloc(dq, dk, dv, (const int32_t*)dl, scale, dout, &dm, s);
  } else {
    const size_t ws_bytes = gqa_decode_workspace_bytes(&dm, 1);
    void* ws = to_device(NULL, ws_bytes);
    st = gqa_decode(dq, dk, dv, (const int32_t*)dl, scale, dout, &dm, ws, ws_bytes, s);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipFree(ws));
  }
  HIP_OK(hipStreamSynchronize(s));
  float* out = (float*)malloc(nq * 4);
  HIP_OK(hipMemcpy(out, dout, nq * 4, hipMemcpyDeviceToHost));

  int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * (B + 1));
  for (int b = 0; b <= B; ++b) offs[b] = (int64_t)b * T_max;
  double* ref = (double*)malloc(nq * sizeof(double));
  const int rc = oracle_gqa_decode(B, H_q, H_kv, d, 1, q, k, v, offs, lens, (double)scale, 0, NULL, ref);
  const double e = rc == 0 ? max_err(out, ref, nq) : INFINITY;
  char msg[256];
  snprintf(msg, sizeof msg, "%s: status %s, max |gpu - oracle| = %.3e (bar 2e-3)", label, gqa_status_string(st), e);
  check(st == GQA_OK && rc == 0 && e <= 2e-3, msg);

  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dl));
  HIP_OK(hipFree(dout));
  free(q);
  free(k);
  free(v);
  free(out);
  free(offs);
  free(ref);
}

/* L layers in one launch on the packed layout (capacity per sequence equal to
 * its length), each layer against the oracle on its own slice. */
static void layers_case(hipStream_t s) {
  const int L = 3, B = 4, H_q = 16, H_kv = 4, d = 64, T_max = 900;
  const int32_t lens[4] = {900, 17, 0, 450};
  int64_t offs[5] = {0};
  for (int b = 0; b < B; ++b) offs[b + 1] = offs[b] + lens[b];
  const size_t per_layer = (size_t)offs[B] * H_kv * d, nq = (size_t)B * H_q * d;
  uint16_t* q = (uint16_t*)malloc(L * nq * 2);
  uint16_t* k = (uint16_t*)malloc(L * per_layer * 2);
  uint16_t* v = (uint16_t*)malloc(L * per_layer * 2);
  fill(q, L * nq, 101);
  fill(k, L * per_layer, 102);
  fill(v, L * per_layer, 103);
  const float scale = 0.125f;
  gqa_dims dm = make_dims(B, H_q, H_kv, d, T_max);
  const size_t ws_bytes = gqa_decode_workspace_bytes(&dm, L);
  void *dq = to_device(q, L * nq * 2), *dk = to_device(k, L * per_layer * 2), *dv = to_device(v, L * per_layer * 2);
  void *doffs = to_device(offs, sizeof offs), *dl = to_device(lens, sizeof lens);
  void *dout = to_device(NULL, L * nq * 4), *ws = to_device(NULL, ws_bytes);
  const gqa_status st = gqa_decode_layers(L, dq, dk, dv, (const int64_t*)doffs, (const int32_t*)dl, scale, dout,
                                          &dm, ws, ws_bytes, s);
  HIP_OK(hipStreamSynchronize(s));
  float* out = (float*)malloc(L * nq * 4);
  HIP_OK(hipMemcpy(out, dout, L * nq * 4, hipMemcpyDeviceToHost));
  double* ref = (double*)malloc(nq * sizeof(double));
  double e = 0.0;
  int rc = 0;
  for (int l = 0; l < L && rc == 0; ++l) {
    rc = oracle_gqa_decode(B, H_q, H_kv, d, 1, q + l * nq, k + l * per_layer, v + l * per_layer, offs, lens,
                           (double)scale, 0, NULL, ref);
    const double el = max_err(out + l * nq, ref, nq);
    if (el > e) e = el;
  }
  char msg[256];
  snprintf(msg, sizeof msg, "gqa_decode_layers (3 layers, packed, a sequence of 0 tokens): status %s, "
           "max |gpu - oracle| = %.3e (bar 2e-3)", gqa_status_string(st), e);
  check(st == GQA_OK && rc == 0 && e <= 2e-3, msg);
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(doffs));
  HIP_OK(hipFree(dl));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(ws));
  free(q);
  free(k);
  free(v);
  free(out);
  free(ref);
}

/* Argument errors come back as status codes, and a rejected call writes
 * nothing: the output buffer keeps its sentinel bytes. */
static void error_cases(hipStream_t s) {
  const int B = 2, H_q = 32, H_kv = 8, d = 128, T_max = 4096;
  gqa_dims dm = make_dims(B, H_q, H_kv, d, T_max);
  const int32_t lens[2] = {4096, 4096};
  const size_t nq = (size_t)B * H_q * d, nkv = (size_t)B * H_kv * T_max * d;
  void *dq = to_device(NULL, nq * 2), *dk = to_device(NULL, nkv * 2), *dv = to_device(NULL, nkv * 2);
  void *dl = to_device(lens, sizeof lens), *dout = to_device(NULL, nq * 4);
  HIP_OK(hipMemset(dout, 0x7f, nq * 4));
  int32_t chunk = -1, groups = -1;
  const gqa_status sp = gqa_decode_plan(&dm, 1, &chunk, &groups);
  char msg[256];
  snprintf(msg, sizeof msg, "gqa_decode_plan: status %s, %d workgroups, forced span %d", gqa_status_string(sp),
           groups, chunk);
  check(sp == GQA_OK && groups >= 1 && chunk == 0, msg);
  const size_t need = gqa_decode_workspace_bytes(&dm, 1);
  void* ws = to_device(NULL, need);
  const gqa_status s1 = gqa_decode(dq, dk, dv, (const int32_t*)dl, 0.1f, dout, &dm, ws, need / 2, s);
  const gqa_status s2 = gqa_decode(dq, NULL, dv, (const int32_t*)dl, 0.1f, dout, &dm, ws, need, s);
  gqa_dims bad = dm;
  bad.head_dim = 96;
  const gqa_status s3 = gqa_decode(dq, dk, dv, (const int32_t*)dl, 0.1f, dout, &bad, ws, need, s);
  HIP_OK(hipStreamSynchronize(s));
  unsigned char* out = (unsigned char*)malloc(nq * 4);
  HIP_OK(hipMemcpy(out, dout, nq * 4, hipMemcpyDeviceToHost));
  int untouched = 1;
  for (size_t i = 0; i < nq * 4; ++i) untouched &= out[i] == 0x7f;
  snprintf(msg, sizeof msg, "errors: half workspace -> %s, null k_cache -> %s, d = 96 -> %s, output untouched: %d",
           gqa_status_string(s1), gqa_status_string(s2), gqa_status_string(s3), untouched);
  check(need > 0 && s1 == GQA_ERR_WORKSPACE && s2 == GQA_ERR_INVALID_ARG && s3 == GQA_ERR_UNSUPPORTED && untouched,
        msg);
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dl));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(ws));
  free(out);
}

/* One host thread's calls: its own inputs, stream and workspace. */
typedef struct {
  int B, H_q, H_kv, d, T_max;
  int32_t lens[4];
  uint64_t seed;
  uint16_t *q, *k, *v;
  float* out;
  gqa_status st[3];
} thread_case;

static void* thread_calls(void* arg) {
  thread_case* c = (thread_case*)arg;
  const size_t nq = (size_t)c->B * c->H_q * c->d, nkv = (size_t)c->B * c->H_kv * c->T_max * c->d;
  gqa_dims dm = make_dims(c->B, c->H_q, c->H_kv, c->d, c->T_max);
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  const size_t ws_bytes = gqa_decode_workspace_bytes(&dm, 1);
  void *dq = to_device(c->q, nq * 2), *dk = to_device(c->k, nkv * 2), *dv = to_device(c->v, nkv * 2);
  void *dl = to_device(c->lens, (size_t)c->B * 4), *dout = to_device(NULL, nq * 4), *ws = to_device(NULL, ws_bytes);
  for (int r = 0; r < 3; ++r)
    c->st[r] = gqa_decode(dq, dk, dv, (const int32_t*)dl, 1.0f / sqrtf((float)c->d), dout, &dm, ws, ws_bytes, s);
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(c->out, dout, nq * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dl));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(ws));
  HIP_OK(hipStreamDestroy(s));
  return NULL;
}

static void threads_case(void) {
  thread_case cs[4] = {
      {2, 32, 8, 128, 3000, {3000, 2500, 0, 0}, 41, NULL, NULL, NULL, NULL, {0}},
      {3, 32, 1, 128, 1500, {1500, 700, 1, 0}, 42, NULL, NULL, NULL, NULL, {0}},
      {4, 16, 2, 64, 900, {900, 1, 450, 899}, 43, NULL, NULL, NULL, NULL, {0}},
      {1, 64, 8, 128, 5000, {4999, 0, 0, 0}, 44, NULL, NULL, NULL, NULL, {0}},
  };
  pthread_t th[4];
  for (int i = 0; i < 4; ++i) {
    thread_case* c = &cs[i];
    const size_t nq = (size_t)c->B * c->H_q * c->d, nkv = (size_t)c->B * c->H_kv * c->T_max * c->d;
    c->q = (uint16_t*)malloc(nq * 2);
    c->k = (uint16_t*)malloc(nkv * 2);
    c->v = (uint16_t*)malloc(nkv * 2);
    c->out = (float*)malloc(nq * 4);
    fill(c->q, nq, c->seed);
    fill(c->k, nkv, c->seed + 1);
    fill(c->v, nkv, c->seed + 2);
  }
  for (int i = 0; i < 4; ++i)
    if (pthread_create(&th[i], NULL, thread_calls, &cs[i]) != 0) {
      fprintf(stderr, "pthread_create failed\n");
      exit(2);
    }
  for (int i = 0; i < 4; ++i) pthread_join(th[i], NULL);
  double e = 0.0;
  int ok = 1;
  for (int i = 0; i < 4; ++i) {
    thread_case* c = &cs[i];
    const size_t nq = (size_t)c->B * c->H_q * c->d;
    int64_t offs[5];
    for (int b = 0; b <= c->B; ++b) offs[b] = (int64_t)b * c->T_max;
    double* ref = (double*)malloc(nq * sizeof(double));
    const float scale = 1.0f / sqrtf((float)c->d);
    const int rc = oracle_gqa_decode(c->B, c->H_q, c->H_kv, c->d, 1, c->q, c->k, c->v, offs, c->lens, (double)scale,
                                     0, NULL, ref);
    const double ei = rc == 0 ? max_err(c->out, ref, nq) : INFINITY;
    if (ei > e) e = ei;
    for (int r = 0; r < 3; ++r) ok &= c->st[r] == GQA_OK;
    ok &= rc == 0;
    free(ref);
    free(c->q);
    free(c->k);
    free(c->v);
    free(c->out);
  }
  char msg[256];
  snprintf(msg, sizeof msg, "four host threads, first calls of the process at once (own streams and workspaces): "
           "statuses %s, max |gpu - oracle| = %.3e (bar 2e-3)", ok ? "GQA_OK" : "not all GQA_OK", e);
  check(ok && e <= 2e-3, msg);
}

int main(void) {
  int n = 0;
  HIP_OK(hipGetDeviceCount(&n));
  if (n < 1) {
    fprintf(stderr, "no GPU\n");
    return 2;
  }
  HIP_OK(hipSetDevice(0));
  threads_case();
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  {
    /* ragged lengths: the planner's split cuts the long units across workgroups */
    const int32_t lens[3] = {3000, 1, 1777};
    dense_case(3, 32, 8, 128, 3000, lens, 11, s, 0, "gqa_decode (B 3, H_q 32, H_kv 8, d 128, ragged)");
  }
  {
    const int32_t lens[2] = {2000, 1200};
    dense_case(2, 32, 1, 128, 2000, lens, 21, s, 0, "gqa_decode (MQA, G 32)");
  }
  {
    const int32_t lens[4] = {4096, 4096, 4096, 4096};
    dense_case(4, 32, 8, 128, 4096, lens, 31, s, 1, "gqa_decode_noalloc (B 4, T 4096)");
    const int32_t lens2[2] = {700, 64};
    dense_case(2, 16, 2, 64, 700, lens2, 32, s, 1, "gqa_decode_noalloc again, smaller (B 2, d 64)");
  }
  layers_case(s);
  error_cases(s);
  HIP_OK(hipStreamDestroy(s));
  printf("%s\n", failures ? "C ABI CHECK FAILED" : "C ABI CHECK OK");
  return failures ? 1 : 0;
}
