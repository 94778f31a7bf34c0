/*
 * gqa_probe.h -- measurement kernels of the MI355X (gfx950) GQA decode
 * library (same shared library as gqa_decode.h).
 *
 * "Grouped-Query Attention (GQA) and Multi-Query Attention (MQA):
 * Mathematical Foundations, Arithmetic Intensity, and KV-Cache Scaling
 * Mechanics", section 1 ("Arithmetic Intensity in Autoregressive Decoding"),
 * places a decode step far below the roofline's balance point: its time is
 * the time to stream the KV cache out of HBM once.  The probe below measures
 * what a plain read of a buffer achieves on this part, the ceiling a decode
 * step that reads the same bytes can approach.
 */
#ifndef GQA_PROBE_H
#define GQA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "gqa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `a_bytes` bytes at `a` and then `b_bytes` bytes at `b` once, in one
 * launch, with 16-byte non-temporal vector loads (the loads of the decode
 * kernels), and nothing else.  The two buffers form one stream (a, then b)
 * cut into equal contiguous spans, one per workgroup, as the decode kernel's
 * token split cuts the K and V it reads; each thread issues its loads in
 * rounds of eight and issues the next round before folding the current
 * one, so eight to sixteen loads are in flight.  What a wavefront reads is
 * folded by XOR and stored to *sink only when the fold equals one fixed
 * word, so that no load can be dropped and no workgroups contend for the
 * sink (the value left in *sink means nothing; it may stay untouched).
 *   a, b              : device memory, 16-byte aligned; caller-owned, only
 *                       read.  b may be NULL when b_bytes is 0.
 *   a_bytes, b_bytes  : multiples of 16 (both 0: a no-op)
 *   workgroups_per_cu : 1 to 8 workgroups of 256 threads per compute unit
 *   sink              : one device uint32, caller-owned, 4-byte aligned
 *   stream            : hipStream_t (NULL: the default stream)
 * Enqueues one kernel and returns; GQA_ERR_INVALID_ARG for a null or
 * misaligned pointer, a size that is not a multiple of 16 or
 * workgroups_per_cu out of range, GQA_ERR_LAUNCH if the runtime refuses the
 * launch.  Reentrant.
 */
gqa_status gqa_hbm_read_probe(const void* a, size_t a_bytes, const void* b, size_t b_bytes,
                              int32_t workgroups_per_cu, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PROBE_H */
