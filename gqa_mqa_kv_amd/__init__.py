"""MI355X (gfx950) grouped-query-attention decode step behind a C ABI.

The computation ("Grouped-Query Attention (GQA) and Multi-Query Attention
(MQA): Mathematical Foundations, Arithmetic Intensity, and KV-Cache Scaling
Mechanics", section 2): each query head i attends over its sequence's cached
tokens with the key/value head g = i / G of its contiguous group.  All work
runs in hand-written HIP kernels (gqa_mqa_kv_amd/csrc); Python only marshals
arguments.  See include/gqa_decode.h for the ABI.

    from gqa_mqa_kv_amd import decode, decode_layers, decode_paged, decode_fp8, append_rope

append_rope is the step before a decode step: it turns the new token's
queries and keys by the rotary position embedding of section 4 of the same
page and appends its key and value to the cache.  decode_paged reads a cache
held in fixed-size pages of a pool through a per-sequence table of page ids
(append_rope_paged appends to such a cache).
decode_fp8 reads a cache of one-byte E4M3 elements with one scale for the
keys and one for the values (the bytes-per-element term of section 1 of the
same page, halved); decode_layers_fp8 does the same for the layer-batched
call.
"""
from ._binding import (GqaDims, GqaError, Prepared, append_rope, append_rope_fp8, append_rope_paged,
                       append_rope_paged_fp8, decode, decode_append_rope, decode_append_rope_fp8, decode_append_rope_paged, decode_append_rope_paged_fp8, decode_fp8, decode_layers, decode_noalloc, decode_layers_fp8, decode_paged,
                       decode_paged_fp8, default_workspace, hbm_read_probe, lib, make_dims, plan, prepare, prepare_append,
                       prepare_decode_append, prepare_decode_append_fp8, prepare_decode_append_paged, prepare_decode_append_paged_fp8, prepare_append_fp8, prepare_append_paged_fp8, prepare_append_paged, prepare_fp8, prepare_layers_fp8, prepare_paged, prepare_paged_fp8, status_string,
                       workspace_bytes)

__all__ = ["GqaDims", "GqaError", "Prepared", "prepare", "decode", "decode_append_rope", "decode_append_rope_fp8", "decode_append_rope_paged", "decode_append_rope_paged_fp8", "decode_layers", "decode_noalloc", "decode_layers_fp8",
           "decode_paged", "decode_fp8", "decode_paged_fp8", "hbm_read_probe", "append_rope", "append_rope_fp8", "append_rope_paged",
           "append_rope_paged_fp8", "default_workspace", "lib", "make_dims", "plan", "prepare_append", "prepare_decode_append", "prepare_decode_append_fp8", "prepare_decode_append_paged", "prepare_decode_append_paged_fp8", "prepare_append_fp8", "prepare_append_paged_fp8", "prepare_append_paged", "prepare_fp8",
           "prepare_layers_fp8", "prepare_paged", "prepare_paged_fp8", "status_string", "workspace_bytes"]
