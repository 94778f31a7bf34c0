"""ctypes binding of include/gqa_decode.h (argument marshalling only).

Every step of the decode runs in the HIP library; this module only turns
torch tensors into device pointers and a gqa_dims struct, provides a zeroed
workspace, and raises on a non-zero status.  It never falls back to any other
implementation: when the built library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import build as _build

GQA_DTYPE = {torch.float32: 0, torch.bfloat16: 1}
PATHS = {"auto": 0, "valu": 1, "mfma": 2}
MERGES = {"auto": 0, "fused": 1, "kernel": 2}
STATUS = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_UNSUPPORTED", 3: "GQA_ERR_WORKSPACE",
          4: "GQA_ERR_LAUNCH", 5: "GQA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20   # GQA_NOALLOC_SCRATCH_BYTES
SYMBOLS = ("gqa_append_rope", "gqa_append_rope_fp8", "gqa_append_rope_paged", "gqa_append_rope_paged_fp8",
           "gqa_decode", "gqa_decode_append_rope", "gqa_decode_append_rope_fp8", "gqa_decode_append_rope_paged",
           "gqa_decode_append_rope_paged_fp8", "gqa_decode_fp8", "gqa_decode_layers", "gqa_decode_layers_fp8",
           "gqa_decode_paged",
           "gqa_decode_paged_fp8", "gqa_decode_noalloc",
           "gqa_decode_workspace_bytes", "gqa_decode_plan", "gqa_status_string",
           "gqa_hbm_read_probe")


class GqaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_seq_len", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("seq_len_hint", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("path", ctypes.c_int32), ("workgroup_waves", ctypes.c_int32),
                ("tiles_in_flight", ctypes.c_int32), ("merge", ctypes.c_int32),
                ("workgroups_per_cu", ctypes.c_int32)]


class GqaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = _build.LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError("HIP library not built: %s is missing (run gqa_mqa_kv_amd/build.py or "
                               "__graft_entry__.build())" % path)
        L = ctypes.CDLL(path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dims_p = ctypes.POINTER(GqaDims)
        L.gqa_decode.restype = ctypes.c_int
        L.gqa_decode.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, dims_p, vp, sz, vp]
        L.gqa_decode_noalloc.restype = ctypes.c_int
        L.gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, dims_p, vp]
        L.gqa_decode_layers.restype = ctypes.c_int
        L.gqa_decode_layers.argtypes = [i32, vp, vp, vp, vp, vp, ctypes.c_float, vp, dims_p, vp, sz, vp]
        L.gqa_decode_append_rope.restype = ctypes.c_int
        L.gqa_decode_append_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp, vp,
                                             dims_p, vp, sz, vp]
        L.gqa_decode_append_rope_paged.restype = ctypes.c_int
        L.gqa_decode_append_rope_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, ctypes.c_float,
                                                   ctypes.c_float, vp, vp, dims_p, vp, sz, vp]
        f = ctypes.c_float
        L.gqa_decode_append_rope_fp8.restype = ctypes.c_int
        L.gqa_decode_append_rope_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f, f, f, f, vp, vp, dims_p, vp, sz,
                                                 vp]
        L.gqa_decode_append_rope_paged_fp8.restype = ctypes.c_int
        L.gqa_decode_append_rope_paged_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, f, f, f, f, vp, vp,
                                                       dims_p, vp, sz, vp]
        L.gqa_decode_layers_fp8.restype = ctypes.c_int
        L.gqa_decode_layers_fp8.argtypes = [i32, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                            vp, dims_p, vp, sz, vp]
        L.gqa_decode_paged.restype = ctypes.c_int
        L.gqa_decode_paged.argtypes = [vp, vp, vp, vp, i32, i32, vp, ctypes.c_float, vp, dims_p, vp, sz, vp]
        L.gqa_decode_paged_fp8.restype = ctypes.c_int
        L.gqa_decode_paged_fp8.argtypes = [vp, vp, vp, vp, i32, i32, vp, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_float, vp, dims_p, vp, sz, vp]
        L.gqa_decode_fp8.restype = ctypes.c_int
        L.gqa_decode_fp8.argtypes = [vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, ctypes.c_float, vp, dims_p, vp,
                                     sz, vp]
        L.gqa_decode_workspace_bytes.restype = sz
        L.gqa_decode_workspace_bytes.argtypes = [dims_p, i32]
        L.gqa_decode_plan.restype = ctypes.c_int
        L.gqa_decode_plan.argtypes = [dims_p, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.gqa_append_rope.restype = ctypes.c_int
        L.gqa_append_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, dims_p, vp]
        L.gqa_append_rope_paged.restype = ctypes.c_int
        L.gqa_append_rope_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, ctypes.c_float, vp, dims_p, vp]
        f32 = ctypes.c_float
        L.gqa_append_rope_fp8.restype = ctypes.c_int
        L.gqa_append_rope_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, f32, f32, vp, dims_p, vp]
        L.gqa_append_rope_paged_fp8.restype = ctypes.c_int
        L.gqa_append_rope_paged_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, f32, f32, f32, vp, dims_p, vp]
        L.gqa_hbm_read_probe.restype = ctypes.c_int
        L.gqa_hbm_read_probe.argtypes = [vp, sz, vp, sz, i32, vp, vp]
        L.gqa_status_string.restype = ctypes.c_char_p
        L.gqa_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gqa_status_string(status).decode()


def _check(status: int):
    if status != 0:
        raise GqaError(status, status_string(status))


def make_dims(B, H_q, H_kv, d, T_max, dtype, out_dtype=None, seq_len_hint=0, chunk_tokens=0,
              path="auto", waves=0, tiles=0, merge="auto", per_cu=0) -> GqaDims:
    if dtype not in GQA_DTYPE or (out_dtype is not None and out_dtype not in GQA_DTYPE):
        raise TypeError("dtypes must be float32 or bfloat16")
    return GqaDims(int(B), int(H_q), int(H_kv), int(d), int(T_max), GQA_DTYPE[dtype],
                   GQA_DTYPE[out_dtype if out_dtype is not None else dtype], int(seq_len_hint),
                   int(chunk_tokens), PATHS[path], int(waves), int(tiles), MERGES[merge], int(per_cu))


def workspace_bytes(dims: GqaDims, num_layers: int = 1) -> int:
    return int(lib().gqa_decode_workspace_bytes(ctypes.byref(dims), int(num_layers)))


def plan(dims: GqaDims, num_layers: int = 1):
    """The library's work split: (tokens per workgroup or 0 for an even split,
    workgroups) on the matrix-core path; (tokens per chunk, chunks of the
    longest sequence) on the vector path."""
    c, n = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().gqa_decode_plan(ctypes.byref(dims), int(num_layers), ctypes.byref(c), ctypes.byref(n)))
    return c.value, n.value


_workspaces = {}   # (device type, device index, stream handle) -> zero-filled workspace
_retired = []      # workspaces replaced by larger ones: kept alive for the life of the process


def _stream_handle(device: torch.device, stream) -> int:
    return int(torch.cuda.current_stream(device).cuda_stream if stream is None else stream)


def default_workspace(nbytes: int, device: torch.device, stream=None) -> Optional[torch.Tensor]:
    """A zero-filled device buffer of at least ``nbytes`` (256-byte aligned),
    cached per (device, stream): calls on one stream are ordered, so they may
    share it (the library leaves its arrival counters at zero after each
    call), while calls on different streams, which may overlap in time, get
    buffers of their own.  ``stream``: a hipStream_t handle (None: the
    current stream).  A buffer is zero-filled on the stream that uses it.  A
    buffer replaced by a larger one is never freed: a kernel still running on
    that stream, or a captured graph, may hold its address.  Sizes are
    rounded up to a power of two, so a stream replaces its buffer a few
    times at most.  Every stream used keeps its buffer for the life of the
    process (the handle says nothing of when the stream is destroyed): a
    caller that creates streams per call should pass ``workspace=`` (a
    zero-filled buffer of ``workspace_bytes(dims)`` bytes it owns) instead."""
    if nbytes == 0:
        return None
    s = _stream_handle(device, stream)
    key = (device.type, device.index, s)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        size = 1 << (int(nbytes) - 1).bit_length()
        if s == int(torch.cuda.current_stream(device).cuda_stream):
            new = torch.zeros(size, dtype=torch.uint8, device=device)
        else:
            with torch.cuda.stream(torch.cuda.ExternalStream(s, device=device)):
                new = torch.zeros(size, dtype=torch.uint8, device=device)
        if ws is not None:
            _retired.append(ws)
        _workspaces[key] = ws = new
    return ws


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(t: torch.Tensor, name: str, device: torch.device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s must be on %s (got %s)" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _decode_args(q, k_cache, v_cache, seq_lens, scale, out, out_dtype, chunk_tokens, path, seq_len_hint, workspace,
                 stream, waves, tiles, merge, per_cu):
    """Validated arguments of gqa_decode (nothing is enqueued)."""
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _require(t, n, dev)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,H_q,d] and k/v [B,H_kv,T_max,d]")
    B, H_q, d = q.shape
    _, H_kv, T_max, _ = k_cache.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != d or seq_lens.shape != (B,) or seq_lens.dtype != torch.int32:
        raise ValueError("shape mismatch between q, caches and seq_lens")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    dims = make_dims(B, H_q, H_kv, d, T_max, q.dtype, out_dtype, seq_len_hint, chunk_tokens, path, waves, tiles, merge,
                     per_cu)
    if out is None:
        out = torch.empty(B, H_q, d, dtype=out_dtype or q.dtype, device=dev)
    _require(out, "out", dev)
    if out.shape != (B, H_q, d) or GQA_DTYPE.get(out.dtype) != dims.out_dtype:
        raise ValueError("out must be [B,H_q,d] of the output dtype")
    s = _stream_handle(dev, stream)
    ws = default_workspace(workspace_bytes(dims), dev, s) if workspace is None else workspace
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), float(scale), _ptr(out), ctypes.byref(dims),
            _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), s)
    return args, (out, q, k_cache, v_cache, seq_lens, ws, dims)


def decode(q, k_cache, v_cache, seq_lens, scale: float, out=None, out_dtype=None, chunk_tokens: int = 0,
           path: str = "auto", seq_len_hint: int = 0, workspace=None, stream=None, waves: int = 0,
           tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """One decode step of one layer.  q [B,H_q,d]; k_cache/v_cache
    [B,H_kv,T_max,d]; seq_lens int32 [B] on the same device.  Returns out
    [B,H_q,d] (dtype ``out_dtype``, default q's)."""
    args, keep = _decode_args(q, k_cache, v_cache, seq_lens, scale, out, out_dtype, chunk_tokens, path, seq_len_hint,
                              workspace, stream, waves, tiles, merge, per_cu)
    _check(lib().gqa_decode(*args))
    return keep[0]


def decode_noalloc(q, k_cache, v_cache, seq_lens, scale: float, out=None, out_dtype=None, chunk_tokens: int = 0,
                   path: str = "auto", seq_len_hint: int = 0, stream=None, waves: int = 0, tiles: int = 0,
                   merge: str = "auto", per_cu: int = 0):
    """decode through gqa_decode_noalloc: the partial states live in the
    library's static device buffer (GQA_NOALLOC_SCRATCH_BYTES per GPU), so
    the call allocates nothing on the device beyond ``out`` when ``out`` is
    None (pass ``out`` to allocate nothing at all).  Calls that may overlap in
    time on one GPU race on that buffer."""
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _require(t, n, dev)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,H_q,d] and k/v [B,H_kv,T_max,d]")
    B, H_q, d = q.shape
    _, H_kv, T_max, _ = k_cache.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != d or seq_lens.shape != (B,) or seq_lens.dtype != torch.int32:
        raise ValueError("shape mismatch between q, caches and seq_lens")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    dims = make_dims(B, H_q, H_kv, d, T_max, q.dtype, out_dtype, seq_len_hint, chunk_tokens, path, waves, tiles,
                     merge, per_cu)
    if out is None:
        out = torch.empty(B, H_q, d, dtype=out_dtype or q.dtype, device=dev)
    _require(out, "out", dev)
    if out.shape != (B, H_q, d) or GQA_DTYPE.get(out.dtype) != dims.out_dtype:
        raise ValueError("out must be [B,H_q,d] of the output dtype")
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    _check(lib().gqa_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), float(scale), _ptr(out),
                                    ctypes.byref(dims), s))
    return out


def hbm_read_probe(a: torch.Tensor, workgroups_per_cu: int, sink: torch.Tensor, stream=None, b=None):
    """Enqueue gqa_hbm_read_probe: one plain read of tensor ``a`` and then of
    tensor ``b`` (optional), contiguous device tensors, in one launch, with
    ``workgroups_per_cu`` workgroups per CU; ``sink`` is a one-element int32
    device tensor the kernel folds what it reads into.  Measurement only."""
    dev = a.device
    _require(a, "a", dev)
    _require(sink, "sink", dev)
    if b is not None:
        _require(b, "b", dev)
    if sink.dtype != torch.int32 or sink.numel() < 1:
        raise ValueError("sink must be an int32 device tensor")
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    nb = 0 if b is None else b.numel() * b.element_size()
    _check(lib().gqa_hbm_read_probe(_ptr(a), a.numel() * a.element_size(), _ptr(b), nb, int(workgroups_per_cu),
                                    _ptr(sink), s))


def _paged_args(q, k_pool, v_pool, block_table, seq_lens, scale, out, out_dtype, max_seq_len, chunk_tokens,
                seq_len_hint, workspace, stream, tiles, merge, per_cu, scales=None):
    dev = q.device
    for t, n in ((q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool"), (block_table, "block_table"),
                 (seq_lens, "seq_lens")):
        _require(t, n, dev)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape or block_table.dim() != 2:
        raise ValueError("expected q [B,H_q,d], k/v pools [num_pages,H_kv,page,d] and block_table [B,max_pages]")
    B, H_q, d = q.shape
    _, H_kv, page, _ = k_pool.shape
    max_pages = block_table.shape[1]
    if (k_pool.shape[3] != d or block_table.shape[0] != B or block_table.dtype != torch.int32
            or seq_lens.shape != (B,) or seq_lens.dtype != torch.int32):
        raise ValueError("shape mismatch between q, pools, block_table and seq_lens")
    if scales is None and (k_pool.dtype != q.dtype or v_pool.dtype != q.dtype):
        raise TypeError("q, k_pool and v_pool must share one dtype")
    if scales is not None and (q.dtype != torch.bfloat16 or k_pool.dtype not in E4M3_DTYPES
                               or v_pool.dtype not in E4M3_DTYPES):
        raise TypeError("expected bf16 q and one-byte E4M3 pools (uint8 or float8_e4m3fn)")
    T = max_pages * page if max_seq_len is None else int(max_seq_len)
    dims = make_dims(B, H_q, H_kv, d, T, q.dtype, out_dtype, seq_len_hint, chunk_tokens, "mfma", 0, tiles, merge,
                     per_cu)
    if out is None:
        out = torch.empty(B, H_q, d, dtype=out_dtype or q.dtype, device=dev)
    _require(out, "out", dev)
    if out.shape != (B, H_q, d) or GQA_DTYPE.get(out.dtype) != dims.out_dtype:
        raise ValueError("out must be [B,H_q,d] of the output dtype")
    s = _stream_handle(dev, stream)
    ws = default_workspace(workspace_bytes(dims), dev, s) if workspace is None else workspace
    sc = (float(scale),) if scales is None else (float(scale), float(scales[0]), float(scales[1]))
    args = (_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), int(max_pages), int(page), _ptr(seq_lens)) + \
        sc + (_ptr(out), ctypes.byref(dims), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), s)
    return args, (out, q, k_pool, v_pool, block_table, seq_lens, ws, dims)


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale: float, out=None, out_dtype=None,
                 max_seq_len: Optional[int] = None, chunk_tokens: int = 0, seq_len_hint: int = 0, workspace=None,
                 stream=None, tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """One decode step of one layer whose cache lives in pages of a pool.
    q [B,H_q,d]; k_pool/v_pool [num_pages,H_kv,page,d]; block_table int32
    [B,max_pages] (token t of sequence b in page block_table[b, t // page]);
    seq_lens int32 [B].  max_seq_len defaults to max_pages * page.  Returns
    out [B,H_q,d]."""
    args, keep = _paged_args(q, k_pool, v_pool, block_table, seq_lens, scale, out, out_dtype, max_seq_len,
                             chunk_tokens, seq_len_hint, workspace, stream, tiles, merge, per_cu)
    _check(lib().gqa_decode_paged(*args))
    return keep[0]


E4M3_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _fp8_args(q, k8, v8, seq_lens, scale, k_scale, v_scale, out, out_dtype, chunk_tokens, seq_len_hint, workspace,
              stream, tiles, merge, per_cu):
    dev = q.device
    for t, n in ((q, "q"), (k8, "k_cache"), (v8, "v_cache"), (seq_lens, "seq_lens")):
        _require(t, n, dev)
    if q.dim() != 3 or k8.dim() != 4 or v8.shape != k8.shape:
        raise ValueError("expected q [B,H_q,d] and k/v [B,H_kv,T_max,d]")
    if q.dtype != torch.bfloat16 or k8.dtype not in E4M3_DTYPES or v8.dtype not in E4M3_DTYPES:
        raise TypeError("expected bf16 q and one-byte E4M3 caches (uint8 or float8_e4m3fn)")
    B, H_q, d = q.shape
    _, H_kv, T_max, _ = k8.shape
    if k8.shape[0] != B or k8.shape[3] != d or seq_lens.shape != (B,) or seq_lens.dtype != torch.int32:
        raise ValueError("shape mismatch between q, caches and seq_lens")
    dims = make_dims(B, H_q, H_kv, d, T_max, q.dtype, out_dtype, seq_len_hint, chunk_tokens, "mfma", 0, tiles, merge,
                     per_cu)
    if out is None:
        out = torch.empty(B, H_q, d, dtype=out_dtype or q.dtype, device=dev)
    _require(out, "out", dev)
    if out.shape != (B, H_q, d) or GQA_DTYPE.get(out.dtype) != dims.out_dtype:
        raise ValueError("out must be [B,H_q,d] of the output dtype")
    s = _stream_handle(dev, stream)
    ws = default_workspace(workspace_bytes(dims), dev, s) if workspace is None else workspace
    args = (_ptr(q), _ptr(k8), _ptr(v8), _ptr(seq_lens), float(scale), float(k_scale), float(v_scale), _ptr(out),
            ctypes.byref(dims), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), s)
    return args, (out, q, k8, v8, seq_lens, ws, dims)


def decode_fp8(q, k_cache, v_cache, seq_lens, scale: float, k_scale: float, v_scale: float, out=None, out_dtype=None,
               chunk_tokens: int = 0, seq_len_hint: int = 0, workspace=None, stream=None, tiles: int = 0,
               merge: str = "auto", per_cu: int = 0):
    """One decode step of one layer over one-byte OCP E4M3 caches: q bf16
    [B,H_q,d]; k_cache/v_cache uint8 or float8_e4m3fn [B,H_kv,T_max,d], a key
    (value) element standing for k_scale (v_scale) times its E4M3 value.
    Returns out [B,H_q,d]."""
    args, keep = _fp8_args(q, k_cache, v_cache, seq_lens, scale, k_scale, v_scale, out, out_dtype, chunk_tokens,
                           seq_len_hint, workspace, stream, tiles, merge, per_cu)
    _check(lib().gqa_decode_fp8(*args))
    return keep[0]


def decode_paged_fp8(q, k_pool, v_pool, block_table, seq_lens, scale: float, k_scale: float, v_scale: float,
                     out=None, out_dtype=None, max_seq_len: Optional[int] = None, chunk_tokens: int = 0,
                     seq_len_hint: int = 0, workspace=None, stream=None, tiles: int = 0, merge: str = "auto",
                     per_cu: int = 0):
    """decode_paged over pools of one-byte OCP E4M3 elements (uint8 or
    float8_e4m3fn [num_pages,H_kv,page,d]) with the scales of decode_fp8."""
    args, keep = _paged_args(q, k_pool, v_pool, block_table, seq_lens, scale, out, out_dtype, max_seq_len,
                             chunk_tokens, seq_len_hint, workspace, stream, tiles, merge, per_cu, (k_scale, v_scale))
    _check(lib().gqa_decode_paged_fp8(*args))
    return keep[0]


def _layers_args(q, k_cache, v_cache, seq_lens, scale, kv_offsets, max_seq_len, num_kv_heads, out, out_dtype,
                 chunk_tokens, path, seq_len_hint, workspace, stream, waves, tiles, merge, per_cu, scales=None):
    """Validated arguments of gqa_decode_layers, or of gqa_decode_layers_fp8
    when ``scales`` = (k_scale, v_scale)."""
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _require(t, n, dev)
    if q.dim() != 4:
        raise ValueError("q must be [L,B,H_q,d]")
    L, B, H_q, d = q.shape
    if kv_offsets is None:
        if k_cache.dim() != 5 or v_cache.shape != k_cache.shape or k_cache.shape[:2] != (L, B) or k_cache.shape[4] != d:
            raise ValueError("dense caches must be [L,B,H_kv,T_max,d]")
        H_kv, T_max = k_cache.shape[2], k_cache.shape[3]
    else:
        _require(kv_offsets, "kv_offsets", dev)
        if kv_offsets.dtype != torch.int64 or kv_offsets.shape != (B + 1,):
            raise ValueError("kv_offsets must be int64 [B+1]")
        if max_seq_len is None or num_kv_heads is None:
            raise ValueError("packed caches need max_seq_len and num_kv_heads")
        if v_cache.numel() != k_cache.numel() or k_cache.numel() % (L * num_kv_heads * d):
            raise ValueError("packed cache size mismatch")
        H_kv, T_max = num_kv_heads, max_seq_len
    if seq_lens.shape != (B,) or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32 [B]")
    if scales is None:
        if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
            raise TypeError("q, k_cache and v_cache must share one dtype")
    elif q.dtype != torch.bfloat16 or k_cache.dtype not in E4M3_DTYPES or v_cache.dtype not in E4M3_DTYPES:
        raise TypeError("expected bf16 q and one-byte E4M3 caches (uint8 or float8_e4m3fn)")
    dims = make_dims(B, H_q, H_kv, d, T_max, q.dtype, out_dtype, seq_len_hint, chunk_tokens, path, waves, tiles, merge,
                     per_cu)
    if out is None:
        out = torch.empty(L, B, H_q, d, dtype=out_dtype or q.dtype, device=dev)
    _require(out, "out", dev)
    if out.shape != (L, B, H_q, d) or GQA_DTYPE.get(out.dtype) != dims.out_dtype:
        raise ValueError("out must be [L,B,H_q,d] of the output dtype")
    s = _stream_handle(dev, stream)
    ws = default_workspace(workspace_bytes(dims, L), dev, s) if workspace is None else workspace
    sc = () if scales is None else (float(scales[0]), float(scales[1]))
    args = (int(L), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_offsets), _ptr(seq_lens), float(scale)) + sc + (
        _ptr(out), ctypes.byref(dims), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), s)
    return args, (out, q, k_cache, v_cache, kv_offsets, seq_lens, ws, dims)


def decode_layers(q, k_cache, v_cache, seq_lens, scale: float, kv_offsets=None, max_seq_len: Optional[int] = None,
                  num_kv_heads: Optional[int] = None, out=None, out_dtype=None, chunk_tokens: int = 0,
                  path: str = "auto", seq_len_hint: int = 0, workspace=None, stream=None, waves: int = 0,
                  tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """One decode step of L independent layers in one launch.  q [L,B,H_q,d].
    Dense caches are [L,B,H_kv,T_max,d]; with ``kv_offsets`` (int64 [B+1] on
    the device) the caches are packed (any shape holding L*kv_offsets[B]*H_kv*d
    elements), and ``max_seq_len`` (the largest capacity) and ``num_kv_heads``
    must be given."""
    args, keep = _layers_args(q, k_cache, v_cache, seq_lens, scale, kv_offsets, max_seq_len, num_kv_heads, out,
                              out_dtype, chunk_tokens, path, seq_len_hint, workspace, stream, waves, tiles, merge,
                              per_cu)
    _check(lib().gqa_decode_layers(*args))
    return keep[0]


def decode_layers_fp8(q, k_cache, v_cache, seq_lens, scale: float, k_scale: float, v_scale: float, kv_offsets=None,
                      max_seq_len: Optional[int] = None, num_kv_heads: Optional[int] = None, out=None,
                      out_dtype=None, chunk_tokens: int = 0, seq_len_hint: int = 0, workspace=None, stream=None,
                      tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """decode_layers over one-byte OCP E4M3 caches (uint8 or float8_e4m3fn, in
    the dense or packed layout), with the scales of decode_fp8 shared by every
    layer.  q bf16 [L,B,H_q,d]."""
    args, keep = _layers_args(q, k_cache, v_cache, seq_lens, scale, kv_offsets, max_seq_len, num_kv_heads, out,
                              out_dtype, chunk_tokens, "mfma", seq_len_hint, workspace, stream, 0, tiles, merge, per_cu,
                              (k_scale, v_scale))
    _check(lib().gqa_decode_layers_fp8(*args))
    return keep[0]


def _append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, kv_offsets, max_seq_len, q_out,
                 new_seq_lens, stream, scales):
    """Validated (function, arguments, tensors kept) of gqa_append_rope, or of
    gqa_append_rope_fp8 with ``scales`` (nothing is enqueued)."""
    dev = q.device
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (seq_lens, "seq_lens")):
        _require(t, n, dev)
    if q.dim() != 3 or k_new.dim() != 3 or v_new.shape != k_new.shape:
        raise ValueError("expected q [B,H_q,d] and k_new/v_new [B,H_kv,d]")
    B, H_q, d = q.shape
    H_kv = k_new.shape[1]
    if k_new.shape[0] != B or k_new.shape[2] != d or seq_lens.shape != (B,) or seq_lens.dtype != torch.int32:
        raise ValueError("shape mismatch between q, k_new/v_new and seq_lens")
    if kv_offsets is None:
        if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_cache.shape[:2] != (B, H_kv) or \
                k_cache.shape[3] != d:
            raise ValueError("dense caches must be [B,H_kv,T_max,d]")
        T_max = k_cache.shape[2]
    else:
        _require(kv_offsets, "kv_offsets", dev)
        if kv_offsets.dtype != torch.int64 or kv_offsets.shape != (B + 1,) or max_seq_len is None:
            raise ValueError("packed caches need kv_offsets int64 [B+1] and max_seq_len")
        if v_cache.numel() != k_cache.numel() or k_cache.numel() % (H_kv * d):
            raise ValueError("packed cache size mismatch")
        T_max = max_seq_len
    for t in (k_new, v_new) + (() if scales else (k_cache, v_cache)):
        if t.dtype != q.dtype:
            raise TypeError("q, k_new, v_new and the caches must share one dtype")
    if scales and (k_cache.dtype not in E4M3_DTYPES or v_cache.dtype not in E4M3_DTYPES):
        raise TypeError("E4M3 caches are uint8 or float8_e4m3fn")
    dims = make_dims(B, H_q, H_kv, d, T_max, q.dtype)
    if q_out is None:
        q_out = torch.empty_like(q)
    _require(q_out, "q_out", dev)
    if q_out.shape != q.shape or q_out.dtype != q.dtype:
        raise ValueError("q_out must match q")
    if new_seq_lens is None:
        new_seq_lens = torch.empty_like(seq_lens)
    _require(new_seq_lens, "new_seq_lens", dev)
    if new_seq_lens.shape != (B,) or new_seq_lens.dtype != torch.int32:
        raise ValueError("new_seq_lens must be int32 [B]")
    s = _stream_handle(dev, stream)
    head = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(kv_offsets), _ptr(seq_lens),
            _ptr(new_seq_lens), float(rope_base))
    if scales:
        fn, args = lib().gqa_append_rope_fp8, head + (float(scales[0]), float(scales[1]), _ptr(q_out),
                                                      ctypes.byref(dims), s)
    else:
        fn, args = lib().gqa_append_rope, head + (_ptr(q_out), ctypes.byref(dims), s)
    return fn, args, (q_out, new_seq_lens, q, k_new, v_new, k_cache, v_cache, seq_lens, kv_offsets, dims)


def append_rope(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base: float, kv_offsets=None,
                max_seq_len: Optional[int] = None, q_out=None, new_seq_lens=None, stream=None, scales=None):
    """Append each sequence's new token to one layer's cache with rotary
    position embedding at position seq_lens[b] (see gqa_append_rope in
    include/gqa_decode.h).  q [B,H_q,d]; k_new/v_new [B,H_kv,d]; caches dense
    [B,H_kv,T_max,d], or packed with ``kv_offsets`` (int64 [B+1]) and
    ``max_seq_len``.  Writes the caches in place; returns (q_out,
    new_seq_lens): the rotated queries (a new tensor unless ``q_out`` is
    given, which may be q itself) and the lengths after the append (a new
    int32 tensor unless ``new_seq_lens`` is given, which may be seq_lens)."""
    fn, args, keep = _append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, kv_offsets, max_seq_len,
                                  q_out, new_seq_lens, stream, scales)
    _check(fn(*args))
    return keep[0], keep[1]


def _decode_append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, scale, kv_offsets, max_seq_len, q_out,
                        new_seq_lens, out, out_dtype, chunk_tokens, workspace, stream, tiles, merge, per_cu,
                        scales=None):
    """Validated arguments of gqa_decode_append_rope, or of
    gqa_decode_append_rope_fp8 when ``scales`` = (k_scale, v_scale)."""
    dev = q.device
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (seq_lens, "seq_lens")):
        _require(t, n, dev)
    if q.dim() != 3 or k_new.dim() != 3 or v_new.shape != k_new.shape:
        raise ValueError("expected q [B,H_q,d] and k_new/v_new [B,H_kv,d]")
    B, H_q, d = q.shape
    H_kv = k_new.shape[1]
    if k_new.shape[0] != B or k_new.shape[2] != d or seq_lens.shape != (B,) or seq_lens.dtype != torch.int32:
        raise ValueError("shape mismatch between q, k_new/v_new and seq_lens")
    if kv_offsets is None:
        if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_cache.shape[:2] != (B, H_kv) or \
                k_cache.shape[3] != d:
            raise ValueError("dense caches must be [B,H_kv,T_max,d]")
        T_max = k_cache.shape[2]
    else:
        _require(kv_offsets, "kv_offsets", dev)
        if kv_offsets.dtype != torch.int64 or kv_offsets.shape != (B + 1,) or max_seq_len is None:
            raise ValueError("packed caches need kv_offsets int64 [B+1] and max_seq_len")
        if v_cache.numel() != k_cache.numel() or k_cache.numel() % (H_kv * d):
            raise ValueError("packed cache size mismatch")
        T_max = max_seq_len
    for t in (k_new, v_new) + (() if scales else (k_cache, v_cache)):
        if t.dtype != q.dtype:
            raise TypeError("q, k_new, v_new and the caches must share one dtype")
    if scales and (k_cache.dtype not in E4M3_DTYPES or v_cache.dtype not in E4M3_DTYPES):
        raise TypeError("E4M3 caches are uint8 or float8_e4m3fn")
    dims = make_dims(B, H_q, H_kv, d, T_max, q.dtype, out_dtype, 0, chunk_tokens, "mfma", 0, tiles, merge, per_cu)
    if q_out is None:
        q_out = torch.empty_like(q)
    lens_out = new_seq_lens is not False   # False: the grown lengths are not written
    if new_seq_lens is None or new_seq_lens is False:
        new_seq_lens = torch.empty_like(seq_lens) if lens_out else None
    if out is None:
        out = torch.empty(B, H_q, d, dtype=out_dtype or q.dtype, device=dev)
    for t, n in ((q_out, "q_out"), (new_seq_lens, "new_seq_lens"), (out, "out")):
        if t is not None:
            _require(t, n, dev)
    if q_out.shape != q.shape or q_out.dtype != q.dtype or \
            (lens_out and (new_seq_lens.shape != (B,) or new_seq_lens.dtype != torch.int32)):
        raise ValueError("q_out must match q and new_seq_lens seq_lens")
    if out.shape != (B, H_q, d) or GQA_DTYPE.get(out.dtype) != dims.out_dtype:
        raise ValueError("out must be [B,H_q,d] of the output dtype")
    s = _stream_handle(dev, stream)
    ws = default_workspace(workspace_bytes(dims), dev, s) if workspace is None else workspace
    sc = (float(scale),) if scales is None else (float(scale), float(scales[0]), float(scales[1]))
    args = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(kv_offsets), _ptr(seq_lens),
            _ptr(new_seq_lens), float(rope_base)) + sc + (_ptr(q_out), _ptr(out), ctypes.byref(dims), _ptr(ws),
                                                          0 if ws is None else ws.numel() * ws.element_size(), s)
    return args, (out, q_out, new_seq_lens, q, k_new, v_new, k_cache, v_cache, kv_offsets, seq_lens, ws, dims)


def decode_append_rope(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base: float, scale: float, kv_offsets=None,
                       max_seq_len: Optional[int] = None, q_out=None, new_seq_lens=None, out=None, out_dtype=None,
                       chunk_tokens: int = 0, workspace=None, stream=None, tiles: int = 0, merge: str = "auto",
                       per_cu: int = 0):
    """append_rope followed by decode (gqa_decode_append_rope): bf16 q
    [B,H_q,d], k_new/v_new [B,H_kv,d], a plain [B,H_kv,T_max,d] or packed
    (``kv_offsets``, ``max_seq_len``) cache written in place.  Returns (out,
    q_out, new_seq_lens); q_out and new_seq_lens are new tensors unless given
    (they may not be q and seq_lens).  ``new_seq_lens=False`` writes no
    lengths (returned as None); the call is then one kernel at every G (with
    lengths and G > 16 it is the append kernel and the decode)."""
    args, keep = _decode_append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, scale, kv_offsets,
                                     max_seq_len, q_out, new_seq_lens, out, out_dtype, chunk_tokens, workspace, stream,
                                     tiles, merge, per_cu)
    _check(lib().gqa_decode_append_rope(*args))
    return keep[0], keep[1], keep[2]


def _decode_append_paged_args(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base, scale, max_seq_len,
                              q_out, new_seq_lens, out, out_dtype, chunk_tokens, workspace, stream, tiles, merge,
                              per_cu, scales=None):
    """Validated arguments of gqa_decode_append_rope_paged, or of
    gqa_decode_append_rope_paged_fp8 when ``scales`` = (k_scale, v_scale)."""
    dev = q.device
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_pool, "k_pool"), (v_pool, "v_pool"),
                 (block_table, "block_table"), (seq_lens, "seq_lens")):
        _require(t, n, dev)
    if q.dim() != 3 or k_new.dim() != 3 or v_new.shape != k_new.shape or k_pool.dim() != 4 or \
            v_pool.shape != k_pool.shape or block_table.dim() != 2:
        raise ValueError("expected q [B,H_q,d], k_new/v_new [B,H_kv,d], pools [num_pages,H_kv,page,d] and "
                         "block_table [B,max_pages]")
    B, H_q, d = q.shape
    _, H_kv, page, _ = k_pool.shape
    max_pages = block_table.shape[1]
    if k_new.shape != (B, H_kv, d) or k_pool.shape[3] != d or block_table.shape[0] != B or \
            block_table.dtype != torch.int32 or seq_lens.shape != (B,) or seq_lens.dtype != torch.int32:
        raise ValueError("shape mismatch between q, k_new/v_new, pools, block_table and seq_lens")
    for t in (k_new, v_new) + (() if scales else (k_pool, v_pool)):
        if t.dtype != q.dtype:
            raise TypeError("q, k_new, v_new and the pools must share one dtype")
    if scales and (k_pool.dtype not in E4M3_DTYPES or v_pool.dtype not in E4M3_DTYPES):
        raise TypeError("E4M3 pools are uint8 or float8_e4m3fn")
    T = max_pages * page if max_seq_len is None else int(max_seq_len)
    dims = make_dims(B, H_q, H_kv, d, T, q.dtype, out_dtype, 0, chunk_tokens, "mfma", 0, tiles, merge, per_cu)
    if q_out is None:
        q_out = torch.empty_like(q)
    lens_out = new_seq_lens is not False
    if new_seq_lens is None or new_seq_lens is False:
        new_seq_lens = torch.empty_like(seq_lens) if lens_out else None
    if out is None:
        out = torch.empty(B, H_q, d, dtype=out_dtype or q.dtype, device=dev)
    for t, n in ((q_out, "q_out"), (new_seq_lens, "new_seq_lens"), (out, "out")):
        if t is not None:
            _require(t, n, dev)
    if q_out.shape != q.shape or q_out.dtype != q.dtype or \
            (lens_out and (new_seq_lens.shape != (B,) or new_seq_lens.dtype != torch.int32)):
        raise ValueError("q_out must match q and new_seq_lens seq_lens")
    if out.shape != (B, H_q, d) or GQA_DTYPE.get(out.dtype) != dims.out_dtype:
        raise ValueError("out must be [B,H_q,d] of the output dtype")
    s = _stream_handle(dev, stream)
    ws = default_workspace(workspace_bytes(dims), dev, s) if workspace is None else workspace
    sc = (float(scale),) if scales is None else (float(scale), float(scales[0]), float(scales[1]))
    args = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), int(max_pages),
            int(page), _ptr(seq_lens), _ptr(new_seq_lens), float(rope_base)) + sc + (
        _ptr(q_out), _ptr(out), ctypes.byref(dims), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), s)
    return args, (out, q_out, new_seq_lens, q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, ws, dims)


def decode_append_rope_paged(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base: float, scale: float,
                             max_seq_len: Optional[int] = None, q_out=None, new_seq_lens=None, out=None,
                             out_dtype=None, chunk_tokens: int = 0, workspace=None, stream=None, tiles: int = 0,
                             merge: str = "auto", per_cu: int = 0):
    """append_rope_paged followed by decode_paged (gqa_decode_append_rope_paged):
    bf16 q [B,H_q,d], k_new/v_new [B,H_kv,d], pools [num_pages,H_kv,page,d]
    written in place, block_table int32 [B,max_pages] (only read).  Returns
    (out, q_out, new_seq_lens) as decode_append_rope does (new_seq_lens=False:
    no lengths written, None returned)."""
    args, keep = _decode_append_paged_args(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base, scale,
                                           max_seq_len, q_out, new_seq_lens, out, out_dtype, chunk_tokens, workspace,
                                           stream, tiles, merge, per_cu)
    _check(lib().gqa_decode_append_rope_paged(*args))
    return keep[0], keep[1], keep[2]


def decode_append_rope_fp8(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base: float, scale: float,
                           k_scale: float, v_scale: float, kv_offsets=None, max_seq_len: Optional[int] = None,
                           q_out=None, new_seq_lens=None, out=None, out_dtype=None, chunk_tokens: int = 0,
                           workspace=None, stream=None, tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """decode_append_rope on caches of one-byte E4M3 codes (uint8 or
    float8_e4m3fn, plain or packed): append_rope_fp8 followed by decode_fp8
    (gqa_decode_append_rope_fp8).  Returns (out, q_out, new_seq_lens)."""
    args, keep = _decode_append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, scale, kv_offsets,
                                     max_seq_len, q_out, new_seq_lens, out, out_dtype, chunk_tokens, workspace, stream,
                                     tiles, merge, per_cu, (k_scale, v_scale))
    _check(lib().gqa_decode_append_rope_fp8(*args))
    return keep[0], keep[1], keep[2]


def decode_append_rope_paged_fp8(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base: float,
                                 scale: float, k_scale: float, v_scale: float, max_seq_len: Optional[int] = None,
                                 q_out=None, new_seq_lens=None, out=None, out_dtype=None, chunk_tokens: int = 0,
                                 workspace=None, stream=None, tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """decode_append_rope_paged on pools of one-byte E4M3 codes:
    append_rope_paged_fp8 followed by decode_paged_fp8
    (gqa_decode_append_rope_paged_fp8).  Returns (out, q_out, new_seq_lens)."""
    args, keep = _decode_append_paged_args(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base, scale,
                                           max_seq_len, q_out, new_seq_lens, out, out_dtype, chunk_tokens, workspace,
                                           stream, tiles, merge, per_cu, (k_scale, v_scale))
    _check(lib().gqa_decode_append_rope_paged_fp8(*args))
    return keep[0], keep[1], keep[2]


def prepare_decode_append_fp8(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base: float, scale: float,
                              k_scale: float, v_scale: float, kv_offsets=None, max_seq_len=None, out_dtype=None,
                              chunk_tokens: int = 0, stream=None, tiles: int = 0, merge: str = "auto",
                              per_cu: int = 0):
    """As prepare_decode_append, for gqa_decode_append_rope_fp8."""
    args, keep = _decode_append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, scale, kv_offsets,
                                     max_seq_len, None, None, None, out_dtype, chunk_tokens, None, stream, tiles, merge,
                                     per_cu, (k_scale, v_scale))
    return Prepared(lib().gqa_decode_append_rope_fp8, args, keep)


def prepare_decode_append_paged_fp8(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base: float,
                                    scale: float, k_scale: float, v_scale: float, max_seq_len=None, out_dtype=None,
                                    chunk_tokens: int = 0, stream=None, tiles: int = 0, merge: str = "auto",
                                    per_cu: int = 0):
    """As prepare_decode_append_paged, for gqa_decode_append_rope_paged_fp8."""
    args, keep = _decode_append_paged_args(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base, scale,
                                           max_seq_len, None, None, None, out_dtype, chunk_tokens, None, stream, tiles,
                                           merge, per_cu, (k_scale, v_scale))
    return Prepared(lib().gqa_decode_append_rope_paged_fp8, args, keep)


def prepare_decode_append_paged(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base: float,
                                scale: float, max_seq_len=None, out_dtype=None, chunk_tokens: int = 0, stream=None,
                                tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """As prepare, for gqa_decode_append_rope_paged (each call appends again:
    the new token overwrites the same pool rows with the same values; the
    first call is the first append)."""
    args, keep = _decode_append_paged_args(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base, scale,
                                           max_seq_len, None, None, None, out_dtype, chunk_tokens, None, stream, tiles,
                                           merge, per_cu)
    return Prepared(lib().gqa_decode_append_rope_paged, args, keep)


def prepare_append_paged(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base: float,
                         max_seq_len: Optional[int] = None, stream=None, q_out=None, new_seq_lens=None):
    """As prepare_append, for append_rope_paged."""
    fn, args, keep = _append_paged_args(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base,
                                        max_seq_len, q_out, new_seq_lens, stream, None)
    return Prepared(fn, args, keep)


def prepare_decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base: float, scale: float,
                          kv_offsets=None, max_seq_len=None, out_dtype=None, chunk_tokens: int = 0, stream=None,
                          tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """As prepare, for gqa_decode_append_rope (each call appends again: the
    new token overwrites the same cache rows with the same values; the first
    call is the first append)."""
    args, keep = _decode_append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, scale, kv_offsets,
                                     max_seq_len, None, None, None, out_dtype, chunk_tokens, None, stream, tiles, merge,
                                     per_cu)
    return Prepared(lib().gqa_decode_append_rope, args, keep)


def append_rope_fp8(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base: float, k_scale: float, v_scale: float,
                    kv_offsets=None, max_seq_len: Optional[int] = None, q_out=None, new_seq_lens=None, stream=None):
    """append_rope into caches of one-byte E4M3 codes (uint8 or float8_e4m3fn;
    dense or packed): the rotated key is stored as the code of key / k_scale,
    the value as the code of value / v_scale (nearest, ties to even,
    saturating at +-448)."""
    return append_rope(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, kv_offsets=kv_offsets,
                       max_seq_len=max_seq_len, q_out=q_out, new_seq_lens=new_seq_lens, stream=stream,
                       scales=(k_scale, v_scale))


def _append_paged_args(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base, max_seq_len, q_out,
                       new_seq_lens, stream, scales):
    """Validated (function, arguments, tensors kept) of gqa_append_rope_paged,
    or of gqa_append_rope_paged_fp8 with ``scales`` (nothing is enqueued)."""
    dev = q.device
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_pool, "k_pool"), (v_pool, "v_pool"),
                 (block_table, "block_table"), (seq_lens, "seq_lens")):
        _require(t, n, dev)
    if q.dim() != 3 or k_new.dim() != 3 or v_new.shape != k_new.shape:
        raise ValueError("expected q [B,H_q,d] and k_new/v_new [B,H_kv,d]")
    B, H_q, d = q.shape
    H_kv = k_new.shape[1]
    if k_new.shape[0] != B or k_new.shape[2] != d or seq_lens.shape != (B,) or seq_lens.dtype != torch.int32:
        raise ValueError("shape mismatch between q, k_new/v_new and seq_lens")
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape or k_pool.shape[1] != H_kv or k_pool.shape[3] != d:
        raise ValueError("pools must be [num_pages,H_kv,page,d]")
    if block_table.dim() != 2 or block_table.shape[0] != B or block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32 [B,max_pages]")
    for t in (k_new, v_new) + (() if scales else (k_pool, v_pool)):
        if t.dtype != q.dtype:
            raise TypeError("q, k_new, v_new and the pools must share one dtype")
    if scales and (k_pool.dtype not in E4M3_DTYPES or v_pool.dtype not in E4M3_DTYPES):
        raise TypeError("E4M3 pools are uint8 or float8_e4m3fn")
    page, max_pages = k_pool.shape[2], block_table.shape[1]
    dims = make_dims(B, H_q, H_kv, d, max_pages * page if max_seq_len is None else int(max_seq_len), q.dtype)
    q_out = torch.empty_like(q) if q_out is None else q_out
    new_seq_lens = torch.empty_like(seq_lens) if new_seq_lens is None else new_seq_lens
    _require(q_out, "q_out", dev)
    _require(new_seq_lens, "new_seq_lens", dev)
    if q_out.shape != q.shape or q_out.dtype != q.dtype or new_seq_lens.shape != (B,) or \
            new_seq_lens.dtype != torch.int32:
        raise ValueError("q_out must match q and new_seq_lens be int32 [B]")
    s = _stream_handle(dev, stream)
    head = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), int(max_pages),
            int(page), _ptr(seq_lens), _ptr(new_seq_lens), float(rope_base))
    if scales:
        fn, args = lib().gqa_append_rope_paged_fp8, head + (float(scales[0]), float(scales[1]), _ptr(q_out),
                                                            ctypes.byref(dims), s)
    else:
        fn, args = lib().gqa_append_rope_paged, head + (_ptr(q_out), ctypes.byref(dims), s)
    return fn, args, (q_out, new_seq_lens, q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, dims)




def append_rope_paged(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base: float,
                      max_seq_len: Optional[int] = None, q_out=None, new_seq_lens=None, stream=None, scales=None):
    """append_rope for a cache held in pages of a pool (the layout of
    decode_paged): k_pool/v_pool [num_pages,H_kv,page,d], block_table int32
    [B,max_pages]; the new token of sequence b goes to row seq_lens[b] % page
    of page block_table[b, seq_lens[b] // page].  max_seq_len (the capacity)
    defaults to max_pages * page.  Returns (q_out, new_seq_lens)."""
    fn, args, keep = _append_paged_args(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base,
                                        max_seq_len, q_out, new_seq_lens, stream, scales)
    _check(fn(*args))
    return keep[0], keep[1]


def append_rope_paged_fp8(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base: float, k_scale: float,
                          v_scale: float, max_seq_len: Optional[int] = None, q_out=None, new_seq_lens=None,
                          stream=None):
    """append_rope_paged into pools of one-byte E4M3 codes, quantised as in
    append_rope_fp8."""
    return append_rope_paged(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base,
                             max_seq_len=max_seq_len, q_out=q_out, new_seq_lens=new_seq_lens, stream=stream,
                             scales=(k_scale, v_scale))


def prepare_append(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base: float, kv_offsets=None,
                   max_seq_len: Optional[int] = None, stream=None, q_out=None, new_seq_lens=None):
    """A callable that enqueues append_rope with these arguments (for timing
    loops); it returns the rotated queries.  The arguments are checked on the
    host here and nothing is enqueued until the first call, which is the
    first append.  The new lengths go to a tensor of their own
    (``new_seq_lens`` if given, else a new one), so every call appends at the
    same rows."""
    fn, args, keep = _append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, kv_offsets, max_seq_len,
                                  q_out, new_seq_lens, stream, None)
    return Prepared(fn, args, keep)


def prepare_append_fp8(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base: float, k_scale: float,
                       v_scale: float, kv_offsets=None, max_seq_len: Optional[int] = None, stream=None, q_out=None,
                       new_seq_lens=None):
    """As prepare_append, for append_rope_fp8."""
    fn, args, keep = _append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, rope_base, kv_offsets, max_seq_len,
                                  q_out, new_seq_lens, stream, (k_scale, v_scale))
    return Prepared(fn, args, keep)


def prepare_append_paged_fp8(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base: float,
                             k_scale: float, v_scale: float, max_seq_len: Optional[int] = None, stream=None,
                             q_out=None, new_seq_lens=None):
    """As prepare_append, for append_rope_paged_fp8."""
    fn, args, keep = _append_paged_args(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, rope_base,
                                        max_seq_len, q_out, new_seq_lens, stream, (k_scale, v_scale))
    return Prepared(fn, args, keep)


class Prepared:
    """A call of the library with every argument marshalled and checked on the
    host once; calling it only enqueues the launch (for timing loops and
    graph capture, where per-call argument checks would cost more host time
    than the kernel takes).  Construction enqueues nothing; argument errors
    the library itself detects surface at the first call."""

    def __init__(self, fn, args: tuple, keep: tuple):
        self._fn = fn
        self._args = args
        self._keep = keep   # tensors whose memory the pointers refer to

    def __call__(self):
        _check(self._fn(*self._args))
        return self._keep[0]


def prepare(q, k_cache, v_cache, seq_lens, scale: float, kv_offsets=None, max_seq_len=None, num_kv_heads=None,
            out_dtype=None, chunk_tokens: int = 0, path: str = "auto", seq_len_hint: int = 0, stream=None,
            waves: int = 0, tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """A Prepared launcher writing into a fresh output tensor, which each call
    returns.  q [B,H_q,d] selects gqa_decode, q [L,B,H_q,d] selects
    gqa_decode_layers."""
    if q.dim() == 4:
        args, keep = _layers_args(q, k_cache, v_cache, seq_lens, scale, kv_offsets, max_seq_len, num_kv_heads, None,
                                  out_dtype, chunk_tokens, path, seq_len_hint, None, stream, waves, tiles, merge,
                                  per_cu)
        return Prepared(lib().gqa_decode_layers, args, keep)
    args, keep = _decode_args(q, k_cache, v_cache, seq_lens, scale, None, out_dtype, chunk_tokens, path, seq_len_hint,
                              None, stream, waves, tiles, merge, per_cu)
    return Prepared(lib().gqa_decode, args, keep)


def prepare_paged(q, k_pool, v_pool, block_table, seq_lens, scale: float, out_dtype=None, max_seq_len=None,
                  chunk_tokens: int = 0, seq_len_hint: int = 0, stream=None, tiles: int = 0, merge: str = "auto",
                  per_cu: int = 0):
    """As prepare, for gqa_decode_paged."""
    args, keep = _paged_args(q, k_pool, v_pool, block_table, seq_lens, scale, None, out_dtype, max_seq_len,
                             chunk_tokens, seq_len_hint, None, stream, tiles, merge, per_cu)
    return Prepared(lib().gqa_decode_paged, args, keep)


def prepare_fp8(q, k_cache, v_cache, seq_lens, scale: float, k_scale: float, v_scale: float, out_dtype=None,
                chunk_tokens: int = 0, seq_len_hint: int = 0, stream=None, tiles: int = 0, merge: str = "auto",
                per_cu: int = 0):
    """As prepare, for gqa_decode_fp8."""
    args, keep = _fp8_args(q, k_cache, v_cache, seq_lens, scale, k_scale, v_scale, None, out_dtype, chunk_tokens,
                           seq_len_hint, None, stream, tiles, merge, per_cu)
    return Prepared(lib().gqa_decode_fp8, args, keep)


def prepare_layers_fp8(q, k_cache, v_cache, seq_lens, scale: float, k_scale: float, v_scale: float, kv_offsets=None,
                       max_seq_len=None, num_kv_heads=None, out_dtype=None, chunk_tokens: int = 0,
                       seq_len_hint: int = 0, stream=None, tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """As prepare, for gqa_decode_layers_fp8."""
    args, keep = _layers_args(q, k_cache, v_cache, seq_lens, scale, kv_offsets, max_seq_len, num_kv_heads, None,
                              out_dtype, chunk_tokens, "mfma", seq_len_hint, None, stream, 0, tiles, merge, per_cu,
                              (k_scale, v_scale))
    return Prepared(lib().gqa_decode_layers_fp8, args, keep)


def prepare_paged_fp8(q, k_pool, v_pool, block_table, seq_lens, scale: float, k_scale: float, v_scale: float,
                      out_dtype=None, max_seq_len=None, chunk_tokens: int = 0, seq_len_hint: int = 0, stream=None,
                      tiles: int = 0, merge: str = "auto", per_cu: int = 0):
    """As prepare, for gqa_decode_paged_fp8."""
    args, keep = _paged_args(q, k_pool, v_pool, block_table, seq_lens, scale, None, out_dtype, max_seq_len,
                             chunk_tokens, seq_len_hint, None, stream, tiles, merge, per_cu, (k_scale, v_scale))
    return Prepared(lib().gqa_decode_paged_fp8, args, keep)
