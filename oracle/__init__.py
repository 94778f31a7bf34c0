"""Plain fp64 CPU oracle for one grouped-query-attention decode step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never loads it and shares no code with it.

Contents
--------
* :class:`Oracle` -- ctypes wrapper around ``gqa_oracle.c`` (fp64 softmax
  attention per query head with the contiguous head-to-group map), following
  "Grouped-Query Attention (GQA) and Multi-Query Attention (MQA): Mathematical
  Foundations, Arithmetic Intensity, and KV-Cache Scaling Mechanics",
  section 2, subsection "Grouped-Query Attention (GQA)".
* :meth:`Oracle.decode_paged` -- the same attention with the cache held in
  pages of a pool, found through a per-sequence block table.
* :meth:`Oracle.decode_fp8` -- the same attention over a cache of one-byte
  OCP E4M3 elements with one scale for the keys and one for the values (the
  bytes-per-element term of section 1, "KV Cache Memory Footprint", below
  two); :meth:`Oracle.e4m3` decodes such bytes, and
  :meth:`Oracle.decode_paged_fp8` reads such a cache from pages of a pool.
* :meth:`Oracle.rope` -- fp64 rotary position embedding (section 4 of the
  same page, "Rotary Position Embeddings (RoPE) Interaction"), for the step
  that appends the new token's keys and values.
* :func:`kv_cache_bytes` -- the KV-cache size formula of the same page,
  section 1, "KV Cache Memory Footprint" (also stated on "Grouped-Query
  Attention Shares Keys Without Sharing Every Query").
* :func:`cache_element_ratio` -- cached key/value elements of a layer relative
  to full multi-head attention ("Grouped-Query Attention Shares Keys Without
  Sharing Every Query", the 32-query-head example).
* :func:`roofline_balance` -- I_sat = peak FLOP/s / peak bytes/s (section 1,
  "Arithmetic Intensity in Autoregressive Decoding").

Every function is pinned by CPU tests (closed forms, invariants, a library
routine, the pages' printed tables); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gqa_oracle.c")
LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")

_DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float64: 2}


def build(source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the C oracle with gcc (fp64, no fast-math, OpenMP)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", "-std=c11",
           source, "-lm", "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """Handle on one compiled copy of the C oracle."""

    def __init__(self, lib_path: Optional[str] = None):
        path = lib_path or LIB_PATH
        if lib_path is None and not os.path.exists(path):
            build()
        self.path = path
        lib = ctypes.CDLL(path)
        i64, vp, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.oracle_group_of.restype = i64
        lib.oracle_group_of.argtypes = [i64, i64]
        lib.oracle_gqa_decode.restype = ctypes.c_int
        lib.oracle_gqa_decode.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, dbl,
                                          i64, vp, vp]
        lib.oracle_gqa_head_weights.restype = ctypes.c_int
        lib.oracle_gqa_head_weights.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp,
                                                dbl, i64, i64, vp, vp]
        lib.oracle_gqa_decode_paged.restype = ctypes.c_int
        lib.oracle_gqa_decode_paged.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, i64, i64, vp, dbl,
                                                i64, vp, vp]
        lib.oracle_gqa_decode_fp8.restype = ctypes.c_int
        lib.oracle_gqa_decode_fp8.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, dbl, dbl, dbl,
                                              i64, vp, vp]
        lib.oracle_gqa_decode_paged_fp8.restype = ctypes.c_int
        lib.oracle_gqa_decode_paged_fp8.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, i64, i64, vp,
                                                    dbl, dbl, dbl, i64, vp, vp]
        lib.oracle_e4m3_encode.restype = ctypes.c_int
        lib.oracle_e4m3_encode.argtypes = [i64, vp, vp]
        lib.oracle_e4m3_decode.restype = ctypes.c_int
        lib.oracle_e4m3_decode.argtypes = [i64, vp, vp]
        lib.oracle_rope.restype = ctypes.c_int
        lib.oracle_rope.argtypes = [i64, i64, ctypes.c_int, vp, vp, dbl, vp]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        self._lib = lib

    def num_threads(self) -> int:
        """Threads the oracle's OpenMP loops run on."""
        return int(self._lib.oracle_num_threads())

    # -- head -> group map -------------------------------------------------
    def group_of(self, i: int, R: int) -> int:
        """KV head of query head ``i`` (0-based) when ``R`` query heads share one."""
        return int(self._lib.oracle_group_of(int(i), int(R)))

    # -- helpers ----------------------------------------------------------
    @staticmethod
    def _prep(q, k, v, seq_lens, kv_offsets):
        if q.dtype not in _DTYPE_CODE:
            raise TypeError("oracle takes float32, bfloat16 or float64 tensors")
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise TypeError("q, k and v must share one dtype")
        q = q.detach().to("cpu").contiguous()
        k = k.detach().to("cpu").contiguous()
        v = v.detach().to("cpu").contiguous()
        if q.dim() != 3:
            raise ValueError("q must be [B, H_q, d]")
        B, H_q, d = q.shape
        if kv_offsets is None:
            if k.dim() != 4 or k.shape[0] != B or k.shape[3] != d or v.shape != k.shape:
                raise ValueError("dense cache must be [B, H_kv, T_max, d]")
            H_kv, T_max = k.shape[1], k.shape[2]
            offs = np.arange(B + 1, dtype=np.int64) * T_max
        else:
            offs = np.ascontiguousarray(np.asarray(kv_offsets, dtype=np.int64))
            if offs.shape != (B + 1,):
                raise ValueError("kv_offsets must have B+1 entries")
            rows = k.numel() // d
            if rows * d != k.numel() or v.numel() != k.numel():
                raise ValueError("packed cache size mismatch")
            total = int(offs[-1]) if B else 0
            if total == 0:
                H_kv = None
            else:
                if rows % total:
                    raise ValueError("packed cache rows not a multiple of kv_offsets[B]")
                H_kv = rows // total
        sl = np.ascontiguousarray(np.asarray(
            seq_lens.cpu() if isinstance(seq_lens, torch.Tensor) else seq_lens, dtype=np.int32))
        if sl.shape != (B,):
            raise ValueError("seq_lens must have B entries")
        return q, k, v, sl, offs, B, H_q, H_kv, d

    def decode(self, q, k, v, seq_lens, scale: float, kv_offsets=None, heads=None,
               num_kv_heads: Optional[int] = None) -> np.ndarray:
        """fp64 outputs for query tensor ``q`` [B, H_q, d].

        ``k``/``v`` are dense [B, H_kv, T_max, d] when ``kv_offsets`` is None,
        otherwise a packed array whose sequence ``b`` occupies rows
        ``[kv_offsets[b]*H_kv, kv_offsets[b+1]*H_kv)``, KV head after KV head.
        ``heads`` optionally lists flat head ids ``b*H_q + i``; the result is
        then [len(heads), d] instead of [B, H_q, d].  ``scale`` is widened from
        float32, exactly as a float32 argument reaches the GPU path.
        """
        q, k, v, sl, offs, B, H_q, H_kv, d = self._prep(q, k, v, seq_lens, kv_offsets)
        if H_kv is None:
            H_kv = num_kv_heads if num_kv_heads else H_q
        sc = float(np.float32(scale))
        if heads is None:
            out = np.zeros((B, H_q, d), dtype=np.float64)
            ids_ptr, n = None, B * H_q
        else:
            ids = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
            out = np.zeros((ids.shape[0], d), dtype=np.float64)
            ids_ptr, n = ids.ctypes.data, ids.shape[0]
        rc = self._lib.oracle_gqa_decode(B, H_q, H_kv, d, _DTYPE_CODE[q.dtype], q.data_ptr(),
                                         k.data_ptr(), v.data_ptr(), offs.ctypes.data, sl.ctypes.data,
                                         sc, n, ids_ptr, out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return out

    def decode_paged(self, q, k_pool, v_pool, block_table, page: int, seq_lens, scale: float) -> np.ndarray:
        """fp64 outputs for q [B, H_q, d] with the cache in pages: k_pool and
        v_pool [num_pages, H_kv, page, d]; sequence b's token t is in page
        block_table[b, t // page] (block_table int32 [B, max_pages])."""
        if q.dtype not in _DTYPE_CODE or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
            raise TypeError("q and the pools must share one of float32, bfloat16, float64")
        q = q.detach().to("cpu").contiguous()
        k_pool = k_pool.detach().to("cpu").contiguous()
        v_pool = v_pool.detach().to("cpu").contiguous()
        B, H_q, d = q.shape
        if k_pool.dim() != 4 or k_pool.shape[2] != page or k_pool.shape[3] != d or v_pool.shape != k_pool.shape:
            raise ValueError("pools must be [num_pages, H_kv, page, d]")
        H_kv = k_pool.shape[1]
        bt = np.ascontiguousarray(np.asarray(
            block_table.cpu() if isinstance(block_table, torch.Tensor) else block_table, dtype=np.int32))
        if bt.ndim != 2 or bt.shape[0] != B:
            raise ValueError("block_table must be [B, max_pages]")
        if bt.size and (bt.min() < 0 or bt.max() >= k_pool.shape[0]):
            raise ValueError("page id out of the pool")
        sl = np.ascontiguousarray(np.asarray(
            seq_lens.cpu() if isinstance(seq_lens, torch.Tensor) else seq_lens, dtype=np.int32))
        out = np.zeros((B, H_q, d), dtype=np.float64)
        rc = self._lib.oracle_gqa_decode_paged(B, H_q, H_kv, d, _DTYPE_CODE[q.dtype], q.data_ptr(), k_pool.data_ptr(),
                                               v_pool.data_ptr(), bt.ctypes.data, bt.shape[1], int(page),
                                               sl.ctypes.data, float(np.float32(scale)), B * H_q, None,
                                               out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return out

    def decode_paged_fp8(self, q, k_pool, v_pool, block_table, page: int, seq_lens, scale: float, k_scale: float,
                         v_scale: float) -> np.ndarray:
        """decode_fp8 with the E4M3 cache held in pages of a pool (uint8 or
        float8_e4m3fn pools [num_pages, H_kv, page, d] and a block table, as
        in :meth:`decode_paged`)."""
        if q.dtype not in _DTYPE_CODE:
            raise TypeError("oracle takes float32, bfloat16 or float64 queries")
        q = q.detach().to("cpu").contiguous()
        k_pool = k_pool.detach().to("cpu").contiguous().view(torch.uint8)
        v_pool = v_pool.detach().to("cpu").contiguous().view(torch.uint8)
        B, H_q, d = q.shape
        if k_pool.dim() != 4 or k_pool.shape[2] != page or k_pool.shape[3] != d or v_pool.shape != k_pool.shape:
            raise ValueError("pools must be [num_pages, H_kv, page, d]")
        bt = np.ascontiguousarray(np.asarray(
            block_table.cpu() if isinstance(block_table, torch.Tensor) else block_table, dtype=np.int32))
        if bt.ndim != 2 or bt.shape[0] != B:
            raise ValueError("block_table must be [B, max_pages]")
        if bt.size and (bt.min() < 0 or bt.max() >= k_pool.shape[0]):
            raise ValueError("page id out of the pool")
        sl = np.ascontiguousarray(np.asarray(
            seq_lens.cpu() if isinstance(seq_lens, torch.Tensor) else seq_lens, dtype=np.int32))
        out = np.zeros((B, H_q, d), dtype=np.float64)
        f32 = lambda x: float(np.float32(x))
        rc = self._lib.oracle_gqa_decode_paged_fp8(B, H_q, k_pool.shape[1], d, _DTYPE_CODE[q.dtype], q.data_ptr(),
                                                   k_pool.data_ptr(), v_pool.data_ptr(), bt.ctypes.data, bt.shape[1],
                                                   int(page), sl.ctypes.data, f32(scale), f32(k_scale), f32(v_scale),
                                                   B * H_q, None, out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return out

    def e4m3_encode(self, x) -> np.ndarray:
        """OCP E4M3 bytes of ``x`` (any shape; widened to fp64): nearest value,
        ties to even, saturating at +-448, NaN to 0x7F."""
        v = np.ascontiguousarray(np.asarray(x.detach().cpu().double() if isinstance(x, torch.Tensor) else x,
                                            dtype=np.float64))
        out = np.zeros(v.shape, dtype=np.uint8)
        self._lib.oracle_e4m3_encode(v.size, v.ctypes.data, out.ctypes.data)
        return out

    def e4m3(self, codes) -> np.ndarray:
        """fp64 values of OCP E4M3 bytes (uint8 array or tensor, any shape)."""
        c = np.ascontiguousarray(np.asarray(codes.cpu() if isinstance(codes, torch.Tensor) else codes,
                                            dtype=np.uint8))
        out = np.zeros(c.shape, dtype=np.float64)
        self._lib.oracle_e4m3_decode(c.size, c.ctypes.data, out.ctypes.data)
        return out

    def decode_fp8(self, q, k8, v8, seq_lens, scale: float, k_scale: float, v_scale: float, kv_offsets=None,
                   heads=None, num_kv_heads: Optional[int] = None) -> np.ndarray:
        """fp64 outputs for q [B, H_q, d] over a cache of E4M3 bytes: ``k8`` and
        ``v8`` (uint8, or float8_e4m3fn tensors, which are read as their bytes)
        in the dense [B, H_kv, T_max, d] or packed layout of :meth:`decode`; a
        key element stands for k_scale times its E4M3 value, a value element for
        v_scale times its own.  The three scales are widened from float32, as
        float32 arguments reach the GPU path."""
        if q.dtype not in _DTYPE_CODE:
            raise TypeError("oracle takes float32, bfloat16 or float64 queries")
        k8 = k8.detach().to("cpu").contiguous().view(torch.uint8)
        v8 = v8.detach().to("cpu").contiguous().view(torch.uint8)
        if v8.shape != k8.shape:
            raise ValueError("k8 and v8 must have one shape")
        q = q.detach().to("cpu").contiguous()
        B, H_q, d = q.shape
        if kv_offsets is None:
            if k8.dim() != 4 or k8.shape[0] != B or k8.shape[3] != d:
                raise ValueError("dense cache must be [B, H_kv, T_max, d]")
            H_kv, T_max = k8.shape[1], k8.shape[2]
            offs = np.arange(B + 1, dtype=np.int64) * T_max
        else:
            offs = np.ascontiguousarray(np.asarray(kv_offsets, dtype=np.int64))
            H_kv = num_kv_heads if num_kv_heads else H_q
        sl = np.ascontiguousarray(np.asarray(
            seq_lens.cpu() if isinstance(seq_lens, torch.Tensor) else seq_lens, dtype=np.int32))
        if heads is None:
            out = np.zeros((B, H_q, d), dtype=np.float64)
            ids_ptr, n = None, B * H_q
        else:
            ids = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
            out = np.zeros((ids.shape[0], d), dtype=np.float64)
            ids_ptr, n = ids.ctypes.data, ids.shape[0]
        f32 = lambda x: float(np.float32(x))
        rc = self._lib.oracle_gqa_decode_fp8(B, H_q, H_kv, d, _DTYPE_CODE[q.dtype], q.data_ptr(), k8.data_ptr(),
                                             v8.data_ptr(), offs.ctypes.data, sl.ctypes.data, f32(scale),
                                             f32(k_scale), f32(v_scale), n, ids_ptr, out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return out

    def rope(self, x, positions, base: float) -> np.ndarray:
        """fp64 rotary embedding of ``x`` [..., d] at ``positions`` (one per
        vector: broadcastable to x.shape[:-1]), base ``base``."""
        if x.dtype not in _DTYPE_CODE:
            raise TypeError("oracle takes float32, bfloat16 or float64 tensors")
        x = x.detach().to("cpu").contiguous()
        d = x.shape[-1]
        n = x.numel() // d if d else 0
        pos = np.ascontiguousarray(np.broadcast_to(np.asarray(
            positions.cpu() if isinstance(positions, torch.Tensor) else positions, dtype=np.int64),
            tuple(x.shape[:-1])).reshape(-1))
        out = np.zeros(tuple(x.shape), dtype=np.float64)
        rc = self._lib.oracle_rope(n, d, _DTYPE_CODE[x.dtype], x.data_ptr(), pos.ctypes.data, float(base),
                                   out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return out

    def head_weights(self, q, k, v, seq_lens, scale: float, b: int, i: int, kv_offsets=None,
                     num_kv_heads: Optional[int] = None):
        """Softmax weights over the n valid tokens, and the output, of head (b, i)."""
        q, k, v, sl, offs, B, H_q, H_kv, d = self._prep(q, k, v, seq_lens, kv_offsets)
        if H_kv is None:
            H_kv = num_kv_heads if num_kv_heads else H_q
        n = int(sl[b])
        w = np.zeros(max(n, 1), dtype=np.float64)
        out = np.zeros(d, dtype=np.float64)
        rc = self._lib.oracle_gqa_head_weights(B, H_q, H_kv, d, _DTYPE_CODE[q.dtype], q.data_ptr(),
                                               k.data_ptr(), v.data_ptr(), offs.ctypes.data,
                                               sl.ctypes.data, float(np.float32(scale)), b, i,
                                               w.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return w[:n], out


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def decode(*args, **kwargs) -> np.ndarray:
    return default().decode(*args, **kwargs)


def group_of(i: int, R: int) -> int:
    return default().group_of(i, R)


def rope(x, positions, base: float) -> np.ndarray:
    return default().rope(x, positions, base)


def kv_cache_bytes(b: int, s: int, L: int, H_kv: int, d_k: int, bytes_per_elem: int = 2) -> int:
    """Bytes of keys plus values cached for b sequences of s tokens over L layers.

    "Grouped-Query Attention (GQA) and Multi-Query Attention (MQA): ...",
    section 1, "KV Cache Memory Footprint": one factor 2 for keys and values,
    one for the element width, times b, s, L, H_KV and d_k.  "Grouped-Query
    Attention Shares Keys Without Sharing Every Query" states the same product
    per sequence (2 x layers x tokens x groups x head dimension x bytes).
    """
    return 2 * bytes_per_elem * b * s * L * H_kv * d_k


def cache_element_ratio(H_kv: int, H_q: int) -> float:
    """Cached K/V elements per token of a layer with H_kv heads, relative to H_q
    heads (multi-head attention), at fixed head dimension and precision."""
    return H_kv / H_q


def roofline_balance(peak_flops: float, peak_bytes_per_s: float) -> float:
    """I_sat = peak FLOP/s divided by peak memory bytes/s (section 1)."""
    return peak_flops / peak_bytes_per_s
