"""Seeded synthetic inputs for the GQA decode step.

This module only draws and lays out random inputs; it holds none of the
attention arithmetic.  Both the GPU path's tests/benchmark and the CPU oracle's
tests take their inputs from here.

Workloads (shapes follow the model table of "Grouped-Query Attention (GQA) and
Multi-Query Attention (MQA): Mathematical Foundations, Arithmetic Intensity,
and KV-Cache Scaling Mechanics", section 5, and the example layer of
"Grouped-Query Attention Shares Keys Without Sharing Every Query"):

==========================  ==  ===  ====  ===  ======================  =====  ======
name                        B   H_q  H_kv  d    cached tokens           L      dtype
==========================  ==  ===  ====  ===  ======================  =====  ======
tiny-gqa-fp32               1   8    2     64   128                     1      fp32
llama3-8b-layer             16  32   8     128  4096                    1      bf16
llama-70b-ragged-layer      32  64   8     128  U[1024, 16384]          1      bf16
grouping-sweep-mha          8   32   32    128  32768                   1      bf16
grouping-sweep-gqa          8   32   8     128  32768                   1      bf16
grouping-sweep-mqa          8   32   1     128  32768                   1      bf16
llama3-8b-32-layer-stack    64  32   8     128  U[4096, 32768]          32     bf16
llama-70b-tp8-shard         32  8    1     128  U[1024, 16384]          1      bf16
==========================  ==  ===  ====  ===  ======================  =====  ======

llama-70b-tp8-shard is one GPU's share of llama-70b-ragged-layer under
tensor parallelism over 8 GPUs by heads (section 4 of the first page,
"Tensor Parallelism (TP) Head Partitioning"): one KV head and its 8 query
heads, with the same sequence lengths (same seed for the lengths; its own
values).  tp_shard cuts such a share out of a whole layer's inputs.

Values are N(0, 1) drawn in float32 and rounded to nearest-even into the
storage dtype.  Draw order: sequence lengths, then q, then K, then V.  Ragged
lengths are integers uniform on the closed interval.  The three grouping-sweep
runs share one set of queries (seed 1004); their caches use seed 1004 + H_kv.

to_pages lays a dense cache out in pages of a pool (any workload can be
read through a block table that way); the order of the pages in the pool is a
seeded random permutation.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    d: int
    seq_lo: int          # inclusive lower bound on cached tokens
    seq_hi: int          # inclusive upper bound (== seq_lo for uniform lengths)
    dtype: torch.dtype
    seed: int
    layers: int = 1
    q_seed: Optional[int] = None   # separate query seed (shared queries)
    packed: bool = False           # packed ragged layout (only valid tokens stored)

    @property
    def T_max(self) -> int:
        return self.seq_hi

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny-gqa-fp32", 1, 8, 2, 64, 128, 128, torch.float32, 1001),
        Workload("llama3-8b-layer", 16, 32, 8, 128, 4096, 4096, torch.bfloat16, 1002),
        Workload("llama-70b-ragged-layer", 32, 64, 8, 128, 1024, 16384, torch.bfloat16, 1003),
        Workload("grouping-sweep-mha", 8, 32, 32, 128, 32768, 32768, torch.bfloat16, 1004 + 32, q_seed=1004),
        Workload("grouping-sweep-gqa", 8, 32, 8, 128, 32768, 32768, torch.bfloat16, 1004 + 8, q_seed=1004),
        Workload("grouping-sweep-mqa", 8, 32, 1, 128, 32768, 32768, torch.bfloat16, 1004 + 1, q_seed=1004),
        Workload("llama3-8b-32-layer-stack", 64, 32, 8, 128, 4096, 32768, torch.bfloat16, 1005, layers=32,
                 packed=True),
        Workload("llama-70b-tp8-shard", 32, 8, 1, 128, 1024, 16384, torch.bfloat16, 1003),
    ]
}


def tp_shard(inputs: dict, tp: int, rank: int) -> dict:
    """GPU ``rank``'s share of a one-layer dense input under tensor
    parallelism over ``tp`` GPUs by heads: KV heads [rank*H_kv/tp,
    (rank+1)*H_kv/tp) and the query heads [rank*H_q/tp, (rank+1)*H_q/tp)
    that read them under the contiguous grouping (contiguous copies; the
    lengths and scale are shared).  H_kv must be a multiple of tp."""
    B, H_q, d = inputs["q"].shape
    H_kv = inputs["k"].shape[1]
    if inputs["k"].dim() != 4 or H_kv % tp or H_q % tp or not 0 <= rank < tp:
        raise ValueError("tp_shard takes a dense one-layer input with H_kv divisible by tp")
    qs, ks = H_q // tp, H_kv // tp
    out = dict(inputs)
    out["q"] = inputs["q"][:, rank * qs:(rank + 1) * qs].contiguous()
    out["k"] = inputs["k"][:, rank * ks:(rank + 1) * ks].contiguous()
    out["v"] = inputs["v"][:, rank * ks:(rank + 1) * ks].contiguous()
    return out


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, gen, device, dtype) -> torch.Tensor:
    """N(0,1) in float32, rounded to nearest-even into ``dtype``.  Large
    tensors are drawn in slabs to bound the float32 temporary."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    slab = 1 << 28
    for s in range(0, n, slab):
        e = min(n, s + slab)
        flat[s:e].copy_(torch.randn(e - s, generator=gen, device=device, dtype=torch.float32))
    return out


def seq_lens_for(w: Workload, device="cpu") -> torch.Tensor:
    """Cached-token counts [B] (int32), seeded; the first draw of the workload."""
    g = _gen(w.seed, "cpu")
    if w.seq_lo == w.seq_hi:
        sl = torch.full((w.B,), w.seq_lo, dtype=torch.int32)
    else:
        sl = torch.randint(w.seq_lo, w.seq_hi + 1, (w.B,), generator=g, dtype=torch.int64).to(torch.int32)
    return sl.to(device)


def packed_offsets(seq_lens: torch.Tensor) -> torch.Tensor:
    """kv_offsets [B+1] (int64) of the packed layout: sequence b owns tokens
    [off[b], off[b+1]) per KV head, its capacity being exactly seq_lens[b]."""
    sl = seq_lens.to("cpu", torch.int64)
    off = torch.zeros(sl.numel() + 1, dtype=torch.int64)
    off[1:] = torch.cumsum(sl, 0)
    return off


def generate(w: Workload, device="cpu", poison_padding: bool = False, replica: int = 0,
             seq_lens: Optional[torch.Tensor] = None) -> dict:
    """Inputs of one decode step of workload ``w``.

    Returns a dict with q [L,B,H_q,d] (L dropped when layers == 1), k/v caches,
    seq_lens (int32, on ``device``), kv_offsets (int64 [B+1], packed layouts
    only; on ``device``), scale, and the workload.

    Dense caches are [L][B][H_kv][T_max][d]; positions t >= seq_lens[b] are
    zero, or NaN with ``poison_padding`` (they must never be read).  Packed
    caches are flat [L * kv_offsets[B] * H_kv, d].  ``replica`` > 0 draws an
    independent batch of the same shapes (new values, same lengths).
    """
    dev = torch.device(device)
    sl = seq_lens_for(w, "cpu") if seq_lens is None else seq_lens.to("cpu", torch.int32)
    q_seed = (w.q_seed if w.q_seed is not None else w.seed) + 7919 * replica
    kv_seed = w.seed + 7919 * replica + (1000003 if w.q_seed is None else 0)
    gq = _gen(q_seed, dev)
    gk = _gen(kv_seed, dev)
    L = w.layers
    q = _normal((L, w.B, w.H_q, w.d), gq, dev, w.dtype)
    out = {"workload": w, "scale": w.scale, "seq_lens": sl.to(dev)}
    if w.packed:
        off = packed_offsets(sl)
        rows = int(off[-1]) * w.H_kv
        k = _normal((L * rows, w.d), gk, dev, w.dtype)
        v = _normal((L * rows, w.d), gk, dev, w.dtype)
        out["kv_offsets"] = off.to(dev)
    else:
        shape = (L, w.B, w.H_kv, w.T_max, w.d)
        k = _normal(shape, gk, dev, w.dtype)
        v = _normal(shape, gk, dev, w.dtype)
        pad = float("nan") if poison_padding else 0.0
        for b in range(w.B):
            n = int(sl[b])
            if n < w.T_max:
                k[:, b, :, n:, :] = pad
                v[:, b, :, n:, :] = pad
    if L == 1:
        q = q[0]
        if not w.packed:
            k, v = k[0], v[0]
    out.update(q=q, k=k, v=v)
    return out


def layer_view(inputs: dict, l: int) -> dict:
    """Single-layer slice (q [B,H_q,d], k/v of layer l) of a multi-layer input."""
    w: Workload = inputs["workload"]
    if w.layers == 1:
        return inputs
    res = dict(inputs)
    res["q"] = inputs["q"][l]
    if w.packed:
        rows = inputs["k"].shape[0] // w.layers
        res["k"] = inputs["k"][l * rows:(l + 1) * rows]
        res["v"] = inputs["v"][l * rows:(l + 1) * rows]
    else:
        res["k"] = inputs["k"][l]
        res["v"] = inputs["v"][l]
    return res


def to_pages(inputs: dict, page: int, seed: int, spare: int = 3, share_first_page: bool = False,
             shuffle: bool = True):
    """The dense cache of ``inputs`` (k, v [B, H_kv, T, d]) in pages of
    ``page`` tokens: returns (k_pool, v_pool [num_pages, H_kv, page, d],
    block_table int32 [B, ceil(T / page)]) on the cache's device.

    Sequence b (its length clamped to [0, T]) gets ceil(len / page) pages,
    taken in the order of a seeded permutation of the pool (in pool order
    when ``shuffle`` is false), which has ``spare`` pages more than the
    sequences use.  Spare pages and the rows of a last page past the
    sequence's length are NaN (the E4M3 NaN code 0x7F for uint8 caches);
    table entries past a sequence's last page name the last page of the
    permutation, which is spare (spare >= 1).  ``share_first_page`` points sequence 1's first entry at
    sequence 0's first page (a shared prefix), when sequence 0 fills that page
    and sequence 1 uses a page.
    """
    if spare < 1:
        raise ValueError("spare must be at least 1")
    k, v = inputs["k"], inputs["v"]
    B, H_kv, T, d = k.shape
    dev = k.device
    lens = [max(0, min(int(n), T)) for n in inputs["seq_lens"].tolist()]
    used = [-(-n // page) for n in lens]
    total = sum(used) + spare
    perm = (torch.randperm(total, generator=torch.Generator().manual_seed(seed)) if shuffle
            else torch.arange(total)).tolist()
    pad = float("nan") if k.dtype.is_floating_point else 0x7F   # NaN, or the E4M3 NaN code for byte caches
    k_pool = torch.full((total, H_kv, page, d), pad, dtype=k.dtype, device=dev)
    v_pool = torch.full_like(k_pool, pad)
    table = torch.full((B, -(-T // page)), perm[-1], dtype=torch.int32)
    o = 0
    for b in range(B):
        u = used[b]
        if u == 0:
            continue
        ids = perm[o:o + u]
        o += u
        for src, pool in ((k, k_pool), (v, v_pool)):
            rows = torch.full((H_kv, u * page, d), pad, dtype=k.dtype, device=dev)
            rows[:, :lens[b]] = src[b, :, :lens[b]]
            pool[torch.tensor(ids, device=dev)] = rows.view(H_kv, u, page, d).permute(1, 0, 2, 3)
        table[b, :u] = torch.tensor(ids, dtype=torch.int32)
    if share_first_page and B > 1 and lens[0] >= page and used[1] > 0:
        table[1, 0] = table[0, 0]
    return k_pool, v_pool, table.to(dev)


E4M3_MAX = 448.0   # largest finite OCP E4M3 value


_E4M3_CHUNK = 1 << 26   # elements converted at a time (bounds the float32 temporaries)


def quantize_e4m3(x: torch.Tensor):
    """``x`` as one-byte OCP E4M3 codes and one scale: scale = max|x| / 448
    over the finite elements (a float32 value), codes = torch's
    round-to-nearest-even conversion of x / scale to float8_e4m3fn, as uint8.
    Non-finite elements become NaN codes.  Returns (codes, scale).  Works
    through x in slices, so a cache of any size needs only its codes as
    extra memory."""
    flat = x.reshape(-1)
    amax = 0.0
    for i in range(0, flat.numel(), _E4M3_CHUNK):
        xf = flat[i:i + _E4M3_CHUNK].float()
        fin = torch.isfinite(xf)
        if bool(fin.any()):
            amax = max(amax, float(xf[fin].abs().max()))
    scale = float(torch.tensor(amax / E4M3_MAX if amax > 0 else 1.0, dtype=torch.float32))
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    cf = codes.view(-1)
    for i in range(0, flat.numel(), _E4M3_CHUNK):
        xf = flat[i:i + _E4M3_CHUNK].float()
        y = torch.where(torch.isfinite(xf), xf / scale, torch.full_like(xf, float("nan")))
        cf[i:i + _E4M3_CHUNK] = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def to_e4m3(inputs: dict, release: bool = False) -> dict:
    """A copy of ``inputs`` whose k and v are E4M3 codes (uint8, same layout)
    with their scales k_scale and v_scale; NaN padding stays NaN.  release:
    drop ``inputs``' k (v) as soon as its codes exist, so that a cache near
    the device's capacity is never held twice."""
    out = dict(inputs)
    for name in ("k", "v"):
        out[name], out[name + "_scale"] = quantize_e4m3(inputs[name])
        if release:
            inputs[name] = None
    return out
