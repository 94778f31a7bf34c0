"""The decode step over a cache held in pages of a pool, on the GPU against the
fp64 oracle, through the C ABI.

Bars as for the plain layout: bf16 inputs, fp32 output, max |gpu - oracle|
<= 2e-3; a bf16 output is bitwise the round-to-nearest-even of the fp32
output of the same call.

Every pool here is shuffled and holds, besides the pages the sequences use,
spare pages filled with NaN; table entries past a sequence's last page and
the tail of its last page hold NaN too (the entries point at a spare page),
so a read of anything but a valid token shows up as a NaN output.
"""
import numpy as np
import pytest
import torch

import gqa_mqa_kv_amd as gqa
import oracle
from gqa_mqa_kv_amd import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = 2e-3


def note(*a):
    print("[gpu-case]", *a, flush=True)


def paged(x, page, seed, share=False):
    return workloads.to_pages(x, page, seed, share_first_page=share)


def small(B, H_q, H_kv, d, T, seed, lo=None, lens=None):
    """Seeded bf16 inputs, NaN past each length; ``lens`` replaces the drawn
    lengths."""
    w = workloads.Workload("paged", B, H_q, H_kv, d, lo if lo is not None else T, T, torch.bfloat16, seed)
    if lens is None:
        return workloads.generate(w, "cpu", poison_padding=True)
    x = workloads.generate(w, "cpu")
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
    for b, n in enumerate(lens):
        x["k"][b, :, n:] = float("nan")
        x["v"][b, :, n:] = float("nan")
    return x


def check(x, page, seed=0, share=False, label="", **kw):
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    kp, vp, table = paged(xd, page, seed, share=share)
    note(label, tuple(x["q"].shape), tuple(x["k"].shape), "page", page, kw)
    T = x["k"].shape[2]
    clamped = x["seq_lens"].clamp(0, T)        # the call clamps lengths to max_seq_len = T
    ref = oracle.default().decode_paged(x["q"], kp.cpu(), vp.cpu(), table.cpu(), page, clamped, x["scale"])
    o32 = gqa.decode_paged(xd["q"], kp, vp, table, xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                           max_seq_len=T, **kw)
    o16 = gqa.decode_paged(xd["q"], kp, vp, table, xd["seq_lens"], x["scale"], out_dtype=torch.bfloat16,
                           max_seq_len=T, **kw)
    torch.cuda.synchronize()
    o = o32.double().cpu().numpy()
    assert np.isfinite(o).all(), "non-finite output"
    e = float(np.abs(o - ref).max())
    assert e <= TOL, "%s: max err %.3e" % (label, e)
    assert torch.equal(o16.cpu(), o32.cpu().to(torch.bfloat16)), "bf16 out is not RNE(fp32 out)"
    return o32


SHAPES = [
    # B, H_q, H_kv, d, T_max, lo   (ragged lengths U[lo, T_max])
    (3, 32, 8, 128, 300, 1),        # Llama-3-8B grouping
    (2, 64, 8, 128, 777, 1),        # G = 8
    (2, 16, 1, 128, 520, 33),       # MQA, G = 16
    (2, 32, 1, 128, 600, 100),      # MQA, G = 32
    (3, 8, 8, 64, 300, 1),          # MHA, d = 64
    (2, 40, 1, 64, 257, 1),         # G = 40, d = 64
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_Hq%d_Hkv%d_d%d_T%d" % s[:5])
@pytest.mark.parametrize("page", [16, 32, 64, 256])
def test_paged_small(shape, page):
    B, hq, hkv, d, T, lo = shape
    x = small(B, hq, hkv, d, T, seed=sum(shape[:5]) * 7 + page, lo=lo)
    check(x, page, seed=page, label="paged")


@pytest.mark.parametrize("chunk", [64, 128, 192])
@pytest.mark.parametrize("merge", ["fused", "kernel"])
@pytest.mark.parametrize("page", [16, 48])
def test_paged_forced_spans_and_merges(chunk, merge, page):
    """Spans that cut units (and pages) at many places; both ways of merging
    the pieces of a unit."""
    x = small(4, 32, 8, 128, 500, seed=chunk + page, lens=[1, 17, 255, 500])
    check(x, page, seed=3, chunk_tokens=chunk, merge=merge, label="paged-span")


def test_paged_edges():
    """Empty sequences, one token, lengths one below, at and one past a
    multiple of 16 and of the page, and lengths beyond the capacity
    (clamped to it)."""
    T, page = 320, 32
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 0, 319, 320, 1000]
    x = small(len(lens), 16, 4, 128, T, seed=11, lens=lens)
    out = check(x, page, seed=5, label="paged-edges")
    assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[8]) == 0
    for merge in ("fused", "kernel"):
        check(x, page, seed=6, chunk_tokens=64, merge=merge, label="paged-edges-span")


def test_paged_shared_prefix_page():
    """Two sequences whose tables name the same first page."""
    x = small(3, 32, 8, 128, 200, seed=21, lens=[200, 150, 90])
    check(x, 32, seed=9, share=True, label="paged-shared")


def test_paged_matches_plain_layout_and_repeats_bitwise():
    """The same cache in pages and in the plain layout gives the same
    attention (to the bar: the work split differs), and a paged call
    repeated gives bitwise the same output."""
    x = small(4, 32, 8, 128, 1000, seed=31, lo=100)
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    kp, vp, table = paged(xd, 64, 4)
    plain = gqa.decode(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32)
    a = gqa.decode_paged(xd["q"], kp, vp, table, xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                         max_seq_len=1000)
    b = gqa.decode_paged(xd["q"], kp, vp, table, xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                         max_seq_len=1000)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert float((a - plain).abs().max()) <= TOL


def full_paged(name, page, sample):
    w = workloads.WORKLOADS[name]
    note("full-paged", w.name, "page", page, "generate")
    x = workloads.generate(w, DEV, poison_padding=True)
    kp, vp, table = paged(x, page, seed=page)
    del x["k"], x["v"]
    note("full-paged", w.name, "decode")
    o32 = gqa.decode_paged(x["q"], kp, vp, table, x["seq_lens"], x["scale"], out_dtype=torch.float32,
                           max_seq_len=w.T_max)
    o16 = gqa.decode_paged(x["q"], kp, vp, table, x["seq_lens"], x["scale"], out_dtype=torch.bfloat16,
                           max_seq_len=w.T_max)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert bool(torch.isfinite(o32).all())
    g = torch.Generator().manual_seed(77)
    heads = sorted(set(torch.randperm(w.B * w.H_q, generator=g)[:sample].tolist()) | {0, w.B * w.H_q - 1})
    note("full-paged", w.name, "oracle on %d sampled heads" % len(heads))
    tab = table.cpu()
    e = 0.0
    for hid in heads:
        b, i = divmod(hid, w.H_q)
        gi = i // w.G
        n = int(x["seq_lens"][b])
        u = -(-n // page)
        # the sequence's rows, gathered from its pages (only its own table row)
        ids = tab[b, :u].long().to(DEV)
        k1 = kp[ids, gi].reshape(1, 1, u * page, w.d)[:, :, :n].cpu()
        v1 = vp[ids, gi].reshape(1, 1, u * page, w.d)[:, :, :n].cpu()
        q1 = x["q"][b:b + 1, i:i + 1].cpu()
        ref = oracle.decode(q1, k1, v1, torch.tensor([n], dtype=torch.int32), w.scale)[0, 0]
        e = max(e, float(np.abs(o32[b, i].double().cpu().numpy() - ref).max()))
    note("full-paged", w.name, "max err %.3e" % e)
    assert e <= TOL


@pytest.mark.timeout(600)
def test_full_llama3_8b_layer_paged():
    full_paged("llama3-8b-layer", 16, 64)


@pytest.mark.timeout(600)
def test_full_70b_ragged_layer_paged():
    full_paged("llama-70b-ragged-layer", 64, 64)
