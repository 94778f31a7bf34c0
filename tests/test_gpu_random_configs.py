"""Seeded random configurations across the whole option space, each against
the fp64 oracle through the C ABI.

Every case draws its shape (B, H_q, H_kv, d, T and ragged lengths, zeros
included), its layout (dense, paged, E4M3, paged E4M3), its kernel options
(path, forced span, merge, tiles, workgroups per CU) and its output dtype
from one seed, so the list of cases is fixed.  Bars: 1e-5 for fp32 inputs,
2e-3 for bf16 (and E4M3) caches; a bf16 output may add one rounding of the
result: bf16 carries 8 significant bits, so rounding to nearest-even moves
a value by at most its unit roundoff, 2^-8 of its magnitude (half a unit in
the last place, which is 2^-7 of the binade's lower end).
"""
import random

import numpy as np
import pytest
import torch

import gqa_mqa_kv_amd as gqa
import oracle
from gqa_mqa_kv_amd import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
N_CASES = 64


def draw(i):
    r = random.Random(1000 + i)
    H_kv = r.choice([1, 1, 2, 4, 8])
    G = r.choice([1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 40, 48, 64])
    d = r.choice([64, 128])
    B = r.randint(1, 9)
    T = r.randint(1, 640)
    layout = r.choice(["dense", "dense", "paged", "fp8", "paged_fp8"])
    dtype = torch.float32 if layout == "dense" and r.random() < 0.4 else torch.bfloat16
    if dtype == torch.float32:
        path = "valu"
    else:
        path = r.choice(["auto", "mfma", "valu"]) if layout == "dense" else "mfma"
    lens = [r.choice([0, r.randint(0, T), T, r.randint(max(0, T - 20), T)]) for _ in range(B)]
    c = dict(i=i, B=B, H_q=G * H_kv, H_kv=H_kv, d=d, T=T, lens=lens, layout=layout, dtype=dtype, path=path,
             chunk=r.choice([0, 0, 64, 128, 256, 512]), merge=r.choice(["auto", "fused", "kernel"]),
             tiles=r.choice([0, 1, 2, 4]) if layout in ("fp8", "paged_fp8") else r.choice([0, 1, 2]),
             per_cu=r.choice([0, 0, 1, 2]), page=r.choice([16, 32, 48, 64, 128]),
             out=r.choice([torch.float32, torch.bfloat16]))
    return c


def make(c):
    w = workloads.Workload("rand", c["B"], c["H_q"], c["H_kv"], c["d"], c["T"], c["T"], c["dtype"], 7000 + c["i"])
    x = workloads.generate(w, "cpu")
    x["seq_lens"] = torch.tensor(c["lens"], dtype=torch.int32)
    for b, n in enumerate(c["lens"]):
        x["k"][b, :, n:] = float("nan")
        x["v"][b, :, n:] = float("nan")
    return x


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_config(i):
    c = draw(i)
    x = make(c)
    note = {k: v for k, v in c.items() if k != "lens"}
    print("[gpu-case] random", note, "lens", c["lens"], flush=True)
    orc = oracle.default()
    kw = dict(out_dtype=c["out"], chunk_tokens=c["chunk"], merge=c["merge"], tiles=c["tiles"], per_cu=c["per_cu"])
    sl = x["seq_lens"].to(DEV)
    q = x["q"].to(DEV)
    if c["layout"] in ("fp8", "paged_fp8"):
        x8 = workloads.to_e4m3(x)
        if c["layout"] == "fp8":
            ref = orc.decode_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], x["scale"], x8["k_scale"], x8["v_scale"])
            out = gqa.decode_fp8(q, x8["k"].to(DEV), x8["v"].to(DEV), sl, x["scale"], x8["k_scale"], x8["v_scale"],
                                 **kw)
        else:
            kp, vp, tb = workloads.to_pages(x8, c["page"], seed=c["i"])
            ref = orc.decode_paged_fp8(x["q"], kp, vp, tb, c["page"], x["seq_lens"], x["scale"], x8["k_scale"],
                                       x8["v_scale"])
            out = gqa.decode_paged_fp8(q, kp.to(DEV), vp.to(DEV), tb.to(DEV), sl, x["scale"], x8["k_scale"],
                                       x8["v_scale"], max_seq_len=c["T"], **kw)
    elif c["layout"] == "paged":
        kp, vp, tb = workloads.to_pages(x, c["page"], seed=c["i"])
        ref = orc.decode_paged(x["q"], kp, vp, tb, c["page"], x["seq_lens"], x["scale"])
        out = gqa.decode_paged(q, kp.to(DEV), vp.to(DEV), tb.to(DEV), sl, x["scale"], max_seq_len=c["T"], **kw)
    else:
        ref = orc.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"])
        out = gqa.decode(q, x["k"].to(DEV), x["v"].to(DEV), sl, x["scale"], path=c["path"], **kw)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    assert np.isfinite(o).all(), "non-finite output"
    tol = 1e-5 if c["dtype"] == torch.float32 else 2e-3
    if c["out"] == torch.bfloat16:
        # the fp32 result (within tol of ref) rounded once to bf16
        bar = tol + 2.0 ** -8 * (np.abs(ref) + tol)
    else:
        bar = tol
    err = np.abs(o - ref)
    assert (err <= bar).all(), "max err %.3e" % float(err.max())
    for b, n in enumerate(c["lens"]):
        if n == 0:
            assert not o[b].any(), "empty sequence %d not zero" % b


N_LAYER_CASES = 32


def draw_layers(i):
    r = random.Random(5000 + i)
    H_kv = r.choice([1, 2, 4, 8])
    G = r.choice([g for g in (1, 2, 4, 4, 8, 16, 24, 32, 48) if g * H_kv <= 128])
    T = r.randint(1, 900)
    B = r.randint(1, 8)
    cache = r.choice(["bf16", "bf16", "fp8"])
    lens = [r.choice([0, r.randint(0, T), T]) for _ in range(B)]
    packed = r.random() < 0.5
    if packed and not any(lens):
        lens[-1] = T   # a packed cache of no rows has no storage (a null pointer, which the call rejects)
    return dict(i=i, B=B, H_q=G * H_kv, H_kv=H_kv, d=r.choice([64, 128]), T=T, L=r.randint(2, 6),
                lens=lens, cache=cache, packed=packed,
                chunk=r.choice([0, 0, 0, 64, 256]), merge=r.choice(["auto", "fused", "kernel"]),
                tiles=r.choice([0, 1, 2, 4]) if cache == "fp8" else r.choice([0, 1, 2]),
                per_cu=r.choice([0, 0, 1, 2]), out=r.choice([torch.float32, torch.bfloat16]))


@pytest.mark.parametrize("i", range(N_LAYER_CASES))
def test_random_layer_batch(i):
    """Seeded random layer batches (2 to 6 layers, dense or packed, bf16 or
    E4M3 caches, ragged lengths with zeros, the planner's split with its
    claimed last layer or forced spans, either merge, tiles and workgroups
    per CU): every output of every layer against the oracle, at the bars of
    the one-layer cases above."""
    c = draw_layers(i)
    note = {k: v for k, v in c.items() if k != "lens"}
    print("[gpu-case] random layers", note, "lens", c["lens"], flush=True)
    sl = torch.tensor(c["lens"], dtype=torch.int32)
    w = workloads.Workload("rand-layers", c["B"], c["H_q"], c["H_kv"], c["d"], 1, c["T"], torch.bfloat16,
                           9000 + i, layers=c["L"], packed=c["packed"])
    x = workloads.generate(w, "cpu", poison_padding=True, seq_lens=sl)
    if c["cache"] == "fp8":
        x = workloads.to_e4m3(x)
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    kw = dict(out_dtype=c["out"], chunk_tokens=c["chunk"], merge=c["merge"], tiles=c["tiles"], per_cu=c["per_cu"])
    if c["packed"]:
        kw.update(kv_offsets=xd["kv_offsets"], max_seq_len=c["T"], num_kv_heads=c["H_kv"])
    if c["cache"] == "fp8":
        out = gqa.decode_layers_fp8(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], x["k_scale"],
                                    x["v_scale"], **kw)
    else:
        out = gqa.decode_layers(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], **kw)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    assert np.isfinite(o).all(), "non-finite output"
    orc = oracle.default()
    offs = x["kv_offsets"].numpy() if c["packed"] else None
    for l in range(c["L"]):
        xl = workloads.layer_view(x, l)
        if c["cache"] == "fp8":
            ref = orc.decode_fp8(xl["q"], xl["k"], xl["v"], x["seq_lens"], x["scale"], x["k_scale"], x["v_scale"],
                                 kv_offsets=offs, num_kv_heads=c["H_kv"])
        else:
            ref = orc.decode(xl["q"], xl["k"], xl["v"], x["seq_lens"], x["scale"], kv_offsets=offs,
                             num_kv_heads=c["H_kv"])
        bar = 2e-3 + (2.0 ** -8 * (np.abs(ref) + 2e-3) if c["out"] == torch.bfloat16 else 0.0)
        e = np.abs(o[l] - ref)
        assert (e <= bar).all(), "layer %d: max err %.3e" % (l, float(e.max()))
        for b, n in enumerate(c["lens"]):
            if n == 0:
                assert not o[l, b].any(), "layer %d: empty sequence %d not zero" % (l, b)
