"""The decode step over a cache of one-byte OCP E4M3 elements, on the GPU
against the fp64 oracle (oracle_gqa_decode_fp8), through the C ABI.

Both sides read the same bytes and scales, so the bar is the bf16-input bar:
max |gpu - oracle| <= 2e-3 with an fp32 output (the E4M3 values are widened
to bf16 exactly; the remaining error is that of the fp32 accumulation and of
the softmax weights' bf16 split).  A bf16 output is bitwise the
round-to-nearest-even of the fp32 output of the same call.  The hardware's
decoding of every one of the 256 codes is checked exactly (a one-token
attention returns v_scale times the value row).
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


def small(B, H_q, H_kv, d, T, seed, lo=None, lens=None):
    """Seeded bf16 inputs, NaN past each length, as E4M3 codes with scales."""
    w = workloads.Workload("fp8", B, H_q, H_kv, d, lo if lo is not None else T, T, torch.bfloat16, seed)
    x = workloads.generate(w, "cpu", poison_padding=lens is None)
    if lens is not None:
        x["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
        for b, n in enumerate(lens):
            x["k"][b, :, n:] = float("nan")
            x["v"][b, :, n:] = float("nan")
    return workloads.to_e4m3(x)


def check(x, label="", **kw):
    T = x["k"].shape[2]
    clamped = x["seq_lens"].clamp(0, T)
    ref = oracle.default().decode_fp8(x["q"], x["k"], x["v"], clamped, x["scale"], x["k_scale"], x["v_scale"])
    note(label, tuple(x["q"].shape), tuple(x["k"].shape), kw)
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    args = (xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], x["k_scale"], x["v_scale"])
    o32 = gqa.decode_fp8(*args, out_dtype=torch.float32, **kw)
    o16 = gqa.decode_fp8(*args, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    o = o32.double().cpu().numpy()
    assert np.isfinite(o).all(), "non-finite output"
    e = float(np.abs(o - ref).max())
    assert e <= TOL, "%s: max err %.3e" % (label, e)
    assert torch.equal(o16.cpu(), o32.cpu().to(torch.bfloat16)), "bf16 out is not RNE(fp32 out)"
    return o32


def test_every_code_decodes_exactly():
    """One cached token: every output column is v_scale times the value
    element (weights are exactly 1).  The value rows hold all 256 codes; the
    two NaN codes give NaN in their own column only."""
    B, H_q, H_kv, d = 1, 8, 2, 128
    g = torch.Generator().manual_seed(3)
    q = torch.randn(B, H_q, d, generator=g).to(torch.bfloat16)
    k8 = torch.randint(0, 0x7E, (B, H_kv, 16, d), generator=g, dtype=torch.uint8)   # finite keys
    v8 = torch.zeros(B, H_kv, 16, d, dtype=torch.uint8)
    v8[0, :, 0, :] = torch.arange(256, dtype=torch.uint8).view(H_kv, d)
    sl = torch.tensor([1], dtype=torch.int32)
    note("every E4M3 code")
    out = gqa.decode_fp8(q.to(DEV), k8.to(DEV), v8.to(DEV), sl.to(DEV), d ** -0.5, 0.5, 0.25,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = 0.25 * oracle.default().e4m3(torch.arange(256, dtype=torch.uint8)).reshape(H_kv, d)
    got = out[0].double().cpu().numpy().reshape(H_kv, H_q // H_kv, d)
    for j in range(H_q // H_kv):
        assert np.array_equal(got[:, j], want, equal_nan=True)


SHAPES = [
    # B, H_q, H_kv, d, T_max, lo   (ragged lengths U[lo, T_max])
    (1, 8, 2, 64, 128, None),
    (3, 8, 8, 64, 300, 1),           # MHA, d = 64
    (2, 32, 8, 128, 1000, 200),      # Llama-3-8B grouping
    (2, 64, 8, 128, 777, 1),         # G = 8
    (2, 16, 1, 128, 520, 33),        # MQA, G = 16
    (2, 32, 1, 128, 600, 100),       # MQA, G = 32
    (1, 64, 1, 128, 450, None),      # G = 64
    (2, 12, 4, 128, 333, 10),        # G = 3
    (2, 48, 1, 64, 300, 7),          # G = 48, d = 64
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_Hq%d_Hkv%d_d%d_T%d" % s[:5])
@pytest.mark.parametrize("chunk", [0, 256])
def test_fp8_small(shape, chunk):
    B, hq, hkv, d, T, lo = shape
    x = small(B, hq, hkv, d, T, seed=sum(shape[:5]) * 13 + chunk, lo=lo)
    check(x, chunk_tokens=chunk, label="fp8")


@pytest.mark.parametrize("chunk", [64, 128, 192])
@pytest.mark.parametrize("merge", ["fused", "kernel"])
@pytest.mark.parametrize("tiles", [1, 2, 4])
def test_fp8_forced_spans_merges_tiles(chunk, merge, tiles):
    x = small(4, 32, 8, 128, 500, seed=chunk + tiles, lens=[1, 17, 255, 500])
    check(x, chunk_tokens=chunk, merge=merge, tiles=tiles, label="fp8-span")


def test_fp8_edges():
    """Empty sequences, one token, lengths around multiples of 16, and lengths
    beyond the capacity (clamped)."""
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 0, 319, 320, 1000]
    x = small(len(lens), 16, 4, 128, 320, seed=11, lens=lens)
    out = check(x, label="fp8-edges")
    assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[8]) == 0
    check(x, chunk_tokens=64, merge="kernel", label="fp8-edges-span")


def test_fp8_uniform_codes_and_scales():
    """Caches of uniformly drawn finite codes (every magnitude from the
    subnormals to 448), with scales far from 1."""
    B, H_q, H_kv, d, T = 3, 32, 8, 128, 257
    g = torch.Generator().manual_seed(19)
    codes = torch.randint(0, 254, (2, B, H_kv, T, d), generator=g)
    codes = codes + (codes >= 0x7F).long()                      # skip the NaN code 0x7F (0xFF is out of range)
    x = {"q": torch.randn(B, H_q, d, generator=g).to(torch.bfloat16), "k": codes[0].to(torch.uint8),
         "v": codes[1].to(torch.uint8), "seq_lens": torch.tensor([257, 100, 33], dtype=torch.int32),
         "scale": d ** -0.5, "k_scale": 1.0 / 448.0, "v_scale": 3.0e-3}
    check(x, label="fp8-uniform-codes")


def test_fp8_repeats_bitwise():
    x = small(4, 32, 8, 128, 1000, seed=31, lo=100)
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    args = (xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], x["k_scale"], x["v_scale"])
    a = gqa.decode_fp8(*args, out_dtype=torch.float32)
    b = gqa.decode_fp8(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def full_fp8(name, sample):
    w = workloads.WORKLOADS[name]
    note("full-fp8", w.name, "generate")
    x = workloads.to_e4m3(workloads.generate(w, DEV, poison_padding=True))
    note("full-fp8", w.name, "decode")
    args = (x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], x["k_scale"], x["v_scale"])
    o32 = gqa.decode_fp8(*args, out_dtype=torch.float32)
    o16 = gqa.decode_fp8(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert bool(torch.isfinite(o32).all())
    g = torch.Generator().manual_seed(78)
    heads = sorted(set(torch.randperm(w.B * w.H_q, generator=g)[:sample].tolist()) | {0, w.B * w.H_q - 1})
    note("full-fp8", w.name, "oracle on %d sampled heads" % len(heads))
    e = 0.0
    for hid in heads:
        b, i = divmod(hid, w.H_q)
        gi = i // w.G
        n = int(x["seq_lens"][b])
        ref = oracle.default().decode_fp8(x["q"][b:b + 1, i:i + 1].cpu(), x["k"][b:b + 1, gi:gi + 1, :n].cpu(),
                                          x["v"][b:b + 1, gi:gi + 1, :n].cpu(), torch.tensor([n], dtype=torch.int32),
                                          w.scale, x["k_scale"], x["v_scale"])[0, 0]
        e = max(e, float(np.abs(o32[b, i].double().cpu().numpy() - ref).max()))
    note("full-fp8", w.name, "max err %.3e" % e)
    assert e <= TOL


@pytest.mark.timeout(600)
def test_full_llama3_8b_layer_fp8():
    full_fp8("llama3-8b-layer", 64)


@pytest.mark.timeout(600)
def test_full_70b_ragged_layer_fp8():
    full_fp8("llama-70b-ragged-layer", 64)


# ------------------------------------------------ E4M3 caches in pages --
def check_paged(x, page, seed=0, label="", **kw):
    """gqa_decode_paged_fp8 on the E4M3 codes of ``x`` laid out in shuffled
    pages (spare pages and page tails hold the NaN code), against the oracle
    on the same pool."""
    T = x["k"].shape[2]
    clamped = x["seq_lens"].clamp(0, T)
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    kp, vp, table = workloads.to_pages(xd, page, seed=seed)
    note(label, tuple(x["q"].shape), tuple(x["k"].shape), "page", page, kw)
    ref = oracle.default().decode_paged_fp8(x["q"], kp.cpu(), vp.cpu(), table.cpu(), page, clamped, x["scale"],
                                            x["k_scale"], x["v_scale"])
    args = (xd["q"], kp, vp, table, xd["seq_lens"], x["scale"], x["k_scale"], x["v_scale"])
    o32 = gqa.decode_paged_fp8(*args, out_dtype=torch.float32, max_seq_len=T, **kw)
    o16 = gqa.decode_paged_fp8(*args, out_dtype=torch.bfloat16, max_seq_len=T, **kw)
    torch.cuda.synchronize()
    o = o32.double().cpu().numpy()
    assert np.isfinite(o).all(), "non-finite output"
    e = float(np.abs(o - ref).max())
    assert e <= TOL, "%s: max err %.3e" % (label, e)
    assert torch.equal(o16.cpu(), o32.cpu().to(torch.bfloat16)), "bf16 out is not RNE(fp32 out)"
    return o32


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_Hq%d_Hkv%d_d%d_T%d" % s[:5])
@pytest.mark.parametrize("page", [16, 64])
def test_fp8_paged_small(shape, page):
    B, hq, hkv, d, T, lo = shape
    x = small(B, hq, hkv, d, T, seed=sum(shape[:5]) * 17 + page, lo=lo)
    check_paged(x, page, seed=page, label="fp8-paged")


@pytest.mark.parametrize("chunk", [64, 192])
@pytest.mark.parametrize("merge", ["fused", "kernel"])
@pytest.mark.parametrize("tiles", [1, 2, 4])
def test_fp8_paged_spans_merges_tiles(chunk, merge, tiles):
    x = small(4, 32, 8, 128, 500, seed=chunk + tiles + 7, lens=[1, 17, 255, 500])
    check_paged(x, 48, seed=2, chunk_tokens=chunk, merge=merge, tiles=tiles, label="fp8-paged-span")


def test_fp8_paged_edges():
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 0, 319, 320, 1000]
    x = small(len(lens), 16, 4, 128, 320, seed=12, lens=lens)
    out = check_paged(x, 32, seed=5, label="fp8-paged-edges")
    assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[8]) == 0


@pytest.mark.timeout(600)
def test_full_llama3_8b_layer_paged_fp8():
    """The full 8B layer as E4M3 codes in shuffled pages of 16 tokens, on
    sampled heads (each against the dense E4M3 oracle on its sequence's
    rows gathered from its own pages)."""
    w = workloads.WORKLOADS["llama3-8b-layer"]
    page = 16
    note("full-fp8-paged", w.name, "generate")
    x = workloads.to_e4m3(workloads.generate(w, DEV, poison_padding=True))
    kp, vp, table = workloads.to_pages(x, page, seed=page)
    note("full-fp8-paged", w.name, "decode")
    args = (x["q"], kp, vp, table, x["seq_lens"], x["scale"], x["k_scale"], x["v_scale"])
    o32 = gqa.decode_paged_fp8(*args, out_dtype=torch.float32, max_seq_len=w.T_max)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o32).all())
    g = torch.Generator().manual_seed(79)
    heads = sorted(set(torch.randperm(w.B * w.H_q, generator=g)[:48].tolist()) | {0, w.B * w.H_q - 1})
    tab = table.cpu()
    e = 0.0
    for hid in heads:
        b, i = divmod(hid, w.H_q)
        gi = i // w.G
        n = int(x["seq_lens"][b])
        u = -(-n // page)
        ids = tab[b, :u].long().to(DEV)
        k1 = kp[ids, gi].reshape(1, 1, u * page, w.d)[:, :, :n].cpu()
        v1 = vp[ids, gi].reshape(1, 1, u * page, w.d)[:, :, :n].cpu()
        ref = oracle.default().decode_fp8(x["q"][b:b + 1, i:i + 1].cpu(), k1, v1, torch.tensor([n], dtype=torch.int32),
                                          w.scale, x["k_scale"], x["v_scale"])[0, 0]
        e = max(e, float(np.abs(o32[b, i].double().cpu().numpy() - ref).max()))
    note("full-fp8-paged", w.name, "max err %.3e" % e)
    assert e <= TOL


# ------------------------------------------------------------ layer batches --
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("H_kv,d", [(8, 128), (1, 128), (8, 64)])
@pytest.mark.parametrize("span,merge", [(0, "auto"), (192, "fused"), (192, "kernel")])
def test_layers_fp8(packed, H_kv, d, span, merge):
    """gqa_decode_layers_fp8: four layers of E4M3 caches (one scale pair for
    all of them), dense and packed, G = 4 and G = 32, d = 128 and 64, the
    planner's split (its last layer claimed in chunks at G = 4) and forced
    spans with both merges; each layer against the oracle on the same
    bytes."""
    w = workloads.Workload("layers-fp8", 3, 32, H_kv, d, 100, 900, torch.bfloat16, 61 + H_kv + d, layers=4,
                           packed=packed)
    x8 = workloads.to_e4m3(workloads.generate(w, "cpu", poison_padding=True))
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x8.items()}
    note("layers fp8", packed, H_kv, d, span, merge)
    kw = dict(kv_offsets=xd["kv_offsets"], max_seq_len=w.T_max, num_kv_heads=w.H_kv) if packed else {}
    run = lambda dt: gqa.decode_layers_fp8(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x8["scale"], x8["k_scale"],
                                           x8["v_scale"], out_dtype=dt, chunk_tokens=span, merge=merge, **kw)
    out32, out16 = run(torch.float32), run(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out16.cpu(), out32.cpu().to(torch.bfloat16)), "bf16 out is not RNE(fp32 out)"
    orc = oracle.default()
    for l in range(w.layers):
        xl = workloads.layer_view(x8, l)
        ref = orc.decode_fp8(xl["q"], xl["k"], xl["v"], x8["seq_lens"], x8["scale"], x8["k_scale"], x8["v_scale"],
                             kv_offsets=x8["kv_offsets"].numpy() if packed else None, num_kv_heads=w.H_kv)
        e = float(np.abs(out32[l].double().cpu().numpy() - ref).max())
        assert e <= TOL, "layer %d: max err %.3e" % (l, e)


@pytest.mark.timeout(900)
def test_full_32_layer_stack_fp8():
    """The 32-layer packed stack with its cache as E4M3 codes (about 77 GB),
    one launch (its last layer claimed in chunks): every output of every
    layer against the oracle on the same bytes, layer by layer (each layer's
    codes copied to the host)."""
    w = workloads.WORKLOADS["llama3-8b-32-layer-stack"]
    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info(DEV)
    sl = workloads.seq_lens_for(w)
    need = 2 * w.layers * int(sl.sum()) * w.H_kv * w.d * 2 + w.layers * int(sl.sum()) * w.H_kv * w.d
    if need > free - (8 << 30):
        pytest.skip("needs %.1f GB of device memory, %.1f free" % (need / 1e9, free / 1e9))
    note("full fp8", w.name, "generate")
    x = workloads.generate(w, DEV)
    x8 = workloads.to_e4m3(x, release=True)
    del x
    torch.cuda.empty_cache()
    note("full fp8", w.name, "decode")
    out = gqa.decode_layers_fp8(x8["q"], x8["k"], x8["v"], x8["seq_lens"], x8["scale"], x8["k_scale"],
                                x8["v_scale"], kv_offsets=x8["kv_offsets"], max_seq_len=w.T_max,
                                num_kv_heads=w.H_kv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    offs = x8["kv_offsets"].cpu().numpy()
    sl = x8["seq_lens"].cpu()
    orc = oracle.default()
    e = 0.0
    for l in range(w.layers):
        xl = workloads.layer_view(x8, l)
        ref = orc.decode_fp8(xl["q"].cpu(), xl["k"].cpu(), xl["v"].cpu(), sl, w.scale, x8["k_scale"], x8["v_scale"],
                             kv_offsets=offs, num_kv_heads=w.H_kv)
        el = float(np.abs(out[l].double().cpu().numpy() - ref).max())
        note("full fp8", w.name, "layer %d: max err %.3e" % (l, el))
        e = max(e, el)
    note("full fp8", w.name, "max err %.3e" % e)
    assert e <= TOL
    del x8
    torch.cuda.empty_cache()
