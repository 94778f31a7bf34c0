"""GPU path vs the fp64 CPU oracle, element by element, through the C ABI.

Bars (written here, derived in the design notes):
  * fp32 inputs: max |gpu - oracle| <= 1e-5.
  * bf16 inputs, fp32 accumulation, fp32 output: max |gpu - oracle| <= 2e-3.
  * bf16 output: bitwise equal to the fp32 output of the same call rounded to
    nearest-even (the kernels differ only in the final store), so it is the
    correctly rounded value of a result that meets the bar above.
Every input is seeded; padding positions of dense caches hold NaN so that a
read past seq_len shows up as a NaN output.
"""
import numpy as np
import pytest
import torch

import gqa_mqa_kv_amd as gqa
import oracle
from gqa_mqa_kv_amd import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}


def note(*a):
    print("[gpu-case]", *a, flush=True)


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def small(B, H_q, H_kv, d, T, seed, dtype=torch.bfloat16, lo=None, poison=True):
    w = workloads.Workload("case", B, H_q, H_kv, d, lo if lo is not None else T, T, dtype, seed)
    return workloads.generate(w, "cpu", poison_padding=poison)


def seed_of(shape, salt):
    return sum((j + 1) * (v or 0) for j, v in enumerate(shape)) * 31 + salt


def gpu_decode(x, **kw):
    xd = to_dev(x)
    out = gqa.decode(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], **kw)
    torch.cuda.synchronize()
    return out


def err(out, ref):
    o = out.double().cpu().numpy()
    assert np.isfinite(o).all(), "non-finite output"
    return float(np.abs(o - ref).max())


def check(x, tol=None, label="", **kw):
    dt = x["q"].dtype
    tol = TOL[dt] if tol is None else tol
    ref = oracle.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"])
    note(label, tuple(x["q"].shape), tuple(x["k"].shape), dt, kw)
    out32 = gpu_decode(x, out_dtype=torch.float32, **kw)
    e = err(out32, ref)
    assert e <= tol, "%s: max err %.3e > %.1e" % (label, e, tol)
    if dt == torch.bfloat16:
        out16 = gpu_decode(x, out_dtype=torch.bfloat16, **kw)
        assert torch.equal(out16.cpu(), out32.cpu().to(torch.bfloat16)), "bf16 out is not RNE(fp32 out)"
    return e


# ------------------------------------------------------------ small shapes --
SHAPES = [
    # B, H_q, H_kv, d, T_max, lo     (lo < T_max: ragged lengths U[lo, T_max])
    (1, 8, 2, 64, 128, None),        # the tiny fp32 workload's shape
    (3, 8, 8, 64, 300, 1),           # MHA, ragged, d=64
    (2, 32, 8, 128, 1000, 200),      # Llama-3-8B grouping, several chunks, ragged tail
    (2, 64, 8, 128, 777, 1),         # G = 8
    (2, 16, 1, 128, 520, 33),        # MQA, G = 16
    (2, 32, 1, 128, 600, 100),       # MQA, G = 32 (two head blocks)
    (1, 64, 1, 128, 450, None),      # G = 64 (four head blocks)
    (2, 12, 4, 128, 333, 10),        # G = 3 (partial head block)
    (2, 48, 1, 64, 300, 7),          # G = 48: three head blocks (run as four, one empty), d = 64
    (2, 40, 1, 64, 257, 1),          # G = 40, d = 64
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_Hq%d_Hkv%d_d%d_T%d" % s[:5])
@pytest.mark.parametrize("path", ["mfma", "valu"])
@pytest.mark.parametrize("chunk", [0, 256])
def test_small_bf16(shape, path, chunk):
    """chunk_tokens: tokens per workgroup on the matrix-core path, per chunk on
    the vector path (0: planner)."""
    B, hq, hkv, d, T, lo = shape
    x = small(B, hq, hkv, d, T, seed=seed_of(shape, 17), lo=lo)
    check(x, path=path, chunk_tokens=chunk, label="small-bf16")


@pytest.mark.parametrize("shape", SHAPES[:5], ids=lambda s: "B%d_Hq%d_Hkv%d_d%d_T%d" % s[:5])
@pytest.mark.parametrize("chunk", [0, 128])
def test_small_fp32(shape, chunk):
    B, hq, hkv, d, T, lo = shape
    x = small(B, hq, hkv, d, T, seed=seed_of(shape, 23), dtype=torch.float32, lo=lo)
    check(x, chunk_tokens=chunk, label="small-fp32")


def test_tiny_workload():
    w = workloads.WORKLOADS["tiny-gqa-fp32"]
    x = workloads.generate(w, "cpu")
    check(x, label=w.name)
    check(x, label=w.name, chunk_tokens=64)


# --------------------------------------------------------------- edge cases --
@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_empty_and_single_token(path):
    x = small(4, 16, 4, 128, 300, seed=5)
    x["seq_lens"] = torch.tensor([0, 1, 0, 257], dtype=torch.int32)
    for b, n in enumerate([0, 1, 0, 257]):
        x["k"][b, :, n:] = float("nan")
        x["v"][b, :, n:] = float("nan")
    check(x, path=path, chunk_tokens=128, label="empty+single")
    out = gpu_decode(x, path=path, out_dtype=torch.bfloat16).cpu()
    assert (out[0] == 0).all() and (out[2] == 0).all()
    # one cached token: weight 1, output = V exactly (also in bf16)
    for i in range(16):
        assert torch.equal(out[1, i], x["v"][1, i // 4, 0])


@pytest.mark.parametrize("path", ["mfma", "valu"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_spike_at_tile_and_chunk_edges(path, dtype):
    """Give one token per sequence all the weight; its position walks over
    tile (32) and chunk (256) boundaries and the ragged end.  A dropped or
    duplicated token there is an O(1) error, not a 2e-3 one."""
    if path == "mfma" and dtype == torch.float32:
        pytest.skip("matrix-core path takes bf16 only")
    chunk, n = 256, 700
    pos = [0, 1, 31, 32, 33, 63, 64, 255, 256, 257, 511, 512, 600, 671, 672, 699]
    B, hq, hkv, d = len(pos), 8, 2, 128
    x = small(B, hq, hkv, d, n, seed=77, dtype=dtype)
    x["q"].zero_()
    x["q"][:, :, 0] = 8.0
    for b, t in enumerate(pos):
        x["k"][b, :, t, :] = 0.0
        x["k"][b, :, t, 0] = 64.0            # score 8*64/sqrt(128) = 45 vs <= ~3.5 elsewhere
    out = gpu_decode(x, path=path, chunk_tokens=chunk, out_dtype=dtype).cpu()
    for b, t in enumerate(pos):
        want = x["v"][b, :, t, :].repeat_interleave(hq // hkv, dim=0)
        if dtype == torch.bfloat16:
            assert torch.equal(out[b], want), "spike at %d" % t
        else:
            assert (out[b] - want).abs().max() < 1e-6, "spike at %d" % t


def test_seq_lens_beyond_capacity_are_clamped():
    x = small(2, 8, 2, 64, 200, seed=9, poison=False)
    sl = torch.tensor([500, 37], dtype=torch.int32)
    xd = to_dev(x)
    out = gqa.decode(xd["q"], xd["k"], xd["v"], sl.to(DEV), x["scale"], out_dtype=torch.float32)
    ref = oracle.decode(x["q"], x["k"], x["v"], torch.tensor([200, 37], dtype=torch.int32), x["scale"])
    assert err(out, ref) <= 2e-3


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_deterministic_and_workspace_reuse(path):
    """Bitwise identical results run to run, also with a different-shaped call
    sharing the workspace in between."""
    x = small(3, 32, 8, 128, 2000, seed=31, lo=900)
    y = small(2, 8, 1, 128, 1500, seed=32, lo=1)
    a = gpu_decode(x, path=path, chunk_tokens=256).cpu()
    gpu_decode(y, path=path, chunk_tokens=128)
    b = gpu_decode(x, path=path, chunk_tokens=256).cpu()
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [SHAPES[2], SHAPES[3], SHAPES[5], SHAPES[8], (3, 32, 8, 128, 4000, 1)],
                         ids=lambda s: "B%d_Hq%d_Hkv%d_d%d_T%d" % s[:5])
@pytest.mark.parametrize("waves,tiles", [(4, 1), (4, 2), (8, 1)])
@pytest.mark.parametrize("span", [0, 64, 192])
@pytest.mark.parametrize("merge", ["fused", "kernel"])
def test_kernel_variants(shape, waves, tiles, span, merge):
    """Every instantiated matrix-core variant (workgroup size, tiles in flight),
    with the even token split and with short forced spans that cut units at
    arbitrary token positions (many pieces per unit to merge), merged inside
    the decode kernel or by the merge kernel."""
    B, hq, hkv, d, T, lo = shape
    x = small(B, hq, hkv, d, T, seed=seed_of(shape, 29), lo=lo)
    check(x, path="mfma", chunk_tokens=span, waves=waves, tiles=tiles, merge=merge, label="variant-" + merge)


@pytest.mark.parametrize("per_cu", [1, 2, 3, 4])
@pytest.mark.parametrize("merge", ["fused", "kernel"])
def test_workgroups_per_cu(per_cu, merge):
    """The even token split over one to four resident workgroups per CU."""
    for shape in (SHAPES[3], SHAPES[5], (3, 32, 8, 128, 4000, 1)):
        B, hq, hkv, d, T, lo = shape
        x = small(B, hq, hkv, d, T, seed=seed_of(shape, 37), lo=lo)
        check(x, path="mfma", per_cu=per_cu, merge=merge, label="per_cu %d %s" % (per_cu, merge))


@pytest.mark.parametrize("rate", [0.5, 4.0, 7.9, 8.1, 20.0])
def test_growing_scores_move_the_reference(rate):
    """Scores that grow by `rate` (base-2 units) per 16-token tile, so the
    running maximum moves on every tile: below the kernel's rescale slack
    (8) the reference stays put and the weights grow up to 2^8, above it the
    state is rescaled on each tile.  Each head of a group grows at its own
    rate, and spans of 64 tokens split units across workgroups whose states
    then differ by many powers of two."""
    B, H_q, H_kv, d, T = 2, 32, 8, 128, 700
    x = small(B, H_q, H_kv, d, T, seed=int(rate * 10) + 5)
    x["seq_lens"] = torch.tensor([700, 523], dtype=torch.int32)
    G = H_q // H_kv
    gen = torch.Generator().manual_seed(77)
    u = torch.zeros(d)
    u[3] = 1.0
    step = rate / 16 / (x["scale"] * np.log2(np.e))     # score growth per token, in K units
    t = torch.arange(T, dtype=torch.float32)
    for b in range(B):
        for g in range(H_kv):
            kk = step * t[:, None] * u[None, :] + 0.01 * torch.randn(T, d, generator=gen)
            x["k"][b, g] = kk.to(x["k"].dtype)
        for i in range(H_q):
            x["q"][b, i] = (u * (1.0 + (i % G) / G)).to(x["q"].dtype)
    for b, n in enumerate(x["seq_lens"].tolist()):
        x["k"][b, :, n:] = float("nan")
        x["v"][b, :, n:] = float("nan")
    for path, span, merge in (("mfma", 0, "auto"), ("mfma", 64, "fused"), ("mfma", 64, "kernel"), ("valu", 64, "auto")):
        check(x, path=path, chunk_tokens=span, merge=merge, label="growth %.1f %s span %d %s" % (rate, path, span, merge))


@pytest.mark.parametrize("shape", [(2, 32, 1, 128, 16000), (2, 16, 2, 128, 9000)], ids=["G32", "G8"])
@pytest.mark.parametrize("span", [64, 192])
def test_merge_of_many_pieces(shape, span):
    """Units split into up to 250 pieces (spans of 64 and 192 tokens): the
    merge kernel's lanes each take several load rounds of their strided
    pieces before the butterfly combines them; the fused merge reads them all
    in one workgroup."""
    B, H_q, H_kv, d, T = shape
    x = small(B, H_q, H_kv, d, T, seed=span + H_kv)
    x["seq_lens"] = torch.tensor([T, T * 2 // 3 + 1], dtype=torch.int32)
    for b, n in enumerate(x["seq_lens"].tolist()):
        x["k"][b, :, n:] = float("nan")
        x["v"][b, :, n:] = float("nan")
    for merge in ("kernel", "fused"):
        check(x, path="mfma", chunk_tokens=span, merge=merge, label="many pieces span %d %s" % (span, merge))


def test_token_split_with_empty_and_tiny_sequences():
    """Sequences of 0, 1, 15, 16, 17 and many tokens in one batch: the token
    stream skips empty sequences (their outputs are zero) and spans cross
    sequence and head boundaries at every kind of offset."""
    lens = [0, 1, 15, 16, 17, 0, 333, 1000, 64, 0, 129, 2]
    x = small(len(lens), 16, 2, 128, 1000, seed=71)
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
    for b, n in enumerate(lens):
        x["k"][b, :, n:] = float("nan")
        x["v"][b, :, n:] = float("nan")
    for span in (0, 64, 128, 320, 1024):
        for merge in ("fused", "kernel"):
            check(x, path="mfma", chunk_tokens=span, merge=merge, label="token-split span %d %s" % (span, merge))
    out = gpu_decode(x, path="mfma", out_dtype=torch.bfloat16).cpu()
    assert (out[0] == 0).all() and (out[5] == 0).all() and (out[9] == 0).all()


def test_all_sequences_empty():
    x = small(3, 8, 2, 64, 100, seed=72)
    x["seq_lens"] = torch.zeros(3, dtype=torch.int32)
    for path in ("mfma", "valu"):
        out = gpu_decode(x, path=path, out_dtype=torch.float32).cpu()
        assert (out == 0).all()


def test_workspace_shared_across_shapes():
    """Differently shaped calls share one workspace in stream order: every
    result stays correct."""
    cases = [small(3, 32, 8, 128, 900, seed=61, lo=100), small(2, 64, 8, 128, 2000, seed=62, lo=1500),
             small(5, 16, 2, 64, 700, seed=63, lo=1)]
    refs = [oracle.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"]) for x in cases]
    for rep in range(3):
        for x, ref, path, merge in zip(cases, refs, ["mfma", "valu", "mfma"], ["fused", "auto", "kernel"]):
            out = gpu_decode(x, path=path, chunk_tokens=64 * (rep + 2), merge=merge, out_dtype=torch.float32)
            assert err(out, ref) <= 2e-3
            out = gpu_decode(x, path=path, chunk_tokens=64 * (rep + 3), merge="fused", out_dtype=torch.float32)
            assert err(out, ref) <= 2e-3


def test_workspace_shared_across_paths():
    """The vector path's partial states never land in the counter region the
    fused merge relies on: alternate paths on one workspace."""
    x = small(3, 32, 8, 128, 1500, seed=64, lo=200)
    ref = oracle.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"])
    for rep in range(4):
        for path in ("valu", "mfma"):
            out = gpu_decode(x, path=path, chunk_tokens=256, merge="fused", out_dtype=torch.float32)
            assert err(out, ref) <= 2e-3, (rep, path)


@pytest.mark.parametrize("merge", ["fused", "kernel"])
def test_repeats_bitwise(merge):
    """Many calls in a row on one workspace give the same bits (the fused
    merge leaves its arrival counters at zero)."""
    x = small(4, 32, 8, 128, 3000, seed=33, lo=100)
    first = gpu_decode(x, path="mfma", chunk_tokens=256, merge=merge).cpu()
    for _ in range(20):
        assert torch.equal(gpu_decode(x, path="mfma", chunk_tokens=256, merge=merge).cpu(), first)


@pytest.mark.parametrize("merge", ["fused", "kernel"])
def test_graph_replays_match_eager(merge):
    """Decode calls captured in a HIP graph (a decode loop is commonly
    captured): the library records no memset and leaves its arrival counters
    at zero, so every replay gives the eager result bitwise, with eager work
    and synchronisations between the replays."""
    shapes = [(3, 32, 8, 128, 4000, 1), (2, 32, 1, 128, 600, 100)]
    xs = [to_dev(small(*sh[:5], seed=seed_of(sh, 41), lo=sh[5])) for sh in shapes]
    # and a layer batch under the planner's split, whose last layer is
    # claimed in chunks: its arrival ticket must be back at zero for the
    # next call in the graph and for every replay
    wl = workloads.Workload("graph-layers", 4, 32, 8, 128, 1, 1500, torch.bfloat16, 44, layers=3, packed=True)
    xl = to_dev(workloads.generate(wl, "cpu"))
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ls = [gqa.prepare(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], merge=merge, stream=s.cuda_stream,
                          chunk_tokens=256) for x in xs]
        ls.append(gqa.prepare(xl["q"], xl["k"], xl["v"], xl["seq_lens"], xl["scale"], kv_offsets=xl["kv_offsets"],
                              max_seq_len=1500, num_kv_heads=8, merge=merge, stream=s.cuda_stream))
        eager = [l().clone() for l in ls]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = [l() for l in ls] + [l() for l in ls]
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager + eager):
            assert torch.equal(o, e), "replay %d differs from the eager result" % rep
        gpu_decode(small(2, 8, 2, 64, 100, seed=43))   # eager work on the device between replays


def test_two_streams_use_their_own_default_workspaces():
    """Calls of different shapes issued on two streams that may overlap in
    time, each on the binding's default workspace and each using the fused
    merge's arrival counters: every stream gets a buffer of its own, and
    every result matches the oracle."""
    x = small(3, 32, 8, 128, 3000, seed=81, lo=1000)
    y = small(2, 64, 8, 128, 2500, seed=82, lo=500)
    rx = oracle.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"])
    ry = oracle.decode(y["q"], y["k"], y["v"], y["seq_lens"], y["scale"])
    xd, yd = to_dev(x), to_dev(y)
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    torch.cuda.synchronize()
    outs = []
    for rep in range(8):
        with torch.cuda.stream(s1):
            a = gqa.decode(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], chunk_tokens=64, merge="fused",
                           out_dtype=torch.float32)
        with torch.cuda.stream(s2):
            b = gqa.decode(yd["q"], yd["k"], yd["v"], yd["seq_lens"], y["scale"], chunk_tokens=128, merge="fused",
                           out_dtype=torch.float32)
        outs.append((a, b))
    torch.cuda.synchronize()
    w1 = gqa.default_workspace(1, DEV, s1.cuda_stream)
    w2 = gqa.default_workspace(1, DEV, s2.cuda_stream)
    assert w1.data_ptr() != w2.data_ptr()
    for a, b in outs:
        assert err(a, rx) <= 2e-3 and err(b, ry) <= 2e-3


def test_paths_and_chunkings_agree():
    x = small(2, 32, 8, 128, 1500, seed=41, lo=1000)
    ref = oracle.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"])
    for path in ("mfma", "valu"):
        for chunk in (0, 64, 128, 1024, 1536):
            assert err(gpu_decode(x, path=path, chunk_tokens=chunk, out_dtype=torch.float32), ref) <= 2e-3


def test_explicit_stream_and_workspace():
    x = small(2, 32, 8, 128, 1200, seed=43)
    xd = to_dev(x)
    dims = gqa.make_dims(2, 32, 8, 128, 1200, torch.bfloat16, torch.float32, chunk_tokens=256)
    ws = torch.zeros(gqa.workspace_bytes(dims), dtype=torch.uint8, device=DEV)   # zero-filled once, as required
    s = torch.cuda.Stream(DEV)
    with torch.cuda.stream(s):
        out = gqa.decode(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                         chunk_tokens=256, workspace=ws)
    s.synchronize()
    ref = oracle.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"])
    assert err(out, ref) <= 2e-3
    assert int(ws[:1 << 20].view(torch.int32).abs().sum()) == 0   # arrival counters back at zero


# ------------------------------------------------------------ layer batches --
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_layers(packed, path):
    w = workloads.Workload("layers", 3, 32, 8, 128, 100, 900, torch.bfloat16, 51, layers=4, packed=packed)
    x = workloads.generate(w, "cpu", poison_padding=True)
    xd = to_dev(x)
    note("layers", packed, path)
    kw = dict(kv_offsets=xd["kv_offsets"], max_seq_len=w.T_max, num_kv_heads=w.H_kv) if packed else {}
    out = gqa.decode_layers(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                            path=path, chunk_tokens=256, **kw)
    torch.cuda.synchronize()
    for l in range(w.layers):
        xl = workloads.layer_view(x, l)
        ref = oracle.decode(xl["q"], xl["k"], xl["v"], x["seq_lens"], x["scale"],
                            kv_offsets=x["kv_offsets"].numpy() if packed else None, num_kv_heads=w.H_kv)
        assert err(out[l], ref) <= 2e-3, l


LAYER_SPLIT_CASES = [
    # (H_q, H_kv, d), cached tokens per sequence, layers, packed layouts too
    ((16, 2, 128), [0, 1, 15, 16, 17, 0, 333, 1000, 64, 0, 129, 2], 5, True),   # G = 8, every kind of edge
    ((32, 1, 128), [700, 0, 1, 450], 3, True),    # MQA, G = 32: units split into many pieces per layer
    ((32, 8, 128), [3, 0, 5], 4, True),           # 64 positions per layer: most workgroups hold no span
    ((64, 8, 128), [17, 250], 2, True),           # G = 8, the whole layer inside few spans
    ((8, 2, 64), [0, 0, 0], 3, False),            # no tokens in any layer
    ((16, 4, 64), [5, 700, 0, 129, 2048], 3, True),   # d = 64, G = 4
]


@pytest.mark.parametrize("case", [(i, p) for i, c in enumerate(LAYER_SPLIT_CASES) for p in (False, True)
                                  if c[3] or not p], ids=lambda c: "case%d_%s" % (c[0], "packed" if c[1] else "dense"))
def test_layer_interleaved_split(case):
    """Layer batches: every workgroup streams its span of layer 0, then of
    layer 1, and so on.  Each layer meets the bar against the oracle under
    the planner's split and under forced spans (spans ending on a layer's
    last position, workgroups without a span in any layer, units split over
    many spans of one layer), with both merges; and since the spans of a
    layer are those a one-layer call plans, each layer's output is bitwise
    that of the one-layer call, except the last layer under the planner's
    split at G <= 16, which the workgroups claim in smaller chunks."""
    i, packed = case
    (H_q, H_kv, d), lens, L, _ = LAYER_SPLIT_CASES[i]
    sl = torch.tensor(lens, dtype=torch.int32)
    T = max(max(lens), 1)
    w = workloads.Workload("layer-split", len(lens), H_q, H_kv, d, 1, T, torch.bfloat16, 80 + i, layers=L,
                           packed=packed)
    x = workloads.generate(w, "cpu", poison_padding=True, seq_lens=sl)
    xd = to_dev(x)
    kw = dict(kv_offsets=xd["kv_offsets"], max_seq_len=T, num_kv_heads=H_kv) if packed else {}
    refs = []
    for l in range(L):
        xl = workloads.layer_view(x, l)
        refs.append(oracle.decode(xl["q"], xl["k"], xl["v"], x["seq_lens"], x["scale"],
                                  kv_offsets=x["kv_offsets"].numpy() if packed else None, num_kv_heads=H_kv))
    for span in (0, 64, 192):
        for merge in ("fused", "kernel"):
            note("layer split", i, packed, span, merge)
            run = lambda dt: gqa.decode_layers(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"],
                                               out_dtype=dt, path="mfma", chunk_tokens=span, merge=merge, **kw)
            out32, out16 = run(torch.float32), run(torch.bfloat16)
            torch.cuda.synchronize()
            assert torch.equal(out16, out32.to(torch.bfloat16))
            claimed = span == 0 and L >= 2 and H_q // H_kv <= 16
            for l in range(L):
                assert err(out32[l], refs[l]) <= 2e-3, (span, merge, l)
                if claimed and l == L - 1:
                    continue
                xl = workloads.layer_view(xd, l)
                if packed:
                    one = gqa.decode_layers(xl["q"][None], xl["k"], xl["v"], xd["seq_lens"], x["scale"],
                                            out_dtype=torch.float32, path="mfma", chunk_tokens=span, merge=merge,
                                            **kw)[0]
                else:
                    one = gqa.decode(xl["q"], xl["k"], xl["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                                     path="mfma", chunk_tokens=span, merge=merge)
                assert torch.equal(one, out32[l]), (span, merge, l)


@pytest.mark.parametrize("merge", ["fused", "kernel"])
@pytest.mark.parametrize("packed", [False, True])
def test_claimed_last_layer_is_deterministic(merge, packed):
    """A layer batch under the planner's split hands its last layer out in
    chunks claimed at run time: which workgroup streams a chunk changes from
    call to call, the results do not (a chunk's pieces depend only on its
    bounds, and merges run in slot order), and the arrival ticket and merge
    counters are back at zero after every call, so that calls of any shape
    can follow on the workspace."""
    lens = [0, 1, 300, 17, 2000, 0, 64, 931]
    w = workloads.Workload("claims", len(lens), 32, 8, 128, 1, 2000, torch.bfloat16, 91, layers=3, packed=packed)
    x = workloads.generate(w, "cpu", poison_padding=True, seq_lens=torch.tensor(lens, dtype=torch.int32))
    xd = to_dev(x)
    kw = dict(kv_offsets=xd["kv_offsets"], max_seq_len=2000, num_kv_heads=8) if packed else {}
    dims = gqa.make_dims(len(lens), 32, 8, 128, 2000, torch.bfloat16, out_dtype=torch.float32, merge=merge)
    nbytes = gqa.workspace_bytes(dims, 3)
    ws = torch.zeros(nbytes // 4 + 64, dtype=torch.int32, device=DEV)
    note("claims", merge, packed, nbytes)
    outs = [gqa.decode_layers(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                              merge=merge, workspace=ws, **kw) for _ in range(6)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    assert int(ws[:1 << 18].abs().sum()) == 0   # the counter region (ticket included) is back at zero
    l = w.layers - 1
    xl = workloads.layer_view(x, l)
    ref = oracle.decode(xl["q"], xl["k"], xl["v"], x["seq_lens"], x["scale"],
                        kv_offsets=x["kv_offsets"].numpy() if packed else None, num_kv_heads=8)
    assert err(outs[0][l], ref) <= 2e-3
    # a one-layer call on the same workspace afterwards
    x1 = workloads.layer_view(xd, 0)
    if packed:
        one = gqa.decode_layers(x1["q"][None], x1["k"], x1["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                                merge=merge, workspace=ws, **kw)[0]
    else:
        one = gqa.decode(x1["q"], x1["k"], x1["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                         merge=merge, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(one, outs[0][0])


# -------------------------------------------------------- full-size loads --
def sample_heads(B, H_q, n, seed):
    g = torch.Generator().manual_seed(seed)
    ids = torch.randperm(B * H_q, generator=g)[:n]
    return sorted(set(ids.tolist()) | {0, B * H_q - 1})


def full_check(name, sample=None, dtype=None, path="auto", extra_tol=None):
    w = workloads.WORKLOADS[name]
    if dtype is not None:
        w = w.replace(dtype=dtype)
    note("full", w.name, w.dtype, "generate")
    x = workloads.generate(w, DEV, poison_padding=True)
    note("full", w.name, "decode")
    out32 = gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], out_dtype=torch.float32, path=path)
    out16 = None
    if w.dtype == torch.bfloat16:
        out16 = gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], out_dtype=torch.bfloat16, path=path)
    torch.cuda.synchronize()
    tol = TOL[w.dtype] if extra_tol is None else extra_tol
    if out16 is not None:
        assert torch.equal(out16, out32.to(torch.bfloat16))
    if sample is None:
        note("full", w.name, "oracle on every head")
        xc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
        ref = oracle.decode(xc["q"], xc["k"], xc["v"], xc["seq_lens"], w.scale)
        e = err(out32, ref)
    else:
        heads = sample_heads(w.B, w.H_q, sample, 99)
        note("full", w.name, "oracle on %d sampled heads" % len(heads))
        e = 0.0
        for hid in heads:
            b, i = divmod(hid, w.H_q)
            g = i // w.G
            n = int(x["seq_lens"][b])
            q1 = x["q"][b:b + 1, i:i + 1].cpu()
            k1 = x["k"][b:b + 1, g:g + 1, :n].cpu()
            v1 = x["v"][b:b + 1, g:g + 1, :n].cpu()
            ref = oracle.decode(q1, k1, v1, torch.tensor([n], dtype=torch.int32), w.scale)[0, 0]
            e = max(e, err(out32[b, i], ref))
    note("full", w.name, "max err %.3e" % e)
    assert e <= tol
    return e


@pytest.mark.timeout(600)
def test_full_llama3_8b_layer():
    full_check("llama3-8b-layer")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layout", ["dense", "paged", "e4m3"])
@pytest.mark.parametrize("B,lo,hi", [(1024, 64, 64), (2048, 1, 100), (256, 256, 256)])
def test_many_short_units_every_head(B, lo, hi, layout):
    """Many short units in the planner's launch (one workgroup per CU): each
    span holds tens of whole units, so the incremental step to the next unit
    and the per-piece combine run thousands of times; every head against the
    oracle, for the plain cache, the same cache in shuffled pages of 16 and
    as E4M3 codes."""
    w = workloads.Workload("short-units", B, 32, 8, 128, lo, hi, torch.bfloat16, 1234 + B + hi)
    x = workloads.generate(w, "cpu", poison_padding=True)
    xd = to_dev(x)
    note("short units", B, lo, hi, layout)
    orc = oracle.default()
    if layout == "dense":
        run = lambda dt: gqa.decode(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], out_dtype=dt)
        ref = orc.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"])
    elif layout == "paged":
        kp, vp, tb = workloads.to_pages(x, 16, seed=B)
        kpd, vpd, tbd = kp.to(DEV), vp.to(DEV), tb.to(DEV)
        run = lambda dt: gqa.decode_paged(xd["q"], kpd, vpd, tbd, xd["seq_lens"], x["scale"], out_dtype=dt,
                                          max_seq_len=hi)
        ref = orc.decode_paged(x["q"], kp, vp, tb, 16, x["seq_lens"], x["scale"])
    else:
        x8 = workloads.to_e4m3(x)
        k8, v8 = x8["k"].to(DEV), x8["v"].to(DEV)
        run = lambda dt: gqa.decode_fp8(xd["q"], k8, v8, xd["seq_lens"], x["scale"], x8["k_scale"], x8["v_scale"],
                                        out_dtype=dt)
        ref = orc.decode_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], x["scale"], x8["k_scale"], x8["v_scale"])
    out32, out16 = run(torch.float32), run(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out16, out32.to(torch.bfloat16))
    assert err(out32, ref) <= TOL[torch.bfloat16]


@pytest.mark.timeout(600)
def test_full_llama3_8b_layer_fp32_inputs():
    """fp32 copy of the same shape at the fp32 bar: one dropped token at
    T = 4096 moves an output by ~1e-3, two orders above 1e-5."""
    full_check("llama3-8b-layer", dtype=torch.float32, path="valu")


@pytest.mark.timeout(600)
def test_full_70b_ragged_layer():
    full_check("llama-70b-ragged-layer")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["grouping-sweep-mha", "grouping-sweep-gqa", "grouping-sweep-mqa"])
def test_full_grouping_sweep(name):
    """Every output of the three grouping-sweep runs (8 x 32 heads over
    32768 tokens each) against the oracle."""
    full_check(name)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama-70b-ragged-layer", "grouping-sweep-mha", "grouping-sweep-gqa",
                                  "grouping-sweep-mqa"])
def test_full_size_fp32_inputs(name):
    """fp32 copies of the ragged 70B layer and of the grouping sweep, every
    output at the fp32 bar (vector path): one dropped or doubled token among
    32768 moves an output by ~1.5e-4, fifteen times the bar."""
    full_check(name, dtype=torch.float32, path="valu")


@pytest.mark.timeout(600)
def test_tp8_shards_of_the_70b_layer():
    """The ragged 70B layer split over eight GPUs by heads ([GQA-math]
    section 4, "Tensor Parallelism (TP) Head Partitioning"): GPU r holds KV
    head r and query heads 8r .. 8r+7, and runs this library's call on that
    share alone (one KV head, the per-GPU shape).  Every output of every
    share against the oracle of the whole layer's heads 8r .. 8r+7, and the
    bf16 output the rounding of the fp32 one."""
    w = workloads.WORKLOADS["llama-70b-ragged-layer"]
    note("tp8", "generate")
    x = workloads.generate(w, DEV, poison_padding=True)
    xc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    note("tp8", "oracle on the whole layer")
    ref = oracle.decode(xc["q"], xc["k"], xc["v"], xc["seq_lens"], w.scale)
    e = 0.0
    for r in range(8):
        s = workloads.tp_shard(x, 8, r)
        note("tp8", "rank %d" % r)
        out32 = gqa.decode(s["q"], s["k"], s["v"], s["seq_lens"], s["scale"], out_dtype=torch.float32)
        out16 = gqa.decode(s["q"], s["k"], s["v"], s["seq_lens"], s["scale"], out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(out16, out32.to(torch.bfloat16))
        e = max(e, err(out32, ref[:, 8 * r:8 * r + 8]))
        del s
    note("tp8", "max err %.3e" % e)
    assert e <= 2e-3
    del x
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_full_32_layer_stack():
    """The 32-layer packed stack at full size (about 160 GB of cache), one
    launch: every output of every layer against the oracle, layer by layer
    (each layer's cache copied to the host), and the bf16 output bitwise the
    rounding of the fp32 one."""
    w = workloads.WORKLOADS["llama3-8b-32-layer-stack"]
    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info(DEV)
    sl = workloads.seq_lens_for(w)
    need = 2 * w.layers * int(sl.sum()) * w.H_kv * w.d * 2
    if need > free - (8 << 30):
        pytest.skip("needs %.1f GB of device memory, %.1f free" % (need / 1e9, free / 1e9))
    note("full", w.name, "generate %.1f GB" % (need / 1e9))
    x = workloads.generate(w, DEV)
    note("full", w.name, "decode")
    kw = dict(kv_offsets=x["kv_offsets"], max_seq_len=w.T_max, num_kv_heads=w.H_kv)
    out = gqa.decode_layers(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], out_dtype=torch.float32, **kw)
    out16 = gqa.decode_layers(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out16, out.to(torch.bfloat16))
    offs = x["kv_offsets"].cpu().numpy()
    sl = x["seq_lens"].cpu()
    e = 0.0
    for l in range(w.layers):
        xl = workloads.layer_view(x, l)
        ref = oracle.decode(xl["q"].cpu(), xl["k"].cpu(), xl["v"].cpu(), sl, w.scale, kv_offsets=offs,
                            num_kv_heads=w.H_kv)
        el = err(out[l], ref)
        note("full", w.name, "layer %d: max err %.3e" % (l, el))
        e = max(e, el)
    assert e <= 2e-3
    del x
    torch.cuda.empty_cache()


# ------------------------------------------ cuts of the planner's own split --
def planner_cuts(B, H_q, H_kv, d, T_max, lens):
    """Stream positions where the planner's even token split cuts the
    (sequence, KV head, token) stream of one layer: every workgroup owns
    span = ceil(total / workgroups) positions rounded up to a multiple of 16
    (the split the header describes, with the workgroup count the library
    reports), as (b, g, t) with t the first token of the later piece."""
    _, groups = gqa.plan(gqa.make_dims(B, H_q, H_kv, d, T_max, torch.bfloat16))
    total = H_kv * sum(lens)
    span = max(16, -(-(-(-total // groups)) // 16) * 16)
    starts = []   # (stream position of the unit's token 0, b, g, n)
    pos = 0
    for b, n in enumerate(lens):
        for g in range(H_kv):
            if n > 0:
                starts.append((pos, b, g, n))
            pos += n
    cuts, u = [], 0
    for w in range(1, groups):
        x = w * span
        if x >= total:
            break
        while u + 1 < len(starts) and starts[u + 1][0] <= x:
            u += 1
        p0, b, g, n = starts[u]
        cuts.append((b, g, x - p0, u))
    return cuts, starts


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama3-8b-layer", "llama-70b-ragged-layer"])
def test_spikes_at_the_planners_cuts(name):
    """Full-size layers under the planner's own split (no forced span): every
    cache token on either side of each cut, and the tiles around it, gets an
    equal, overwhelming score (a "spike"), so each head's output is the plain
    mean of its unit's spike values.  A token dropped or doubled at a cut
    moves that mean by O(0.1), ten thousand times the fp32-output bar here;
    units the split does not cut get one spike.  Also checked against the
    oracle on the same inputs."""
    w = workloads.WORKLOADS[name]
    x = workloads.generate(w, DEV, poison_padding=True)
    lens = x["seq_lens"].cpu().tolist()
    cuts, starts = planner_cuts(w.B, w.H_q, w.H_kv, w.d, w.T_max, lens)
    spikes = {}   # unit index -> token positions
    for b, g, t, u in cuts:
        n = lens[b]
        if t == 0:   # a cut between units: the previous unit's last token and this one's first
            spikes.setdefault(u - 1, set()).add(starts[u - 1][3] - 1)
            spikes.setdefault(u, set()).add(0)
            continue
        for tt in (t - 16, t - 1, t, t + 15):
            if 0 <= tt < n:
                spikes.setdefault(u, set()).add(tt)
    gen = torch.Generator().manual_seed(11)
    for u, (_, b, g, n) in enumerate(starts):
        if u not in spikes:
            spikes[u] = {int(torch.randint(n, (1,), generator=gen))}
    note("planner cuts", name, "%d cuts, %d units" % (len(cuts), len(starts)))
    x["q"].zero_()
    x["q"][..., 0] = 8.0
    for u, ts in spikes.items():
        _, b, g, n = starts[u]
        idx = torch.tensor(sorted(ts), device=DEV)
        row = torch.zeros(w.d, dtype=x["k"].dtype, device=DEV)
        row[0] = 64.0                      # score 8 * 64 / sqrt(128) = 45 against |score| < 4 elsewhere
        x["k"][b, g, idx] = row
    out = gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], out_dtype=torch.float32)
    out16 = gqa.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out16, out.to(torch.bfloat16))
    o = out.double().cpu()
    e = 0.0
    for u, ts in spikes.items():
        _, b, g, n = starts[u]
        want = x["v"][b, g, torch.tensor(sorted(ts), device=DEV)].double().mean(0).cpu()
        e = max(e, float((o[b, g * w.G:(g + 1) * w.G] - want).abs().max()))
    note("planner cuts", name, "max |out - spike mean| %.3e" % e)
    assert e <= 1e-5
    xc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    ref = oracle.decode(xc["q"], xc["k"], xc["v"], xc["seq_lens"], w.scale)
    assert err(out, ref) <= 2e-3


# -------------------------------------------------------- largest batches --
@pytest.mark.timeout(300)
def test_batch_at_the_matrix_core_limit():
    """4096 sequences (the most whose prefix sums the matrix-core path keeps
    in LDS: 16 per thread), lengths 0 .. 40, dense and paged; 4097 sequences
    on the automatic path run on the vector path, which has no such limit."""
    g = torch.Generator().manual_seed(4096)
    for B, path, expect_mfma in ((4096, "auto", True), (4097, "auto", False)):
        x = small(B, 8, 2, 64, 40, seed=B)
        x["seq_lens"] = torch.randint(0, 41, (B,), generator=g, dtype=torch.int32)
        for b, n in enumerate(x["seq_lens"].tolist()):
            x["k"][b, :, n:] = float("nan")
            x["v"][b, :, n:] = float("nan")
        d = gqa.make_dims(B, 8, 2, 64, 40, torch.bfloat16, path=path)
        chunk, n = gqa.plan(d)
        assert (chunk == 0) == expect_mfma, (B, chunk, n)   # the matrix-core split reports no chunk size
        check(x, label="B=%d %s" % (B, path))
        if B == 4096:
            xd = to_dev(x)
            kp, vp, tb = workloads.to_pages(xd, 16, seed=1)
            out = gqa.decode_paged(xd["q"], kp, vp, tb, xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                                   max_seq_len=40)
            torch.cuda.synchronize()
            ref = oracle.default().decode_paged(x["q"], kp.cpu(), vp.cpu(), tb.cpu(), 16, x["seq_lens"], x["scale"])
            assert err(out, ref) <= 2e-3
    with pytest.raises(gqa.GqaError):   # forcing the matrix-core path beyond its limit is refused
        xd = to_dev(small(4097, 8, 2, 64, 16, seed=1))
        gqa.decode(xd["q"], xd["k"], xd["v"], xd["seq_lens"], xd["scale"], path="mfma")
