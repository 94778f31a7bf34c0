"""gqa_decode_noalloc (partial states in the library's static device buffer)
against gqa_decode (caller workspace), through the C ABI: bitwise equal
results, and both within the oracle's bar, on calls in a row whose second
input is smaller than the first."""
import numpy as np
import pytest
import torch

import gqa_mqa_kv_amd as gqa
import oracle
from gqa_mqa_kv_amd import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}


def case(B, H_q, H_kv, d, T, lo, seed, dtype=torch.bfloat16):
    w = workloads.Workload("noalloc", B, H_q, H_kv, d, lo, T, dtype, seed)
    x = workloads.generate(w, "cpu", poison_padding=True)
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    return x, xd


def run_pair(x, xd, **kw):
    """The same step through gqa_decode_noalloc and through gqa_decode."""
    print("[gpu-case] noalloc", tuple(x["q"].shape), tuple(x["k"].shape), x["q"].dtype, kw, flush=True)
    a = gqa.decode_noalloc(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32, **kw)
    b = gqa.decode(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"])
    assert torch.equal(a, b), "noalloc differs from the workspace call"
    o = a.double().cpu().numpy()
    assert np.isfinite(o).all()
    assert float(np.abs(o - ref).max()) <= TOL[x["q"].dtype]
    return a


# Each pair: the larger input first, then a smaller one.
PAIRS = [
    # (shape of the first call, shape of the second), extra kwargs
    (((4, 32, 8, 128, 3000, 900), (2, 8, 2, 64, 500, 1)), dict()),                            # even split
    (((3, 32, 8, 128, 2000, 1), (2, 16, 4, 128, 700, 100)), dict(chunk_tokens=64, merge="fused")),
    (((2, 32, 1, 128, 4000, 3000), (1, 32, 1, 128, 900, 900)), dict(chunk_tokens=128, merge="kernel")),
    (((2, 64, 8, 128, 1500, 1), (1, 16, 2, 64, 300, 1)), dict(chunk_tokens=192)),
]


@pytest.mark.parametrize("pair,kw", PAIRS, ids=["even", "fused-spans", "kernel-merge", "g8-spans"])
def test_noalloc_matches_workspace_call(pair, kw):
    for i, sh in enumerate(pair):
        x, xd = case(*sh, seed=1000 + 17 * i + sh[0])
        first = run_pair(x, xd, **kw)
        # again on the same buffer: the counters the fused merge used are back at zero
        again = gqa.decode_noalloc(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], out_dtype=torch.float32,
                                   **kw)
        torch.cuda.synchronize()
        assert torch.equal(first, again)


def test_noalloc_vector_path_and_bf16_out():
    """fp32 inputs (vector path: chunk states in the static buffer), then a
    smaller bf16 call with bf16 output."""
    x, xd = case(2, 32, 8, 128, 2500, 700, seed=5, dtype=torch.float32)
    run_pair(x, xd, chunk_tokens=256)
    y, yd = case(1, 8, 2, 64, 400, 1, seed=6)
    a = gqa.decode_noalloc(yd["q"], yd["k"], yd["v"], yd["seq_lens"], y["scale"])
    b = gqa.decode(yd["q"], yd["k"], yd["v"], yd["seq_lens"], y["scale"])
    torch.cuda.synchronize()
    assert a.dtype == torch.bfloat16 and torch.equal(a, b)


def test_noalloc_under_graph_capture():
    """The entry point is for callers that cannot allocate, such as code under
    HIP graph capture: calls captured in a graph (two shapes, the fused
    merge's counters in use) replay bitwise like the eager calls, with eager
    work between the replays."""
    x, xd = case(3, 32, 8, 128, 2000, 500, seed=41)
    y, yd = case(2, 32, 1, 128, 1500, 1000, seed=42)
    s = torch.cuda.Stream(DEV)
    outs = [torch.empty(3, 32, 128, dtype=torch.float32, device=DEV),
            torch.empty(2, 32, 128, dtype=torch.float32, device=DEV)]
    f32 = torch.float32
    calls = [lambda: gqa.decode_noalloc(xd["q"], xd["k"], xd["v"], xd["seq_lens"], x["scale"], out=outs[0],
                                        out_dtype=f32, chunk_tokens=128, merge="fused", stream=s.cuda_stream),
             lambda: gqa.decode_noalloc(yd["q"], yd["k"], yd["v"], yd["seq_lens"], y["scale"], out=outs[1],
                                        out_dtype=f32, chunk_tokens=64, merge="kernel", stream=s.cuda_stream)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for c in calls:
            c()
    s.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), "replay %d differs" % rep
        run_pair(x, xd, chunk_tokens=256)   # eager work between the replays
