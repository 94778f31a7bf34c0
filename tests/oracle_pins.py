"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an oracle handle (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with:
  * the printed tables/figures of the pages (``tests/golden/``),
  * closed forms and invariants of softmax attention,
  * a library routine: ``torch.nn.functional.scaled_dot_product_attention``
    (CPU, float64), whose ``enable_gqa`` mode expands K/V with
    repeat_interleave -- the equivalent formulation printed in "Grouped-Query
    Attention (GQA) and Multi-Query Attention (MQA): ...", section 2,
    subsection "Grouped-Query Attention (GQA)".

The same pins run against deliberately broken copies of the oracle
(test_oracle_mutants.py) to show that a plausible mistake anywhere in it fails
at least one of them.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle as oracle_mod
from gqa_mqa_kv_amd import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def case(B, H_q, H_kv, d, T, seed, dtype=torch.float64, lo=None, poison=False):
    """Small seeded input (dense layout); lengths U[lo, T] when ``lo`` is given."""
    w = workloads.Workload("pin", B, H_q, H_kv, d, lo if lo is not None else T, T, dtype, seed)
    return workloads.generate(w, "cpu", poison_padding=poison)


def sdpa_reference(x):
    """Library routine: SDPA (float64 CPU) per sequence over its valid tokens,
    with enable_gqa (repeat_interleave of K/V along heads)."""
    q, k, v, sl = x["q"].double(), x["k"].double(), x["v"].double(), x["seq_lens"]
    B, H_q, d = q.shape
    out = torch.zeros(B, H_q, d, dtype=torch.float64)
    for b in range(B):
        n = int(sl[b])
        if n == 0:
            continue
        o = F.scaled_dot_product_attention(q[b:b + 1, :, None, :], k[b:b + 1, :, :n, :], v[b:b + 1, :, :n, :],
                                           scale=float(np.float32(x["scale"])), enable_gqa=True)
        out[b] = o[0, :, 0, :]
    return out.numpy()


def run(orc, x, **kw):
    return orc.decode(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], **kw)


# ---------------------------------------------------------------- group map --
def pin_group_count_theorem(orc):
    """E contiguous heads in groups of G touch exactly (E+G-1)/G groups
    ("Exact-head packing attains the bound: placing E exact heads contiguously
    in groups of G hits exactly ceil(E/G) groups", the theorem statement)."""
    for G in range(1, 65):
        for E in range(0, 65):
            touched = {orc.group_of(i, G) for i in range(E)}
            assert len(touched) == (E + G - 1) // G, (E, G, len(touched))


def pin_tp_partition_figure(orc):
    """Figure "TENSOR PARALLEL PARTITIONING (Llama 3 70B on TP=8)": query heads
    8k..8k+7 read KV head k (H_Q=64, H_KV=8, R=8)."""
    for gpu, lo, hi, kv in golden_rows("tp8_head_partition_llama3_70b.txt"):
        for i in range(int(lo), int(hi) + 1):
            assert orc.group_of(i, 64 // 8) == int(kv), (i, kv)


def pin_production_shapes(orc):
    """Table "ATTENTION ARCHITECTURES IN PRODUCTION": R = H_Q/H_KV, and the
    contiguous map sends exactly R query heads to each of the H_KV KV heads."""
    for model, hq, hkv, r, comp in golden_rows("production_attention_shapes.txt"):
        hq, hkv, r = int(hq), int(hkv), int(r)
        assert hq // hkv == r and float(comp) == hq / hkv, model
        counts = np.bincount([orc.group_of(i, r) for i in range(hq)], minlength=hkv)
        assert counts.shape == (hkv,) and (counts == r).all(), model


# ------------------------------------------------------- library routine --
def pin_gqa_equals_sdpa(orc):
    """GQA output == SDPA with repeat_interleave'd K/V (float64), several G,
    ragged lengths, d=64 and 128."""
    for (B, hq, hkv, d, T, lo, seed) in [(3, 8, 2, 64, 37, 1, 11), (2, 32, 8, 128, 70, 5, 12),
                                         (2, 64, 8, 128, 33, 1, 13), (2, 12, 3, 64, 50, 20, 14)]:
        x = case(B, hq, hkv, d, T, seed, lo=lo)
        got = run(orc, x)
        ref = sdpa_reference(x)
        assert np.abs(got - ref).max() < 1e-12, (B, hq, hkv, np.abs(got - ref).max())


def pin_mha_equals_sdpa(orc):
    """H_KV = H_Q reduces to independent per-head attention ("Multi-Head
    Attention (MHA)" subsection): compare with plain SDPA, no grouping."""
    x = case(2, 6, 6, 64, 40, 21, lo=3)
    got = run(orc, x)
    q, k, v = x["q"], x["k"], x["v"]
    for b in range(2):
        n = int(x["seq_lens"][b])
        ref = F.scaled_dot_product_attention(q[b, :, None, :], k[b, :, :n], v[b, :, :n],
                                             scale=float(np.float32(x["scale"])))[:, 0]
        assert np.abs(got[b] - ref.numpy()).max() < 1e-12


def pin_mqa_shared_kv(orc):
    """H_KV = 1 ("Multi-Query Attention (MQA)" subsection): every head reads
    the one K/V head; heads with equal query rows give equal outputs; equals
    SDPA with K/V broadcast over heads."""
    x = case(2, 8, 1, 64, 30, 31, lo=7)
    x["q"][:, 5] = x["q"][:, 2]
    got = run(orc, x)
    assert np.array_equal(got[:, 5], got[:, 2])
    q, k, v = x["q"], x["k"], x["v"]
    for b in range(2):
        n = int(x["seq_lens"][b])
        kb = k[b, 0:1, :n].expand(8, n, 64)
        vb = v[b, 0:1, :n].expand(8, n, 64)
        ref = F.scaled_dot_product_attention(q[b, :, None, :], kb, vb, scale=float(np.float32(x["scale"])))[:, 0]
        assert np.abs(got[b] - ref.numpy()).max() < 1e-12


# -------------------------------------------------------------- invariants --
def pin_weights_sum_to_one(orc):
    x = case(2, 8, 2, 64, 50, 41, lo=1)
    for b in range(2):
        for i in range(8):
            w, out = orc.head_weights(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], b, i)
            assert w.shape == (int(x["seq_lens"][b]),)
            assert abs(w.sum() - 1.0) < 1e-14 and (w > 0).all()
            # the output is the weighted sum of the group's value rows
            g = i // 4
            n = w.shape[0]
            assert np.abs(out - w @ x["v"][b, g, :n].numpy()).max() < 1e-14


def pin_permutation_invariance(orc):
    x = case(1, 8, 2, 64, 45, 51)
    base = run(orc, x)
    perm = torch.randperm(45, generator=torch.Generator().manual_seed(5))
    y = dict(x, k=x["k"][:, :, perm].contiguous(), v=x["v"][:, :, perm].contiguous())
    assert np.abs(run(orc, y) - base).max() < 1e-13


def pin_single_token(orc):
    """One cached token: the weight is exactly 1 and the output is V exactly."""
    x = case(2, 8, 2, 64, 1, 61)
    got = run(orc, x)
    for b in range(2):
        for i in range(8):
            assert np.array_equal(got[b, i], x["v"][b, i // 4, 0].numpy())


def pin_constant_values(orc):
    x = case(1, 8, 4, 64, 33, 71)
    row = torch.linspace(-2, 2, 64, dtype=torch.float64)
    x["v"][:] = row
    got = run(orc, x)
    assert np.abs(got - row.numpy()).max() < 1e-14


def pin_zero_query_is_mean(orc):
    """q = 0 makes every score 0, so the output is the mean of the valid V rows."""
    x = case(2, 8, 2, 64, 29, 81, lo=4)
    x["q"].zero_()
    got = run(orc, x)
    for b in range(2):
        n = int(x["seq_lens"][b])
        for i in range(8):
            assert np.abs(got[b, i] - x["v"][b, i // 4, :n].mean(0).numpy()).max() < 1e-14


def pin_key_shift_invariance(orc):
    """Adding one vector to every key shifts all scores of a head equally."""
    x = case(1, 8, 2, 64, 31, 91)
    base = run(orc, x)
    shift = torch.randn(1, 2, 1, 64, dtype=torch.float64, generator=torch.Generator().manual_seed(9))
    y = dict(x, k=x["k"] + shift)
    assert np.abs(run(orc, y) - base).max() < 1e-12


def pin_linearity_in_values(orc):
    x = case(1, 8, 2, 64, 27, 101)
    v2 = torch.randn(x["v"].shape, dtype=torch.float64, generator=torch.Generator().manual_seed(3))
    a = run(orc, x)
    b = run(orc, dict(x, v=v2))
    c = run(orc, dict(x, v=2.0 * x["v"] - 3.0 * v2))
    assert np.abs(c - (2.0 * a - 3.0 * b)).max() < 1e-12


def pin_hand_example(orc):
    """Worked by hand: d=1, scale=1, q=1, keys 0 and ln 3 give weights 1/4 and
    3/4; values 4 and 8 give 4/4 + 3*8/4 = 7."""
    q = torch.ones(1, 1, 1, dtype=torch.float64)
    k = torch.tensor([0.0, math.log(3.0)], dtype=torch.float64).view(1, 1, 2, 1)
    v = torch.tensor([4.0, 8.0], dtype=torch.float64).view(1, 1, 2, 1)
    got = orc.decode(q, k, v, [2], 1.0)
    assert abs(got[0, 0, 0] - 7.0) < 1e-13


def pin_empty_sequence_is_zero(orc):
    x = case(2, 8, 2, 64, 16, 111)
    x["seq_lens"][1] = 0
    got = run(orc, x)
    assert (got[1] == 0).all() and np.isfinite(got[0]).all() and np.abs(got[0]).max() > 0


def pin_padding_never_read(orc):
    """Positions at or beyond seq_len (NaN here) do not reach the output, and
    the result equals the same cache cut to its valid length."""
    x = case(3, 8, 2, 64, 40, 121, lo=3, poison=True)
    got = run(orc, x)
    assert np.isfinite(got).all()
    for b in range(3):
        n = int(x["seq_lens"][b])
        y = dict(x, q=x["q"][b:b + 1], k=x["k"][b:b + 1, :, :n].contiguous(), v=x["v"][b:b + 1, :, :n].contiguous(),
                 seq_lens=x["seq_lens"][b:b + 1])
        assert np.array_equal(run(orc, y)[0], got[b])


def pin_bf16_and_fp32_widening(orc):
    """bf16/fp32 inputs are widened exactly: same result as their float64 copies."""
    for dt in (torch.bfloat16, torch.float32):
        x = case(2, 8, 2, 64, 19, 131, dtype=dt, lo=2)
        y = dict(x, q=x["q"].double(), k=x["k"].double(), v=x["v"].double())
        assert np.array_equal(run(orc, x), run(orc, y))


def pin_packed_layout(orc):
    """The packed ragged layout addresses the same tokens as the dense one."""
    x = case(3, 8, 2, 64, 25, 141, lo=1)
    dense = run(orc, x)
    sl = x["seq_lens"]
    offs = workloads.packed_offsets(sl)
    rows = []
    for b in range(3):
        n = int(sl[b])
        rows.append(x["k"][b, :, :n].reshape(-1, 64))
    kp = torch.cat(rows)
    vp = torch.cat([x["v"][b, :, :int(sl[b])].reshape(-1, 64) for b in range(3)])
    packed = orc.decode(x["q"], kp, vp, sl, x["scale"], kv_offsets=offs.numpy())
    assert np.array_equal(packed, dense)


def pin_head_subset(orc):
    x = case(2, 8, 2, 64, 21, 151, lo=5)
    full = run(orc, x).reshape(16, 64)
    ids = [15, 0, 7, 8]
    assert np.array_equal(run(orc, x, heads=ids), full[ids])


def paged_copy(x, page, seed, spare=3):
    """The dense cache of ``x`` cut into pages of ``page`` tokens, spread over
    a shuffled pool with ``spare`` unused pages (NaN), and its block table."""
    B, H_kv, T, d = x["k"].shape
    mp = -(-T // page)
    n_pages = B * mp + spare
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(seed))
    kp = torch.full((n_pages, H_kv, page, d), float("nan"), dtype=x["k"].dtype)
    vp = torch.full((n_pages, H_kv, page, d), float("nan"), dtype=x["k"].dtype)
    table = torch.zeros(B, mp, dtype=torch.int32)
    for b in range(B):
        for j in range(mp):
            pid = int(perm[b * mp + j])
            table[b, j] = pid
            n = min(page, T - j * page)
            kp[pid, :, :n] = x["k"][b, :, j * page:j * page + n]
            vp[pid, :, :n] = x["v"][b, :, j * page:j * page + n]
    return kp, vp, table


def pin_paged_layout(orc):
    """A cache held in shuffled pages of a pool (unused pages and page tails
    NaN) gives bitwise the dense cache's result, for pages of 1, 16 and the
    whole capacity."""
    x = case(3, 8, 2, 64, 48, 161, lo=1, poison=True)
    dense = run(orc, x)
    for page in (1, 16, 48):
        kp, vp, table = paged_copy(x, page, seed=page)
        got = orc.decode_paged(x["q"], kp, vp, table, page, x["seq_lens"], x["scale"])
        assert np.array_equal(got, dense), page


# ------------------------------------------------ one-byte E4M3 caches --
# The bytes-per-element factor of "Grouped-Query Attention (GQA) and
# Multi-Query Attention (MQA): ...", section 1, "KV Cache Memory Footprint"
# (2 for FP16/BF16), taken to one byte: OCP E4M3 elements with one scale per
# array (the pages give no format; this is the reading the oracle states).
def pin_e4m3_decode(orc):
    """All 256 codes against torch's float8_e4m3fn widening (a library
    routine), and the format's landmarks: 0x38 = 1, 0x7E = 448 (largest
    finite), 0x08 = 2^-6 (smallest normal), 0x07 = 7 * 2^-9 and 0x01 = 2^-9
    (subnormals), 0x80 = -0, 0x7F and 0xFF NaN."""
    codes = torch.arange(256, dtype=torch.uint8)
    got = orc.e4m3(codes)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, lib, equal_nan=True)
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x08] == 2.0 ** -6 and got[0x07] == 7 * 2.0 ** -9 and got[0x01] == 2.0 ** -9
    assert got[0x80] == 0.0 and np.signbit(got[0x80])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.isfinite(np.delete(got, [0x7F, 0xFF])).all()


def pin_fp8_attention_is_dequantised_attention(orc):
    """The E4M3-cache attention equals the fp64 attention over K =
    k_scale * E4M3(k8) and V = v_scale * E4M3(v8), widened by torch; ragged
    lengths with NaN codes in the padding, GQA and MQA, distinct scales."""
    for shape, seed in (((3, 8, 2, 64, 40), 71), ((2, 16, 1, 32, 33), 72)):
        x = case(*shape, seed=seed, dtype=torch.bfloat16, lo=0, poison=True)
        x8 = workloads.to_e4m3(x)
        ks, vs = x8["k_scale"], x8["v_scale"] * 1.5
        got = orc.decode_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], x["scale"], ks, vs)
        kd = x8["k"].view(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(ks))
        vd = x8["v"].view(torch.float8_e4m3fn).to(torch.float64) * float(np.float32(vs))
        want = orc.decode(x["q"].double(), kd, vd, x["seq_lens"], x["scale"])
        assert np.isfinite(got).all() and np.abs(got - want).max() <= 1e-12, shape


def pin_e4m3_encode(orc):
    """The encoder the quantising append follows: every finite code
    re-encodes to itself; float32 values across the whole range, every
    midpoint between neighbouring codes (ties go to the even mantissa) and
    the float32 neighbours of those midpoints agree with torch's
    float8_e4m3fn conversion (a library routine) below 448; beyond it the
    encoder saturates (448, infinities), and NaN gives 0x7F."""
    codes = torch.arange(256, dtype=torch.uint8)
    vals = orc.e4m3(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(orc.e4m3_encode(vals[fin]), codes.numpy()[fin])
    pos = np.sort(vals[(vals >= 0) & fin & ~np.signbit(vals)])
    mids = (pos[:-1] + pos[1:]) / 2                       # exact in float32 (4 significant bits)
    m32 = torch.tensor(mids, dtype=torch.float32)
    around = torch.cat([m32, torch.nextafter(m32, torch.tensor(np.inf, dtype=torch.float32)),
                        torch.nextafter(m32, torch.tensor(-np.inf, dtype=torch.float32))])
    g = torch.Generator().manual_seed(31)
    rnd = torch.randn(100000, generator=g) * torch.exp(torch.empty(100000).uniform_(-14, 6, generator=g))
    x = torch.cat([around, -around, rnd])
    x = x[x.abs() < 448]
    lib = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(x.double()), lib)
    # ties: 1 + 1/16 -> 1, 1 + 3/16 -> 1.25, 2^-10 -> 0, 3 * 2^-11 -> 2^-9
    assert orc.e4m3_encode([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11]).tolist() == [0x38, 0x3A, 0x00, 0x01]
    sat = orc.e4m3_encode([448.0, 460.0, 1e9, np.inf, -1e9, -np.inf, np.nan, -0.0])
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80]


def pin_fp8_paged_layout(orc):
    """An E4M3 cache held in shuffled pages (spare pages and page tails hold
    the NaN code) gives bitwise the dense E4M3 cache's result."""
    x = case(3, 8, 2, 64, 48, 161, dtype=torch.bfloat16, lo=1, poison=True)
    x8 = workloads.to_e4m3(x)
    dense = orc.decode_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], x["scale"], x8["k_scale"], x8["v_scale"])
    for page in (16, 48):
        kp, vp, table = workloads.to_pages(x8, page, seed=page)
        got = orc.decode_paged_fp8(x["q"], kp, vp, table, page, x["seq_lens"], x["scale"], x8["k_scale"],
                                   x8["v_scale"])
        assert np.array_equal(got, dense), page


def pin_fp8_scale_placement(orc):
    """k_scale multiplies the scores and v_scale the output: with powers of
    two every product stays exact, so trading k_scale against ``scale`` and
    pulling v_scale out of the sum change nothing, bitwise."""
    x = case(2, 8, 2, 32, 24, 73, dtype=torch.bfloat16, lo=1)
    x8 = workloads.to_e4m3(x)
    a = orc.decode_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], x["scale"], 2.0, 1.0)
    b = orc.decode_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], 2.0 * x["scale"], 1.0, 1.0)
    c = orc.decode_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], x["scale"], 1.0, 4.0)
    d = orc.decode_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], x["scale"], 1.0, 1.0)
    assert np.array_equal(a, b)
    assert np.array_equal(c, 4.0 * d)
    assert not np.allclose(a, d)


# --------------------------------------------- rotary position embedding --
# "Grouped-Query Attention (GQA) and Multi-Query Attention (MQA): ...",
# section 4, "Rotary Position Embeddings (RoPE) Interaction".
def pin_rope_closed_form(orc):
    """Block-diagonal rotation of consecutive pairs, by m * base^(-2j/d):
    d = 4, base 100 -> theta = (1, 1/10).  e_0 at position m goes to
    (cos m, sin m, 0, 0); e_3 to (0, 0, -sin(m/10), cos(m/10))."""
    x = torch.zeros(2, 4, dtype=torch.float64)
    x[0, 0] = 1.0
    x[1, 3] = 1.0
    for m in (0, 1, 7, 1000):
        got = orc.rope(x, [m, m], 100.0)
        want = np.array([[math.cos(m), math.sin(m), 0.0, 0.0],
                         [0.0, 0.0, -math.sin(m / 10.0), math.cos(m / 10.0)]])
        assert np.abs(got - want).max() < 1e-12, m


def pin_rope_identity_norm_composition(orc):
    """Position 0 is the identity; every pair keeps its length; turning by a
    then by b is turning by a + b."""
    g = torch.Generator().manual_seed(201)
    x = torch.randn(6, 128, dtype=torch.float64, generator=g)
    assert np.array_equal(orc.rope(x, 0, 10000.0), x.numpy())
    pos = [0, 1, 17, 4095, 32767, 131071]
    y = orc.rope(x, pos, 10000.0)
    n0 = (x.numpy().reshape(6, 64, 2) ** 2).sum(-1)
    n1 = (y.reshape(6, 64, 2) ** 2).sum(-1)
    assert np.abs(n0 - n1).max() < 1e-11
    a, b = [3, 100, 5000, 1, 0, 77], [9, 28, 11111, 32766, 131071, 2]
    two = orc.rope(torch.from_numpy(orc.rope(x, a, 10000.0)), b, 10000.0)
    one = orc.rope(x, [i + j for i, j in zip(a, b)], 10000.0)
    assert np.abs(two - one).max() < 1e-9


def pin_rope_relative_position(orc):
    """The page's identity: <R_m q, R_n k> = <R_(m-n) q, k> (the score of a
    query head with its group's key depends on the distance only)."""
    g = torch.Generator().manual_seed(202)
    q = torch.randn(1, 64, dtype=torch.float64, generator=g)
    k = torch.randn(1, 64, dtype=torch.float64, generator=g)
    for m, n in ((5, 3), (0, 9), (4096, 4000), (30000, 12)):
        lhs = float((orc.rope(q, m, 10000.0) * orc.rope(k, n, 10000.0)).sum())
        rhs = float((orc.rope(q, m - n, 10000.0) * k.numpy()).sum())
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(rhs)), (m, n)


def pin_rope_attention_shift(orc):
    """Rotating every query at position p and every cached key at its own
    position t leaves the GQA outputs unchanged when all positions move by
    the same offset (scores depend on p - t only)."""
    x = case(2, 8, 2, 64, 12, 211, lo=3)
    T = x["k"].shape[2]
    outs = []
    for off in (0, 1000):
        pq = torch.tensor([int(n) - 1 + off for n in x["seq_lens"]])
        q = torch.from_numpy(orc.rope(x["q"], pq.view(2, 1), 10000.0))
        k = torch.from_numpy(orc.rope(x["k"], (torch.arange(T) + off).view(1, 1, T), 10000.0))
        outs.append(run(orc, dict(x, q=q, k=k)))
    assert np.abs(outs[0] - outs[1]).max() < 1e-10


# ------------------------------------------------------ page formulas --
def pin_kv_cache_table():
    """Reproduce all nine cells of the printed 70B KV-cache table."""
    for s, hkv, gb in golden_rows("kv_cache_table_70b.txt"):
        got = oracle_mod.kv_cache_bytes(b=1, s=int(s), L=80, H_kv=int(hkv), d_k=128, bytes_per_elem=2)
        assert f"{got / 1e9:.2f}" == gb, (s, hkv, got)


def pin_cache_element_ratios():
    for hq, hkv, num, den in golden_rows("cache_element_ratios.txt"):
        assert oracle_mod.cache_element_ratio(int(hkv), int(hq)) == int(num) / int(den)


def pin_roofline_balance():
    for f, bw, isat in golden_rows("h100_roofline.txt"):
        assert f"{oracle_mod.roofline_balance(float(f), float(bw)):.1f}" == isat


ORACLE_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and v.__code__.co_argcount == 1]
FORMULA_PINS = [pin_kv_cache_table, pin_cache_element_ratios, pin_roofline_balance]
