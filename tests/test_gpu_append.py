"""The append step (rotary position embedding of the new token, written into
the cache) on the GPU against the fp64 oracle, through the C ABI.

Bars:
  * rotated fp32 values: max |gpu - oracle| <= 1e-5 (the rotation runs in
    fp32 with cosines and sines of double-precision angles: a few fp32
    roundings of values of size ~5 at most);
  * rotated bf16 values: |gpu - oracle| <= 2^-8 |oracle| + 1e-6 (one rounding
    to bf16 of such an fp32 result, plus its own tiny error);
  * values copied into the cache, rows that must not change, and the new
    lengths: bitwise;
  * an append followed by a decode step: the attention bars (1e-5 fp32,
    2e-3 bf16 inputs).
"""
import numpy as np
import pytest
import torch

import gqa_mqa_kv_amd as gqa
import oracle
from gqa_mqa_kv_amd import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def note(*a):
    print("[gpu-case]", *a, flush=True)


def rot_err_ok(gpu, ref, dtype):
    g = gpu.double().cpu().numpy()
    assert np.isfinite(g).all()
    if dtype == torch.float32:
        return float(np.abs(g - ref).max()) <= 1e-5
    return bool((np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6).all())


def make(B, H_q, H_kv, d, T_max, dtype, seed, lens):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g).to(dtype)
    x = dict(q=r(B, H_q, d), k_new=r(B, H_kv, d), v_new=r(B, H_kv, d),
             k=r(B, H_kv, T_max, d), v=r(B, H_kv, T_max, d),
             seq_lens=torch.tensor(lens, dtype=torch.int32))
    return x


CASES = [
    # B, H_q, H_kv, d, T_max, lengths before the append (T_max = full: not appended)
    (4, 32, 8, 128, 64, [0, 17, 63, 64]),
    (3, 8, 8, 64, 40, [1, 39, 40]),            # MHA, d = 64
    (2, 32, 1, 128, 33, [32, 5]),              # MQA
    (2, 12, 4, 128, 300, [299, 150]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d_T%d" % c[:5])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("base", [10000.0, 500000.0])
def test_append_rope_matches_oracle(case, dtype, base):
    B, H_q, H_kv, d, T_max, lens = case
    x = make(B, H_q, H_kv, d, T_max, dtype, seed=sum(case[:5]) + len(lens), lens=lens)
    note("append", case, dtype, base)
    xd = {k: v.to(DEV) for k, v in x.items()}
    q_out, new_lens = gqa.append_rope(xd["q"], xd["k_new"], xd["v_new"], xd["k"], xd["v"], xd["seq_lens"], base)
    torch.cuda.synchronize()
    pos = torch.tensor(lens).clamp(min=0)
    orc = oracle.default()
    assert rot_err_ok(q_out, orc.rope(x["q"], pos.view(B, 1), base), dtype)
    k_rot = orc.rope(x["k_new"], pos.view(B, 1), base)
    k_after, v_after = xd["k"].cpu(), xd["v"].cpu()
    for b in range(B):
        m = int(pos[b])
        if m < T_max:
            assert rot_err_ok(k_after[b, :, m], k_rot[b], dtype)
            assert torch.equal(v_after[b, :, m], x["v_new"][b])
            keep = [t for t in range(T_max) if t != m]
            assert int(new_lens[b]) == m + 1
        else:
            keep = list(range(T_max))
            assert int(new_lens[b]) == lens[b]
        assert torch.equal(k_after[b, :, keep], x["k"][b, :, keep])
        assert torch.equal(v_after[b, :, keep], x["v"][b, :, keep])


def test_append_in_place_and_large_positions():
    """q_out may be q and new_seq_lens may be seq_lens; angles at positions
    near 131072 (m * theta up to 1.3e5 radians) stay accurate in fp32."""
    B, H_q, H_kv, d, T_max = 2, 16, 2, 128, 131072
    lens = [131071, 100000]
    x = make(B, H_q, H_kv, d, 4, torch.float32, seed=5, lens=[0, 0])
    k = torch.zeros(B, H_kv, T_max, d, device=DEV)
    v = torch.zeros(B, H_kv, T_max, d, device=DEV)
    q = x["q"].to(DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    note("append in place, large positions")
    q_out, nl = gqa.append_rope(q, x["k_new"].to(DEV), x["v_new"].to(DEV), k, v, sl, 10000.0, q_out=q,
                                new_seq_lens=sl)
    torch.cuda.synchronize()
    assert q_out.data_ptr() == q.data_ptr() and nl.data_ptr() == sl.data_ptr()
    orc = oracle.default()
    pos = torch.tensor(lens)
    assert rot_err_ok(q, orc.rope(x["q"], pos.view(B, 1), 10000.0), torch.float32)
    kr = orc.rope(x["k_new"], pos.view(B, 1), 10000.0)
    for b in range(B):
        assert rot_err_ok(k[b, :, lens[b]], kr[b], torch.float32)
    assert sl.cpu().tolist() == [l + 1 for l in lens]


def test_append_packed_layout():
    """The packed layout (one layer): row kv_offsets[b]*H_kv + g*cap_b + m."""
    B, H_q, H_kv, d = 3, 16, 4, 64
    caps = [10, 3, 7]
    lens = [4, 3, 0]                       # sequence 1 is full
    offs = torch.tensor([0, 10, 13, 20], dtype=torch.int64)
    g = torch.Generator().manual_seed(9)
    q = torch.randn(B, H_q, d, generator=g).to(torch.bfloat16)
    kn = torch.randn(B, H_kv, d, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, H_kv, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(int(offs[-1]) * H_kv, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(int(offs[-1]) * H_kv, d, generator=g).to(torch.bfloat16)
    kd, vd = kc.to(DEV), vc.to(DEV)
    note("append packed")
    q_out, nl = gqa.append_rope(q.to(DEV), kn.to(DEV), vn.to(DEV), kd, vd,
                                torch.tensor(lens, dtype=torch.int32, device=DEV), 10000.0,
                                kv_offsets=offs.to(DEV), max_seq_len=max(caps))
    torch.cuda.synchronize()
    orc = oracle.default()
    kr = orc.rope(kn, torch.tensor(lens).view(B, 1), 10000.0)
    k_after, v_after = kd.cpu(), vd.cpu()
    changed = set()
    for b in range(B):
        if lens[b] < caps[b]:
            for h in range(H_kv):
                row = int(offs[b]) * H_kv + h * caps[b] + lens[b]
                changed.add(row)
                assert rot_err_ok(k_after[row], kr[b, h], torch.bfloat16)
                assert torch.equal(v_after[row], vn[b, h])
    keep = [r for r in range(kc.shape[0]) if r not in changed]
    assert torch.equal(k_after[keep], kc[keep]) and torch.equal(v_after[keep], vc[keep])
    assert nl.cpu().tolist() == [5, 3, 1]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_append_then_decode(dtype):
    """A whole decode step: append the new token with its rotation, then
    attend with the rotated query over the cache including it.  Reference:
    the oracle's rotation of q and of every cached key at its own position,
    then the oracle's attention, all in fp64."""
    B, H_q, H_kv, d, T_max = 3, 32, 8, 128, 700
    g = torch.Generator().manual_seed(77)
    lens = torch.randint(0, T_max, (B,), generator=g, dtype=torch.int32)
    raw_k = torch.randn(B, H_kv, T_max, d, generator=g).to(dtype)     # unrotated keys of every position
    v = torch.randn(B, H_kv, T_max, d, generator=g).to(dtype)
    q = torch.randn(B, H_q, d, generator=g).to(dtype)
    base = 10000.0
    orc = oracle.default()
    # the cache as earlier appends left it: keys rotated at their positions
    rot_k = torch.from_numpy(orc.rope(raw_k, torch.arange(T_max).view(1, 1, T_max), base)).to(dtype)
    kd, vd = rot_k.clone().to(DEV), v.clone().to(DEV)
    m = lens.long()
    kn = raw_k[torch.arange(B), :, m]                                     # the new token's key and value
    vn = v[torch.arange(B), :, m]
    note("append then decode", dtype)
    q_rot, nl = gqa.append_rope(q.to(DEV), kn.contiguous().to(DEV), vn.contiguous().to(DEV), kd, vd,
                                lens.to(DEV), base)
    out = gqa.decode(q_rot, kd, vd, nl, d ** -0.5, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_q = torch.from_numpy(orc.rope(q.double(), m.view(B, 1), base))
    ref_k = torch.from_numpy(orc.rope(raw_k.double(), torch.arange(T_max).view(1, 1, T_max), base))
    ref = orc.decode(ref_q, ref_k, v.double(), (lens + 1).tolist(), d ** -0.5)
    tol = 1e-5 if dtype == torch.float32 else 2e-3
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    assert err <= tol, err


def paged_for_append(x, page, seed):
    """Pool and table for the dense cache of ``x`` with a page allocated for
    position seq_lens[b] too (where the append writes), when it is inside T."""
    T = x["k"].shape[2]
    alloc = dict(x, seq_lens=(x["seq_lens"] + 1).clamp(max=T))
    return workloads.to_pages(alloc, page, seed=seed)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("page", [16, 48])
def test_append_paged_matches_oracle(dtype, page):
    """The paged append writes the rotated key and the value at row m % page
    of page table[b][m // page] of every KV head, and nothing else."""
    B, H_q, H_kv, d, T = 6, 32, 8, 128, 192
    lens = [0, 15, 16, 47, 191, 192]                       # page boundaries, last row, full
    x = make(B, H_q, H_kv, d, T, dtype, seed=40 + page, lens=lens)
    kp, vp, table = paged_for_append({k: x[k] for k in ("k", "v", "seq_lens")}, page, seed=page)
    kd, vd, td = kp.to(DEV), vp.to(DEV), table.to(DEV)
    note("append paged", dtype, page)
    q_out, nl = gqa.append_rope_paged(x["q"].to(DEV), x["k_new"].to(DEV), x["v_new"].to(DEV), kd, vd, td,
                                      x["seq_lens"].to(DEV), 10000.0, max_seq_len=T)
    torch.cuda.synchronize()
    orc = oracle.default()
    pos = torch.tensor(lens)
    assert rot_err_ok(q_out, orc.rope(x["q"], pos.view(B, 1), 10000.0), dtype)
    k_rot = orc.rope(x["k_new"], pos.view(B, 1), 10000.0)
    k_after, v_after = kd.cpu(), vd.cpu()
    written = torch.zeros(kp.shape[:3], dtype=torch.bool)
    for b in range(B):
        m = lens[b]
        if m < T:
            pid = int(table[b, m // page])
            written[pid, :, m % page] = True
            assert rot_err_ok(k_after[pid, :, m % page], k_rot[b], dtype)
            assert torch.equal(v_after[pid, :, m % page], x["v_new"][b])
            assert int(nl[b]) == m + 1
        else:
            assert int(nl[b]) == m
    keep = ~written
    assert torch.equal(k_after[keep].view(-1).view(torch.int8), kp[keep].view(-1).view(torch.int8))
    assert torch.equal(v_after[keep].view(-1).view(torch.int8), vp[keep].view(-1).view(torch.int8))


def test_append_then_decode_paged():
    """A whole decode step on a paged cache: append with rotation, then
    attend, against the oracle's rotation of every position and its
    attention."""
    B, H_q, H_kv, d, T, page = 3, 32, 8, 128, 700, 32
    g = torch.Generator().manual_seed(78)
    lens = torch.tensor([0, 350, 699], dtype=torch.int32)
    raw_k = torch.randn(B, H_kv, T, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H_kv, T, d, generator=g).to(torch.bfloat16)
    q = torch.randn(B, H_q, d, generator=g).to(torch.bfloat16)
    base = 10000.0
    orc = oracle.default()
    rot_k = torch.from_numpy(orc.rope(raw_k, torch.arange(T).view(1, 1, T), base)).to(torch.bfloat16)
    kp, vp, table = paged_for_append({"k": rot_k, "v": v, "seq_lens": lens}, page, seed=5)
    m = lens.long()
    kn, vn = raw_k[torch.arange(B), :, m], v[torch.arange(B), :, m]
    note("append then decode, paged")
    kd, vd, td = kp.to(DEV), vp.to(DEV), table.to(DEV)
    q_rot, nl = gqa.append_rope_paged(q.to(DEV), kn.contiguous().to(DEV), vn.contiguous().to(DEV), kd, vd, td,
                                      lens.to(DEV), base, max_seq_len=T)
    out = gqa.decode_paged(q_rot, kd, vd, td, nl, d ** -0.5, out_dtype=torch.float32, max_seq_len=T)
    torch.cuda.synchronize()
    ref_q = torch.from_numpy(orc.rope(q.double(), m.view(B, 1), base))
    ref_k = torch.from_numpy(orc.rope(raw_k.double(), torch.arange(T).view(1, 1, T), base))
    ref = orc.decode(ref_q, ref_k, v.double(), (lens + 1).tolist(), d ** -0.5)
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    assert err <= 2e-3, err


@pytest.mark.parametrize("H_q,H_kv", [(32, 8), (64, 8), (32, 1)], ids=["G4", "G8", "G32"])
@pytest.mark.parametrize("span", [0, 64])
def test_decode_append_rope_paged_matches_oracle(H_q, H_kv, span):
    """The fused paged step (gqa_decode_append_rope_paged) against the oracle
    directly: its rotation of the queries and of every cached key at its own
    position (the new token's at m = seq_lens[b]), then its attention over
    the cache including the new token.  G = 32 with lengths runs as the
    append kernel and the decode; spans of 64 tokens cut units into pieces,
    so the new token lies in a unit's last piece."""
    B, d, T, page = 3, 128, 700, 32
    g = torch.Generator().manual_seed(79 + H_q + H_kv + span)
    lens = torch.tensor([0, 350, 699], dtype=torch.int32)
    raw_k = torch.randn(B, H_kv, T, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H_kv, T, d, generator=g).to(torch.bfloat16)
    q = torch.randn(B, H_q, d, generator=g).to(torch.bfloat16)
    base, scale = 10000.0, d ** -0.5
    orc = oracle.default()
    rot_k = torch.from_numpy(orc.rope(raw_k, torch.arange(T).view(1, 1, T), base)).to(torch.bfloat16)
    kp, vp, table = paged_for_append({"k": rot_k, "v": v, "seq_lens": lens}, page, seed=6 + span)
    m = lens.long()
    kn, vn = raw_k[torch.arange(B), :, m], v[torch.arange(B), :, m]
    note("fused paged append vs oracle", H_q, H_kv, span)
    kd, vd, td = kp.to(DEV), vp.to(DEV), table.to(DEV)
    out, q_rot, nl = gqa.decode_append_rope_paged(q.to(DEV), kn.contiguous().to(DEV), vn.contiguous().to(DEV), kd,
                                                  vd, td, lens.to(DEV), base, scale, out_dtype=torch.float32,
                                                  max_seq_len=T, chunk_tokens=span)
    torch.cuda.synchronize()
    ref_q = orc.rope(q.double(), m.view(B, 1), base)
    assert rot_err_ok(q_rot, ref_q, torch.bfloat16)
    assert nl.cpu().tolist() == (lens + 1).tolist()
    ref_k = torch.from_numpy(orc.rope(raw_k.double(), torch.arange(T).view(1, 1, T), base))
    ref = orc.decode(torch.from_numpy(ref_q), ref_k, v.double(), (lens + 1).tolist(), scale)
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    assert err <= 2e-3, err


# ------------------------------------------------ quantising append (E4M3) --
def codes_within(gpu_codes, y, eps):
    """Each code decodes to a value the E4M3 encoder gives for some point of
    [y - eps, y + eps] (the encoder is monotone): the GPU's fp32 rotation and
    division may move y by eps, which only matters next to a rounding
    boundary.  Away from boundaries this is exact equality."""
    orc = oracle.default()
    got = orc.e4m3(gpu_codes)
    lo = orc.e4m3(orc.e4m3_encode(y - eps))
    hi = orc.e4m3(orc.e4m3_encode(y + eps))
    return bool(((got >= lo) & (got <= hi)).all())


def e4m3_cache(shape, seed):
    g = torch.Generator().manual_seed(seed)
    c = torch.randint(0, 0x7E, shape, generator=g, dtype=torch.uint8)
    return c | (torch.randint(0, 2, shape, generator=g, dtype=torch.uint8) << 7)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("paged", [False, True], ids=["dense", "paged"])
def test_append_fp8_matches_oracle(dtype, paged):
    """Rotated keys and values written as E4M3 codes of key / k_scale and
    value / v_scale (nearest, ties to even, saturating), every other byte
    unchanged; sequence 3's new token is large enough to saturate."""
    B, H_q, H_kv, d, T, page = 6, 32, 8, 128, 192, 32
    lens = [0, 15, 16, 47, 191, 192]
    x = make(B, H_q, H_kv, d, T, dtype, seed=61, lens=lens)
    x["k_new"][3] *= 40
    x["v_new"][3] *= 40
    ks, vs = 0.03125, 0.0125
    kc, vc = e4m3_cache((B, H_kv, T, d), 1), e4m3_cache((B, H_kv, T, d), 2)
    note("append fp8", dtype, "paged" if paged else "dense")
    args = (x["q"].to(DEV), x["k_new"].to(DEV), x["v_new"].to(DEV))
    if paged:
        pk, pv, table = paged_for_append({"k": kc, "v": vc, "seq_lens": x["seq_lens"]}, page, seed=8)
        kd, vd = pk.to(DEV), pv.to(DEV)
        q_out, nl = gqa.append_rope_paged_fp8(*args, kd, vd, table.to(DEV), x["seq_lens"].to(DEV), 10000.0, ks, vs,
                                              max_seq_len=T)
        row = lambda t, b, m: t[int(table[b, m // page]), :, m % page]
        before_k, before_v = pk, pv
    else:
        kd, vd = kc.to(DEV), vc.to(DEV)
        q_out, nl = gqa.append_rope_fp8(*args, kd, vd, x["seq_lens"].to(DEV), 10000.0, ks, vs)
        row = lambda t, b, m: t[b, :, m]
        before_k, before_v = kc, vc
    torch.cuda.synchronize()
    orc = oracle.default()
    pos = torch.tensor(lens)
    assert rot_err_ok(q_out, orc.rope(x["q"], pos.view(B, 1), 10000.0), dtype)
    k_rot = orc.rope(x["k_new"], pos.view(B, 1), 10000.0)                  # fp64 [B, H_kv, d]
    k_after, v_after = kd.cpu(), vd.cpu()
    written_k, written_v = before_k.clone(), before_v.clone()
    for b in range(B):
        m = lens[b]
        if m >= T:
            assert int(nl[b]) == m
            continue
        assert int(nl[b]) == m + 1
        xk = x["k_new"][b].double().numpy()
        pair_mag = np.abs(xk.reshape(H_kv, d // 2, 2)).sum(-1).repeat(2, -1)   # |x0| + |x1| of each element's pair
        yk = k_rot[b] / ks
        assert codes_within(row(k_after, b, m), yk, 4 * 2.0 ** -23 * pair_mag / ks + 2.0 ** -22 * np.abs(yk))
        yv = x["v_new"][b].double().numpy() / vs
        assert codes_within(row(v_after, b, m), yv, 2.0 ** -22 * np.abs(yv))
        row(written_k, b, m)[...] = row(k_after, b, m)
        row(written_v, b, m)[...] = row(v_after, b, m)
    assert torch.equal(k_after, written_k) and torch.equal(v_after, written_v)   # nothing else changed
    assert (row(k_after, 3, lens[3]).numpy() & 0x7F).max() == 0x7E                 # the large token saturates


def test_append_then_decode_fp8():
    """A whole decode step on an E4M3 cache: the quantising append, then the
    E4M3 decode, against the oracle's rotation, encoder and E4M3 attention."""
    B, H_q, H_kv, d, T = 3, 32, 8, 128, 700
    g = torch.Generator().manual_seed(79)
    lens = torch.tensor([0, 350, 699], dtype=torch.int32)
    raw_k = torch.randn(B, H_kv, T, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H_kv, T, d, generator=g).to(torch.bfloat16)
    q = torch.randn(B, H_q, d, generator=g).to(torch.bfloat16)
    base, ks, vs = 10000.0, 4.0 / 448, 4.0 / 448
    orc = oracle.default()
    rot_k = orc.rope(raw_k, torch.arange(T).view(1, 1, T), base)
    k8 = torch.from_numpy(orc.e4m3_encode(rot_k / float(np.float32(ks))))          # the cache earlier appends left
    v8 = torch.from_numpy(orc.e4m3_encode(v.double() / float(np.float32(vs))))
    m = lens.long()
    kn, vn = raw_k[torch.arange(B), :, m], v[torch.arange(B), :, m]
    note("append then decode, E4M3")
    kd, vd = k8.clone().to(DEV), v8.clone().to(DEV)
    q_rot, nl = gqa.append_rope_fp8(q.to(DEV), kn.contiguous().to(DEV), vn.contiguous().to(DEV), kd, vd, lens.to(DEV),
                                    base, ks, vs)
    out = gqa.decode_fp8(q_rot, kd, vd, nl, d ** -0.5, ks, vs, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_q = torch.from_numpy(orc.rope(q.double(), m.view(B, 1), base))
    ref_k8, ref_v8 = k8.clone(), v8.clone()                                     # the oracle's own append
    for b in range(B):
        ref_k8[b, :, int(m[b])] = torch.from_numpy(orc.e4m3_encode(orc.rope(kn[b], int(m[b]), base)
                                                                   / float(np.float32(ks))))
        ref_v8[b, :, int(m[b])] = torch.from_numpy(orc.e4m3_encode(vn[b].double() / float(np.float32(vs))))
    ref = orc.decode_fp8(ref_q, ref_k8, ref_v8, (lens + 1).tolist(), d ** -0.5, ks, vs)
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    assert err <= 2e-3, err


def test_e4m3_encoder_exact():
    """The kernel's E4M3 encoder, exactly: with scales of 1 it sees the
    values themselves, so every value code must equal the oracle encoder's.
    Keys are turned at position 0 (cos 1, sin 0): x0 - x1 * 0 is x0 exactly
    unless the partner x1 is infinite or NaN (inf * 0) or x0 is a zero (whose
    sign the subtraction may flip), so key codes are compared where neither
    happens.  Inputs:
    every midpoint between neighbouring codes and its two float32
    neighbours (ties and near-ties, both signs), values across the whole
    range, and the saturating and special values."""
    orc = oracle.default()
    vals = orc.e4m3(torch.arange(256, dtype=torch.uint8))
    pos = np.sort(vals[np.isfinite(vals) & (vals >= 0) & ~np.signbit(vals)])
    mids = torch.tensor((pos[:-1] + pos[1:]) / 2, dtype=torch.float32)
    up = torch.nextafter(mids, torch.tensor(np.inf, dtype=torch.float32))
    dn = torch.nextafter(mids, torch.tensor(-np.inf, dtype=torch.float32))
    g = torch.Generator().manual_seed(5)
    rnd = torch.randn(60000, generator=g) * torch.exp(torch.empty(60000).uniform_(-16, 8, generator=g))
    special = torch.tensor([0.0, -0.0, 448.0, -448.0, 447.9, 464.0, 465.0, 1e9, -1e9, float("inf"), float("-inf"),
                            float("nan"), 2.0 ** -6, 2.0 ** -7, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 1e-30])
    x = torch.cat([mids, up, dn, -mids, -up, -dn, torch.from_numpy(pos).float(), rnd, special])
    H_kv, d = 8, 128
    per = H_kv * d
    B = -(-x.numel() // per)
    x = torch.cat([x, torch.zeros(B * per - x.numel())]).view(B, H_kv, d)
    q = torch.zeros(B, 8, d)
    kc = torch.zeros(B, H_kv, 1, d, dtype=torch.uint8)
    vc = torch.zeros(B, H_kv, 1, d, dtype=torch.uint8)
    kd, vd = kc.to(DEV), vc.to(DEV)
    note("E4M3 encoder exact", B * per, "values")
    gqa.append_rope_fp8(q.to(DEV), x.to(DEV), x.to(DEV), kd, vd, torch.zeros(B, dtype=torch.int32, device=DEV),
                        10000.0, 1.0, 1.0)
    torch.cuda.synchronize()
    want = orc.e4m3_encode(x.double())
    got_v, got_k = vd.cpu()[:, :, 0].numpy(), kd.cpu()[:, :, 0].numpy()
    bad = np.argwhere(got_v != want)
    assert len(bad) == 0, ("value codes differ", [(float(x[tuple(i)]), int(got_v[tuple(i)]), int(want[tuple(i)]))
                                                  for i in bad[:8]])
    xv = x.numpy()
    partner = xv.reshape(B, H_kv, d // 2, 2)[..., ::-1].reshape(B, H_kv, d)
    ok = np.isfinite(partner) & (xv != 0)
    bad = np.argwhere((got_k != want) & ok)
    assert len(bad) == 0, ("key codes differ", [(float(x[tuple(i)]), int(got_k[tuple(i)]), int(want[tuple(i)]))
                                                for i in bad[:8]])


# ------------------------------------------------------ append fused into decode --
FUSED_CASES = [
    # B, H_q, H_kv, d, T_max, lengths before the append (T_max = full: not appended; negative: position 0)
    (6, 32, 8, 128, 300, [0, 15, 16, 17, 299, 300]),     # G = 4, tile edges and a full cache
    (3, 64, 8, 128, 777, [776, 1, 500]),                 # G = 8
    (2, 32, 1, 128, 1000, [999, 313]),                   # G = 32 (two head blocks)
    (2, 64, 1, 64, 257, [256, 100]),                     # G = 64 (two head groups), d = 64
    (3, 12, 4, 128, 200, [-3, 31, 150]),                 # G = 3, a negative length
]


def fused_vs_pipeline(x, base, scale, packed=None, lens_out=True, **kw):
    """The fused call and append_rope + decode on copies of the same inputs:
    outputs, turned queries, caches and lengths bitwise equal (lens_out
    False: the fused call writes no lengths, and is then one kernel at every
    G).  Returns the pipeline's (out, caches, new lengths)."""
    xd = {k: v.to(DEV) for k, v in x.items()}
    ka, va, kb, vb = xd["k"].clone(), xd["v"].clone(), xd["k"].clone(), xd["v"].clone()
    ext = dict(kv_offsets=packed[0].to(DEV), max_seq_len=packed[1]) if packed else {}
    qo, nl = gqa.append_rope(xd["q"], xd["k_new"], xd["v_new"], ka, va, xd["seq_lens"], base, **ext)
    if packed:
        ref = gqa.decode_layers(qo[None], ka, va, nl, scale, kv_offsets=ext["kv_offsets"], max_seq_len=packed[1],
                                num_kv_heads=x["k_new"].shape[1], out_dtype=torch.float32, **kw)[0]
    else:
        ref = gqa.decode(qo, ka, va, nl, scale, out_dtype=torch.float32, **kw)
    out, qf, nlf = gqa.decode_append_rope(xd["q"], xd["k_new"], xd["v_new"], kb, vb, xd["seq_lens"], base, scale,
                                          out_dtype=torch.float32, new_seq_lens=None if lens_out else False,
                                          **ext, **kw)
    torch.cuda.synchronize()
    assert torch.equal(qf, qo), "turned queries differ"
    assert (nlf is None) if not lens_out else torch.equal(nlf, nl), "new lengths differ"
    assert torch.equal(kb, ka) and torch.equal(vb, va), "caches differ"
    assert torch.equal(out, ref), "outputs differ: max %.3e" % float((out - ref).abs().max())
    return ref, ka, va, nl


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d_T%d" % c[:5])
@pytest.mark.parametrize("span,merge,tiles", [(0, "auto", 0), (64, "fused", 0), (64, "kernel", 0), (128, "auto", 2)])
def test_decode_append_rope_equals_the_two_calls(case, span, merge, tiles):
    """gqa_decode_append_rope against gqa_append_rope followed by gqa_decode
    (plain cache): every output bitwise, with the planner's split and with
    forced spans that cut units into pieces (the new token then lies in a
    unit's last piece, its queries' first piece another workgroup), both
    merges and two tiles per batch; and the attention against the oracle on
    the updated cache."""
    B, H_q, H_kv, d, T, lens = case
    x = make(B, H_q, H_kv, d, T, torch.bfloat16, 91 + B + d, lens)
    note("fused append", case, span, merge, tiles)
    scale = d ** -0.5
    ref, ka, va, nl = fused_vs_pipeline(x, 10000.0, scale, chunk_tokens=span, merge=merge, tiles=tiles)
    qo, _ = gqa.append_rope(x["q"].to(DEV), x["k_new"].to(DEV), x["v_new"].to(DEV), x["k"].to(DEV).clone(),
                            x["v"].to(DEV).clone(), x["seq_lens"].to(DEV), 10000.0)
    want = oracle.decode(qo.cpu(), ka.cpu(), va.cpu(), nl.cpu(), scale)
    assert float(np.abs(ref.double().cpu().numpy() - want).max()) <= 2e-3


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d_T%d" % c[:5])
@pytest.mark.parametrize("span,merge", [(0, "auto"), (64, "fused"), (64, "kernel")])
def test_decode_append_rope_one_kernel_without_lengths(case, span, merge):
    """With no lengths to write the call is the fused kernel at every G (with
    lengths, G > 16 runs as the append kernel and the decode): bitwise equal
    to the two calls."""
    B, H_q, H_kv, d, T, lens = case
    x = make(B, H_q, H_kv, d, T, torch.bfloat16, 93 + B + d, lens)
    note("fused append without lengths", case, span, merge)
    fused_vs_pipeline(x, 10000.0, d ** -0.5, lens_out=False, chunk_tokens=span, merge=merge)


def test_decode_append_rope_packed_cache():
    """The fused call on the packed layout (capacities of their own, one of
    them full, one empty), against the two calls."""
    g = torch.Generator().manual_seed(5)
    caps = [40, 0, 17, 300]
    lens = [12, 0, 17, 299]
    H_q, H_kv, d = 32, 8, 128
    offs = torch.tensor([0] + list(np.cumsum(caps)), dtype=torch.int64)
    rows = int(offs[-1]) * H_kv
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    x = dict(q=r(4, H_q, d), k_new=r(4, H_kv, d), v_new=r(4, H_kv, d), k=r(rows, d), v=r(rows, d),
             seq_lens=torch.tensor(lens, dtype=torch.int32))
    for span in (0, 64):
        fused_vs_pipeline(x, 500000.0, d ** -0.5, packed=(offs, max(caps)), chunk_tokens=span)


def test_decode_append_rope_full_8b_layer():
    """The Llama-3-8B-shaped layer (16 x 4096 cached tokens, one appended
    each: 4097 attended), fused against the two calls, bitwise."""
    w = workloads.WORKLOADS["llama3-8b-layer"]
    g = torch.Generator().manual_seed(8)
    T = w.T_max + 64
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    x = dict(q=r(w.B, w.H_q, w.d), k_new=r(w.B, w.H_kv, w.d), v_new=r(w.B, w.H_kv, w.d),
             k=r(w.B, w.H_kv, T, w.d), v=r(w.B, w.H_kv, T, w.d),
             seq_lens=torch.full((w.B,), w.T_max, dtype=torch.int32))
    fused_vs_pipeline(x, 500000.0, w.scale)


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d_T%d" % c[:5])
@pytest.mark.parametrize("page", [16, 48])
@pytest.mark.parametrize("span,merge,lens_out", [(0, "auto", True), (0, "auto", False), (64, "fused", False),
                                                 (64, "kernel", True)])
def test_decode_append_rope_paged_equals_the_two_calls(case, page, span, merge, lens_out):
    """gqa_decode_append_rope_paged against gqa_append_rope_paged followed by
    gqa_decode_paged on copies of one shuffled pool: outputs, turned queries,
    pools and lengths bitwise equal (the new token's page is allocated, also
    for a negative length, whose token goes to position 0)."""
    B, H_q, H_kv, d, T, lens = case
    x = make(B, H_q, H_kv, d, T, torch.bfloat16, 97 + B + d + page, lens)
    note("fused paged append", case, page, span, merge, lens_out)
    alloc = dict(x, seq_lens=(x["seq_lens"].clamp(min=0) + 1).clamp(max=T))
    kp, vp, table = workloads.to_pages(alloc, page, seed=11 + page)
    kp, vp, table = kp.to(DEV), vp.to(DEV), table.to(DEV)
    ka, va, kb, vb = kp.clone(), vp.clone(), kp.clone(), vp.clone()
    q, kn, vn, sl = (x[n].to(DEV) for n in ("q", "k_new", "v_new", "seq_lens"))
    scale, base = d ** -0.5, 10000.0
    kw = dict(chunk_tokens=span, merge=merge, max_seq_len=T)
    qo, nl = gqa.append_rope_paged(q, kn, vn, ka, va, table, sl, base, max_seq_len=T)
    ref = gqa.decode_paged(qo, ka, va, table, nl, scale, out_dtype=torch.float32, **kw)
    out, qf, nlf = gqa.decode_append_rope_paged(q, kn, vn, kb, vb, table, sl, base, scale, out_dtype=torch.float32,
                                                new_seq_lens=None if lens_out else False, **kw)
    torch.cuda.synchronize()
    assert torch.equal(qf, qo), "turned queries differ"
    assert (nlf is None) if not lens_out else torch.equal(nlf, nl), "new lengths differ"
    # the pools hold NaN in unused rows: compare bit patterns
    assert torch.equal(kb.view(torch.int16), ka.view(torch.int16)), "key pools differ"
    assert torch.equal(vb.view(torch.int16), va.view(torch.int16)), "value pools differ"
    assert torch.equal(out, ref), "outputs differ: max %.3e" % float((out - ref).abs().max())


def test_prepared_paged_calls_repeat_the_direct_ones():
    """prepare_decode_append_paged and prepare_append_paged (the timing
    loops' callables) enqueue the same calls as the direct ones: a repeated
    call rewrites the same rows with the same values and gives the same
    outputs, bitwise."""
    B, H_q, H_kv, d, T, page = 4, 32, 8, 128, 600, 32
    x = make(B, H_q, H_kv, d, T, torch.bfloat16, 131, [100, 599, 0, 345])
    note("prepared paged calls")
    alloc = dict(x, seq_lens=(x["seq_lens"].clamp(min=0) + 1).clamp(max=T))
    kp, vp, table = (t.to(DEV) for t in workloads.to_pages(alloc, page, seed=17))
    q, kn, vn, sl = (x[n].to(DEV) for n in ("q", "k_new", "v_new", "seq_lens"))
    scale, base = d ** -0.5, 10000.0
    ka, va, kb, vb = kp.clone(), vp.clone(), kp.clone(), vp.clone()
    out, qo, nl = gqa.decode_append_rope_paged(q, kn, vn, ka, va, table, sl, base, scale, max_seq_len=T)
    pr = gqa.prepare_decode_append_paged(q, kn, vn, kb, vb, table, sl, base, scale, max_seq_len=T)
    torch.cuda.synchronize()
    assert torch.equal(kb.view(torch.int16), kp.view(torch.int16))   # preparing enqueues nothing
    pr()
    again = pr().clone()
    torch.cuda.synchronize()
    assert torch.equal(again, out)
    assert torch.equal(kb.view(torch.int16), ka.view(torch.int16))
    assert torch.equal(vb.view(torch.int16), va.view(torch.int16))
    kc, vc = kp.clone(), vp.clone()
    app = gqa.prepare_append_paged(q, kn, vn, kc, vc, table, sl, base, max_seq_len=T)
    app()
    q2 = app().clone()
    torch.cuda.synchronize()
    assert torch.equal(q2, qo)
    assert torch.equal(kc.view(torch.int16), ka.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), va.view(torch.int16))



# ------------------------------------------------ fused append into E4M3 caches --
def e4m3_case(B, H_q, H_kv, d, T, lens, seed, packed_caps=None):
    """bf16 queries and new rows, and an E4M3 cache (codes drawn from N(0, 1)
    keys and values with per-array scales) of T rows per (sequence, KV head),
    or packed with the capacities ``packed_caps``."""
    x = make(B, H_q, H_kv, d, T, torch.bfloat16, seed, lens)
    if packed_caps is not None:
        offs = torch.tensor([0] + list(np.cumsum(packed_caps)), dtype=torch.int64)
        g = torch.Generator().manual_seed(seed + 1)
        rows = int(offs[-1]) * H_kv
        x["k"] = torch.randn(rows, d, generator=g).to(torch.bfloat16)
        x["v"] = torch.randn(rows, d, generator=g).to(torch.bfloat16)
        x["kv_offsets"] = offs
    k8, ks = workloads.quantize_e4m3(x["k"])
    v8, vs = workloads.quantize_e4m3(x["v"])
    x.update(k=k8, v=v8, k_scale=ks, v_scale=vs)
    return x


def fused_vs_pipeline_fp8(x, base, scale, lens_out=True, paged=None, **kw):
    """gqa_decode_append_rope_fp8 (or its paged form) against
    gqa_append_rope_fp8 + gqa_decode_fp8 (or the paged pair) on copies of the
    same cache: outputs, turned queries, cache bytes and lengths bitwise.
    Returns the pipeline's (out, k cache, v cache, lengths)."""
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    ks, vs = x["k_scale"], x["v_scale"]
    if paged:
        page, table = paged
        kpool, vpool = xd["k"], xd["v"]
        td = table.to(DEV)
        T = kw.pop("max_seq_len")
        ka, va, kb, vb = kpool.clone(), vpool.clone(), kpool.clone(), vpool.clone()
        qo, nl = gqa.append_rope_paged_fp8(xd["q"], xd["k_new"], xd["v_new"], ka, va, td, xd["seq_lens"], base, ks, vs,
                                           max_seq_len=T)
        ref = gqa.decode_paged_fp8(qo, ka, va, td, nl, scale, ks, vs, out_dtype=torch.float32, max_seq_len=T, **kw)
        out, qf, nlf = gqa.decode_append_rope_paged_fp8(xd["q"], xd["k_new"], xd["v_new"], kb, vb, td,
                                                        xd["seq_lens"], base, scale, ks, vs, max_seq_len=T,
                                                        out_dtype=torch.float32,
                                                        new_seq_lens=None if lens_out else False, **kw)
    else:
        ext = dict(kv_offsets=xd["kv_offsets"], max_seq_len=kw.pop("max_seq_len")) if "kv_offsets" in x else {}
        ka, va, kb, vb = xd["k"].clone(), xd["v"].clone(), xd["k"].clone(), xd["v"].clone()
        qo, nl = gqa.append_rope_fp8(xd["q"], xd["k_new"], xd["v_new"], ka, va, xd["seq_lens"], base, ks, vs, **ext)
        if ext:
            H_kv = x["k_new"].shape[1]
            ref = gqa.decode_layers_fp8(qo[None], ka, va, nl, scale, ks, vs, kv_offsets=ext["kv_offsets"],
                                        max_seq_len=ext["max_seq_len"], num_kv_heads=H_kv, out_dtype=torch.float32,
                                        **kw)[0]
        else:
            ref = gqa.decode_fp8(qo, ka, va, nl, scale, ks, vs, out_dtype=torch.float32, **kw)
        out, qf, nlf = gqa.decode_append_rope_fp8(xd["q"], xd["k_new"], xd["v_new"], kb, vb, xd["seq_lens"], base,
                                                  scale, ks, vs, out_dtype=torch.float32,
                                                  new_seq_lens=None if lens_out else False, **ext, **kw)
    torch.cuda.synchronize()
    assert torch.equal(qf, qo), "turned queries differ"
    assert (nlf is None) if not lens_out else torch.equal(nlf, nl), "new lengths differ"
    assert torch.equal(kb, ka) and torch.equal(vb, va), "cache bytes differ"
    assert torch.equal(out, ref), "outputs differ: max %.3e" % float((out - ref).abs().max())
    return ref, ka, va, nl, qo


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d_T%d" % c[:5])
@pytest.mark.parametrize("span,merge,tiles,lens_out", [(0, "auto", 0, True), (0, "auto", 0, False),
                                                       (64, "fused", 1, False), (64, "kernel", 2, True),
                                                       (128, "auto", 4, False)])
def test_decode_append_rope_fp8_equals_the_two_calls(case, span, merge, tiles, lens_out):
    """gqa_decode_append_rope_fp8 against gqa_append_rope_fp8 followed by
    gqa_decode_fp8 (plain E4M3 cache): every output bitwise, with the
    planner's split and forced spans that cut units into pieces, both merges
    and one, two or four tiles per batch, with and without lengths written;
    and the attention against the oracle on the updated cache."""
    B, H_q, H_kv, d, T, lens = case
    x = e4m3_case(B, H_q, H_kv, d, T, lens, 151 + B + d)
    note("fused append e4m3", case, span, merge, tiles, lens_out)
    scale = d ** -0.5
    ref, ka, va, nl, qo = fused_vs_pipeline_fp8(x, 10000.0, scale, lens_out=lens_out, chunk_tokens=span, merge=merge,
                                                tiles=tiles)
    want = oracle.default().decode_fp8(qo.cpu(), ka.cpu(), va.cpu(), nl.cpu(), scale, x["k_scale"], x["v_scale"])
    assert float(np.abs(ref.double().cpu().numpy() - want).max()) <= 2e-3


def test_decode_append_rope_fp8_packed_cache():
    """The fused E4M3 step on the packed layout (capacities of their own, one
    full, one empty), against the two calls."""
    caps, lens = [40, 0, 17, 300], [12, 0, 17, 299]
    x = e4m3_case(4, 32, 8, 128, 1, lens, 161, packed_caps=caps)
    for span in (0, 64):
        fused_vs_pipeline_fp8(x, 500000.0, 128 ** -0.5, chunk_tokens=span, max_seq_len=max(caps))


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d_T%d" % c[:5])
@pytest.mark.parametrize("page", [16, 48])
@pytest.mark.parametrize("span,merge,lens_out", [(0, "auto", True), (64, "fused", False), (64, "kernel", True)])
def test_decode_append_rope_paged_fp8_equals_the_two_calls(case, page, span, merge, lens_out):
    """gqa_decode_append_rope_paged_fp8 against gqa_append_rope_paged_fp8
    followed by gqa_decode_paged_fp8 on copies of one shuffled E4M3 pool:
    outputs, turned queries, pool bytes (NaN codes in unused rows included)
    and lengths bitwise."""
    B, H_q, H_kv, d, T, lens = case
    x = e4m3_case(B, H_q, H_kv, d, T, lens, 171 + B + d + page)
    alloc = dict(x, seq_lens=(x["seq_lens"].clamp(min=0) + 1).clamp(max=T))
    kp, vp, table = workloads.to_pages(alloc, page, seed=13 + page)
    xp = dict(x, k=kp, v=vp)
    note("fused paged append e4m3", case, page, span, merge, lens_out)
    fused_vs_pipeline_fp8(xp, 10000.0, d ** -0.5, lens_out=lens_out, paged=(page, table), chunk_tokens=span,
                          merge=merge, max_seq_len=T)


def test_decode_append_rope_fp8_matches_oracle():
    """The fused E4M3 step against the oracle directly: its rotation of q and
    of the new key, its E4M3 encoder for the new row (the key turned in fp32
    on the GPU, so a code may sit one step off where the fp64 value lies
    within fp32 rounding of a code boundary: the new row is compared code by
    code within that slack), and its attention over the updated cache."""
    B, H_q, H_kv, d, T = 3, 32, 8, 128, 500
    lens = [0, 250, 499]
    x = e4m3_case(B, H_q, H_kv, d, T, lens, 181)
    xd = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    kc, vc = xd["k"].clone(), xd["v"].clone()
    out, q_rot, nl = gqa.decode_append_rope_fp8(xd["q"], xd["k_new"], xd["v_new"], kc, vc, xd["seq_lens"], 10000.0,
                                                d ** -0.5, x["k_scale"], x["v_scale"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    orc = oracle.default()
    m = torch.tensor(lens)
    ref_q = orc.rope(x["q"].double(), m.view(B, 1), 10000.0)
    assert rot_err_ok(q_rot, ref_q, torch.bfloat16)
    k_rot = orc.rope(x["k_new"].double(), m.view(B, 1), 10000.0)
    ks, vs = float(np.float32(x["k_scale"])), float(np.float32(x["v_scale"]))
    kn, vn = kc.cpu(), vc.cpu()
    for b in range(B):
        xk = x["k_new"][b].double().numpy()
        pair_mag = np.abs(xk.reshape(H_kv, d // 2, 2)).sum(-1).repeat(2, -1)   # |x0| + |x1| of each element's pair
        yk = k_rot[b] / ks
        assert codes_within(kn[b, :, lens[b]], yk, 4 * 2.0 ** -23 * pair_mag / ks + 2.0 ** -22 * np.abs(yk))
        yv = x["v_new"][b].double().numpy() / vs
        assert codes_within(vn[b, :, lens[b]], yv, 2.0 ** -22 * np.abs(yv))
    keep = torch.ones(kn.shape[:3], dtype=torch.bool)
    for b in range(B):
        keep[b, :, lens[b]] = False
    assert torch.equal(kn[keep], x["k"][keep]) and torch.equal(vn[keep], x["v"][keep])
    ref = orc.decode_fp8(q_rot.cpu(), kn, vn, nl.cpu(), d ** -0.5, x["k_scale"], x["v_scale"])
    assert float(np.abs(out.double().cpu().numpy() - ref).max()) <= 2e-3
