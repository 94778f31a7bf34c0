"""The C-ABI library on the host, without a GPU: it loads, exports every
function include/gqa_decode.h declares, validates arguments before touching
the device, and plans split-KV chunks as documented.  No kernel is launched."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import gqa_mqa_kv_amd as gqa
from gqa_mqa_kv_amd import _binding, build, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_decode.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x100000          # 16-byte aligned stand-in address; never dereferenced on these error paths


def declared_functions():
    """Every function include/*.h declares."""
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(gqa_\w+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(_binding.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = gqa.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", build.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (gqa_\w+)", nm))
    assert set(declared_functions()) <= exported


def test_product_never_links_or_imports_the_oracle():
    nm = subprocess.run(["nm", "-D", build.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in nm
    ldd = subprocess.run(["ldd", build.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in ldd
    pkg = os.path.join(ROOT, "gqa_mqa_kv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".h", ".hip", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "gqa_oracle" not in text and "liboracle" not in text, f


def dims(**kw):
    base = dict(B=2, H_q=8, H_kv=2, d=64, T_max=1024, dtype=torch.bfloat16)
    base.update({k: v for k, v in kw.items() if k in base})
    extra = {k: v for k, v in kw.items() if k not in base}
    return _binding.make_dims(**base, **extra)


def call(d, q=FAKE, k=FAKE, v=FAKE, sl=FAKE, out=FAKE, ws=None, ws_bytes=0, scale=0.125):
    return gqa.lib().gqa_decode(q, k, v, sl, scale, out, ctypes.byref(d), ws, ws_bytes, None)


def call_layers(L, d, offs=None, **kw):
    return gqa.lib().gqa_decode_layers(L, FAKE, FAKE, FAKE, offs, FAKE, 0.125, FAKE, ctypes.byref(d), None, 0, None)


def test_status_strings():
    for code, name in _binding.STATUS.items():
        assert gqa.status_string(code).startswith(name)
    assert gqa.status_string(99) == "unknown gqa_status"


@pytest.mark.parametrize("kw,expect", [
    (dict(H_q=8, H_kv=3), INVALID),            # H_q not a multiple of H_kv
    (dict(H_q=0), INVALID),
    (dict(H_kv=0), INVALID),
    (dict(B=-1), INVALID),
    (dict(T_max=0), INVALID),
    (dict(d=96), UNSUPPORTED),
    (dict(d=256), UNSUPPORTED),
    (dict(H_q=130, H_kv=1), UNSUPPORTED),      # G > 64
    (dict(dtype=torch.float32, path="mfma"), UNSUPPORTED),
    (dict(chunk_tokens=100), INVALID),         # not a multiple of 64
    (dict(chunk_tokens=-64), INVALID),
    (dict(seq_len_hint=2048), INVALID),        # hint above T_max
    (dict(waves=2), INVALID),                  # workgroup size not 4, 8 or 16 wavefronts
    (dict(waves=32), INVALID),
    (dict(tiles=3), INVALID),                  # tiles in flight not 1, 2 or 4
    (dict(tiles=5), INVALID),
    (dict(tiles=-1), INVALID),
    (dict(per_cu=5), INVALID),                 # workgroups per CU: 0 (default) or 1 to 4
    (dict(per_cu=-1), INVALID),
])
def test_dims_validation(kw, expect):
    d = dims(**kw)
    assert call(d) == expect
    assert gqa.lib().gqa_decode_workspace_bytes(ctypes.byref(d), 1) == 0
    assert call_layers(3, d) == expect


def test_enum_validation():
    for field in ("dtype", "out_dtype", "path", "merge"):
        d = dims()
        setattr(d, field, 7)
        assert call(d) == INVALID, field


def test_null_and_misaligned_pointers():
    d = dims()
    assert gqa.lib().gqa_decode(FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, None, 0, None) == INVALID
    for pos in range(5):
        ptrs = [FAKE] * 5
        ptrs[pos] = None
        assert call(d, *ptrs) == INVALID, pos
        ptrs[pos] = FAKE + 2          # misaligned
        assert call(d, *ptrs) == INVALID, pos
    assert call(d, scale=float("nan")) == INVALID
    assert call(d, scale=float("inf")) == INVALID
    assert gqa.lib().gqa_decode_layers(2, FAKE, FAKE, FAKE, FAKE + 4, FAKE, 0.1, FAKE, ctypes.byref(d), None, 0,
                                       None) == INVALID     # kv_offsets not 8-byte aligned
    assert call_layers(0, d) == INVALID


def test_empty_batch_is_a_noop():
    d = dims(B=0)
    assert gqa.lib().gqa_decode(None, None, None, None, 0.1, None, ctypes.byref(d), None, 0, None) == OK


def test_workspace_checked_before_launch():
    d = dims(T_max=4096, chunk_tokens=256)
    need = gqa.workspace_bytes(d)
    assert need > 0
    assert call(d) == WORKSPACE
    assert call(d, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    assert call(d, ws=FAKE + 128, ws_bytes=need) == WORKSPACE   # not 256-byte aligned


def test_workspace_size_formula():
    up = lambda x: (x + 255) // 256 * 256
    # vector path: one partial state per (unit, chunk)
    d = dims(B=3, H_q=32, H_kv=4, d=128, T_max=5000, chunk_tokens=512, path="valu")
    assert gqa.plan(d) == (512, 10)
    units, G, n = 3 * 4, 8, 10
    assert gqa.workspace_bytes(d) == (1 << 20) + up(units * n * G * 2 * 4) + units * n * G * 128 * 4
    assert gqa.workspace_bytes(d, 5) > gqa.workspace_bytes(d, 1)
    assert gqa.workspace_bytes(dims(T_max=256, chunk_tokens=256, path="valu")) == 0   # one chunk: no partial state
    # matrix-core path with a forced span: two state slots per workgroup
    d = dims(B=3, H_q=32, H_kv=4, d=128, T_max=5000, chunk_tokens=512)
    span, groups = gqa.plan(d)
    assert (span, groups) == (512, -(-units * 5000 // 512))
    assert gqa.workspace_bytes(d) == (1 << 20) + up(4 * 8 * groups) + up(2 * groups * G * 2 * 4) + 2 * groups * G * 128 * 4


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_plan(name):
    w = workloads.WORKLOADS[name]
    d = _binding.make_dims(w.B, w.H_q, w.H_kv, w.d, w.T_max, w.dtype)
    a, b = gqa.plan(d, w.layers)
    units = w.layers * w.B * w.H_kv
    if w.dtype == torch.bfloat16:
        # token split: valid tokens shared evenly at run time by about two workgroups per CU
        assert a == 0
        assert 1 <= b <= 2 * 256 and b <= -(-units * w.T_max // 16)
    else:
        chunk, n = a, b
        assert chunk % 64 == 0 and chunk >= 256
        assert n * chunk >= w.T_max > (n - 1) * chunk


def test_matrix_core_path_limits():
    assert call(dims(B=5000, path="mfma")) == UNSUPPORTED           # prefix sums of lengths live in LDS
    assert gqa.plan(dims(B=5000))[0] == 256 or True                  # auto falls back to the vector path
    assert call(dims(B=64, T_max=1 << 26)) == UNSUPPORTED            # 32-bit prefix sums of lengths


def call_append(d, ptrs=None, base=10000.0, offs=None, new_lens=FAKE):
    p = [FAKE] * 5 if ptrs is None else ptrs
    return gqa.lib().gqa_append_rope(p[0], p[1], p[2], p[3], p[4], offs, FAKE, new_lens, base, FAKE,
                                     ctypes.byref(d), None)


def test_append_rope_validation():
    """The append step checks its arguments before touching the device."""
    assert call_append(dims(d=96)) == UNSUPPORTED
    assert call_append(dims(H_q=8, H_kv=3)) == INVALID
    assert call_append(dims(T_max=0)) == INVALID
    d = dims()
    for base in (0.0, -1.0, float("nan"), float("inf")):
        assert call_append(d, base=base) == INVALID, base
    for pos in range(5):
        ptrs = [FAKE] * 5
        ptrs[pos] = None
        assert call_append(d, ptrs) == INVALID, pos
        ptrs[pos] = FAKE + 1                       # not bf16-aligned
        assert call_append(d, ptrs) == INVALID, pos
    ptrs = [FAKE + 2] * 5                          # bf16-aligned but not fp32-aligned
    assert call_append(dims(dtype=torch.float32), ptrs) == INVALID
    assert call_append(d, offs=FAKE + 4) == INVALID     # kv_offsets not 8-byte aligned
    assert call_append(d, new_lens=FAKE + 2) == INVALID
    d0 = dims(B=0)
    assert gqa.lib().gqa_append_rope(None, None, None, None, None, None, None, None, 10000.0, None,
                                     ctypes.byref(d0), None) == OK
    assert gqa.lib().gqa_append_rope(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 10000.0, FAKE, None,
                                     None) == INVALID


def call_paged(d, ptrs=None, bt=FAKE, max_pages=64, page=16, scale=0.125):
    q, k, v, sl, out = ptrs or [FAKE] * 5
    return gqa.lib().gqa_decode_paged(q, k, v, bt, max_pages, page, sl, scale, out, ctypes.byref(d), None, 0, None)


def test_decode_paged_validation():
    """The paged entry point checks its arguments before touching the device."""
    d = dims(T_max=1024)
    for page in (0, -16, 8, 24, 100):
        assert call_paged(d, page=page) == INVALID, page
    assert call_paged(d, max_pages=0) == INVALID
    assert call_paged(d, max_pages=63, page=16) == INVALID       # 63 * 16 < max_seq_len
    assert call_paged(d, max_pages=16, page=64) == WORKSPACE     # exactly max_seq_len: valid, needs a workspace
    assert call_paged(dims(dtype=torch.float32)) == UNSUPPORTED  # fp32 runs on the vector path only
    assert call_paged(dims(path="valu")) == UNSUPPORTED
    assert call_paged(dims(d=96)) == UNSUPPORTED
    assert call_paged(d, bt=None) == INVALID
    assert call_paged(d, bt=FAKE + 2) == INVALID                 # not 4-byte aligned
    for pos in range(5):
        ptrs = [FAKE] * 5
        ptrs[pos] = None
        assert call_paged(d, ptrs) == INVALID, pos
    assert call_paged(d, scale=float("nan")) == INVALID
    assert gqa.lib().gqa_decode_paged(FAKE, FAKE, FAKE, FAKE, 64, 16, FAKE, 0.125, FAKE, None, None, 0,
                                      None) == INVALID
    assert call_paged(dims(B=0), [None] * 5, bt=None) == OK


def call_fp8(d, ptrs=None, scale=0.125, ks=0.01, vs=0.02):
    q, k, v, sl, out = ptrs or [FAKE] * 5
    return gqa.lib().gqa_decode_fp8(q, k, v, sl, scale, ks, vs, out, ctypes.byref(d), None, 0, None)


def test_decode_fp8_validation():
    """The E4M3-cache entry point checks its arguments before touching the
    device: bf16 queries on the matrix-core path only, finite scales,
    16-byte aligned caches."""
    d = dims()
    assert call_fp8(d) == WORKSPACE                                    # valid: only the workspace is missing
    assert call_fp8(dims(dtype=torch.float32)) == UNSUPPORTED
    assert call_fp8(dims(path="valu")) == UNSUPPORTED
    assert call_fp8(dims(d=96)) == UNSUPPORTED
    for bad in (float("nan"), float("inf"), -float("inf")):
        assert call_fp8(d, ks=bad) == INVALID
        assert call_fp8(d, vs=bad) == INVALID
        assert call_fp8(d, scale=bad) == INVALID
    for pos in range(5):
        ptrs = [FAKE] * 5
        ptrs[pos] = None
        assert call_fp8(d, ptrs) == INVALID, pos
    for pos in (1, 2):                                                 # caches must be 16-byte aligned
        ptrs = [FAKE] * 5
        ptrs[pos] = FAKE + 8
        assert call_fp8(d, ptrs) == INVALID, pos
    assert gqa.lib().gqa_decode_fp8(FAKE, FAKE, FAKE, FAKE, 0.1, 1.0, 1.0, FAKE, None, None, 0, None) == INVALID
    assert call_fp8(dims(B=0), [None] * 5) == OK


def test_decode_layers_fp8_validation():
    """The layer-batched E4M3 entry point: the checks of gqa_decode_fp8, a
    positive layer count, and the packed layout's offsets aligned."""
    d = dims()
    call = lambda dd=d, L=3, offs=None, ptrs=None, scale=0.125, ks=0.01, vs=0.02: gqa.lib().gqa_decode_layers_fp8(
        L, *(ptrs or [FAKE] * 5)[:3], offs, FAKE if ptrs is None else ptrs[3], scale, ks, vs,
        FAKE if ptrs is None else ptrs[4], ctypes.byref(dd), None, 0, None)
    assert call() == WORKSPACE                                          # dense layers: only the workspace is missing
    assert call(offs=FAKE) == WORKSPACE                                 # packed
    assert call(offs=FAKE + 4) == INVALID                               # offsets not 8-byte aligned
    assert call(L=0) == INVALID
    assert call(dims(dtype=torch.float32)) == UNSUPPORTED
    assert call(dims(path="valu")) == UNSUPPORTED
    for bad in (float("nan"), float("inf")):
        assert call(ks=bad) == INVALID
        assert call(vs=bad) == INVALID
        assert call(scale=bad) == INVALID
    for pos in range(5):
        ptrs = [FAKE] * 5
        ptrs[pos] = None
        assert call(ptrs=ptrs) == INVALID, pos
    assert call(dims(B=0), ptrs=[None] * 5) == OK


def test_decode_append_rope_validation():
    """The fused append-and-decode entry point checks its arguments before
    touching the device: bf16 on the matrix-core path, no length hint, a
    finite positive base, q_out present and distinct from q, new lengths
    distinct from the lengths read, 16-byte aligned new rows."""
    d = dims()
    Q, KN, VN, KC, VC, SL, NL, QO, OUT = (FAKE + 0x1000 * i for i in range(9))
    call = lambda dd=d, q=Q, kn=KN, vn=VN, sl=SL, nl=NL, base=10000.0, qo=QO, offs=None: \
        gqa.lib().gqa_decode_append_rope(q, kn, vn, KC, VC, offs, sl, nl, base, 0.125, qo, OUT, ctypes.byref(dd), None,
                                         0, None)
    assert call() == WORKSPACE                                          # valid: only the workspace is missing
    assert call(nl=None) == WORKSPACE                                   # new lengths are optional
    assert call(dims(dtype=torch.float32)) == UNSUPPORTED
    assert call(dims(path="valu")) == UNSUPPORTED
    assert call(dims(seq_len_hint=100)) == INVALID
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert call(base=bad) == INVALID
    assert call(qo=None) == INVALID
    assert call(qo=Q) == INVALID                                        # q_out may not be q
    assert call(nl=SL) == INVALID                                       # new lengths may not be the lengths
    for kw in (dict(kn=None), dict(vn=None), dict(kn=KN + 8), dict(vn=VN + 8), dict(qo=QO + 8), dict(nl=NL + 2)):
        assert call(**kw) == INVALID, kw
    assert call(dims(B=0), q=None, kn=None, vn=None, sl=None, nl=None, qo=None) == OK


def test_decode_append_rope_paged_validation():
    """The paged fused entry point applies the page rules of gqa_decode_paged
    and the rules of the fused call."""
    d = dims(T_max=1024)
    Q, KN, VN, KP, VP, SL, NL, QO, OUT = (FAKE + 0x1000 * i for i in range(9))
    call = lambda dd=d, bt=FAKE, mp=64, pg=16, qo=QO, nl=NL, base=10000.0: gqa.lib().gqa_decode_append_rope_paged(
        Q, KN, VN, KP, VP, bt, mp, pg, SL, nl, base, 0.125, qo, OUT, ctypes.byref(dd), None, 0, None)
    assert call() == WORKSPACE                                          # valid: only the workspace is missing
    assert call(nl=None) == WORKSPACE                                   # new lengths are optional
    for pg in (0, 8, 24, -16):
        assert call(pg=pg) == INVALID, pg                               # a positive multiple of 16
    assert call(mp=0) == INVALID
    assert call(mp=63) == INVALID                                       # max_pages * page_size < max_seq_len
    assert call(bt=None) == INVALID
    assert call(bt=FAKE + 2) == INVALID                                 # table 4-byte aligned
    assert call(dims(T_max=1024, dtype=torch.float32)) == UNSUPPORTED
    assert call(dims(T_max=1024, seq_len_hint=100)) == INVALID
    assert call(qo=None) == INVALID
    assert call(qo=Q) == INVALID
    assert call(nl=SL) == INVALID
    assert call(base=float("nan")) == INVALID


def test_decode_paged_fp8_validation():
    """The paged E4M3 entry point applies the rules of both parents."""
    d = dims(T_max=1024)
    call = lambda dd=d, bt=FAKE, mp=64, pg=16, ks=0.01, ptrs=None: gqa.lib().gqa_decode_paged_fp8(
        *(ptrs or [FAKE] * 3), bt, mp, pg, FAKE, 0.125, ks, 0.02, FAKE, ctypes.byref(dd), None, 0, None)
    assert call() == WORKSPACE                                          # valid: only the workspace is missing
    for pg in (0, 8, 24):
        assert call(pg=pg) == INVALID, pg
    assert call(mp=63) == INVALID
    assert call(bt=None) == INVALID and call(bt=FAKE + 2) == INVALID
    assert call(ks=float("nan")) == INVALID
    assert call(dd=dims(dtype=torch.float32)) == UNSUPPORTED
    assert call(dd=dims(path="valu")) == UNSUPPORTED
    assert call(ptrs=[FAKE, FAKE + 8, FAKE]) == INVALID                # pools must be 16-byte aligned
    assert call(dd=dims(B=0), bt=None) == OK


def test_append_rope_paged_validation():
    """The paged append checks the page size, the capacity and the table
    before touching the device."""
    d = dims(T_max=1024)
    call = lambda dd=d, bt=FAKE, mp=64, pg=16, base=10000.0: gqa.lib().gqa_append_rope_paged(
        FAKE, FAKE, FAKE, FAKE, FAKE, bt, mp, pg, FAKE, None, base, FAKE, ctypes.byref(dd) if dd else None, None)
    for pg in (0, -16, 8, 24):
        assert call(pg=pg) == INVALID, pg
    assert call(mp=0) == INVALID
    assert call(mp=63) == INVALID                    # 63 * 16 < max_seq_len
    assert call(bt=None) == INVALID
    assert call(bt=FAKE + 2) == INVALID              # table not 4-byte aligned
    assert call(base=0.0) == INVALID
    assert call(dd=dims(d=96)) == UNSUPPORTED
    assert call(dd=None) == INVALID
    assert call(dd=dims(B=0), bt=None) == OK


def test_append_rope_fp8_validation():
    """The quantising appends check their scales on top of their parents'
    rules, before touching the device; E4M3 caches need no alignment."""
    d = dims(T_max=1024)
    dense = lambda dd=d, ks=0.01, vs=0.02, cache=FAKE + 1: gqa.lib().gqa_append_rope_fp8(
        FAKE, FAKE, FAKE, cache, cache, None, FAKE, None, 10000.0, ks, vs, FAKE, ctypes.byref(dd), None)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert dense(ks=bad) == INVALID and dense(vs=bad) == INVALID
    assert dense(dd=dims(d=96)) == UNSUPPORTED
    assert dense(dd=dims(B=0)) == OK
    paged = lambda pg=16, mp=64, bt=FAKE: gqa.lib().gqa_append_rope_paged_fp8(
        FAKE, FAKE, FAKE, FAKE, FAKE, bt, mp, pg, FAKE, None, 10000.0, 0.01, 0.02, FAKE, ctypes.byref(d), None)
    assert paged(pg=24) == INVALID and paged(mp=63) == INVALID and paged(bt=None) == INVALID


def test_library_missing_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding._build, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _binding.lib()


def test_binding_validates_tensors_on_cpu():
    x = torch.zeros(1, 8, 64)
    with pytest.raises((ValueError, TypeError)):
        gqa.decode(x, torch.zeros(1, 2, 16, 64), torch.zeros(1, 2, 16, 64), torch.zeros(1, dtype=torch.int64), 0.1)


def test_page_layout_of_the_input_generator():
    """workloads.to_pages puts every valid row where the block table says and
    nothing else: token t of sequence b, KV head g, is row t % page of page
    table[b, t // page]; spare pages, page tails and unused entries are NaN."""
    w = workloads.Workload("pages", 4, 8, 2, 16, 1, 70, torch.bfloat16, 3)
    x = workloads.generate(w, "cpu")
    x["seq_lens"] = torch.tensor([0, 33, 70, 200], dtype=torch.int32)   # the last is clamped to T = 70
    kp, vp, table = workloads.to_pages(x, 32, seed=1, spare=2)
    lens = [0, 33, 70, 70]
    used = [0, 2, 3, 3]
    assert kp.shape == (sum(used) + 2, 2, 32, 16) and table.shape == (4, 3)
    seen = set()
    for b in range(4):
        for t in range(lens[b]):
            pid = int(table[b, t // 32])
            seen.add(pid)
            assert torch.equal(kp[pid, :, t % 32], x["k"][b, :, t])
            assert torch.equal(vp[pid, :, t % 32], x["v"][b, :, t])
        for j in range(used[b], 3):
            assert bool(torch.isnan(kp[int(table[b, j])]).all())
    assert len(seen) == sum(used)
    spare = [p for p in range(kp.shape[0]) if p not in seen]
    assert len(spare) == 2 and all(bool(torch.isnan(kp[p]).all()) for p in spare)
    assert bool(torch.isnan(kp[int(table[1, 1]), :, 1:]).all())   # tail of sequence 1's last page


def test_noalloc_validates_and_refuses_plans_beyond_its_buffer():
    """gqa_decode_noalloc checks its arguments like gqa_decode and refuses, on
    the host, a plan whose partial states exceed the static buffer."""
    lib = gqa.lib()
    d = dims()
    assert lib.gqa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, None) == INVALID
    assert lib.gqa_decode_noalloc(None, FAKE, FAKE, FAKE, 0.1, FAKE, ctypes.byref(d), None) == INVALID
    assert lib.gqa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, float("nan"), FAKE, ctypes.byref(d), None) == INVALID
    assert lib.gqa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, ctypes.byref(dims(d=96)), None) == UNSUPPORTED
    empty = dims(B=0)
    assert lib.gqa_decode_noalloc(None, None, None, None, 0.1, None, ctypes.byref(empty), None) == OK
    big = dims(B=64, H_q=64, H_kv=1, d=128, T_max=32768, chunk_tokens=64)
    assert gqa.workspace_bytes(big) > _binding.NOALLOC_SCRATCH_BYTES
    assert lib.gqa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, ctypes.byref(big), None) == 5   # GQA_ERR_SCRATCH
    src = open(HEADER).read()
    assert "#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in src
    assert _binding.NOALLOC_SCRATCH_BYTES == 32 << 20


def test_read_probe_validates_its_arguments():
    """gqa_hbm_read_probe refuses bad sizes, pointers and launch shapes on the
    host, and treats an empty read as a no-op."""
    lib = gqa.lib()
    assert lib.gqa_hbm_read_probe(None, 0, None, 0, 1, None, None) == OK
    assert lib.gqa_hbm_read_probe(FAKE, 1000, None, 0, 1, FAKE, None) == INVALID      # not a multiple of 16
    assert lib.gqa_hbm_read_probe(FAKE, 1024, FAKE, 8, 1, FAKE, None) == INVALID      # b not a multiple of 16
    assert lib.gqa_hbm_read_probe(FAKE + 8, 1024, None, 0, 1, FAKE, None) == INVALID  # misaligned
    assert lib.gqa_hbm_read_probe(None, 1024, None, 0, 1, FAKE, None) == INVALID
    assert lib.gqa_hbm_read_probe(FAKE, 1024, None, 16, 1, FAKE, None) == INVALID     # b missing
    assert lib.gqa_hbm_read_probe(FAKE, 1024, None, 0, 1, None, None) == INVALID      # no sink
    assert lib.gqa_hbm_read_probe(FAKE, 1024, None, 0, 1, FAKE + 2, None) == INVALID  # sink misaligned
    for wpc in (0, 9, -1):
        assert lib.gqa_hbm_read_probe(FAKE, 1024, None, 0, wpc, FAKE, None) == INVALID


def test_two_kernel_append_path_checks_everything_before_enqueueing():
    """With G > 16 and new lengths written, gqa_decode_append_rope (and its
    paged form) runs as the append kernel followed by the decode: every
    argument of the decode is checked before the append is enqueued, so a
    missing workspace, or a missing or misaligned output, is reported as
    such (no kernel launch is attempted on this GPU-less host, which would
    report GQA_ERR_LAUNCH)."""
    lib = gqa.lib()
    Q, KN, VN, KC, VC, SL, NL, QO, OUT = (FAKE + 0x1000 * i for i in range(9))
    for H_q in (32, 64):                          # two head blocks; two head groups
        d = dims(H_q=H_q, H_kv=1, T_max=4096, d=128)
        assert gqa.workspace_bytes(d) > 0
        call = lambda out=OUT, ws=None, nb=0: lib.gqa_decode_append_rope(Q, KN, VN, KC, VC, None, SL, NL, 10000.0,
                                                                        0.125, QO, out, ctypes.byref(d), ws, nb, None)
        assert call() == WORKSPACE
        assert call(ws=FAKE, nb=gqa.workspace_bytes(d) - 256) == WORKSPACE
        assert call(out=None) == INVALID
        assert call(out=OUT + 8) == INVALID
        paged = lambda ws=None, nb=0: lib.gqa_decode_append_rope_paged(Q, KN, VN, KC, VC, FAKE, 256, 16, SL, NL,
                                                                       10000.0, 0.125, QO, OUT, ctypes.byref(d), ws,
                                                                       nb, None)
        assert paged() == WORKSPACE



def test_decode_append_rope_fp8_validation():
    """The fused append into E4M3 caches checks what the bf16 fused call
    checks, plus positive finite scales; its paged form the page rules."""
    lib = gqa.lib()
    d = dims(T_max=1024)
    Q, KN, VN, KC, VC, SL, NL, QO, OUT = (FAKE + 0x1000 * i for i in range(9))
    call = lambda dd=d, ks=0.5, vs=0.25, qo=QO, base=10000.0: lib.gqa_decode_append_rope_fp8(
        Q, KN, VN, KC, VC, None, SL, NL, base, 0.125, ks, vs, qo, OUT, ctypes.byref(dd), None, 0, None)
    assert call() == WORKSPACE                                          # valid: only the workspace is missing
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert call(ks=bad) == INVALID and call(vs=bad) == INVALID
    assert call(base=0.0) == INVALID
    assert call(qo=Q) == INVALID
    assert call(dims(T_max=1024, dtype=torch.float32)) == UNSUPPORTED
    assert call(dims(T_max=1024, seq_len_hint=10)) == INVALID
    paged = lambda pg=16, mp=64, bt=FAKE, ks=0.5: lib.gqa_decode_append_rope_paged_fp8(
        Q, KN, VN, KC, VC, bt, mp, pg, SL, NL, 10000.0, 0.125, ks, 0.25, QO, OUT, ctypes.byref(d), None, 0, None)
    assert paged() == WORKSPACE
    assert paged(pg=24) == INVALID and paged(mp=63) == INVALID and paged(bt=None) == INVALID
    assert paged(ks=-1.0) == INVALID
    # G > 16 with lengths: the append kernel and the decode, every argument checked first
    d32 = dims(H_q=32, H_kv=1, T_max=4096)
    assert lib.gqa_decode_append_rope_fp8(Q, KN, VN, KC, VC, None, SL, NL, 10000.0, 0.125, 0.5, 0.25, QO, OUT,
                                          ctypes.byref(d32), None, 0, None) == WORKSPACE


def test_c_boundary_check_compiles_against_the_header(tmp_path):
    """The header is valid C (gcc -std=c11 -Wall -Wextra -Werror) and the C
    check program links against the library, the HIP runtime and the oracle
    (it runs on a GPU, in tests/test_gpu_c_abi.py)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "c_abi_build", os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    out = str(tmp_path / "c_abi_check")
    mod.build(out)
    assert os.path.getsize(out) > 0


def test_tp_shard_follows_the_partition_figure():
    """workloads.tp_shard cuts GPU r's share as the page's figure "TENSOR
    PARALLEL PARTITIONING (Llama 3 70B on TP=8)" lists it (tests/golden):
    query heads first..last and the one KV head they read."""
    import oracle_pins
    w = workloads.Workload("tp", 2, 64, 8, 16, 5, 9, torch.bfloat16, 7)
    x = workloads.generate(w, "cpu")
    rows = oracle_pins.golden_rows("tp8_head_partition_llama3_70b.txt")
    assert len(rows) == 8
    for gpu, lo, hi, kv in rows:
        s = workloads.tp_shard(x, 8, int(gpu))
        assert torch.equal(s["q"], x["q"][:, int(lo):int(hi) + 1])
        assert torch.equal(s["k"], x["k"][:, int(kv):int(kv) + 1])
        assert torch.equal(s["v"], x["v"][:, int(kv):int(kv) + 1])
        assert s["seq_lens"] is x["seq_lens"]
    with pytest.raises(ValueError):
        workloads.tp_shard(x, 3, 0)
