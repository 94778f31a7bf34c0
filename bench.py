"""GQA decode-step benchmark: effective HBM GB/s and microseconds per step.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--paged PAGE] [--kv fp8] [--gpus 1]

One step = one decode step of the workload (every split-KV piece and the
merge of the pieces: one kernel launch when the merge is fused into the
decode kernel, else the decode kernel and a small merge kernel) over one
batch of synthetic inputs that are already resident in HBM.  The default
workload is the 32-layer stack (B 64, H_q 32, H_kv 8, d 128, lengths
U[4096, 32768] shared by the layers, about 160 GB of packed bf16 cache): the
largest configuration, one launch of gqa_decode_layers per step.  Steps
rotate over enough independent input batches (``--replicas``) that one
round of the rotation reads at least 2 GiB of K/V, far beyond the 256 MB
last-level (Infinity) cache, so every step streams its K/V from HBM (with
one batch reused every step, a 1.1 GB step ran 0.7 % faster).  ``--paged PAGE`` lays each batch's cache out in
pages of PAGE tokens (shuffled in a pool, read through a block table) and
times gqa_decode_paged instead.  ``--kv fp8`` stores each batch's cache as
one-byte E4M3 codes with one scale per array and times gqa_decode_fp8 (the
bytes per cached element halve).

Metric: (K + V bytes of the valid tokens + q bytes + out bytes) / time, the
KV traffic formula of "Grouped-Query Attention (GQA) and Multi-Query
Attention (MQA): ...", section 1 ("KV Cache Memory Footprint"), per step.

The single JSON line also carries
  * roofline: the decode kernel's achieved algorithmic GB/s (HIP events
    around the timed region on the launch stream, divided by the launches)
    against the MI355X HBM3E peak of 8 TB/s, and the HBM traffic the
    rocprofv3 counters recorded (profiles/), if they were taken on the
    current kernel source;
  * cpu_baseline: the fp64 CPU oracle timed on this host on a sample of the
    same workload (whole steps of a single-layer workload; a few layers of a
    layer-batched one, scaled to the whole step), about ten seconds of work;
  * read_probe: a plain read of the step's K/V tensors by the library's
    read-probe kernel, the rate a step that reads those bytes can approach;
  * per_step_us: percentiles of the steps of the timed region (long steps)
    or of a pass after it (short steps); for long steps also the first ten
    steps' rate and a sustained pass of more than a second;
  * context: the H100 roofline figures printed on that page (3.35 TB/s,
    989 TFLOP/s, I_sat ~ 295 FLOP/B), hardware context only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "GQA decode effective HBM GB/s (% of MI355X peak) + µs/step"
DEFAULT_WORKLOAD = "llama3-8b-32-layer-stack"
KERNEL_SOURCES = ["common.h", "kernel_mfma.h", "kernel_valu.h", "gqa_decode.hip"]
LONG_STEP_BYTES = 8e9   # steps that move this many bytes (>1 ms) carry events of their own inside the timed region


def traffic_profile(key: str) -> str:
    """The committed counter summary of a workload ("name" or "name/pagedN")."""
    return os.path.join(ROOT, "profiles", "gqa_decode_mfma_%s_counters.txt" % re.sub(r"[-/]", "_", key))


def kernel_source_hash() -> str:
    """Hash of the decode kernels' sources with comments and layout removed,
    so that it changes with the code and not with its comments."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gqa_mqa_kv_amd", "csrc", f)) as fh:
            t = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        h.update(" ".join(t.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, seq_lens, out_elem_bytes, page: int = 0, kv_elem_bytes: int = 0) -> int:
    """K/V of the valid tokens, q and out; with pages, also the block-table
    entries of the pages in use (4 bytes each, read once).  kv_elem_bytes
    overrides the cache element size (1 for E4M3)."""
    e = 2 if str(w.dtype).endswith("bfloat16") else 4
    kv = 2 * w.layers * int(seq_lens.sum()) * w.H_kv * w.d * (kv_elem_bytes or e)
    qb = w.layers * w.B * w.H_q * w.d * e
    ob = w.layers * w.B * w.H_q * w.d * out_elem_bytes
    tb = 4 * sum(-(-int(n) // page) for n in seq_lens.tolist()) if page else 0
    return kv + qb + ob + tb


def read_traffic(workload_name: str, launches_bytes: int):
    """HBM bytes per launch from the committed counter summary, when it was
    recorded on the current kernel source for this workload; else None."""
    path = traffic_profile(workload_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    kv = dict(re.findall(r"^(\w+)\s*[:=]\s*(\S+)\s*$", text, re.M))
    if kv.get("kernel_source_hash") != kernel_source_hash() or kv.get("workload") != workload_name:
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, budget_s: float = 10.0, x=None):
    """Time the fp64 oracle on this host on a sample of the workload.

    Single-layer workloads: whole steps, repeated for about ``budget_s``.
    Layer-batched workloads: the layers are independent and the oracle runs
    layer by layer (each layer's K/V copied to the host first, outside the
    timing), on layers 0, 1, ... until ``budget_s`` is spent; the step's time
    is the mean per-layer time times the number of layers.  ``x``: the
    step's inputs (any device) for a layer-batched workload."""
    import oracle
    from gqa_mqa_kv_amd import workloads

    orc = oracle.default()
    out_bytes = 2 if str(w.dtype).endswith("bfloat16") else 4
    if w.layers == 1:
        x = workloads.generate(w, "cpu")
        args = (x["q"], x["k"], x["v"], x["seq_lens"], x["scale"])
        orc.decode(*args)   # warm
        n, t0 = 0, time.perf_counter()
        while True:
            orc.decode(*args)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 1000:
                break
        per_step = el / n
        sample = "%d whole steps of %s (fp64 C oracle, OpenMP), %.1f s" % (n, w.name, el)
        sl = x["seq_lens"]
    else:
        if x is None:
            x = workloads.generate(w, "cpu")
        sl = x["seq_lens"].cpu()
        offs = x["kv_offsets"].cpu().numpy() if w.packed else None
        spent, n = 0.0, 0
        for l in range(w.layers):
            xl = workloads.layer_view(x, l)
            q, k, v = xl["q"].cpu(), xl["k"].cpu(), xl["v"].cpu()
            t0 = time.perf_counter()
            orc.decode(q, k, v, sl, x["scale"], kv_offsets=offs, num_kv_heads=w.H_kv)
            spent += time.perf_counter() - t0
            n += 1
            del q, k, v
            if spent >= budget_s:
                break
        per_step = spent / n * w.layers
        sample = ("%d of %d layers of %s (fp64 C oracle, OpenMP, each layer's K/V copied to the host first, "
                  "untimed), %.1f s; step time = mean layer time x %d" % (n, w.layers, w.name, spent, w.layers))
    nbytes = algorithmic_bytes(w, sl, out_bytes)
    return {"value": round(nbytes / per_step / 1e9, 4), "unit": "GB/s", "cores": orc.num_threads(),
            "kind": "oracle", "us_per_step": round(per_step * 1e6, 1), "cpu_model": cpu_model(),
            "sample": sample}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def step_percentiles(torch, step, stream, n: int, start: int):
    """Per-step times (µs) of n more steps, each bracketed by its own events
    (a pass after the timed region, so the events do not touch it)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(start + i)
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    pick = lambda f: round(t[min(len(t) - 1, int(f * len(t)))], 2)
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "steps": n}


def copy_calibration(torch, dev, nbytes: int, launches: int) -> None:
    """A plain copy of known size: each launch reads and writes nbytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(launches):
        torch.neg(src, out=dst)     # elementwise: one fp32 read and one fp32 write per element
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "elementwise neg, fp32", "bytes_read_per_launch": nbytes,
                      "bytes_written_per_launch": nbytes, "launches": launches}), flush=True)


def read_probe(torch, gqa, pairs, stream, launches: int = 0, sustained_s: float = 0.0):
    """The library's read-probe kernel over ``pairs`` (the (K, V) tensors of
    each input batch, in the order the steps use them): one launch reads a
    batch's K and then its V, as a decode step does; a pass reads every
    batch once.  Tries 1, 2, 4 and 8 workgroups per CU and reports the best
    rate, each shape's rate, and (``sustained_s``) the first and last ten
    passes of a run of about that many seconds at the best shape."""
    dev = pairs[0][0].device
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = sum(t.numel() * t.element_size() for kv in pairs for t in kv)

    def one_pass(wpc):
        for k, v in pairs:
            gqa.hbm_read_probe(k, wpc, sink, stream.cuda_stream, b=v)

    rates = {}
    for wpc in (1, 2, 4, 8):
        one_pass(wpc)
        torch.cuda.synchronize()
        reps = launches or max(3, min(200, int(2e9 // max(nbytes, 1))))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            one_pass(wpc)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        rates[wpc] = (round(nbytes / (us * 1e-6) / 1e9, 1), round(us, 2))
    best = max(rates, key=lambda k: rates[k][0])
    res = {"GB/s": rates[best][0], "us_per_pass": rates[best][1], "bytes_per_pass": nbytes,
           "launches_per_pass": len(pairs), "workgroups_per_cu": best,
           "GB/s_by_workgroups_per_cu": {str(k): v[0] for k, v in rates.items()},
           "kernel": "gqa_hbm_read_probe: 16-byte non-temporal loads in double-buffered rounds of 8 per thread, one span per workgroup"}
    if sustained_s > 0:
        res["sustained"] = sustained_rates(torch, lambda i: one_pass(best), stream, nbytes,
                                           max(20, int(sustained_s * 1e6 / rates[best][1])))
    return res


def sustained_rates(torch, step, stream, nbytes: int, n: int):
    """n back-to-back steps, each bracketed by events: the rate of the first
    ten, of the last ten, and of all of them (GB/s), and how long the run
    streamed."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n)]
    rate = lambda ts: round(nbytes * len(ts) / (sum(ts) * 1e-6) / 1e9, 1)
    return {"steps": n, "seconds": round(sum(t) * 1e-6, 3), "first_10_GB/s": rate(t[:10]),
            "last_10_GB/s": rate(t[-10:]), "all_GB/s": rate(t), "first_10_us": round(sum(t[:10]) / 10, 1),
            "last_10_us": round(sum(t[-10:]) / 10, 1)}


def time_layers_one_by_one(torch, gqa, workloads, w, x, stream, out_dtype, reps: int = 3, fp8: bool = False):
    """The same step as L launches of one layer each (gqa_decode_layers, or
    gqa_decode_layers_fp8, with L = 1 on each layer's slice), as a model that
    computes layer l's queries from layer l-1 would issue it."""
    launchers = []
    for l in range(w.layers):
        xl = workloads.layer_view(x, l)
        extra = dict(kv_offsets=x["kv_offsets"], max_seq_len=w.T_max, num_kv_heads=w.H_kv) if w.packed else {}
        if fp8:
            launchers.append(gqa.prepare_layers_fp8(xl["q"][None], xl["k"][None] if not w.packed else xl["k"],
                                                    xl["v"][None] if not w.packed else xl["v"], x["seq_lens"],
                                                    x["scale"], x["k_scale"], x["v_scale"], out_dtype=out_dtype,
                                                    **extra))
            continue
        launchers.append(gqa.prepare(xl["q"][None], xl["k"], xl["v"], x["seq_lens"], x["scale"], out_dtype=out_dtype,
                                     **extra))
    for f in launchers:
        f()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for f in launchers:
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e3
        best = t if best is None else min(best, t)
    return {"us_per_step": round(best, 1), "launches": w.layers, "best_of": reps}


def time_append(torch, gqa, w, x, stream, steps: int, warmup: int):
    """The step before a decode step (gqa_append_rope: rotary embedding of the
    new token's H_q queries and H_kv keys, its key and value written into the
    cache) at the workload's shape, timed like the decode step.  Every
    sequence appends at row T_max - 1 (the call never writes anywhere else).
    Bytes: q read and written, the new K/V rows read and written to the
    cache, the lengths read and written."""
    g = torch.Generator(device=x["q"].device).manual_seed(w.seed + 17)
    kn = torch.randn(w.B, w.H_kv, w.d, device=x["q"].device, generator=g).to(w.dtype)
    vn = torch.randn(w.B, w.H_kv, w.d, device=x["q"].device, generator=g).to(w.dtype)
    lens = torch.full((w.B,), w.T_max - 1, dtype=torch.int32, device=x["q"].device)
    call = gqa.prepare_append(x["q"], kn, vn, x["k"], x["v"], lens, 500000.0)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    e = 2
    nbytes = 2 * w.B * w.H_q * w.d * e + 4 * w.B * w.H_kv * w.d * e + 8 * w.B
    return {"us_per_call": round(us, 2), "algorithmic_bytes": nbytes, "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "bound": "launch latency (the call moves %d bytes)" % nbytes, "rope_base": 500000.0}


def time_fused_append(torch, gqa, w, batches, stream, steps: int, warmup: int):
    """One decode step including its append: gqa_append_rope then gqa_decode
    (two launches) against gqa_decode_append_rope (one), over the rotated
    input batches (their paged and E4M3 forms for --paged and --kv fp8).
    Every sequence holds one token fewer than in the plain step and appends
    one, so the attention covers the same tokens.  Both sides rewrite the
    same cache rows with the same values at every step."""
    two, one = [], []
    for x in batches:
        g = torch.Generator(device=x["q"].device).manual_seed(w.seed + 19)
        kn = torch.randn(w.B, w.H_kv, w.d, device=x["q"].device, generator=g).to(w.dtype)
        vn = torch.randn(w.B, w.H_kv, w.d, device=x["q"].device, generator=g).to(w.dtype)
        lens = (x["seq_lens"] - 1).clamp(min=0).to(torch.int32)
        new_lens = torch.empty_like(lens)
        q_out = torch.empty_like(x["q"])
        if "k_scale" in x:   # E4M3 cache: the quantising append and the E4M3 decode
            sc = (x["k_scale"], x["v_scale"])
            if "pool" in x:
                kp, vp, table = x["pool"]
                app = gqa.prepare_append_paged_fp8(x["q"], kn, vn, kp, vp, table, lens, 500000.0, *sc,
                                                   max_seq_len=w.T_max, q_out=q_out, new_seq_lens=new_lens)
                dec = gqa.prepare_paged_fp8(q_out, kp, vp, table, new_lens, x["scale"], *sc, max_seq_len=w.T_max)
                one.append(gqa.prepare_decode_append_paged_fp8(x["q"], kn, vn, kp, vp, table, lens, 500000.0,
                                                               x["scale"], *sc, max_seq_len=w.T_max))
            else:
                app = gqa.prepare_append_fp8(x["q"], kn, vn, x["k"], x["v"], lens, 500000.0, *sc, q_out=q_out,
                                             new_seq_lens=new_lens)
                dec = gqa.prepare_fp8(q_out, x["k"], x["v"], new_lens, x["scale"], *sc)
                one.append(gqa.prepare_decode_append_fp8(x["q"], kn, vn, x["k"], x["v"], lens, 500000.0, x["scale"],
                                                         *sc))
            two.append((app, dec))
            continue
        if "pool" in x:   # paged: the pool and table of the plain step (every appended row has its page)
            kp, vp, table = x["pool"]
            app = gqa.prepare_append_paged(x["q"], kn, vn, kp, vp, table, lens, 500000.0, max_seq_len=w.T_max,
                                           q_out=q_out, new_seq_lens=new_lens)
            dec = gqa.prepare_paged(q_out, kp, vp, table, new_lens, x["scale"], max_seq_len=w.T_max)
            one.append(gqa.prepare_decode_append_paged(x["q"], kn, vn, kp, vp, table, lens, 500000.0, x["scale"],
                                                       max_seq_len=w.T_max))
        else:
            app = gqa.prepare_append(x["q"], kn, vn, x["k"], x["v"], lens, 500000.0, q_out=q_out,
                                     new_seq_lens=new_lens)
            dec = gqa.prepare(q_out, x["k"], x["v"], new_lens, x["scale"])
            one.append(gqa.prepare_decode_append(x["q"], kn, vn, x["k"], x["v"], lens, 500000.0, x["scale"]))
        two.append((app, dec))

    def run(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / steps, 2)

    n = len(batches)
    sep = run(lambda i: (two[i % n][0](), two[i % n][1]()))
    fused = run(lambda i: one[i % n]())
    return {"append_then_decode_us_per_step": sep, "fused_us_per_step": fused,
            "launches": {"append_then_decode": 2, "fused": 1 if w.H_q // w.H_kv <= 16 else 2}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--replicas", type=int, default=0, help="input batches rotated over (0: enough for >= 2 GiB)")
    ap.add_argument("--chunk-tokens", type=int, default=0)
    ap.add_argument("--paged", type=int, default=0, metavar="PAGE",
                    help="cache in shuffled pages of PAGE tokens (a multiple of 16), read through a block table")
    ap.add_argument("--kv", default="same", choices=["same", "fp8"],
                    help="cache elements: the workload's dtype, or one-byte E4M3 codes with per-array scales")
    ap.add_argument("--path", default="auto", choices=["auto", "mfma", "valu"])
    ap.add_argument("--out-dtype", default=None, choices=[None, "bf16", "fp32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed steps: no per-step percentiles, single-layer launches or append timing "
                         "(for kernel traces that should hold one kind of launch)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--sustained-s", type=float, default=1.5,
                    help="long steps: seconds of back-to-back steps (and of probe reads) in the sustained pass")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain N-MiB device copy (counter calibration kernel)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode step is not sharded across GPUs here "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import gqa_mqa_kv_amd as gqa
    from gqa_mqa_kv_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib:
        copy_calibration(torch, dev, args.copy_calibration_mib << 20, args.steps)
        return
    w = workloads.WORKLOADS[args.workload]
    if args.paged and (w.layers != 1 or w.packed or w.dtype != torch.bfloat16 or args.paged % 16):
        print("--paged takes a single-layer bf16 workload and a page that is a multiple of 16", file=sys.stderr)
        sys.exit(2)
    fp8 = args.kv == "fp8"
    if fp8 and w.dtype != torch.bfloat16:
        print("--kv fp8 takes a bf16 workload", file=sys.stderr)
        sys.exit(2)
    out_dtype = {None: w.dtype, "bf16": torch.bfloat16, "fp32": torch.float32}[args.out_dtype]
    seq_lens = workloads.seq_lens_for(w)
    kv_bytes = 2 * w.layers * int(seq_lens.sum()) * w.H_kv * w.d * (2 if w.dtype == torch.bfloat16 else 4)
    resident = kv_bytes if w.packed else 2 * w.layers * w.B * w.H_kv * w.T_max * w.d * (
        2 if w.dtype == torch.bfloat16 else 4)
    if fp8:
        resident //= 2
    # rotate over enough batches that one round reads at least 2 GiB of K/V
    # (counted as read: the valid tokens' bytes, not the allocation)
    step_bytes = kv_bytes // 2 if fp8 else kv_bytes
    reps = args.replicas or max(1, min(16, -(-(2 << 30) // max(step_bytes, 1))))
    free, _ = torch.cuda.mem_get_info(dev)
    reps = max(1, min(reps, int((free * 0.85) // max(resident, 1))))
    print("[bench] workload %s, %d input batch(es) of %.3f GB resident" % (w.name, reps, resident / 1e9),
          file=sys.stderr, flush=True)
    batches = [workloads.generate(w, dev, replica=r) for r in range(reps)]
    print("[bench] inputs generated", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream(dev)
    kw = dict(out_dtype=out_dtype, chunk_tokens=args.chunk_tokens, path=args.path)
    launchers = []
    for r, x in enumerate(batches):
        if fp8:
            x8 = workloads.to_e4m3(x, release=True)   # the E4M3 copy holds the cache now
            batches[r] = x8
            if w.layers > 1:
                extra = dict(kv_offsets=x["kv_offsets"], max_seq_len=w.T_max, num_kv_heads=w.H_kv) if w.packed else {}
                launchers.append(gqa.prepare_layers_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], x["scale"],
                                                        x8["k_scale"], x8["v_scale"], out_dtype=out_dtype,
                                                        chunk_tokens=args.chunk_tokens, **extra))
            elif args.paged:
                kp, vp, table = workloads.to_pages(x8, args.paged, seed=1000 + r, spare=1)
                del x8["k"], x8["v"]   # the pool holds the cache now
                x8["pool"] = (kp, vp, table)
                launchers.append(gqa.prepare_paged_fp8(x["q"], kp, vp, table, x["seq_lens"], x["scale"],
                                                       x8["k_scale"], x8["v_scale"], max_seq_len=w.T_max,
                                                       out_dtype=out_dtype, chunk_tokens=args.chunk_tokens))
            else:
                launchers.append(gqa.prepare_fp8(x["q"], x8["k"], x8["v"], x["seq_lens"], x["scale"], x8["k_scale"],
                                                 x8["v_scale"], out_dtype=out_dtype, chunk_tokens=args.chunk_tokens))
            continue
        if args.paged:
            kp, vp, table = workloads.to_pages(x, args.paged, seed=1000 + r, spare=1)
            del x["k"], x["v"]   # the pool holds the cache now
            x["pool"] = (kp, vp, table)
            launchers.append(gqa.prepare_paged(x["q"], kp, vp, table, x["seq_lens"], x["scale"],
                                               max_seq_len=w.T_max, out_dtype=out_dtype,
                                               chunk_tokens=args.chunk_tokens))
            continue
        extra = dict(kv_offsets=x["kv_offsets"], max_seq_len=w.T_max, num_kv_heads=w.H_kv) if w.packed else {}
        launchers.append(gqa.prepare(x["q"], x["k"], x["v"], x["seq_lens"], x["scale"], **extra, **kw))

    print("[bench] calls prepared%s" % (" (E4M3 caches)" if fp8 else ""), file=sys.stderr, flush=True)

    def step(i):
        return launchers[i % reps]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print("[bench] warm-up done", file=sys.stderr, flush=True)
    nbytes = algorithmic_bytes(w, seq_lens, 2 if out_dtype == torch.bfloat16 else 4, args.paged, 1 if fp8 else 0)
    # Long steps carry an event of their own at every step boundary inside the
    # timed region (a marker between launches that are milliseconds long);
    # short steps are timed as one block (a marker between launches tens of
    # microseconds long would cost a few microseconds each), and their
    # percentiles come from a pass after it.
    long_steps = nbytes >= LONG_STEP_BYTES
    # timed region: exactly K steps, synchronised on both sides
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1 if long_steps else 2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        if long_steps:
            evs[i + 1].record(stream)
    if not long_steps:
        evs[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = total_ms / args.steps
    step_us = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)] if long_steps else None
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9

    # The decode kernel's average launch duration: HIP events bracket the
    # timed region on the launch stream, divided by its launches (one per
    # step when the merge is fused into the decode kernel; with the merge
    # kernel a step is two launches and this figure covers both).
    achieved = gbps
    d = gqa.make_dims(w.B, w.H_q, w.H_kv, w.d, w.T_max, w.dtype, out_dtype, chunk_tokens=args.chunk_tokens,
                      path=args.path)
    a, b = gqa.plan(d, w.layers)
    mfma = args.paged or fp8 or args.path == "mfma" or (args.path == "auto" and w.dtype == torch.bfloat16 and w.B <= 4096)
    if mfma:   # token split: (forced tokens per workgroup or 0 for an even split, workgroups)
        split = {"kernel": "matrix-core, token split", "workgroups": b, "tokens_per_workgroup": a or "even"}
    else:      # vector path: (tokens per chunk, chunks of the longest sequence)
        split = {"kernel": "vector ALU, chunked", "chunk_tokens": a, "chunks_per_sequence": b}
    traffic = (read_traffic(w.name + ("/paged%d" % args.paged if args.paged else "") + ("/fp8" if fp8 else ""), nbytes)
               if args.path in ("auto", "mfma") and not args.chunk_tokens else None)

    result = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_peak_hbm": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8 e4m3 cache, bf16 q" if fp8 else "bf16" if w.dtype == torch.bfloat16 else "fp32"),
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H_q": w.H_q, "H_kv": w.H_kv, "G": w.G, "d": w.d,
                   "cached_tokens": [w.seq_lo, w.seq_hi], "seq_lens_sum": int(seq_lens.sum()), "layers": w.layers,
                   "layout": ("paged, %d tokens per page" % args.paged if args.paged
                              else "packed" if w.packed else "dense"), "accumulate": "fp32",
                   "kv_elements": "OCP E4M3 (1 byte), per-array scales" if fp8 else
                   ("bf16" if w.dtype == torch.bfloat16 else "fp32"),
                   "out_dtype": "bf16" if out_dtype == torch.bfloat16 else "fp32",
                   "path": args.path, "work_split": split,
                   "input_batches_rotated": reps, "algorithmic_bytes_per_step": nbytes,
                   "wall_s_timed_region": round(wall, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "launch_us_avg": round(ms_per_step * 1e3, 2),
                     "launch_us_avg_source": "HIP events around the timed region on the launch stream / steps "
                                             "(one launch per step with the fused merge)",
                     "algorithmic_bytes_per_launch": nbytes, "kernel_source_hash": kernel_source_hash()},
        "cpu_baseline": None,
        "context": {"h100_sxm5_hbm_TBps": 3.35, "h100_sxm5_dense_bf16_TFLOPs": 989, "h100_I_sat_FLOP_per_B": 295.2},
    }
    if long_steps:
        # every step of the timed region, and the first ten steps alone
        t = sorted(step_us)
        pick = lambda f: round(t[min(len(t) - 1, int(f * len(t)))], 2)
        result["per_step_us"] = {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "steps": len(t),
                                 "source": "the timed region's steps"}
        first = step_us[:10]
        result["first_10_steps"] = {"us_per_step": round(sum(first) / len(first), 1),
                                    "GB/s": round(nbytes * len(first) / (sum(first) * 1e-6) / 1e9, 1)}
    if not args.no_extras:
        if not long_steps:
            result["per_step_us"] = dict(step_percentiles(torch, step, stream, min(args.steps, 100), args.steps),
                                         source="a pass of events per step after the timed region")
            # the same step repeated on one input batch: whatever of it fits stays in the caches
            result["warm_one_batch_us_per_step"] = step_percentiles(
                torch, lambda i: launchers[0](), stream, min(args.steps, 50), 0)["p50"]
        else:
            # more than a second of back-to-back steps: the part's sustained rate
            result["sustained_steps"] = sustained_rates(torch, step, stream, nbytes,
                                                        max(20, int(args.sustained_s * 1e3 / ms_per_step)))
        # a plain read of the same K/V tensors (rotated like the steps)
        kv = [(x["pool"][0], x["pool"][1]) if "pool" in x else (x["k"], x["v"]) for x in batches]
        probe = read_probe(torch, gqa, kv, stream, sustained_s=args.sustained_s if long_steps else 0.0)
        probe["step_rate_as_fraction"] = round(gbps / probe["GB/s"], 4)
        result["read_probe"] = probe
    if w.layers > 1 and not args.no_extras:
        result["sequential_single_layer_launches"] = time_layers_one_by_one(torch, gqa, workloads, w, batches[0],
                                                                            stream, out_dtype, fp8=fp8)
    if w.layers == 1 and w.dtype == torch.bfloat16 and not args.no_extras:
        if not args.paged and not fp8:
            result["append_rope"] = time_append(torch, gqa, w, batches[0], stream, args.steps, args.warmup)
        result["step_with_append"] = time_fused_append(torch, gqa, w, batches, stream, min(args.steps, 100),
                                                       args.warmup)
    if not args.no_cpu_baseline and not fp8 and not args.paged:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, batches[0] if w.layers > 1 else None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
