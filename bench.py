"""Benchmark of the pack -> ragged attention -> unpack path on one MI355X.

Headline (the JSON line's `value`): kept tokens per second of the direct
fused launch (one kernel launch = one whole pass of the path: counts and
offsets, row gather, attention, unpack with zero fill) on the peak-throughput
mixed batch -- 1024 DeiT-B-shaped images, 197 tokens, 12 heads, head_dim 64,
fp16, per-image pruning rate uniform in [0, 0.9].  Inputs are resident in
HBM before the timed region.

The same line carries, for every workload: per-call latency (host clock,
launch + synchronise), kernel time (HIP events, warm and cache-scrubbed),
dispatch = latency - kernel, kept tokens/s, attention TFLOP/s, algorithmic
GB/s and the fraction of the binding roofline; the launch floor of an empty
kernel (direct and captured); and the fp64 CPU oracle timed on this host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}  # dense, published
KERNEL_SOURCES = ["ragged_variable_length_amd/csrc/attend.hip",
                  "ragged_variable_length_amd/csrc/rva_device.h",
                  "ragged_variable_length_amd/csrc/rva_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the attention kernel's code with comments and blank space
    removed, so that counters taken on a kernel stay attached to it until
    its code (not its commentary) changes."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def workload_stats(w):
    """Algorithmic sizes of one pass (bytes the method must move, FLOPs)."""
    es = 4 if w.dtype == "f32" else 2
    R = w.H * w.d * es                    # bytes per token row
    n = w.counts.astype("int64")
    T = int(n.sum())
    sum_n2 = int((n * n).sum())
    BN = w.B * w.N
    return {
        "T": T,
        "sum_n2": sum_n2,
        "flops": 4 * w.d * w.H * sum_n2,
        # fused: mask read, kept q/k/v rows read once, every padded O row written, offsets
        "bytes_fused": BN + 3 * T * R + BN * R + 4 * (w.B + 2),
        "bytes_pack": BN + 6 * T * R + 4 * T + 4 * (w.B + 2),
        "bytes_attend": 4 * T * R + 4 * (w.B + 1),
        "bytes_unpack": T * R + BN * R + BN + 4 * (w.B + 1),
        "row_bytes": R,
    }


class Ctx:
    def __init__(self, torch, rva, dev):
        self.torch, self.rva, self.dev = torch, rva, dev
        self.stream = torch.cuda.current_stream()
        self._scrub = None

    def scrub(self, i):
        """Read 1 GiB so the next call starts with cold caches (MALL is 256 MB).
        A read, not a write: written lines would still be draining to HBM
        while the timed call runs."""
        t = self.torch
        if self._scrub is None:
            self._scrub = t.ones(1 << 28, dtype=t.float32, device=self.dev)
            self._sink = t.empty(1, dtype=t.float32, device=self.dev)
        t.sum(self._scrub, dim=0, out=self._sink)

    def events_time(self, fn, reps):
        """Mean device time per call of `reps` back-to-back calls (HIP events on
        the launch stream)."""
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(reps):
            fn()
        e1.record(self.stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # us

    def graph_time(self, fn, per=50, reps=10):
        """Device time per launch of `per` launches captured in one HIP graph
        and replayed `reps` times: the launches run back to back on the
        device, whatever the host needs to issue one call."""
        t = self.torch
        fn()
        t.cuda.synchronize()
        g = t.cuda.CUDAGraph()
        with t.cuda.graph(g):
            for _ in range(per):
                fn()
        g.replay()
        t.cuda.synchronize()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(reps):
            g.replay()
        e1.record(self.stream)
        e1.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / (reps * per)

    def cold_time(self, fn, reps):
        t = self.torch
        out = []
        for i in range(reps):
            self.scrub(i)
            e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3)
        return statistics.median(out)

    def latency(self, fn, reps):
        """Median host time of call + synchronise (dispatch + kernel), us."""
        t = self.torch
        out = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            t.cuda.synchronize()
            out.append((time.perf_counter() - t0) * 1e6)
        return statistics.median(out)


def upload(ctx, w):
    import numpy as np
    t = ctx.torch

    def dev(x):
        a = t.from_numpy(np.ascontiguousarray(x))
        if w.dtype == "bf16":
            return a.view(t.int16).to(ctx.dev).view(t.bfloat16)
        return a.to(ctx.dev)
    return dev(w.q), dev(w.k), dev(w.v), t.from_numpy(w.mask).to(ctx.dev)


def make_plans(ctx, w, tensors, staged=True):
    t, rva = ctx.torch, ctx.rva
    q, k, v, mask = tensors
    B, N, H, d = q.shape
    out = t.empty_like(q)
    cu = t.empty(B + 1, dtype=t.int32, device=ctx.dev)
    mx = t.empty(1, dtype=t.int32, device=ctx.dev)
    hint = int(w.counts.max())
    plans = {"fused_graph": rva.Plan(rva.FUSED, q=q, k=k, v=v, mask=mask, out=out, cu_seqlens=cu,
                                     max_seqlen=mx, max_seqlen_hint=hint),
             "fused_plan_direct": rva.Plan(rva.FUSED_DIRECT, q=q, k=k, v=v, mask=mask, out=out,
                                           cu_seqlens=cu, max_seqlen=mx, max_seqlen_hint=hint)}
    if staged:
        packed = {nm: t.empty((B * N, H, d), dtype=q.dtype, device=ctx.dev) for nm in "qkvo"}
        plans["staged_graph"] = rva.Plan(rva.STAGED, q=q, k=k, v=v, mask=mask, out=out,
                                         packed=packed, cu_seqlens=cu, max_seqlen=mx,
                                         max_seqlen_hint=hint)
    return plans


def fused_call(ctx, tensors, hint, form="fused"):
    """The direct single-launch path (one kernel, no graph); form
    "persistent" launches the persistent grid instead (profiling only)."""
    t, rva = ctx.torch, ctx.rva
    q, k, v, mask = tensors
    out = t.empty_like(q)
    cu = t.empty(q.shape[0] + 1, dtype=t.int32, device=ctx.dev)
    mx = t.empty(1, dtype=t.int32, device=ctx.dev)
    if form == "persistent":
        work = t.zeros(2, dtype=t.int32, device=ctx.dev)
        return lambda: rva.fused_persistent(q, k, v, mask, work, out=out, cu_seqlens=cu,
                                            max_seqlen=mx, max_seqlen_hint=hint)
    return lambda: rva.fused(q, k, v, mask, out=out, cu_seqlens=cu, max_seqlen=mx,
                             max_seqlen_hint=hint)


def roofline(stats, dtype, us, bytes_key):
    gbs = stats[bytes_key] / (us * 1e-6) / 1e9
    tfl = stats["flops"] / (us * 1e-6) / 1e12
    t_hbm = stats[bytes_key] / (HBM_PEAK_GBS * 1e9) * 1e6
    t_mfma = stats["flops"] / (MFMA_PEAK_TFLOPS[dtype] * 1e12) * 1e6
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return {"bound": bound, "t_bound_us": round(max(t_hbm, t_mfma), 3), "GBps": round(gbs, 1),
            "TFLOPs": round(tfl, 2), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "frac_mfma": round(tfl / MFMA_PEAK_TFLOPS[dtype], 4),
            "frac": round(max(t_hbm, t_mfma) / us, 4)}


WARMUP_LAUNCHES = 150  # the first ~100 launches of a fresh process run slower


def timings(ctx, fn, reps, capturable=True):
    """Per-call latency (host: call + synchronise, warm), kernel time warm
    (back to back on the device: graph-captured launches when the call can
    be captured, else back-to-back calls) and cold (after a cache scrub),
    and dispatch = warm latency - warm kernel time: both sides warm."""
    for _ in range(WARMUP_LAUNCHES):
        fn()
    warm = ctx.graph_time(fn) if capturable else ctx.events_time(fn, reps)
    cold = ctx.cold_time(fn, max(5, reps // 10))
    lat = ctx.latency(fn, reps)
    return {"latency_us": round(lat, 2), "kernel_us_warm": round(warm, 2),
            "kernel_us_cold": round(cold, 2), "dispatch_us": round(max(lat - warm, 0.0), 2),
            "warm_timing": "graph" if capturable else "back_to_back_calls"}


def measure_config(ctx, w, reps, floor_us):
    import numpy as np
    stats = workload_stats(w)
    tensors = upload(ctx, w)
    hint = int(w.counts.max())
    res = {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "dtype": w.dtype, "T": stats["T"],
           "gflop": round(stats["flops"] / 1e9, 4), "fused_MB": round(stats["bytes_fused"] / 1e6, 3)}
    # direct single launch (the lowest-dispatch path) and the captured plans
    direct = timings(ctx, fused_call(ctx, tensors, hint), reps)
    direct["kept_tokens_per_s"] = round(stats["T"] / (direct["latency_us"] * 1e-6))
    direct["kept_tokens_per_s_back_to_back"] = round(stats["T"] / (direct["kernel_us_warm"] * 1e-6))
    direct["roofline_cold"] = roofline(stats, w.dtype, direct["kernel_us_cold"], "bytes_fused")
    direct["roofline_warm"] = roofline(stats, w.dtype, direct["kernel_us_warm"], "bytes_fused")
    direct["per_call_frac"] = round(max(direct["roofline_cold"]["t_bound_us"], floor_us) /
                                    direct["latency_us"], 4)
    res["fused_direct"] = direct
    for name, plan in make_plans(ctx, w, tensors).items():
        # a direct-launch plan enqueues one kernel (capturable); the graph
        # plans are timed as back-to-back graph launches
        res[name] = timings(ctx, plan.launch, reps, capturable=(name == "fused_plan_direct"))
        plan.close()
    # the direct-launch plan: arguments validated once, one short call per launch
    pd = res["fused_plan_direct"]
    pd["kept_tokens_per_s"] = round(stats["T"] / (pd["latency_us"] * 1e-6))
    pd["per_call_frac"] = round(max(direct["roofline_cold"]["t_bound_us"], floor_us) /
                                pd["latency_us"], 4)
    # the attention kernel on its own (packed operands), cold
    rva, t = ctx.rva, ctx.torch
    q, k, v, mask = tensors
    pk = rva.pack(q, k, v, mask)
    o = t.empty_like(pk["q"])
    att = lambda: rva.ragged_attend(pk["q"], pk["k"], pk["v"], pk["cu_seqlens"], hint, out=o)
    att()
    a_us = ctx.cold_time(att, max(5, reps // 10))
    res["attend_only"] = {"kernel_us_cold": round(a_us, 2), "kernel_us_warm": round(ctx.graph_time(att), 2),
                          "roofline_cold": roofline(stats, w.dtype, a_us, "bytes_attend")}
    # padded-dense comparator: the same fused kernel with every token kept,
    # so its launch takes the (image, head, query tile) grid of the full length
    full = t.ones_like(mask)
    dense_fn = fused_call(ctx, (q, k, v, full), w.N)
    for _ in range(20):
        dense_fn()
    d_cold = ctx.cold_time(dense_fn, max(5, reps // 10))
    d_warm = ctx.graph_time(dense_fn)
    dense_flops = 4 * w.d * w.H * w.B * w.N * w.N
    res["padded_dense"] = {"kernel_us_cold": round(d_cold, 2), "kernel_us_warm": round(d_warm, 2),
                           "TFLOPs_warm": round(dense_flops / (d_warm * 1e-6) / 1e12, 1),
                           "ragged_speedup_cold": round(d_cold / direct["kernel_us_cold"], 3),
                           "ragged_speedup_warm": round(d_warm / direct["kernel_us_warm"], 3)}
    del pk, o, full
    return res


def measure_threshold(ctx, reps):
    """The Threshold-l2 keep-mask: alone on DeiT-B-width embeddings for 1024
    images, and in front of the fused path on the DeiT-S recipe (direct
    calls and the captured two-kernel plan)."""
    import workloads as W
    t, rva = ctx.torch, ctx.rva
    x = W.embeddings()
    B, N, C = x.shape
    xd = t.from_numpy(x).to(ctx.dev)
    mask = t.empty((B, N), dtype=t.uint8, device=ctx.dev)
    fn = lambda: rva.threshold_l2_mask(xd, 0.5, out=mask)
    for _ in range(3):
        fn()
    cold = ctx.cold_time(fn, max(5, reps // 10))
    warm = ctx.events_time(fn, reps)
    nbytes = B * N * C * x.itemsize + B * N
    res = {"embeddings": {"B": B, "N": N, "C": C, "dtype": "f16", "keep_quantile": 0.5,
                          "kernel_us_cold": round(cold, 2), "kernel_us_warm": round(warm, 2),
                          "bytes": nbytes, "GBps_cold": round(nbytes / (cold * 1e-6) / 1e9, 1),
                          "frac_hbm_cold": round(nbytes / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}
    del xd, mask
    w = W.deit_s_224_threshold_l2()
    q, k, v, _ = upload(ctx, w)
    xs = t.from_numpy(w.meta["x"]).to(ctx.dev)
    m = t.empty((w.B, w.N), dtype=t.uint8, device=ctx.dev)
    out = t.empty_like(q)

    def direct():
        rva.threshold_l2_mask(xs, 0.5, out=m)
        rva.fused(q, k, v, m, out=out)
    plan = rva.Plan(rva.L2_FUSED, q=q, k=k, v=v, mask=m, out=out, x=xs, keep_quantile=0.5)
    res["deit_s_mask_then_fused"] = {"direct": timings(ctx, direct, reps),
                                     "plan": timings(ctx, plan.launch, reps, capturable=False)}
    plan.close()
    return res


def measure_block(ctx, reps, layers=12):
    """The attention block around the ragged path at DeiT-B width on the mixed
    batch (synthetic weights): stage by stage (offsets and kept index, QKV
    gather-product, ragged attention, output product with scatter), then a
    `layers`-deep stack as one multi-layer plan, ragged and padded-dense."""
    import numpy as np
    import workloads as W
    t, rva = ctx.torch, ctx.rva
    w = W.mixed_peak()
    B, N, H = w.B, w.N, w.H
    C = H * 64
    T = w.total_kept
    x = t.from_numpy(W.embeddings(B=B, N=N, C=C)).to(ctx.dev)
    md = t.from_numpy(w.mask).to(ctx.dev)

    def weights(seed):
        return {k: t.from_numpy(v).to(ctx.dev) for k, v in W.projection_weights(seed=seed, C=C).items()}
    wd = weights(2000)
    idx = rva.index(md)
    cu = idx["cu_seqlens"]
    qkv = tuple(t.empty((B * N, C), dtype=t.float16, device=ctx.dev) for _ in range(3))
    o = t.empty((B * N, C), dtype=t.float16, device=ctx.dev)
    y = t.empty((B, N, C), dtype=t.float16, device=ctx.dev)
    q, k, v = qkv
    stages = {
        "index": (lambda: rva.index(md, out=idx), 0),
        "qkv_projection": (lambda: rva.qkv_projection(x, cu, wd["w_qkv"], wd["b_qkv"],
                                                      kept_index=idx["kept_index"], out=qkv),
                           2 * T * C * 3 * C),
        "ragged_attention": (lambda: rva.ragged_attend(q.view(-1, H, 64), k.view(-1, H, 64),
                                                       v.view(-1, H, 64), cu, 197,
                                                       out=o.view(-1, H, 64)),
                             4 * 64 * H * int((w.counts.astype(np.int64) ** 2).sum())),
        "out_projection": (lambda: rva.out_projection(o, cu, wd["w_o"], wd["b_o"],
                                                      kept_index=idx["kept_index"], mask=md, out=y),
                           2 * T * C * C),
    }
    res = {"workload": w.name, "C": C, "T": T, "stages": {}}
    total = 0.0
    for name, (fn, flops) in stages.items():
        for _ in range(3):
            fn()
        us = ctx.events_time(fn, reps)
        total += us
        e = {"kernel_us_warm": round(us, 2)}
        if flops:
            e["TFLOPs"] = round(flops / (us * 1e-6) / 1e12, 1)
            e["mfma_frac"] = round(flops / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS["f16"], 4)
        res["stages"][name] = e
    res["block_us"] = round(total, 2)
    res["attention_share"] = round(res["stages"]["ragged_attention"]["kernel_us_warm"] / total, 4)
    del qkv, q, k, v, o, y
    # the stack, ragged and padded-dense (every token kept)
    wl = [weights(2100 + l) for l in range(layers)]
    out = {}
    for label, mask in (("ragged", md), ("padded_dense", t.ones_like(md))):
        plan = rva.LayersPlan(x, mask, wl, max_seqlen_hint=197)
        for _ in range(2):
            plan.launch()
        us = ctx.events_time(plan.launch, max(3, reps // 10))
        kept = T if label == "ragged" else B * N
        out[label] = {"us": round(us, 1), "us_per_layer": round(us / layers, 1),
                      "kept_tokens_per_s": round(kept / (us * 1e-6))}
        plan.close()
        del plan
        t.cuda.empty_cache()
    out["layers"] = layers
    out["ragged_speedup"] = round(out["padded_dense"]["us"] / out["ragged"]["us"], 3)
    res["stack"] = out
    return res


def measure_ceilings(ctx):
    """What this device reaches on plain streaming and dense matrix-core work,
    with the library's own probe kernels (csrc/probe.hip): a 1 GiB copy
    (read + write counted), a 1 GiB read, and independent fp16 16x16x32
    products on register operands; the vendor library's 8192^3 fp16 product
    beside them for context."""
    t, rva = ctx.torch, ctx.rva
    nbytes = 1 << 30
    a = t.ones(nbytes // 4, dtype=t.float32, device=ctx.dev)
    b = t.empty_like(a)
    cus = t.cuda.get_device_properties(ctx.dev).multi_processor_count
    sink = t.empty(2 * cus * 256, dtype=t.int32, device=ctx.dev)

    def timed(fn, reps):
        for _ in range(5):
            fn()
        return ctx.events_time(fn, reps)
    # launch shapes: the best of a sweep on MI355X (csrc/probe.hip)
    copy_us = timed(lambda: rva.probe_copy(a, b, 4 * cus), 30)
    read_us = timed(lambda: rva.probe_read(a, sink, 2 * cus), 30)
    out = t.empty(8 * cus * 256, dtype=t.float32, device=ctx.dev)
    mflops = rva.probe_mfma(2048, out, 8 * cus)
    mfma_us = timed(lambda: rva.probe_mfma(2048, out, 8 * cus), 10)
    del a, b, sink, out
    m = t.randn(8192, 8192, dtype=t.float16, device=ctx.dev)
    mm_us = timed(lambda: t.matmul(m, m), 5)
    del m
    return {"copy_GBps": round(2 * nbytes / (copy_us * 1e-6) / 1e9, 1),
            "read_GBps": round(nbytes / (read_us * 1e-6) / 1e9, 1),
            "mfma_fp16_TFLOPs": round(mflops / (mfma_us * 1e-6) / 1e12, 1),
            "kernels": "csrc/probe.hip (non-temporal 16-byte copy at 4 workgroups per CU and read "
                       "at 2 per CU, 4 loads in flight per thread; matrix cores: 8 independent "
                       "16x16x32 fp16 chains per wave, 8 waves per SIMD)",
            "vendor_fp16_matmul_8192_TFLOPs": round(2 * 8192 ** 3 / (mm_us * 1e-6) / 1e12, 1)}


def measure_pattern(ctx, w):
    """The headline's fused launch beside the library's gather probe
    (csrc/probe.hip) on the same batch: the same reads and writes with none
    of the arithmetic (non-temporal loads and stores, the fastest policy for
    this pattern measured), both graph-timed warm and interleaved twice
    (best of each).  probe / fused says how much of the
    kernel's time its access pattern alone takes on this device."""
    t, rva = ctx.torch, ctx.rva
    tensors = upload(ctx, w)
    q, k, v, mask = tensors
    idx = rva.index(mask)
    fused = fused_call(ctx, tensors, int(w.counts.max()))
    out = t.empty_like(q)
    probe = lambda: rva.probe_gather(q, k, v, mask, idx["cu_seqlens"], idx["kept_index"], out)
    f_us, p_us = [], []
    for _ in range(2):
        f_us.append(ctx.graph_time(fused))
        p_us.append(ctx.graph_time(probe))
    f, p = min(f_us), min(p_us)
    nbytes = workload_stats(w)["bytes_fused"]
    del tensors, out, idx
    return {"workload": w.name, "fused_us_warm": round(f, 2), "probe_us_warm": round(p, 2),
            "fused_GBps": round(nbytes / (f * 1e-6) / 1e9, 1),
            "probe_GBps": round(nbytes / (p * 1e-6) / 1e9, 1),
            "probe_over_fused": round(p / f, 4),
            "bytes": "the fused kernel's algorithmic bytes for both",
            "kernel": "probe_gather_kernel: one workgroup per (image, head pair), kept rows' q/k/v "
                      "slices read and every o row written, non-temporal loads and stores"}


def _write_workload(path, w):
    """A workload file for csrc/floor_bench.cpp: int32 B, N, H, dtype code,
    length hint; q, k, v bits; the uint8 mask."""
    import numpy as np
    code = {"f32": 0, "f16": 1, "bf16": 2}[w.dtype]
    with open(path, "wb") as f:
        np.array([w.B, w.N, w.H, code, int(w.counts.max())], dtype=np.int32).tofile(f)
        for a in (w.q, w.k, w.v):
            np.ascontiguousarray(a).tofile(f)
        np.ascontiguousarray(w.mask, dtype=np.uint8).tofile(f)


def measure_floor_cpp():
    """The C++ probe's dispatch floor (csrc/floor_bench.cpp, built next to the
    library), run as a child process; None when it has not been built.
    Beside the empty kernel it times the fused call itself from C++ on the
    small workloads (tiny, DeiT-S, DeiT-B 224 at 80% pruning), whose calls
    the dispatch floor dominates."""
    import shutil
    import subprocess
    import tempfile
    import workloads as W
    exe = os.path.join(ROOT, "ragged_variable_length_amd", "floor_bench")
    if not os.path.exists(exe):
        return None
    tmp = tempfile.mkdtemp(prefix="rva_floor_")
    try:
        files = []
        for w in (W.tiny(), W.deit_s_224_threshold_l2(), W.deit_b_224(0.8)):
            files.append(os.path.join(tmp, w.name))
            _write_workload(files[-1], w)
        r = subprocess.run([exe] + files, capture_output=True, text=True, timeout=180)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    if r.returncode != 0:
        log("floor_bench failed:", r.stderr.strip())
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def measure_floor(ctx, reps):
    rva = ctx.rva
    plan = rva.Plan(rva.EMPTY)
    for _ in range(10):
        plan.launch()
    g_lat = ctx.latency(plan.launch, reps)
    g_dev = ctx.events_time(plan.launch, reps)
    d_lat = ctx.latency(lambda: rva.empty(1), reps)
    d_dev = ctx.events_time(lambda: rva.empty(1), reps)
    d_graph = ctx.graph_time(lambda: rva.empty(1))
    plan.close()
    # the staged path's shape: four launches per call, direct and as one captured graph
    t = ctx.torch
    d4_lat = ctx.latency(lambda: rva.empty(4), reps)
    rva.empty(4)
    t.cuda.synchronize()
    g4 = t.cuda.CUDAGraph()
    with t.cuda.graph(g4):
        rva.empty(4)
    for _ in range(10):
        g4.replay()
    g4_lat = ctx.latency(g4.replay, reps)
    del g4
    return {"graph_latency_us": round(g_lat, 2), "graph_back_to_back_us": round(g_dev, 2),
            "direct_latency_us": round(d_lat, 2), "direct_back_to_back_us": round(d_dev, 2),
            "empty_kernel_device_us": round(d_graph, 2),
            "direct_4_kernels_latency_us": round(d4_lat, 2),
            "graph_4_kernels_latency_us": round(g4_lat, 2),
            "note": "the persistent form is one direct launch: its floor is direct_latency_us"}


CPU_POOL_MAX = 16  # worker processes at most (the GPU machine's CPU share for one GPU)


def _oracle_images(args):
    """Pool worker: the oracle's pack + attend + unpack on images [b0, b1) of
    workload `name`, held by the parent (inherited through fork)."""
    import oracle
    name, b0, b1 = args
    w = _CPU_W[name]
    t0 = time.perf_counter()
    oracle.pack_attend_unpack(w.q[b0:b1], w.k[b0:b1], w.v[b0:b1], w.mask[b0:b1], w.dtype)
    return time.perf_counter() - t0


_CPU_W = {}


def _image_ranges(B, parts):
    edges = [round(i * B / parts) for i in range(parts + 1)]
    return [(edges[i], edges[i + 1]) for i in range(parts) if edges[i + 1] > edges[i]]


def cpu_baseline_child(repeats=2):
    """Runs in a child process started with BLAS pinned to one thread (so no
    GPU state is ever inherited): the fp64 oracle, untuned, on the whole
    mixed batch, (i) in this one thread and (ii) over a pool of forked
    processes, one contiguous range of images each, one per available core
    (at most CPU_POOL_MAX).  Prints one JSON line."""
    import multiprocessing as mp
    import oracle
    import workloads as W
    configs = list(W.all_configs())
    for wk in configs:
        _CPU_W[wk.name] = wk
    w = next(wk for wk in configs if wk.B == 1024)  # the headline's mixed batch
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    one = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.pack_attend_unpack(w.q, w.k, w.v, w.mask, w.dtype)
        one.append(time.perf_counter() - t0)
    cores = max(1, min(CPU_POOL_MAX, len(os.sched_getaffinity(0))))
    pool_s = []
    per = []
    with mp.get_context("fork").Pool(cores) as pool:
        pool.map(_oracle_images, [(w.name, 0, 1)] * cores)  # workers up before timing
        for _ in range(repeats):
            t0 = time.perf_counter()
            pool.map(_oracle_images, [(w.name, b0, b1) for b0, b1 in _image_ranges(w.B, cores)],
                     chunksize=1)
            pool_s.append(time.perf_counter() - t0)
        # every configuration, the same two ways (best of `repeats` each)
        for wk in configs:
            t1 = []
            for _ in range(repeats):
                t0 = time.perf_counter()
                oracle.pack_attend_unpack(wk.q, wk.k, wk.v, wk.mask, wk.dtype)
                t1.append(time.perf_counter() - t0)
            rng = _image_ranges(wk.B, cores)
            tp = []
            for _ in range(repeats):
                t0 = time.perf_counter()
                pool.map(_oracle_images, [(wk.name, b0, b1) for b0, b1 in rng], chunksize=1)
                tp.append(time.perf_counter() - t0)
            st = workload_stats(wk)
            per.append({"workload": wk.name, "T": wk.total_kept,
                        "single_thread_s": round(min(t1), 5),
                        "single_thread_kept_tokens_per_s": round(wk.total_kept / min(t1), 1),
                        "single_thread_gflops_fp64": round(st["flops"] / min(t1) / 1e9, 2),
                        "pool_processes": len(rng), "pool_s": round(min(tp), 5),
                        "pool_kept_tokens_per_s": round(wk.total_kept / min(tp), 1)})
    s1, sp = min(one), min(pool_s)
    print(json.dumps({
        "value": round(w.total_kept / sp, 1), "unit": "kept tokens/s", "cores": cores,
        "kind": "oracle",
        "sample": f"whole {w.name} batch ({w.B} images, {w.total_kept} kept tokens), pack+attend+unpack "
                  f"in fp64 over {cores} processes (contiguous image ranges), best of {repeats} "
                  f"({sp:.2f} s)",
        "single_thread": {"value": round(w.total_kept / s1, 1), "cores": 1, "seconds": round(s1, 3),
                          "gflops_fp64": round(workload_stats(w)["flops"] / s1 / 1e9, 2)},
        "all_cores_gflops_fp64": round(workload_stats(w)["flops"] / sp / 1e9, 2),
        "cpu_model": model, "per_config": per}), flush=True)


def cpu_baseline():
    """The CPU oracle leg, in a child process (BLAS pinned to one thread per
    process before numpy loads); None if it fails."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child"],
                       capture_output=True, text=True, timeout=600, env=env)
    if r.returncode != 0:
        log("CPU baseline failed:", r.stderr.strip()[-2000:])
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def load_traffic(name="mixed_b1024"):
    """HBM bytes per fused launch from the committed rocprofv3 counter summary
    of workload `name`, or None if absent or taken on a different kernel
    source."""
    path = traffic_file(name)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


PROFILE_STEPS = 200  # timed launches of a profiled workload (as the default headline)
CALIB_BYTES = 1 << 28  # the calibration probes move 256 MiB each
CALIB_KIB = CALIB_BYTES / 1024
READ_KERNEL = "probe_read_kernel"
COPY_PROBE_KERNEL = "probe_copy_kernel"
# workloads a --profile run can target: the headline mixed batch and the
# DeiT-B configurations the pages' kernel-latency claim is about
PROFILE_WORKLOADS = {
    "mixed_b1024": lambda W: W.mixed_peak(),
    "tiny": lambda W: W.tiny(),
    "deit_s_224": lambda W: W.deit_s_224_threshold_l2(),
    "deit_b_224_p0": lambda W: W.deit_b_224(0.0),
    "deit_b_224_p20": lambda W: W.deit_b_224(0.2),
    "deit_b_224_p50": lambda W: W.deit_b_224(0.5),
    "deit_b_224_p80": lambda W: W.deit_b_224(0.8),
    "deit_b_384_p80": lambda W: W.deit_b_384(),
}
_ROCPROF = "cd /tmp && export TMPDIR=/tmp && "


def profile_commands(name, form="fused"):
    """The rocprofv3 commands (from the repository root R, after building)
    whose output the summaries of workload `name` (launch form `form`) come
    from."""
    tgt = f"-- python3 $R/bench.py --profile {name}" + (f" --form {form}" if form != "fused" else "")
    d = f"$R/gpurun_out/prof_{name}" + (f"_{form}" if form != "fused" else "")
    return {
        "trace": _ROCPROF + f"rocprofv3 --kernel-trace --stats --output-format csv -d {d}_trace "
                 f"-o fused {tgt}   # R = repository root",
        "fetch": _ROCPROF + f"timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv "
                 f"-d {d}_fetch -o fused {tgt}",
        "write": _ROCPROF + f"timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv "
                 f"-d {d}_write -o fused {tgt}",
        "util": _ROCPROF + "timeout -s KILL 90 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                "SQ_ACTIVE_INST_VALU SQ_BUSY_CU_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
                "SQ_INSTS_VALU_TRANS_F32 SQ_WAVE_CYCLES SQ_INSTS_LDS GRBM_GUI_ACTIVE --output-format csv "
                f"-d {d}_util -o fused {tgt}",
        "all": _ROCPROF + "rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof_all_trace "
               "-o bench -- python3 $R/bench.py --no-cpu",
        "short": _ROCPROF + "rocprofv3 --kernel-trace --stats --output-format csv -d "
                 "$R/gpurun_out/prof_short_trace -o bench -- python3 $R/bench.py --gpus 1 --steps 20 "
                 "--warmup 5 > $R/gpurun_out/prof_short_line.json",
    }


PROFILE_COMMANDS = profile_commands("mixed_b1024")
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8


def kernel_label(w):
    """Name of the fused instance a workload's launch runs: the key-split
    form when one workgroup per 16-query block of the longest sequence fits
    one fill of 3 workgroups per CU (on 256 CUs) and that sequence is staged
    whole (208 rows at N = 197)."""
    if w.dtype == "f32":
        return "attend32_kernel<true>"
    nqb = -(-int(w.counts.max()) // 16)
    ks = w.B * w.H * nqb <= 3 * 256 and w.B * w.H < 3 * 256 and int(w.counts.max()) <= 208
    return f"{profile_kernel(w)}, {'true' if ks else 'false'}>"


def profile_kernel(w):
    """Kernel-name fragment of a workload's fused launch (the 16-bit fused
    instances: whole-sequence and streamed forms, or the key-split form of
    small launches)."""
    return {"f16": "attend16_kernel<1, true", "bf16": "attend16_kernel<2, true",
            "f32": "attend32_kernel<true>"}[w.dtype]


def traffic_file(name):
    return os.path.join(ROOT, "profiles", f"fused_{name}_traffic.json")


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_profiles(trace_dir, fetch_dir, write_dir, name="mixed_b1024"):
    """Turns the rocprofv3 output of the --profile runs of workload `name`
    into the committed summaries: per-dispatch kernel time, and HBM bytes per
    launch from the FETCH_SIZE / WRITE_SIZE counters.  The counters are
    calibrated with the library's own probes, whose bytes are known:
    FETCH_SIZE by the pure read of 256 MiB, WRITE_SIZE by the copy's 256 MiB
    of writes; the copy's FETCH_SIZE, scaled the read's way, must come out at
    its 256 MiB of reads too (a cross-check of the factor)."""
    import glob
    import workloads as W
    cmds = profile_commands(name)
    w = PROFILE_WORKLOADS[name](W)
    kern = profile_kernel(w)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    trace = _read_csv(glob.glob(os.path.join(trace_dir, "*kernel_trace.csv"))[0])
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            for r in trace if kern in r["Kernel_Name"]]
    stats_rows = _read_csv(glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))[0])

    def counter(d, cname, kname):
        rows = _read_csv(glob.glob(os.path.join(d, "*counter_collection.csv"))[0])
        v = [float(r["Counter_Value"]) for r in rows
             if r["Counter_Name"] == cname and kname in r["Kernel_Name"]]
        return v

    f_read = statistics.median(counter(fetch_dir, "FETCH_SIZE", READ_KERNEL))
    f_copy = statistics.median(counter(fetch_dir, "FETCH_SIZE", COPY_PROBE_KERNEL))
    w_copy = statistics.median(counter(write_dir, "WRITE_SIZE", COPY_PROBE_KERNEL))
    fk = counter(fetch_dir, "FETCH_SIZE", kern)
    wk = counter(write_dir, "WRITE_SIZE", kern)
    f_kern, w_kern = statistics.mean(fk), statistics.mean(wk)
    f_scale, w_scale = CALIB_KIB / f_read, CALIB_KIB / w_copy
    hbm = (f_kern * f_scale + w_kern * w_scale) * 1024
    alg = workload_stats(w)["bytes_fused"]
    out = {"kernel": kern, "workload": w.name, "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_launch": round(f_kern, 2), "write_kib_per_launch": round(w_kern, 2),
           "read_probe_fetch_kib": round(f_read, 2), "copy_probe_fetch_kib": round(f_copy, 2),
           "copy_probe_write_kib": round(w_copy, 2),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "copy_fetch_check": round(f_copy * f_scale / CALIB_KIB, 4),
           "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": alg,
           "traffic_over_algorithmic": round(hbm / alg, 4)}
    with open(traffic_file(name), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    n = len(durs)
    srt = sorted(durs)
    title = f"Fused kernel, {w.name} ({w.B} images, N={w.N}, H={w.H}, {w.dtype}, T={w.total_kept})"
    lines = [f"# {title}: kernel trace", "",
             "Command (from the repository root, after building):", "",
             "```", cmds["trace"], "```", "",
             f"Dispatches of `{kern}`: {n} (warm-up and timed launches; the first launches of a "
             "fresh process run slower while the device settles)", "",
             "| statistic | us |", "|---|---|",
             f"| mean | {statistics.mean(durs):.2f} |", f"| median | {statistics.median(durs):.2f} |",
             f"| min | {srt[0]:.2f} |", f"| max | {srt[-1]:.2f} |",
             f"| mean of the last {min(n, 100)} | {statistics.mean(durs[-100:]):.2f} |",
             f"| mean of the timed launches (the last {min(n, PROFILE_STEPS)}) | "
             f"{statistics.mean(durs[-PROFILE_STEPS:]):.2f} |", "",
             "rocprofv3 kernel statistics (all kernels of the run, times in ns):", "",
             "| kernel | calls | total | average | min | max |", "|---|---|---|---|---|---|"]
    for r in stats_rows:
        lines.append(f"| {r['Name'][:70]} | {r['Calls']} | {r['TotalDurationNs']} | "
                     f"{float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    with open(os.path.join(ROOT, "profiles", f"fused_{name}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    lines = [f"# {title}: HBM byte counters", "",
             "Commands (from the repository root, after building), one counter per run:", "",
             "```", cmds["fetch"], cmds["write"], "```", "",
             "Each run first launches the library's read probe (256 MiB read) and copy probe (256 MiB "
             "read and 256 MiB written) three times each (csrc/probe.hip); their known bytes "
             "calibrate the counters' units.", "",
             "| | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) |", "|---|---|---|",
             f"| read probe, 256 MiB read | {f_read:.2f} | |",
             f"| copy probe, 256 MiB each way | {f_copy:.2f} | {w_copy:.2f} |",
             f"| scale to bytes moved (read probe / copy probe writes) | {f_scale:.4f} | {w_scale:.4f} |",
             f"| copy probe reads, scaled (check: 1.0 = 256 MiB) | {f_copy * f_scale / CALIB_KIB:.4f} | |",
             f"| fused kernel, mean per dispatch ({len(fk)} / {len(wk)} dispatches) | {f_kern:.2f} | "
             f"{w_kern:.2f} |",
             f"| fused kernel, scaled (MB) | {f_kern * f_scale * 1024 / 1e6:.2f} | "
             f"{w_kern * w_scale * 1024 / 1e6:.2f} |", "",
             f"HBM bytes per launch: {hbm / 1e6:.2f} MB; algorithmic bytes per launch: "
             f"{alg / 1e6:.2f} MB; ratio {hbm / alg:.4f}.", "",
             f"Kernel source hash (attend.hip, rva_device.h, rva_internal.h): "
             f"`{out['kernel_source_hash']}`"]
    with open(os.path.join(ROOT, "profiles", f"fused_{name}_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(out))


def summarize_all(trace_dir, cmds, top=30):
    """Every kernel of a full bench run, grouped by kernel and launch shape
    (each grid size belongs to one workload and launch form): calls and
    median / mean / min duration per dispatch."""
    import glob
    rows = _read_csv(glob.glob(os.path.join(trace_dir, "*kernel_trace.csv"))[0])
    groups = {}
    for r in rows:
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(wg, 1)
        name = r["Kernel_Name"]
        name = name[:60] + ("..." if len(name) > 60 else "")
        groups.setdefault((name, grid, wg), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    order = sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]
    lines = ["# All kernels of a full bench run: durations by kernel and launch shape", "",
             "Command (from the repository root, after building):", "",
             "```", cmds["all"], "```", "",
             "Grouped by kernel name, workgroups per launch and threads per workgroup; each launch shape "
             "belongs to one workload and launch form of the bench (for example the fused kernel with "
             "6529 workgroups is the 1024-image mixed batch: 960 images in head pairs, the last 64 one "
             "head per workgroup, and the offsets workgroup). The largest groups by total time:", "",
             "| kernel | workgroups | threads | calls | median us | mean us | min us |",
             "|---|---|---|---|---|---|---|"]
    for (name, grid, wg), d in order:
        lines.append(f"| `{name}` | {grid} | {wg} | {len(d)} | {statistics.median(d):.2f} | "
                     f"{statistics.mean(d):.2f} | {min(d):.2f} |")
    with open(os.path.join(ROOT, "profiles", "bench_all_kernels_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_short(trace_dir, line_file, warmup=5, steps=20):
    """The headline's own dispatches in a kernel trace of a short bench run
    (`--steps 20 --warmup 5`): the first warmup + steps launches of the mixed batch's fused
    kernel (6529 workgroups; the process's first GPU work), the last `steps`
    of them timed, against the launch time the line reports from HIP events
    in the same run."""
    import glob
    import workloads as W
    w = W.mixed_peak()
    kern = kernel_label(w)
    rows = _read_csv(glob.glob(os.path.join(trace_dir, "*kernel_trace.csv"))[0])
    mine = []
    for r in rows:
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(wg, 1)
        if kern in r["Kernel_Name"] and grid == 6529:
            mine.append((int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    mine.sort()
    durs = [d for _, d in mine[:warmup + steps]]
    timed = durs[warmup:]
    with open(line_file) as f:
        line = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])
    ev = line["roofline"]["avg_launch_us"]
    lines = [f"# Fused kernel, {w.name}: the headline's dispatches in a short bench run (5 warm-ups, 20 timed launches)", "",
             "Command (from the repository root, after building):", "",
             "```", PROFILE_COMMANDS["short"], "```", "",
             f"The headline's launches are the process's first GPU work: `{kern}` with 6529 workgroups, "
             f"{warmup} warm-up and {steps} timed launches (later launches of the same shape belong to the "
             "per-workload section and are not counted here).", "",
             "| launch | us |", "|---|---|"]
    lines += [f"| {'warm-up' if i < warmup else 'timed'} {i + 1} | {d:.2f} |" for i, d in enumerate(durs)]
    lines += ["", "| | us |", "|---|---|",
              f"| mean of the {len(timed)} timed dispatches (rocprofv3) | {statistics.mean(timed):.2f} |",
              f"| the line's `roofline.avg_launch_us` (HIP events, same run) | {ev:.2f} |",
              f"| ratio | {ev / statistics.mean(timed):.4f} |"]
    with open(os.path.join(ROOT, "profiles", "fused_mixed_b1024_short_run_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_util(util_dir, name="mixed_b1024", form="fused"):
    """Matrix-core and VALU utilisation of the fused kernel from the "util"
    counter run: MfmaUtil = MFMA busy cycles / (GUI-active cycles x SIMDs),
    VALUBusy = VALU-active cycles / (GUI-active cycles x CUs), with the
    GUI-active count of the busiest XCD; instruction counts per launch."""
    import glob
    import workloads as W
    cmds = profile_commands(name, form)
    w = PROFILE_WORKLOADS[name](W)
    kern = profile_kernel(w)
    if form == "persistent":
        kern = kern.replace("attend16_kernel<", "attend16_persistent_kernel<").replace(", true>", ">")
    rows = _read_csv(glob.glob(os.path.join(util_dir, "*counter_collection.csv"))[0])
    per = {}
    durs = {}
    for r in rows:
        if kern not in r["Kernel_Name"]:
            continue
        per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        durs[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    m = {k: statistics.mean(v) for k, v in per.items()}
    n = len(per["GRBM_GUI_ACTIVE"])
    gui = m["GRBM_GUI_ACTIVE"] / XCD_NUM  # summed over the XCDs' GRBM instances
    us = statistics.mean(durs.values())
    mfma_util = 100 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMD_NUM)
    valu_busy = 100 * m["SQ_ACTIVE_INST_VALU"] / CU_NUM / gui
    flops = workload_stats(w)["flops"]
    mfma_flops = m["SQ_INSTS_MFMA"] * 16 * 16 * 32 * 2
    lines = [f"# Fused kernel, {w.name} ({w.B} images, N={w.N}, H={w.H}, {w.dtype}): matrix-core and "
             "VALU utilisation", "",
             "Command (from the repository root, after building):", "",
             "```", cmds["util"], "```", "",
             f"Mean over {n} dispatches of `{kern}` (counters summed over the device; "
             f"GRBM_GUI_ACTIVE divided by the {XCD_NUM} XCDs).", "",
             "| counter | per launch |", "|---|---|"]
    for k in sorted(m):
        lines.append(f"| {k} | {m[k]:,.0f} |")
    lines += ["", "| derived | value |", "|---|---|",
              f"| kernel duration under counters (us) | {us:.1f} |",
              f"| GUI-active cycles per XCD | {gui:,.0f} ({gui / us / 1e3:.2f} GHz over the duration) |",
              f"| MfmaUtil: MFMA busy / (GUI-active x {SIMD_NUM} SIMDs) | {mfma_util:.1f}% |",
              f"| VALUBusy: VALU-active / (GUI-active x {CU_NUM} CUs) | {valu_busy:.1f}% |",
              f"| MFMA instructions (16x16x32) | {m['SQ_INSTS_MFMA']:,.0f} |",
              f"| matrix-core FLOPs executed / algorithmic (4 d H sum n^2 = {flops / 1e9:.1f} G) | "
              f"{mfma_flops / flops:.2f} (padding to 16-query blocks and 32-key tiles, row sums) |",
              f"| VALU instructions per MFMA | {m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.1f} |",
              f"| transcendental (exp2, rcp) per MFMA | {m['SQ_INSTS_VALU_TRANS_F32'] / m['SQ_INSTS_MFMA']:.2f} |",
              f"| LDS instructions per MFMA | {m['SQ_INSTS_LDS'] / m['SQ_INSTS_MFMA']:.2f} |", "",
              f"Kernel source hash (attend.hip, rva_device.h, rva_internal.h): `{kernel_source_hash()}`"]
    suffix = "_persistent" if form == "persistent" else ""
    with open(os.path.join(ROOT, "profiles", f"fused_{name}{suffix}_utilisation.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 150 untimed launches (about 30 ms): the first launches of a run on a
    # fresh process run up to 15% slower while the device settles
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--quick", action="store_true", help="headline only (no per-workload sweep)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--profile", nargs="?", const="mixed_b1024", choices=sorted(PROFILE_WORKLOADS),
                    help="profiling target: the calibration probes, then the fused launch of one "
                         "workload (default: the headline's mixed batch) only")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from rocprofv3 output of --profile runs")
    ap.add_argument("--name", default="mixed_b1024", choices=sorted(PROFILE_WORKLOADS),
                    help="workload of --summarize / --summarize-util")
    ap.add_argument("--form", default="fused", choices=["fused", "persistent"],
                    help="launch form of a --profile run, and of --summarize-util")
    ap.add_argument("--summarize-all", metavar="TRACE_DIR",
                    help="write the profiles/ summary of every kernel from a traced full bench run")
    ap.add_argument("--summarize-short", nargs=2, metavar=("TRACE_DIR", "LINE_JSON"),
                    help="summarise a kernel trace of a short run (PROFILE_COMMANDS['short'])")
    ap.add_argument("--summarize-util", metavar="UTIL_DIR",
                    help="write the profiles/ utilisation summary from the rocprofv3 counter run")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_baseline_child:
        cpu_baseline_child()
        return
    if args.summarize_all:
        summarize_all(args.summarize_all, PROFILE_COMMANDS)
        return
    if args.summarize_short:
        summarize_short(*args.summarize_short)
        return
    if args.summarize_util:
        summarize_util(args.summarize_util, args.name, args.form)
        return
    if args.summarize:
        summarize_profiles(*args.summarize, args.name)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the ragged path needs no cross-GPU exchange "
              "(images shard independently), and only the one-GPU figure is reported.",
              file=sys.stderr)
        sys.exit(2)

    # the C++ dispatch floor first, in its own process, before this one
    # touches the GPU (two live contexts on one device would skew it)
    floor_cpp = None if (args.quick or args.profile) else measure_floor_cpp()

    import torch
    import ragged_variable_length_amd as rva
    import workloads as W

    rva.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    ctx = Ctx(torch, rva, dev)

    log(f"generating the {args.profile or 'mixed_b1024'} workload ...")
    w = PROFILE_WORKLOADS[args.profile](W) if args.profile else W.mixed_peak()
    stats = workload_stats(w)
    tensors = upload(ctx, w)
    hint = int(w.counts.max())
    step = fused_call(ctx, tensors, hint, args.form if args.profile else "fused")

    if args.profile:
        # rocprofv3 target: first the library's read and copy probes over 256
        # MiB, three times each (their bytes are known, so they calibrate the
        # HBM byte counters), then exactly the timed loop below on the chosen
        # workload, and nothing else
        a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        sink = torch.empty(2 * cus * 256, dtype=torch.int32, device=dev)
        for _ in range(3):
            rva.probe_read(a, sink, 2 * cus)
        for _ in range(3):
            rva.probe_copy(a, b, 4 * cus)
        torch.cuda.synchronize()
        del a, b, sink
        args.quick = args.no_cpu = True

    # The headline runs first: its W warm-up and K timed launches are the
    # first kernel launches of this process (after the input upload).  A fresh process's first ~100 launches
    # run up to 15% slower while the device's power management settles, so
    # with few warm-ups the line measures that state; the warm figures (the
    # per-workload section's, after its own warm-ups) sit beside it.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()  # (one process: the barrier is trivial)
    t0 = time.perf_counter()
    e0.record(ctx.stream)
    for _ in range(args.steps):
        step()
    e1.record(ctx.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_us = e0.elapsed_time(e1) * 1e3 / args.steps
    value = stats["T"] * args.steps / wall
    log(f"headline: {wall * 1e3 / args.steps:.3f} ms/step wall, {dev_us:.2f} us/launch (events)")

    rl = roofline(stats, w.dtype, dev_us, "bytes_fused")
    traffic = load_traffic(args.profile or "mixed_b1024")
    line = {
        "metric": "ragged attention kept-tokens/s + \u00b5s/call (dispatch+kernel), % MFMA/HBM peak",
        "value": round(value, 1),
        "unit": "kept tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "images": w.B, "tokens": w.N, "heads": w.H, "head_dim": w.d,
                   "kept_tokens": stats["T"], "pruning": "per-image rate ~ U[0, 0.9]",
                   "launch": "direct single launch of the fused kernel (offsets, gather, attention, "
                             "zero-filled padded output)"},
        "roofline": {"bound": rl["bound"], "achieved": rl["GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": rl["frac_hbm"], "traffic": traffic,
                     "kernel": f"{kernel_label(w)} (fused, {w.dtype})",
                     "algorithmic_bytes_per_launch": stats["bytes_fused"],
                     "avg_launch_us": round(dev_us, 3),
                     "mfma_TFLOPs": rl["TFLOPs"], "mfma_frac": rl["frac_mfma"]},
        "warm_state": ("after the calibration probes (profiling run)" if args.profile else
                       "fresh process: the W warm-up launches are its first kernel launches (the first ~100 "
                       "launches of a fresh process run up to 15% slower; per_config's entry for this "
                       "workload gives the warm kernel time)"),
    }
    del tensors, step

    reps = 200
    if not args.quick:
        log("measuring the device ceilings ...")
        ceilings = measure_ceilings(ctx)
        floor = measure_floor(ctx, reps)
        floor["cpp"] = floor_cpp
        line["launch_floor"] = floor
        line["ceilings"] = ceilings
        log("measuring the access pattern alone ...")
        line["ceilings"]["access_pattern"] = measure_pattern(ctx, w)
        torch.cuda.empty_cache()
        per = []
        for wk in W.all_configs():
            log(f"measuring {wk.name} ...")
            per.append(measure_config(ctx, wk, reps if wk.B < 1024 else 50,
                                      floor["direct_latency_us"]))
            torch.cuda.empty_cache()
        line["per_config"] = per
        # the metric's per-call split for the headline workload (direct fused call)
        mix = next((c for c in per if c["workload"] == w.name), None)
        if mix is not None:
            fd = mix["fused_direct"]
            line["us_per_call"] = {"latency": fd["latency_us"], "kernel_warm": fd["kernel_us_warm"],
                                   "dispatch": fd["dispatch_us"],
                                   "form": "direct fused call from Python, call + synchronise"}
        log("measuring the keep-mask ...")
        line["threshold_l2"] = measure_threshold(ctx, reps)
        log("measuring the attention block and the layer stack ...")
        line["attention_block"] = measure_block(ctx, 50)
        torch.cuda.empty_cache()
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
