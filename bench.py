"""Benchmark of the block-sparse top-k attention hot path on one MI355X.

One step = the whole path on one batch of synthetic input already resident in HBM:
bsattn_select (pool q/k, block scores, top-k) then bsattn_forward (gathered-block
attention). Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload sparseformer_n8192_bf16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}        # dense TFLOP/s, MI355X
HBM_PEAK_GBS = 8000.0
METRIC = "tokens/sec + % bf16 MFMA peak, block-sparse attn N=8192 H=16 D=64 top-30%"
ATTN_SOURCE = os.path.join(ROOT, "block_sparse_top_amd", "csrc", "attn_bf16_kernel.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_sparseformer_n8192_traffic.txt")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="sparseformer_n8192_bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-batches", type=int, default=0,
                   help="cap on batch elements in the oracle sample (0: time-bounded, ~10 s)")
    p.add_argument("--causal", action="store_true",
                   help="causal variant (own block forced, earlier blocks only, masked own block)")
    p.add_argument("--pooling", choices=("mean", "max"), default="mean")
    p.add_argument("--group", action="store_true", help="one selection per KV head group")
    p.add_argument("--key-stride", type=int, default=0,
                   help="overlapping key blocks starting every KEY_STRIDE tokens (0: block; "
                        "the overlap ratio 0.25 is 3/4 of the block)")
    p.add_argument("--random-places", type=int, default=0,
                   help="places of each row filled by seeded random blocks (-1: int(0.05 k), the "
                        "MSA page's 5 %% random blocks)")
    p.add_argument("--backward", action="store_true",
                   help="also time bsattn_backward (bf16, block 64) on the same selection")
    p.add_argument("--decode", action="store_true",
                   help="time the decode step instead (workload decode_gqa_l32768)")
    return p.parse_args()


def file_sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_per_launch():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE, encoding="utf-8"):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            vals[key.strip()] = val.strip()
    if vals.get("source_sha256") != file_sha256(ATTN_SOURCE):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def probe_lib():
    """libbsattn_probe.so (include/bsattn_probe.h), the achievable-peak probes: a library of
    their own, separate from the method's libbsattn.so."""
    import ctypes
    path = os.path.join(ROOT, "block_sparse_top_amd", "libbsattn_probe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with block_sparse_top_amd.build.build()")
    L = ctypes.CDLL(path)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.bsattn_probe_last_error.restype = ctypes.c_char_p
    L.bsattn_probe_last_error.argtypes = []
    L.bsattn_probe_sink_floats.restype = sz
    L.bsattn_probe_sink_floats.argtypes = [i32]
    L.bsattn_probe_mfma_bf16.restype = i32
    L.bsattn_probe_mfma_bf16.argtypes = [i64, i32, vp, ctypes.POINTER(ctypes.c_double), vp]
    L.bsattn_probe_mfma_fp8.restype = i32
    L.bsattn_probe_mfma_fp8.argtypes = [i64, i32, vp, ctypes.POINTER(ctypes.c_double), vp]
    L.bsattn_probe_read.restype = i32
    L.bsattn_probe_read.argtypes = [vp, sz, i32, vp, vp]
    L.bsattn_probe_copy.restype = i32
    L.bsattn_probe_copy.argtypes = [vp, vp, sz, i32, vp]
    return L


def achievable_peaks(device, stream, reps=3):
    """What the chip sustains (include/bsattn_probe.h): dense bf16 MFMA TFLOP/s, HBM read GB/s,
    HBM copy GB/s (read + written bytes), each the best of `reps` HIP-event-timed launches."""
    import ctypes
    import torch
    L = probe_lib()
    groups = 2048                                   # 8 work-groups of 4 waves per CU
    sink = torch.empty(L.bsattn_probe_sink_floats(groups), dtype=torch.float32, device=device)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    nbytes = 1 << 30
    src = torch.empty(2 * nbytes, dtype=torch.uint8, device=device)
    src[:nbytes].fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=device)
    flops = ctypes.c_double(0.0)

    def best(call, work):
        call()                                      # warm-up
        out = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            e1.synchronize()
            out = max(out, work / (e0.elapsed_time(e1) / 1e3))
        return out

    def mfma():
        assert L.bsattn_probe_mfma_bf16(20000, groups, P(sink), ctypes.byref(flops), sp) == 0
    mfma()
    tf = best(mfma, flops.value) / 1e12
    flops8 = ctypes.c_double(0.0)

    def mfma8():
        assert L.bsattn_probe_mfma_fp8(10000, groups, P(sink), ctypes.byref(flops8), sp) == 0
    mfma8()
    tf8 = best(mfma8, flops8.value) / 1e12
    rd = best(lambda: L.bsattn_probe_read(P(src), 2 * nbytes, groups, P(sink), sp), 2 * nbytes) / 1e9
    cp = best(lambda: L.bsattn_probe_copy(P(src), P(dst), nbytes, groups, sp), 2 * nbytes) / 1e9
    del src, dst
    return {"mfma_bf16_tflops": round(tf, 1), "mfma_fp8_tflops": round(tf8, 1),
            "hbm_read_gbs": round(rd, 1), "hbm_copy_gbs": round(cp, 1)}


def host_cores():
    """Host cores the CPU leg may use: the process's affinity mask, capped by OMP_NUM_THREADS
    where the environment sets one (the box's share of a shared host)."""
    n = len(os.sched_getaffinity(0))
    how = f"len(os.sched_getaffinity(0)) = {n}"
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and 0 < int(env) < n:
        how += f", capped by OMP_NUM_THREADS = {env}"
        n = int(env)
    return n, how


def cpu_baseline(w, q, k, v, ds, max_batches, budget_s=15.0, causal=False, pooling="mean",
                 group=False, key_stride=0):
    """The fp64 oracle, as it stands, on batch elements 0, 1, ... of the workload until
    `budget_s` seconds of CPU work are done (at least one, at most `max_batches`)."""
    import numpy as np
    import torch
    import oracle.bsattn_oracle as O
    threads, how = host_cores()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads)
    except Exception:  # pragma: no cover
        limiter = None

    def host(t):
        c = t.detach().cpu()
        if c.dtype == torch.bfloat16:
            return c.view(torch.int16).numpy().view(np.uint16), "bf16"
        if c.dtype == torch.float8_e4m3fn:
            return c.view(torch.uint8).numpy(), "fp8"
        return c.numpy(), "f32"

    nkb = len(O.key_block_ranges(w.N, w.block, key_stride)) if key_stride else w.nb
    topk = O.topk_count(w.ratio, nkb)
    dt_s, batches = 0.0, 0
    while batches < max_batches and (batches == 0 or dt_s < budget_s):
        sl = slice(batches, batches + 1)
        (qh, dt), (kh, _), (vh, _) = host(q[sl]), host(k[sl]), host(v[sl])
        t0 = time.perf_counter()
        qo, ko, vo = O.widen(qh, dt, ds[0]), O.widen(kh, dt, ds[1]), O.widen(vh, dt, ds[2])
        stride = key_stride or None
        idx = O.select(qo, ko, w.block, topk, causal=causal, pooling=pooling, group=group,
                       stride=stride)
        if stride:
            O.attend(qo, ko, vo, idx, w.block, 1.0 / math.sqrt(w.D), stride=stride)
        else:
            O.attend_batched(qo, ko, vo, idx, w.block, 1.0 / math.sqrt(w.D), causal=causal)
        dt_s += time.perf_counter() - t0
        batches += 1
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": batches * w.N / dt_s, "unit": "tokens/s", "cores": int(threads),
            "cores_from": how, "kind": "oracle",
            "sample": f"{batches} of {w.B} batch elements (all heads, all query blocks), "
                      f"whole path in fp64 numpy, {dt_s:.1f} s"}


def time_backward(args, w, q, k, v, idx, out, topk, scale, flags, L, P, sp, stream, fwd_flops):
    """HIP-event time of one bsattn_backward call (after a forward that writes the row
    log-sum-exp). Algorithmic flops: the five products S, dP, dV, dK, dQ = 2.5 x forward."""
    import torch
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=q.device)
    dcode = 1
    st = L.bsattn_forward_ex(dcode, w.B, w.N, w.Hq, w.Hkv, w.D, w.block, topk, flags, 0, P(q),
                             P(k), P(v), P(idx), scale, None, P(out), P(lse), sp)
    assert st == 0, L.bsattn_last_error()
    g = torch.Generator(device=q.device).manual_seed(7)
    dout = torch.randn(out.shape, generator=g, device=q.device).to(torch.bfloat16)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    nbytes = L.bsattn_backward_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.block, topk)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)

    def call():
        st = L.bsattn_backward(dcode, w.B, w.N, w.Hq, w.Hkv, w.D, w.block, topk, flags, P(q),
                               P(k), P(v), P(idx), P(out), P(dout), P(lse), scale, P(dq), P(dk),
                               P(dv), P(ws), ws.numel(), sp)
        assert st == 0, L.bsattn_last_error()

    for _ in range(max(1, args.warmup // 2)):
        call()
    torch.cuda.synchronize()
    n = max(1, args.steps // 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    bflops = 2.5 * fwd_flops
    return {"ms": round(ms, 4), "algorithmic_flop": bflops,
            "tflops": round(bflops / ms / 1e9, 2),
            "frac_bf16_peak": round(bflops / ms / 1e9 / PEAK["bf16"], 4)}


def bench_decode(args):
    """One step = bsattn_decode for every sequence of the batch (one new token each) against
    a full cache; the pooled-key cache is built once beforehand (untimed). Prints one line."""
    import ctypes
    import torch
    import block_sparse_top_amd as bst
    from block_sparse_top_amd import synthetic as syn
    w = syn.DECODE_WORKLOADS["decode_gqa_l32768"]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    q, kc, vc = syn.decode_inputs(w, device=dev)
    topk = int(w.ratio * w.nb)
    lens = torch.full((w.B,), w.N, dtype=torch.int32, device=dev)
    kbar = torch.empty((w.B, w.Hkv, w.D, w.nb), dtype=torch.float32, device=dev)
    bst.decode_pool(kc, lens, kbar, w.block)
    L = bst.lib()
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((w.B, w.Hq, topk), dtype=torch.int32, device=dev)
    ws = torch.empty(L.bsattn_decode_workspace_bytes(w.B, w.Hq, w.D, topk), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    scale = 1.0 / math.sqrt(w.D)

    flags = bst.GROUP_SELECT if args.group else 0

    def step():
        st = L.bsattn_decode_ex(1, w.B, w.N, w.Hq, w.Hkv, w.D, w.block, topk, flags, P(q), P(kc),
                                P(vc), P(kbar), P(lens), scale, P(out), P(idx), P(ws), ws.numel(),
                                sp)
        assert st == 0, L.bsattn_last_error()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    # bytes the step must read: keys and values of the chosen blocks (per query head; with a
    # group-shared selection once per KV head, whose query heads read the same blocks), the
    # pooled keys (per selection), the query, the output and idx
    sel_heads = w.Hkv if args.group else w.Hq
    kv_bytes = w.B * sel_heads * topk * w.block * w.D * 2 * 2
    kbar_bytes = w.B * sel_heads * w.nb * w.D * 4
    total = kv_bytes + kbar_bytes + w.B * w.Hq * (w.D * 4 + topk * 4)
    rec = {
        "metric": "decode tokens/s (one new token per sequence, block-sparse attention step)",
        "value": round(w.B / (wall / args.steps), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) caches, resident in HBM)",
        "config": {"workload": w.name, "B": w.B, "cache_len": w.N, "Hq": w.Hq, "Hkv": w.Hkv,
                   "D": w.D, "block": w.block, "topk": topk, "parallelism": "single GPU",
                   **({"group_select": True} if args.group else {})},
        "roofline": {"bound": "hbm", "achieved": round(total / (ms / 1e3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(total / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "bsattn_decode (select + split attention + combine)",
                     "algorithmic_bytes_per_step": total},
        "decode_ms": round(ms, 4),
    }
    ach = achievable_peaks(q.device, stream)
    rec["achievable"] = ach
    rec["roofline"]["achievable_peak"] = ach["hbm_read_gbs"]
    rec["roofline"]["achievable_frac"] = round(rec["roofline"]["achieved"] / ach["hbm_read_gbs"], 4)
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library is a "
              "single-GPU path; it shards over (batch, KV-head group) with no communication, so "
              "N GPUs run N independent copies of this measurement.", file=sys.stderr)
        sys.exit(2)
    if args.decode:
        bench_decode(args)
        return
    import torch
    import block_sparse_top_amd as bst
    from block_sparse_top_amd import synthetic as syn

    w = syn.WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    q, k, v, ds, _ = syn.workload_inputs(w, device=dev)
    ks = args.key_stride or w.block
    if ks != w.block and (args.causal or args.backward):
        sys.exit("bench.py: overlapping key blocks run the non-causal forward only")
    nkb = bst.key_blocks(w.N, w.block, ks)
    topk = int(w.ratio * nkb)                  # k = int(topk_ratio * number of key blocks)
    scale = 1.0 / math.sqrt(w.D)
    ws = torch.empty(bst.select_workspace_bytes(w.B, w.N, w.Hq, w.Hkv, w.D, w.block, ks),
                     dtype=torch.uint8, device=dev)
    idx = torch.empty((w.B, w.Hq, w.nb, topk), dtype=torch.int32, device=dev)
    odt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    out = torch.empty((w.B, w.N, w.Hq, w.D), dtype=odt, device=dev)

    # the C calls run on preallocated buffers (the binding would allocate idx and out per call)
    L = bst.lib()
    import ctypes
    dcode = bst.bsattn._DTYPES[q.dtype]
    dsc = (ctypes.c_float * 3)(*ds)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    flags = (bst.CAUSAL if args.causal else 0) | (bst.POOL_MAX if args.pooling == "max" else 0) \
        | (bst.GROUP_SELECT if args.group else 0)

    nrand = int(0.05 * topk) if args.random_places < 0 else args.random_places

    def do_select():
        st = L.bsattn_select_ex(dcode, w.B, w.N, w.Hq, w.Hkv, w.D, w.block, topk, flags, nrand,
                                12345, ks, P(q), P(k), P(idx), P(ws), ws.numel(), sp)
        assert st == 0, L.bsattn_last_error()

    def do_forward():
        st = L.bsattn_forward_ex(dcode, w.B, w.N, w.Hq, w.Hkv, w.D, w.block, topk, flags, ks,
                                 P(q), P(k), P(v), P(idx), scale, dsc, P(out), None, sp)
        assert st == 0, L.bsattn_last_error()

    for _ in range(args.warmup):
        do_select()
        do_forward()
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps back to back; HIP events on the library's
    # stream around each call give the per-launch durations the roofline uses
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        do_select()
        e[1].record(stream)
        do_forward()
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel_all = [e[0].elapsed_time(e[1]) for e in evs]
    fwd_all = [e[1].elapsed_time(e[2]) for e in evs]
    sel_ms = sum(sel_all) / len(evs)
    fwd_ms = sum(fwd_all) / len(evs)
    ms_per_step = wall * 1e3 / args.steps
    tokens = w.B * w.N
    value = tokens / (ms_per_step / 1e3)

    # A second timing protocol, after the timed region (reported beside it): per call,
    # repeats of up to 50 launches, the median over 5 repeats; each selection launch follows a
    # 512 MB write that evicts the 256 MB MALL (the write is outside the events).
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def protocol(call, est_ms, flush_first):
        n = max(1, min(50, int(round(500.0 / max(est_ms, 1e-3)))))
        reps = []
        for r in range(5):
            if flush_first:
                tot = 0.0
                for _ in range(n):
                    flush.fill_(r & 0xFF)
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    call()
                    b.record(stream)
                    b.synchronize()
                    tot += a.elapsed_time(b)
                reps.append(tot / n)
            else:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(n):
                    call()
                b.record(stream)
                b.synchronize()
                reps.append(a.elapsed_time(b) / n)
        reps.sort()
        return {"median_ms": round(reps[2], 4), "repeats_ms": [round(x, 4) for x in reps],
                "launches_per_repeat": n}
    proto = {"select_after_mall_flush": protocol(do_select, sel_ms, True),
             "forward": protocol(do_forward, fwd_ms, False)}
    del flush

    # QK^T + PV over every computed key block (causal: query block i computes min(topk, i+1)
    # blocks, its own one in full although half of it is masked)
    blocks = sum(min(topk, i + 1) for i in range(w.nb)) if args.causal else w.nb * topk
    flops = 4.0 * w.B * w.Hq * w.block * (blocks * w.block) * w.D
    if ks != w.block:
        # overlapping key blocks: the keys attended are the union of each row's blocks (the
        # rows are ascending; a pair j-1, j shares block - ks tokens, the last block is short)
        adj = (idx[..., 1:] == idx[..., :-1] + 1).sum().item()
        last = (idx == nkb - 1).sum().item()
        keys = (w.B * w.Hq * w.nb * topk * w.block - adj * (w.block - ks)
                - last * (w.block - (w.N - (nkb - 1) * ks)))
        flops = 4.0 * w.block * keys * w.D
    achieved = flops / (fwd_ms / 1e3) / 1e12
    peak = PEAK[w.dtype]
    ebytes = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    # The selection's algorithmic bytes: q and k read once, the
    # pooled blocks written once, idx written; where the score matrix goes through HBM
    # (more than 1024 blocks) also its write and read and the pooled blocks' read by the
    # score product. ("moved": what the kernels move on top of that, e.g. the fused kernel
    # re-reading the pooled keys.)
    sel_heads = w.Hkv if args.group else w.Hq
    sel_bytes = (w.B * w.N * (w.Hq + w.Hkv) * w.D * ebytes             # read q, k
                 + 4 * w.B * (w.nb * w.Hq + nkb * w.Hkv) * w.D         # pooled writes
                 + 4 * w.B * w.Hq * w.nb * topk)                       # idx write
    moved = sel_bytes + 4 * w.B * nkb * w.Hkv * w.D                    # pooled keys read back
    if w.nb > 1024:
        extra = (2 * 4 * w.B * sel_heads * w.nb * w.nb                 # score matrix write + read
                 + 4 * w.B * (w.nb * w.Hq + w.nb * w.Hkv) * w.D)       # pooled rows read
        sel_bytes += extra
        moved = sel_bytes + (4 * w.B * w.nb * w.Hq * w.D if args.group else 0)
    plain = not (args.causal or args.group or args.pooling == "max" or ks != w.block)
    tr = traffic_per_launch() if plain and w.name == "sparseformer_n8192_bf16" else None
    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1), resident in HBM)",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "block": w.block, "topk": topk, "parallelism": "single GPU",
                   **({"causal": True} if args.causal else {}),
                   **({"pooling": "max"} if args.pooling == "max" else {}),
                   **({"group_select": True} if args.group else {}),
                   **({"random_places": nrand} if nrand else {}),
                   **({"key_stride": ks, "key_blocks": nkb} if ks != w.block else {})},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": tr, "kernel": f"attn_{w.dtype}_kernel",
                     "algorithmic_flop_per_launch": flops},
        "select_ms": round(sel_ms, 4), "forward_ms": round(fwd_ms, 4),
        "timed_region": {"select_ms_avg": round(sel_ms, 4), "forward_ms_avg": round(fwd_ms, 4),
                         "forward_ms_min": round(min(fwd_all), 4),
                         "forward_ms_max": round(max(fwd_all), 4)},
        "select_hbm_frac": round(sel_bytes / (sel_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "select_algorithmic_bytes": sel_bytes, "select_moved_bytes": moved,
        "protocol": proto,
        "select_hbm_frac_after_flush": round(
            sel_bytes / (proto["select_after_mall_flush"]["median_ms"] / 1e3) / 1e9
            / HBM_PEAK_GBS, 4),
    }
    if w.dtype in ("bf16", "fp8"):
        ach = achievable_peaks(dev, stream)
        rec["achievable"] = ach
        apeak = ach["mfma_bf16_tflops" if w.dtype == "bf16" else "mfma_fp8_tflops"]
        rec["roofline"]["achievable_peak"] = apeak
        rec["roofline"]["achievable_frac"] = round(achieved / apeak, 4)
        rec["select_achievable_hbm_frac"] = round(
            sel_bytes / (sel_ms / 1e3) / 1e9 / ach["hbm_read_gbs"], 4)
    if args.backward:
        rec["backward"] = time_backward(args, w, q, k, v, idx, out, topk, scale, flags, L, P, sp,
                                        stream, flops)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, ds, args.cpu_batches or w.B,
                                           causal=args.causal, pooling=args.pooling,
                                           group=args.group,
                                           key_stride=ks if ks != w.block else 0)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
