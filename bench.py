#!/usr/bin/env python3
"""Benchmark of msa_index_score on one MI355X.

A step is one call of the operator (one kernel launch through the C ABI) over
one batch of seeded synthetic inputs resident in HBM.  The default workload is
the decode batch: 64 requests of one query token, 16 index heads over one KV
head, kv_len ~ U[1, 32768], bf16 keys in 16384 paged 128-token blocks
(BBND) behind a random block table, right-down causal, local_blocks = 1.

Timed region: W untimed warmup steps, then exactly K steps bracketed by
torch.cuda.synchronize(); one pair of HIP events on the launch stream around
the K launches (nothing recorded between them) gives the kernel's average
duration for the roofline.  The launches are a loop of C-ABI calls from
Python; each line also reports, under 'graph', the same K calls captured
into a HIP graph and replayed once (the GPU-side figure where the host's
call rate, ~8-18 us a call depending on the box, is slower than a short
kernel; where the host keeps up, replays measured no faster, so the loop is
the primary figure; ``--graph`` swaps them).
To keep the 256 MB Infinity Cache from serving repeated reads, the key cache
is replicated into several HBM copies and the steps rotate over them.

Output: one JSON line (rank 0 of 1).  By default its top level is the
headline decode batch, and its ``workloads`` list holds all five base
workloads measured in the same process (the tiny example, the decode batch,
the varlen prefill, the int8 decode batch and the chunked fp8 prefill) and
the MXFP4 variants of three of them (the decode batch and both prefills),
each with its average launch duration, roofline (with HBM traffic from the
committed counter runs when they match the current kernel sources), the
oracle's CPU baseline on this host's available cores (one core too, for the
decode-sized ones) and, for the base prefill workloads, the top-k selection
on their scores.  ``--config all`` prints one full line per workload instead.
``--topk`` times the top-k block selection (msa_block_topk, k = 16) over the
chosen workload's score rows instead, with its own roofline (HBM bytes: every
row's num_valid scores read, its k indices written).  ``--local-mode query``
runs the workload with the local_mask window at each token's own block.
``--config mx`` (or one of ``decode_bbnd_mxfp4``, ``prefill_tnd_mxfp4``,
``prefill_bbnd_mxfp4``) measures the MXFP4 variants of three workloads
(msa_index_score_mxfp4; roofline against FP4's 10.1 PFLOP/s dense peak, or
HBM for the decode batch).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("block scores/s + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill), 1 GPU")
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "i8": 2500.0, "f8e4m3": 5000.0, "f8e5m2": 5000.0,
               "mxfp4": 10100.0}
ESIZE = {"f16": 2, "bf16": 2, "i8": 1, "f8e4m3": 1, "f8e5m2": 1, "mxfp4": 0.5}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_max_qk_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def workload_stats(case) -> dict:
    """Algorithmic work of one step, from the drawn lengths."""
    import torch
    P = case.block_size
    cu = case.cu_seqlens_q.long()
    kv = case.kv_len.long()
    B = case.batch
    scores = 0          # (h, t, beta) entries with >= 1 visible key
    visible = 0         # (h, t, j) visible key positions
    k_bytes = 0
    table_bytes = 0
    esz = ESIZE[case.key_dtype_name()]
    for b in range(B):
        Lq = int(cu[b + 1] - cu[b])
        L = int(kv[b])
        if Lq == 0 or L == 0:
            continue
        i = torch.arange(Lq, dtype=torch.int64)
        qpos = (L - Lq + i) if case.sparse_mode == 3 else torch.full_like(i, L - 1)
        lim = torch.clamp(torch.minimum(qpos, torch.tensor(L - 1)), min=-1)
        lim = torch.minimum(lim, torch.tensor(case.max_blocks * P - 1))
        nvis = torch.where(lim >= 0, lim // P + 1, torch.zeros_like(lim))
        scores += int(nvis.sum()) * case.Hq
        visible += int((lim + 1).sum()) * case.Hq
        lmax = int(lim.max())
        if lmax >= 0:
            k_bytes += int((lmax + 1) * case.Hkv * case.D * esz)  # each visible key read once
            if case.scale is not None:
                k_bytes += (lmax + 1) * case.Hkv * 4
            if case.k_mx_scale is not None:                        # E8M0 per 32 elements
                k_bytes += (lmax + 1) * case.Hkv * (case.D // 32)
            if case.layout != "TND":
                table_bytes += (lmax // P + 1) * 4
    W = ((max(case.max_blocks, 1) + 15) // 16) * 16
    q_bytes = case.query.numel() * case.query.element_size()
    if case.q_mx_scale is not None:
        q_bytes += case.q_mx_scale.numel()
    out_bytes = case.Hq * case.T * W * 4
    return {"scores": scores, "out_entries": case.Hq * case.T * W,
            "flops": 2 * case.D * visible,
            "bytes": k_bytes + q_bytes + out_bytes + table_bytes + 8 * B,
            "k_bytes": k_bytes, "q_bytes": q_bytes, "out_bytes": out_bytes}


def time_launches(launch, steps: int, stream, graph: bool):
    """Time `steps` launches, launch(i, stream_handle) issuing launch i on the
    given stream.  graph: the launches are captured once into a HIP graph and
    the timed region is one replay of it (the K kernel launches with no host
    work between them); otherwise a plain loop of C-ABI calls from Python.
    Returns the average launch duration from one HIP event pair around the K
    launches on `stream` (nothing recorded between them: events between
    launches add their own processing time to each) and the wall time per
    step; both bracketed by torch.cuda.synchronize()."""
    import torch
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap):
            for i in range(steps):
                launch(i, cap.cuda_stream)
        stream.wait_stream(cap)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    if graph:
        with torch.cuda.stream(stream):
            g.replay()
    else:
        for i in range(steps):
            launch(i, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return e0.elapsed_time(e1) / steps, (t1 - t0) * 1e3 / steps


def bench_config(c_idx: int, steps: int, warmup: int, copies: int, family: int,
                 cpu_baseline: bool, args, local_mode: int = 0, topk: bool = False,
                 host: dict = None) -> dict:
    import dataclasses
    import torch
    import block_max_qk_amd as m
    from block_max_qk_amd._binding import describe
    import ctypes
    import synth

    dev = torch.device("cuda:0")
    t_gen = time.time()
    nbase = len(synth.CONFIG_NAMES)
    case = (synth.config_case(c_idx) if c_idx < nbase
            else synth.mx_config_case(synth.MX_CONFIG_NAMES[c_idx - nbase]))
    mx = case.q_mx_scale is not None
    if local_mode:
        case = dataclasses.replace(case, local_mode=local_mode)
    t_gen = time.time() - t_gen
    stats = workload_stats(case)
    kname = case.key_dtype_name()
    is_decode = m.msa_index_score_kernel_family(case.T, case.batch, case.Hq, case.Hkv) == 0 \
        if family < 0 else family == 0

    # inputs resident in HBM; the key cache (and scale) replicated `copies` times
    W = m.msa_index_score_out_width(case.max_blocks)
    q = case.query.to(dev)
    keys, scales, kmx = [], [], []
    for _ in range(copies):
        ks = case.key_storage.to(dev)
        keys.append(ks[:: case.gap + 1] if case.gap else ks)
        scales.append(None if case.scale is None else case.scale.to(dev))
        kmx.append(None if case.k_mx_scale is None else case.k_mx_scale.to(dev))
    qmx = None if case.q_mx_scale is None else case.q_mx_scale.to(dev)
    sl = case.start_loc.to(dev)
    bt = None if case.block_table is None else case.block_table.to(dev)
    cu = case.cu_seqlens_q.to(dev)
    kv = case.kv_len.to(dev)
    out = torch.empty((case.Hq, case.T, W), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    lib = m.load_library()

    # marshal each copy's arguments once; the timed loop only calls the C ABI
    keep = []
    calls = []
    for i in range(copies):
        qd, kd = describe(q), describe(keys[i])
        keep += [qd, kd]
        if mx:
            calls.append((ctypes.byref(qd), ctypes.c_void_p(qmx.data_ptr()), ctypes.byref(kd),
                          ctypes.c_void_p(kmx[i].data_ptr()), ctypes.c_void_p(sl.data_ptr()),
                          None if bt is None else ctypes.c_void_p(bt.data_ptr()),
                          case.max_blocks, ctypes.c_void_p(cu.data_ptr()),
                          ctypes.c_void_p(kv.data_ptr()), case.batch, case.block_size,
                          m._binding.LAYOUT_CODE[case.layout], case.sparse_mode,
                          case.init_blocks, case.local_blocks, case.local_mode,
                          ctypes.c_void_p(out.data_ptr()), W, None))
            continue
        a = (ctypes.byref(qd), ctypes.byref(kd), ctypes.c_void_p(sl.data_ptr()),
             None if bt is None else ctypes.c_void_p(bt.data_ptr()), case.max_blocks,
             None if scales[i] is None else ctypes.c_void_p(scales[i].data_ptr()),
             ctypes.c_void_p(cu.data_ptr()), ctypes.c_void_p(kv.data_ptr()), case.batch,
             case.block_size, m._binding.LAYOUT_CODE[case.layout], case.sparse_mode,
             case.init_blocks,
             case.local_blocks, case.local_mode, ctypes.c_void_p(out.data_ptr()), W,
             None, family)
        calls.append(a)
    fn = lib.msa_index_score_mxfp4 if mx else lib.msa_index_score_ex
    si = 18 if mx else 17          # position of the stream argument

    def launch(i, h):
        a = calls[i % copies]
        st = fn(*a[:si], ctypes.c_void_p(h), *a[si + 1:])
        if st != 0:
            raise RuntimeError(m.msa_status_str(st))

    for i in range(warmup):
        launch(i, stream.cuda_stream)
    torch.cuda.synchronize()
    graph = bool(getattr(args, "graph", False))
    kernel_ms, ms_per_step = time_launches(launch, steps, stream, graph)
    alt_ms, alt_step = time_launches(launch, steps, stream, not graph)

    gbs = stats["bytes"] / (kernel_ms * 1e-3) / 1e9
    tflops = stats["flops"] / (kernel_ms * 1e-3) / 1e12
    if is_decode:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        pk = PEAK_TFLOPS[kname]
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": pk, "unit": "TFLOP/s",
                "frac": round(tflops / pk, 4)}
    # counters were taken with the per-request window (same memory accesses)
    roof["traffic"] = measured_traffic(case.name) if case.local_mode == 0 else None
    roof["kernel"] = ("decode_kernel" if is_decode else "prefill_kernel") + f"<{kname}>"
    roof["kernel_ms_avg"] = round(kernel_ms, 5)
    roof["algorithmic_bytes"] = stats["bytes"]
    roof["algorithmic_flops"] = stats["flops"]

    value = stats["scores"] / (ms_per_step * 1e-3)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "block scores/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": kname, "data": "synthetic",
        "config": {"workload": case.name, "B": case.batch, "T": case.T, "Hq": case.Hq,
                   "Hkv": case.Hkv, "D": case.D, "P": case.block_size, "MB": case.max_blocks,
                   "layout": case.layout, "query_dtype": case.query_dtype_name(),
                   "key_dtype": kname, "sparse_mode": case.sparse_mode,
                   "init_blocks": case.init_blocks, "local_blocks": case.local_blocks,
                   "local_window": "per-query" if case.local_mode else "per-request",
                   "key_cache_copies": copies,
                   "kernel_family": "decode" if is_decode else "prefill"},
        "hbm_gbs": round(gbs, 1), "mfma_tflops": round(tflops, 3),
        "block_scores_per_step": stats["scores"], "out_entries_per_step": stats["out_entries"],
        "roofline": roof,
        "cpu_baseline": None,
        "launch": "hip_graph" if graph else "eager",
        ("eager" if graph else "graph"): {"kernel_ms_avg": round(alt_ms, 5),
                                          "ms_per_step": round(alt_step, 5)},
        "input_generation_s": round(t_gen, 2),
    }
    if topk:
        # the selection that follows the operator, timed on the scores the
        # last step wrote (resident in HBM)
        res["topk"] = time_topk(out, case.max_blocks, steps, warmup, stream, graph=graph)
    del calls, keep, out
    if cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_leg(case, stats, args, host or host_cpu())
    return res


def time_topk(scores, num_valid: int, steps: int, warmup: int, stream, k: int = 16,
              graph: bool = True) -> dict:
    """msa_block_topk (k = 16) over every row of a score tensor already in
    HBM: average launch duration (time_launches), and its HBM roofline (each
    row's num_valid scores read, k indices written)."""
    import torch
    import block_max_qk_amd as m
    Hq, T, W = scores.shape
    out = torch.empty((T, Hq, k), dtype=torch.int32, device=scores.device)
    for _ in range(warmup):
        m.msa_block_topk(scores, num_valid, k, out, stream=stream)
    torch.cuda.synchronize()
    ms, _ = time_launches(lambda i, h: m.msa_block_topk(scores, num_valid, k, out, stream=h),
                          steps, stream, graph)
    alg = Hq * T * (num_valid + k) * 4
    gbs = alg / (ms * 1e-3) / 1e9
    return {"kernel": "topk_kernel", "k": k, "rows": Hq * T, "num_valid": num_valid,
            "kernel_ms_avg": round(ms, 5), "selections_per_s": round(Hq * T / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": alg}}


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, when
    they were taken on the current kernel sources; otherwise null."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def host_cpu() -> dict:
    """The host the oracle runs on: core counts as the OS reports them, the
    share this process may use (CPU affinity, cgroup CPU quota and
    OMP_NUM_THREADS, which a shared GPU host sets to the job's CPU share),
    and the CPU model."""
    info = {"nproc": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        info["affinity"] = os.cpu_count()
    quota = None
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = round(int(q) / int(per), 2)
    except (OSError, ValueError):
        pass
    info["cgroup_cpus"] = quota
    omp = os.environ.get("OMP_NUM_THREADS", "")
    info["omp_num_threads"] = int(omp) if omp.isdigit() and int(omp) > 0 else None
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info["cpu_model"] = model
    avail = info["affinity"] or 1
    if quota:
        avail = min(avail, max(1, int(quota)))
    if info["omp_num_threads"]:
        avail = min(avail, info["omp_num_threads"])
    info["cores_available"] = avail
    return info


def visible_blocks_per_token(case):
    """int64 [T]: blocks with at least one visible key for each query token
    (the window of workload_stats), i.e. the block scores an (h, t) row costs
    whatever local_mask later writes over them."""
    import torch
    P = case.block_size
    cu, kv = case.cu_seqlens_q.long(), case.kv_len.long()
    nvis = torch.zeros(case.T, dtype=torch.int64)
    for b in range(case.batch):
        t0, t1, L = int(cu[b]), int(cu[b + 1]), int(kv[b])
        if t1 == t0 or L == 0:
            continue
        i = torch.arange(t1 - t0, dtype=torch.int64)
        qpos = (L - (t1 - t0) + i) if case.sparse_mode == 3 else torch.full_like(i, L - 1)
        lim = torch.clamp(torch.minimum(qpos, torch.tensor(L - 1)), min=-1)
        lim = torch.minimum(lim, torch.tensor(case.max_blocks * P - 1))
        nvis[t0:t1] = torch.where(lim >= 0, lim // P + 1, torch.zeros_like(lim))
    return nvis


def cpu_baseline_leg(case, stats, args, host: dict) -> dict:
    """The CPU oracle, as it is, timed on this host's available cores on a
    bounded sample of the same workload, scaled to block scores/s.  Decode
    batches and the tiny example: the whole workload on every available core,
    and one core on the whole tiny example or a random eighth of a batch's
    requests.  Prefill workloads: whole random output rows on every available
    core (extrapolated to the workload's rate)."""
    import torch
    import oracle
    nth = host["cores_available"]
    W = ((max(case.max_blocks, 1) + 15) // 16) * 16
    res = {"unit": "block scores/s", "cores": nth, "kind": "oracle", "host": host}
    if case.T <= 256:
        t0 = time.perf_counter()
        oracle.index_score(**oracle.case_args(case), nthreads=nth)
        dt = time.perf_counter() - t0
        res.update(value=round(stats["scores"] / dt, 1), extrapolated=False,
                   sample=f"the whole workload ({stats['scores']} block scores) in {dt:.2f} s "
                          f"on {nth} threads")
        # one core
        g = torch.Generator().manual_seed(11)
        B = case.batch
        nreq = B if case.T <= 32 else max(1, (B + 7) // 8)
        reqs = sorted(torch.randperm(B, generator=g)[:nreq].tolist())
        cu = case.cu_seqlens_q.long()
        ts = torch.cat([torch.arange(int(cu[b]), int(cu[b + 1])) for b in reqs])
        hs = torch.arange(case.Hq)
        pts = torch.stack([hs.repeat_interleave(len(ts) * W), ts.repeat_interleave(W).repeat(case.Hq),
                           torch.arange(W).repeat(len(ts) * case.Hq)], 1)
        t0 = time.perf_counter()
        oracle.index_score_case_points(case, pts, nthreads=1)
        dt1 = time.perf_counter() - t0
        n1 = int(visible_blocks_per_token(case)[ts].sum()) * case.Hq
        res["single_core"] = {"value": round(n1 / dt1, 1), "cores": 1,
                              "sample": f"{nreq} of {B} requests at random, every entry "
                                        f"({n1} block scores) in {dt1:.2f} s",
                              "extrapolated": nreq < B}
        return res
    # prefill: whole rows (h, t, all blocks) of tokens spread over the batch
    g = torch.Generator().manual_seed(7)
    nrows = args.cpu_rows
    ts = torch.randint(0, case.T, (nrows,), generator=g)
    hs = torch.randint(0, case.Hq, (nrows,), generator=g)
    beta = torch.arange(W)
    pts = torch.stack([hs.repeat_interleave(W), ts.repeat_interleave(W), beta.repeat(nrows)], 1)
    t0 = time.perf_counter()
    oracle.index_score_case_points(case, pts, nthreads=nth)
    dt = time.perf_counter() - t0
    sampled = int(visible_blocks_per_token(case)[ts].sum())
    res.update(value=round(sampled / dt, 1), extrapolated=True,
               sample=f"{nrows} whole rows (h, t) at random, {sampled} block scores in "
                      f"{dt:.2f} s on {nth} threads, scaled to block scores/s")
    return res


TOPK_METRIC = "top-k block selections/s (k=16) + achieved HBM GB/s, 1 GPU"


def bench_topk(c_idx: int, steps: int, warmup: int, cpu_baseline: bool, args) -> dict:
    """Time msa_block_topk (k = 16) on the score rows of a workload: the
    scores are computed once by the operator, then each step is one top-k
    launch over all [Hq, T] rows (inputs resident in HBM; the prefill score
    tensors are ~1 GB, beyond the Infinity Cache)."""
    import torch
    import block_max_qk_amd as m
    import synth

    dev = torch.device("cuda:0")
    k = 16
    case = synth.config_case(c_idx)
    W = m.msa_index_score_out_width(case.max_blocks)
    d = dict(query=case.query.to(dev), key=case.key_storage.to(dev))
    key = d["key"][:: case.gap + 1] if case.gap else d["key"]
    scores = torch.empty((case.Hq, case.T, W), dtype=torch.float32, device=dev)
    m.msa_index_score(d["query"], key, case.start_loc.to(dev),
                      None if case.block_table is None else case.block_table.to(dev),
                      None if case.scale is None else case.scale.to(dev),
                      case.cu_seqlens_q.to(dev), case.kv_len.to(dev), case.layout,
                      case.sparse_mode, case.init_blocks, case.local_blocks, scores,
                      case.max_blocks)
    del d, key
    nv = case.max_blocks
    rows = case.Hq * case.T
    out = torch.empty((case.T, case.Hq, k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        m.msa_block_topk(scores, nv, k, out, stream=stream)
    torch.cuda.synchronize()
    graph = bool(getattr(args, "graph", False))
    kernel_ms, ms_per_step = time_launches(
        lambda i, h: m.msa_block_topk(scores, nv, k, out, stream=h), steps, stream, graph)
    alg = rows * (nv + k) * 4      # each row's num_valid scores read, k indices written
    gbs = alg / (kernel_ms * 1e-3) / 1e9
    res = {
        "metric": TOPK_METRIC, "value": round(rows / (ms_per_step * 1e-3), 1),
        "unit": "block selections/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": case.name, "stage": "top-k", "k": k, "rows": rows,
                   "width": W, "num_valid": nv},
        "launch": "hip_graph" if graph else "eager",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("topk:" + case.name),
                     "kernel": "topk_kernel", "kernel_ms_avg": round(kernel_ms, 5),
                     "algorithmic_bytes": alg},
        "cpu_baseline": None,
    }
    if cpu_baseline:
        import oracle
        import torch as _t
        g = _t.Generator().manual_seed(7)
        n = min(rows, args.cpu_topk_rows)
        pick = _t.randperm(rows, generator=g)[:n]
        sample = scores.reshape(rows, W)[pick.to(dev)].cpu()[None]
        t = time.perf_counter()
        oracle.block_topk(sample, nv, k)
        dt = time.perf_counter() - t
        res["cpu_baseline"] = {"value": round(n / dt, 1), "unit": "block selections/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{n} random rows of the workload in {dt:.2f} s"}
    return res


HEADLINE = "decode_bbnd_bf16"


def decode_batch_stats(kv, Hq: int, Hkv: int, D: int, P: int, MB: int, esz: int) -> dict:
    """workload_stats for one-token decode requests (q_len = 1, right-down
    causal window, every kv_len >= 1 and <= MB P): each request scores its
    ceil(kv_len / P) blocks and reads its kv_len keys once."""
    import numpy as np
    kv = np.asarray(kv, dtype=np.int64)
    B = int(kv.size)
    nb = (kv - 1) // P + 1
    W = ((max(MB, 1) + 15) // 16) * 16
    k_bytes = int(kv.sum()) * Hkv * D * esz
    q_bytes = B * Hq * D * 2
    out_bytes = Hq * B * W * 4
    return {"scores": int(nb.sum()) * Hq, "out_entries": Hq * B * W,
            "flops": 2 * D * int(kv.sum()) * Hq,
            "bytes": k_bytes + q_bytes + out_bytes + int(nb.sum()) * 4 + 8 * B,
            "k_bytes": k_bytes, "q_bytes": q_bytes, "out_bytes": out_bytes}


def bench_decode_batch(B: int, steps: int, warmup: int, seed: int = 20261299) -> dict:
    """The bf16 decode workload's distribution at batch size B (kv_len ~
    U[1, 32768], Hq = 16, Hkv = 1, MB = 256, B MB distinct pages in a random
    table), keys drawn on the GPU from a seeded generator (host generation of
    the 8.6 GB cache of B = 1024 would dominate the run).  Times the launch
    with the drawn lengths (HBM roofline) and with every kv_len = 1, where
    one block per request leaves the launch, the request lookup and the fill
    of the unscored blocks."""
    import ctypes
    import numpy as np
    import torch
    import block_max_qk_amd as m
    from block_max_qk_amd._binding import describe, LAYOUT_CODE

    dev = torch.device("cuda:0")
    Hq, Hkv, D, P, MB = 16, 1, 128, 128, 256
    NP = B * MB
    rng = np.random.default_rng(seed + B)
    kv_np = rng.integers(1, 32768 + 1, size=B).astype(np.int64)
    bt = torch.from_numpy(rng.permutation(NP)[: B * MB].reshape(B, MB).astype(np.int32)).to(dev)
    g = torch.Generator(device=dev).manual_seed(seed + B)
    key = torch.empty((NP, P, Hkv, D), dtype=torch.bfloat16, device=dev).normal_(generator=g)
    q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev).normal_(generator=g)
    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    W = m.msa_index_score_out_width(MB)
    out = torch.empty((Hq, B, W), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    lib = m.load_library()
    qd, kd = describe(q), describe(key)

    def timed(kv_host):
        kv = torch.from_numpy(kv_host.astype(np.int32)).to(dev)
        sl = torch.from_numpy(((kv_host - 1) // P).astype(np.int32)).to(dev)
        a = (ctypes.byref(qd), ctypes.byref(kd), ctypes.c_void_p(sl.data_ptr()),
             ctypes.c_void_p(bt.data_ptr()), MB, None, ctypes.c_void_p(cu.data_ptr()),
             ctypes.c_void_p(kv.data_ptr()), B, P, LAYOUT_CODE["BBND"], 3, 0, 1, 0,
             ctypes.c_void_p(out.data_ptr()), W, ctypes.c_void_p(stream.cuda_stream), -1)
        for _ in range(warmup):
            st = lib.msa_index_score_ex(*a)
            if st != 0:
                raise RuntimeError(m.msa_status_str(st))
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            lib.msa_index_score_ex(*a)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(kv_np)
    ms_one = timed(np.ones(B, dtype=np.int64))
    st = decode_batch_stats(kv_np, Hq, Hkv, D, P, MB, 2)
    gbs = st["bytes"] / (ms * 1e-3) / 1e9
    fam = "decode" if m.msa_index_score_kernel_family(B, B, Hq, Hkv) == 0 else "prefill"
    del key, out
    torch.cuda.empty_cache()
    return {"metric": "decode batch scaling", "config": {
                "workload": f"decode_bbnd_bf16 distribution at B={B}", "B": B, "Hq": Hq,
                "Hkv": Hkv, "D": D, "P": P, "MB": MB, "pages": NP, "kernel_family": fam,
                "data": "synthetic, keys drawn on the GPU"},
            "steps": steps, "warmup": warmup,
            "kernel_ms_avg": round(ms, 5), "us_per_request": round(ms * 1e3 / B, 4),
            "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": st["bytes"], "block_scores": st["scores"],
            "kv_len_1_kernel_ms_avg": round(ms_one, 5),
            "kv_len_1_us_per_request": round(ms_one * 1e3 / B, 4)}


def workload_summary(r: dict) -> dict:
    """One workload's figures for the headline line's 'workloads' list."""
    keys = ("value", "unit", "ms_per_step", "dtype", "hbm_gbs", "mfma_tflops",
            "block_scores_per_step", "out_entries_per_step", "roofline", "cpu_baseline", "topk",
            "launch", "eager", "graph")
    out = {"workload": r["config"]["workload"], "config": r["config"]}
    out.update({k: r[k] for k in keys if k in r})
    out["kernel_ms_avg"] = r["roofline"]["kernel_ms_avg"]
    out["latency_us"] = round(r["roofline"]["kernel_ms_avg"] * 1e3, 2)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="default",
                    help="'default': the headline decode line with every workload (the "
                         "five base ones and three MXFP4 variants) measured in the same "
                         "process under 'workloads'; or a workload "
                         "name or index, 'all' (one line per base workload) or 'mx' (their "
                         "MXFP4 variants)")
    ap.add_argument("--copies", type=int, default=0,
                    help="key-cache copies to rotate over (0: 4 for the decode workloads, "
                         "so that the 256 MB Infinity Cache cannot serve a step from the "
                         "one before; 1 otherwise)")
    ap.add_argument("--family", type=int, default=-1, help="-1 auto, 0 decode, 1 prefill tiles")
    ap.add_argument("--graph", action="store_true",
                    help="time the K launches as one replay of a HIP graph that holds them "
                         "instead of a loop of C-ABI calls from Python (each line reports "
                         "the other way's figures too)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=256,
                    help="whole output rows of a prefill workload the oracle computes for "
                         "its CPU baseline")
    ap.add_argument("--topk", action="store_true",
                    help="time the top-k block selection on the workload's scores instead")
    ap.add_argument("--cpu-topk-rows", type=int, default=200000)
    ap.add_argument("--local-mode", choices=["request", "query"], default="request",
                    help="local_mask window at start_loc (the workloads' own setting) or at "
                         "each token's own block")
    ap.add_argument("--decode-batch", default="",
                    help="comma-separated batch sizes: time the bf16 decode workload's "
                         "distribution at each (batch scaling of the request lookup)")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="instead of the operator, run this many MiB device copies "
                         "(counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every block score is independent, so the "
              "operator shards across GPUs with no exchange and there is no multi-GPU step "
              "to time; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.calib_copy:
        n = args.calib_copy * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": max(args.steps, 1)}))
        return

    if args.decode_batch:
        for b in [int(x) for x in args.decode_batch.split(",") if x]:
            print(f"[bench] decode batch {b}", file=sys.stderr, flush=True)
            print(json.dumps(bench_decode_batch(b, args.steps, args.warmup)), flush=True)
        return

    import synth
    names = list(synth.CONFIG_NAMES) + list(synth.MX_CONFIG_NAMES)
    local_mode = 1 if args.local_mode == "query" else 0
    if args.config == "default":
        host = host_cpu() if not args.no_cpu_baseline else None
        recs = []
        for c, name in enumerate(names):
            copies = args.copies if args.copies > 0 else (4 if name.startswith("decode") else 1)
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            base = c < len(synth.CONFIG_NAMES)
            recs.append(bench_config(c, args.steps, args.warmup, copies, args.family,
                                     not args.no_cpu_baseline, args, local_mode=local_mode,
                                     topk=base and name.startswith("prefill"), host=host))
        head = dict(next(r for r in recs if r["config"]["workload"] == HEADLINE))
        head["workloads"] = [workload_summary(r) for r in recs]
        print(json.dumps(head), flush=True)
        return
    if args.config == "all":
        todo = list(range(len(synth.CONFIG_NAMES)))
    elif args.config == "mx":
        todo = list(range(len(synth.CONFIG_NAMES), len(names)))
    elif args.config.isdigit():
        todo = [int(args.config)]
    else:
        todo = [names.index(args.config)]
    for c in todo:
        if args.topk and c >= len(synth.CONFIG_NAMES):
            print("--topk runs on the five base workloads", file=sys.stderr)
            sys.exit(2)
        if args.topk:
            print(json.dumps(bench_topk(c, args.steps, args.warmup, not args.no_cpu_baseline,
                                        args)), flush=True)
            continue
        copies = args.copies
        if copies <= 0:
            copies = 4 if names[c].startswith("decode") else 1
        r = bench_config(c, args.steps, args.warmup, copies, args.family,
                         not args.no_cpu_baseline, args, local_mode=local_mode)
        print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
