"""Throughput of exact attention (forward + backward) on one MI355X.

One step = the whole hot path over one batch of synthetic input: fa_fwd, then
the backward launch sequence (rowsum(dO*O), the dK/dV kernel, the dQ kernel)
through fa_bwd_ex, all on torch's current stream.  Prints ONE JSON line on stdout.

  value      whole-step TFLOP/s, FLOPs counted as 4*B*H*N^2*d for the forward
             (halved when causal) and 2.5x that for the backward, over the
             wall-clock time of the timed steps (inputs resident in HBM).
             Workloads with key padding or a block mask count 4d per visible
             (query, key) pair instead (and also report the dense-equivalent
             rate, labelled as such).
  roofline   the kernel with the largest average duration: algorithmic FLOPs
             of one launch over its average duration from HIP events recorded
             on the launch stream around every timed launch; per visible
             (query, key) pair: forward 4d (S, PV), backward dK/dV kernel 8d
             (S, dP, dV, dK), backward dQ kernel 2d (dQ; it also recomputes S
             and dP, 4d more, reported apart as executed MFMA work); peak =
             dense bf16/fp16 MFMA 2516.6 TFLOP/s.  `traffic` comes from the
             committed rocprofv3 counter summary when it was taken on the
             current kernel sources, else null.
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload.

A forward-only (decoding) workload is timed as one split-KV forward per step
(fa_fwd_splitkv with the library's split count): value = algorithmic HBM
bytes (Q, K, V read; O, LSE written) per second, roofline bound "hbm" on the
split forward kernel.

--dropout P runs the same step with fused dropout (probability P, Philox
counter offset = step index, as a training loop would advance it); FLOPs are
counted as without dropout (the keep decisions are not matrix work).
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
MIN_WARMUP_S = 0.3  # minimum untimed warm-up before a timed region (see time_attention)
DEFAULT_WORKLOAD = "long_causal_n16k"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources the attention kernels of a step (forward, backward, split-KV
# forward and its merge) and their launches are built from; the row
# reductions, the shard merge and the allocation-free entry point are not.
STEP_SOURCES = ("fa_api.cpp", "fa_bwd.hip", "fa_device.hpp", "fa_dropout.hpp", "fa_fwd.hip",
                "fa_internal.hpp")


def kernel_source_hash() -> str:
    """sha256 over STEP_SOURCES and include/fa.h."""
    csrc = os.path.join(ROOT, "exact_io_aware_33_amd", "csrc")
    h = hashlib.sha256()
    for name in STEP_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "fa.h"), "rb").read())
    return h.hexdigest()


def visible_pairs(w, key_lens=None, block_mask=None) -> int:
    """Number of (query, key) pairs no mask removes, summed over batch and heads
    (causal: key j visible to query i iff j <= i + N_k - N_q)."""
    import numpy as np
    Nq, Nk = w.N, w.Nk
    cs = Nk - Nq if w.causal else None
    if w.mb is not None:
        if key_lens is not None:
            raise NotImplementedError("block mask combined with key padding")
        bmk = np.asarray(block_mask).astype(bool)
        mb = w.mb
        if cs is None:
            per_head = int(bmk.sum()) * mb * mb
        else:
            # pairs of block (I, J) under the causal rule depend on
            # delta = I mb - J mb + cs only: sum over its rows r of
            # clamp(delta + r + 1, 0, mb)
            I, J = np.nonzero(bmk)
            delta = (I - J) * mb + cs
            r = np.arange(mb)
            per_head = 0
            for dl, cnt in zip(*np.unique(delta, return_counts=True)):
                per_head += int(cnt) * int(np.clip(dl + r + 1, 0, mb).sum())
        return per_head * w.B * w.H
    total = 0
    i = np.arange(Nq, dtype=np.int64)
    for b in range(w.B):
        L = Nk if key_lens is None else max(0, min(Nk, int(key_lens[b])))
        if cs is not None:
            pairs = int(np.clip(i + cs + 1, 0, L).sum())
        else:
            pairs = Nq * L
        total += pairs * w.H
    return total


def headline_count(w) -> bool:
    """Whether the metric's own FLOP count applies: a square problem whose
    only mask is (optionally) causal."""
    return w.N == w.Nk and w.lens is None and w.mb is None


def forward_flops(w, pairs) -> float:
    """Forward FLOPs of one step: the metric's 4 B H N^2 d (halved when
    causal) for a square dense or causal problem; 4 d per visible (query, key)
    pair whenever padding, a block mask or N_q != N_k removes pairs (the
    dense count would credit work that is never done)."""
    if headline_count(w):
        return 4.0 * w.B * w.H * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    return 4.0 * w.d * pairs


def dense_equivalent_flops(w) -> float:
    """4 B H N_q N_k d: what the same shape would cost with every (query,
    key) pair visible, for context on masked workloads only."""
    return 4.0 * w.B * w.H * w.N * w.Nk * w.d


def traffic_from_profile(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, or None."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k["fetch_bytes"] + k["write_bytes"]


def cpu_baseline(w, inputs, budget_heads=1, dropout=None):
    """The oracle as it stands, timed on this host on one (batch, head) of the
    workload (full N, forward + backward)."""
    import numpy as np

    import oracle
    from exact_io_aware_33_amd.inputs import as_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max((int(i.get("num_threads", 1)) for i in threadpool_info()), default=1)
    except Exception:  # threadpoolctl missing: fall back to the environment
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    sl = (slice(0, 1), slice(0, budget_heads))
    pairs_head = visible_pairs(w, None if inputs["key_lens"] is None else inputs["key_lens"].numpy(),
                               None if inputs["block_mask"] is None else inputs["block_mask"].numpy()
                               ) / (w.B * w.H)
    q, k, v, do = (as_f64(inputs[n][sl]) for n in ("q", "k", "v", "do"))
    lens = None if inputs["key_lens"] is None else inputs["key_lens"].numpy()[:1]
    bm = None if inputs["block_mask"] is None else inputs["block_mask"].numpy()
    t0 = time.perf_counter()
    oracle.backward(q, k, v, do, w.scale, causal=w.causal, key_lens=lens, block_mask=bm,
                    mb=w.mb or 128, dropout=dropout)
    dt = time.perf_counter() - t0
    flops_fwd = forward_flops(w, pairs_head * w.B * w.H) / (w.B * w.H) * budget_heads
    return {"value": round(3.5 * flops_fwd / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": f"1 batch x {budget_heads} head(s) of {w.name} (N_q={w.N}, N_k={w.Nk}, d={w.d}), "
                      f"fp64 numpy two-pass forward + analytic backward"
                      f"{'' if dropout is None else f' with dropout p={dropout[0]}'}, {dt:.1f} s; "
                      f"host os.cpu_count()={os.cpu_count()}"}


def warm_up(fn, n):
    """n untimed calls of fn, then more until MIN_WARMUP_S has passed (the
    shader clock settles under load; see time_attention).  Returns the number
    of extra calls."""
    import torch
    t_w = time.perf_counter()
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    extra = 0
    while time.perf_counter() - t_w < MIN_WARMUP_S:
        fn()
        extra += 1
        if extra % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return extra


def calibration_copy(args, dev):
    """One device-to-device copy of known size, for scaling the HBM counters."""
    if not args.copy_calibration_mib:
        return
    import torch
    n = args.copy_calibration_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done")
    del src, dst


def compulsory_bytes(w, kernel):
    """Bytes a kernel must move at least (each input read once, each output
    written once), for the whole launch: the forward reads Q, K, V and writes
    O and the LSE; the dK/dV pass reads Q, K, V, dO and two floats per query
    row and writes dK, dV; the dQ pass (with the preprocessing of its rows)
    reads Q, K, V, dO, O and the LSE and writes dQ and two floats per row."""
    e = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    bh = w.B * w.H
    q_side, k_side = bh * w.N * w.d * e, bh * w.Nk * w.d * e
    rows = bh * w.N
    if kernel == "fwd_kernel":
        return 2 * q_side + 2 * k_side + 4 * rows
    if kernel == "bwd_main_kernel":
        return 2 * q_side + 4 * k_side + 8 * rows
    return 4 * q_side + 2 * k_side + 12 * rows


def attainable(flops, nbytes, peak_tflops, achieved_tflops):
    """The attainable rate min(MFMA peak, AI x HBM bandwidth) for the kernel's
    arithmetic intensity AI = algorithmic FLOPs / compulsory bytes, and the
    achieved rate as a fraction of it."""
    ai = flops / nbytes
    att = min(peak_tflops, ai * HBM_PEAK_GBS / 1e3)
    return {"arithmetic_intensity": round(ai, 1), "attainable": round(att, 1),
            "frac_of_attainable": round(achieved_tflops / att, 4)}


def gemm_reference(dtype, dev, n=8192, iters=20):
    """TFLOP/s of a plain n^3 matrix product in `dtype` through torch.matmul
    (the vendor GEMM library) on standard-normal operands, timed right after
    the attention step (clock already settled).  The matrix cores' rate
    depends on the data as well as on the instruction stream (the chip is
    power-limited under dense MFMA work; the same product on zeros runs about
    1.35x faster), so this is the practical ceiling for dense 16-bit MFMA work
    on data like the benchmark's -- context for the roofline, not its peak."""
    import torch
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(dtype)
    if dt is None:
        return None
    g = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(n, n, device=dev, dtype=dt, generator=g)
    b = torch.randn(n, n, device=dev, dtype=dt, generator=g)

    def rate(x, y):
        c = x @ y
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:  # the clock settles on the new load
            c = x @ y
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            c = x @ y
        e1.record()
        torch.cuda.synchronize()
        del c
        return 2.0 * n ** 3 / (e0.elapsed_time(e1) / iters * 1e-3) / 1e12

    t_rand = rate(a, b)
    a.zero_()
    t_zero = rate(a, a)
    del a, b
    return {"op": f"torch.matmul {dtype} {n}x{n}x{n}, standard-normal operands",
            "tflops": round(t_rand, 1), "tflops_zero_operands": round(t_zero, 1)}


def decode_main(args, w, dev):
    """One split-KV forward per step on a forward-only (decoding) workload."""
    import numpy as np
    import torch

    from exact_io_aware_33_amd import (fa_fwd_splitkv, fa_fwd_splitkv_num_splits,
                                       fa_fwd_splitkv_workspace_bytes)
    from exact_io_aware_33_amd.inputs import make_workload_inputs

    log(f"[bench] workload {w.name}: B={w.B} H={w.H} N_q={w.N} N_k={w.Nk} d={w.d} {w.dtype} "
        f"causal={w.causal} (forward only, split-KV)")
    inputs = make_workload_inputs(w, seed=0)
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    calibration_copy(args, dev)
    splits = fa_fwd_splitkv_num_splits(q, k, scale=w.scale, causal=w.causal)
    ws = torch.empty(fa_fwd_splitkv_workspace_bytes(q, k, splits, scale=w.scale, causal=w.causal),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        fa_fwd_splitkv(q, k, v, num_splits=splits, scale=w.scale, causal=w.causal, workspace=ws,
                       out=o, lse=lse)

    warm_up(step, args.warmup)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        events[i][0].record(stream)
        step()
        events[i][1].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    e = q.element_size()
    alg_bytes = (2 * w.B * w.H * w.Nk * w.d + 2 * w.B * w.H * w.N * w.d) * e + 4 * w.B * w.H * w.N
    value = alg_bytes / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes / (ev_ms * 1e-3) / 1e9
    log(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step (events {ev_ms:.4f} ms), "
        f"{splits} splits")
    out = {
        "metric": "decode attention HBM GB/s (split-KV forward)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "N_k": w.Nk, "d": w.d,
                   "causal": w.causal, "num_splits": splits},
        "roofline": {"kernel": "fwd_kernel (split) + splitkv_merge_kernel", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (None if traffic_from_profile(w.name, "fwd_kernel") is None
                                 or traffic_from_profile(w.name, "splitkv_merge_kernel") is None
                                 else traffic_from_profile(w.name, "fwd_kernel")
                                 + traffic_from_profile(w.name, "splitkv_merge_kernel")),
                     "bytes_per_launch": alg_bytes, "avg_launch_ms": round(ev_ms, 4)},
    }
    print(json.dumps(out), flush=True)


def time_attention(args, w, dev, steps, warmup):
    """Time `steps` whole steps of workload `w` after `warmup` untimed ones.

    Returns the inputs, the wall-clock ms per step and the HIP-event averages
    (ms) of the forward, of the dQ pass (with the preprocessing of its rows:
    one call with FA_BWD_PRE | FA_BWD_DQ) and of the dK/dV pass -- the launch
    sequence of fa_bwd, split in two calls so each is timed."""
    import numpy as np
    import torch

    from exact_io_aware_33_amd import fa_fwd
    from exact_io_aware_33_amd.inputs import make_workload_inputs

    log(f"[bench] workload {w.name}: B={w.B} H={w.H} N_q={w.N} N_k={w.Nk} d={w.d} {w.dtype} "
        f"causal={w.causal}")
    inputs = make_workload_inputs(w, seed=0)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    kl = None if inputs["key_lens"] is None else inputs["key_lens"].to(dev)
    bm = None if inputs["block_mask"] is None else inputs["block_mask"].to(dev)
    calibration_copy(args, dev)

    from exact_io_aware_33_amd import (FA_BWD_DQ, FA_BWD_MAIN, FA_BWD_PRE, fa_bwd_ex,
                                       fa_bwd_workspace_bytes, fa_fwd_blocksparse)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    ws = torch.empty(fa_bwd_workspace_bytes(q, k, scale=w.scale, causal=w.causal, key_lens=kl),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    common = dict(scale=w.scale, causal=w.causal, key_lens=kl)
    drop_seed = 0x5EED

    qt = dict(query_tile=getattr(args, "query_tile", 0))

    def fwd(i):
        dr = dict(dropout_p=args.dropout, dropout_seed=drop_seed, dropout_offset=i)
        if bm is None:
            fa_fwd(q, k, v, out=o, lse=lse, **common, **dr, **qt)
        else:
            fa_fwd_blocksparse(q, k, v, bm, mask_block=w.mb, out=o, lse=lse, **common, **dr, **qt)

    def bwd(stage, i):
        dr = dict(dropout_p=args.dropout, dropout_seed=drop_seed, dropout_offset=i)
        fa_bwd_ex(q, k, v, o, lse, do, stage, block_mask=bm, mask_block=w.mb or 128,
                  workspace=ws, dq=dq, dk=dk, dv=dv, **common, **dr)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        fwd(i)
        if ev is not None:
            ev[1].record(stream)
        bwd(FA_BWD_PRE | FA_BWD_DQ, i)
        if ev is not None:
            ev[2].record(stream)
        bwd(FA_BWD_MAIN, i)
        if ev is not None:
            ev[3].record(stream)

    # The W warm-up steps asked for, then more until at least MIN_WARMUP_S of
    # warm-up has run: the shader clock takes ~0.1-0.2 s of load to settle,
    # and a timed region that starts cold reads up to ~15% slow on the small
    # problems (measured: the same steps timed again right after, or as a
    # replayed HIP graph, run at the settled rate).
    t_w = time.perf_counter()
    extra = 0
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    while time.perf_counter() - t_w < MIN_WARMUP_S:
        step(warmup + extra)
        extra += 1
        if extra % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    time_attention.extra_warmup = extra
    log(f"[bench] warmup {warmup} steps (+{extra} to reach {MIN_WARMUP_S} s) done")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    # The per-launch breakdown: as many steps again, with HIP events between
    # the launches.  Kept out of the timed region above: at the small
    # problems the events themselves add ~10 us to a step.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(warmup + steps + i, events[i])
    torch.cuda.synchronize()
    per = {"fwd": [e[0].elapsed_time(e[1]) for e in events],
           "bwd_dq": [e[1].elapsed_time(e[2]) for e in events],
           "bwd_main": [e[2].elapsed_time(e[3]) for e in events]}
    fwd_ms, dq_ms, main_ms = (float(np.mean(per[n])) for n in ("fwd", "bwd_dq", "bwd_main"))
    time_attention.spread = {"kernel_ms_median": {n: round(float(np.median(v)), 4) for n, v in per.items()},
                             "kernel_ms_min": {n: round(float(np.min(v)), 4) for n, v in per.items()}}
    log(f"[bench] timed {steps} steps: {ms_step:.3f} ms/step; fwd {fwd_ms:.3f} ms, "
        f"bwd dq (with the preprocessing) {dq_ms:.3f} / main {main_ms:.3f} ms")

    if getattr(args, "cold", False):
        # Cold caches: before each of K more steps, 512 MiB written to a
        # scratch buffer (twice the 256 MB MALL, far more than the L2s), so
        # the step finds none of its inputs cached.  Events around each step
        # only, so the flush is not timed.
        flush = torch.empty(512 << 18, dtype=torch.float32, device=dev)
        cold = []
        for i in range(steps):
            flush.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(warmup + 2 * steps + i)
            e1.record(stream)
            cold.append((e0, e1))
        torch.cuda.synchronize()
        time_attention.cold_ms = float(np.mean([a.elapsed_time(b) for a, b in cold]))
        del flush
        log(f"[bench] cold caches: {time_attention.cold_ms:.3f} ms/step")

    if getattr(args, "graph", False):
        # The same step recorded once into a HIP graph and replayed: what the
        # four launches cost without the host's per-launch work.  Eager and
        # graph blocks of `steps` steps alternate three times (so neither
        # profits from a clock the other warmed up); medians are reported.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(0)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        eager, graph = [], []
        for _ in range(3):
            t0 = time.perf_counter()
            for i in range(steps):
                step(i)
            torch.cuda.synchronize()
            eager.append((time.perf_counter() - t0) * 1e3 / steps)
            t0 = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            graph.append((time.perf_counter() - t0) * 1e3 / steps)
        time_attention.graph_ms = float(np.median(graph))
        time_attention.eager_alt_ms = float(np.median(eager))
        log(f"[bench] interleaved: eager {time_attention.eager_alt_ms:.3f} / graph "
            f"{time_attention.graph_ms:.3f} ms/step")
    return inputs, ms_step, fwd_ms, main_ms, dq_ms


def sweep_main(args, dev):
    """The metric's sequence-length sweep: bf16, d=64, H=16, B=16384/N (the
    same number of tokens at every N), N = 1K..16K, causal and not.  Forward
    TFLOP/s from the forward's HIP events, fwd+bwd TFLOP/s from the wall clock
    of whole steps, FLOPs by the headline count (4 B H N^2 d forward, halved
    when causal; backward 2.5x).  Each point times --steps x 16384/N steps
    (and as many more warm-up steps), so every point runs for about as long."""
    from exact_io_aware_33_amd.inputs import Workload

    rows = []
    for causal in (False, True):
        for N in (1024, 2048, 4096, 8192, 16384):
            w = Workload(f"sweep_n{N}_{'causal' if causal else 'full'}", 16384 // N, 16, N, 64,
                         "bf16", causal=causal)
            # at least ~10 steps' worth of the 16K problem per point, so the
            # short problems are not timed over a few milliseconds only
            reps = max(1, 16384 // N)
            _, ms_step, fwd_ms, main_ms, dq_ms = time_attention(
                args, w, dev, args.steps * reps, args.warmup * reps)
            f_fwd = forward_flops(w, None)
            rows.append({"N": N, "B": w.B, "H": w.H, "causal": causal,
                         "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 1),
                         "bwd_tflops": round(2.5 * f_fwd / ((main_ms + dq_ms) * 1e-3) / 1e12, 1),
                         "fwd_bwd_tflops": round(3.5 * f_fwd / (ms_step * 1e-3) / 1e12, 1),
                         "ms_per_step": round(ms_step, 4),
                         **({"graph_fwd_bwd_tflops": round(
                             3.5 * f_fwd / (time_attention.graph_ms * 1e-3) / 1e12, 1),
                             "eager_fwd_bwd_tflops_interleaved": round(
                             3.5 * f_fwd / (time_attention.eager_alt_ms * 1e-3) / 1e12, 1)}
                            if args.graph else {}),
                         "kernel_ms": {"fwd": round(fwd_ms, 4), "bwd_main": round(main_ms, 4),
                                       "bwd_dq": round(dq_ms, 4)}})
            log(f"[bench] sweep {rows[-1]}")
    print(json.dumps({"metric": "attention TFLOP/s fwd & fwd+bwd, N=1K-16K d=64 bf16; % of MFMA peak",
                      "unit": "TFLOP/s", "peak": MFMA_PEAK_TFLOPS["bf16"], "steps": args.steps,
                      "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
                      "sweep": rows}), flush=True)


def tile_sweep_main(args, dev):
    """The forward at B_r = 64, 128 and 256 queries per workgroup (2, 4 and 8
    wavefronts) on the same inputs: bf16, d = 64, B = 1, H = 16, non-causal,
    N = 8K, 16K and 32K.  Each (N, B_r) point is its own kernel instance
    (template argument W = B_r / 32), so a rocprofv3 counter run of this mode
    gives FETCH_SIZE per launch against B_r: the tile model's K / V re-read
    term, 2 N^2 d e / B_r per head, scales as 1 / B_r unless the L2 holds the
    K / V of a head (summary page, Complexity analysis: Theta(N^2 d^2 / M)).
    Forward TFLOP/s from HIP events around each timed launch."""
    import numpy as np
    import torch

    from exact_io_aware_33_amd import fa_fwd
    from exact_io_aware_33_amd.inputs import make_inputs

    calibration_copy(args, dev)
    rows = []
    stream = torch.cuda.current_stream(dev)
    for N in (8192, 16384, 32768):
        inp = make_inputs(1, 16, N, 64, "bf16", seed=0, with_do=False)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        flops = 4.0 * 16 * N * N * 64
        for qt in (64, 128, 256):
            def run():
                fa_fwd(q, k, v, out=o, lse=lse, query_tile=qt)
            warm_up(run, args.warmup)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for a, b in ev:
                a.record(stream)
                run()
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
            rows.append({"N": N, "B_r": qt, "grid_workgroups": 16 * ((N + qt - 1) // qt),
                         "fwd_ms": round(ms, 4), "fwd_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                         "tile_model_kv_reread_bytes": 16 * 2 * N * 64 * 2 * ((N + qt - 1) // qt)})
            log(f"[bench] tile sweep {rows[-1]}")
        del q, k, v, o, lse
    print(json.dumps({"mode": "tile_sweep", "B": 1, "H": 16, "d": 64, "dtype": "bf16", "causal": False,
                      "steps": args.steps, "rows": rows}), flush=True)


def ring_main(args, dev):
    """One device's share of context-parallel (ring) attention at the per-hop
    shape: bf16, d = 64, B = 1, H = 16, 16K local queries, 4 visiting K / V
    shards of 16K keys (64K keys in all), non-causal.  Times (HIP events on
    the stream) each hop's forward (fa_fwd, 16K x 16K), the merge of the 4
    partial (O_s, LSE_s) (fa_merge_partials), each hop's backward with the
    merged O and LSE (fa_bwd), and, for comparison, one fa_fwd over all 64K
    keys.  The merge is HBM-bound: its algorithmic bytes are the S parts' O_s
    and LSE_s read and O, LSE written."""
    import numpy as np
    import torch

    from exact_io_aware_33_amd import fa_bwd, fa_fwd, fa_merge_partials
    from exact_io_aware_33_amd.inputs import make_inputs

    S, Ns, Nq, H, d = 4, 16384, 16384, 16, 64
    inp = make_inputs(1, H, Nq, d, "bf16", seed=0, n_keys=S * Ns)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    # each visiting shard in a buffer of its own, as it arrives from a peer
    ks = [k[:, :, s * Ns:(s + 1) * Ns].contiguous() for s in range(S)]
    vs = [v[:, :, s * Ns:(s + 1) * Ns].contiguous() for s in range(S)]
    o_parts = [torch.empty_like(q) for _ in range(S)]
    l_parts = [torch.empty(q.shape[:3], dtype=torch.float32, device=dev) for _ in range(S)]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    grads = [(torch.empty_like(q), torch.empty_like(ks[0]), torch.empty_like(ks[0])) for _ in range(S)]
    ws = torch.empty(16 * Nq * 8 + 1024, dtype=torch.uint8, device=dev)
    o_all = torch.empty_like(q)
    lse_all = torch.empty_like(lse)
    stream = torch.cuda.current_stream(dev)

    def hop_fwd(s):
        fa_fwd(q, ks[s], vs[s], out=o_parts[s], lse=l_parts[s])

    def merge():
        fa_merge_partials(o_parts, l_parts, out=o, lse=lse)

    def hop_bwd(s):
        fa_bwd(q, ks[s], vs[s], o, lse, do, workspace=ws, dq=grads[s][0], dk=grads[s][1], dv=grads[s][2])

    def whole():
        fa_fwd(q, k, v, out=o_all, lse=lse_all)

    def step():
        for s in range(S):
            hop_fwd(s)
        merge()
        for s in range(S):
            hop_bwd(s)

    warm_up(step, args.warmup)
    warm_up(whole, args.warmup)
    names = ["hop_fwd", "merge", "hop_bwd", "fwd_all_keys"]
    times = {n: [] for n in names}
    for _ in range(args.steps):
        evs = []
        for fn in ([lambda: hop_fwd(0)], [merge], [lambda: hop_bwd(0)], [whole]):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn[0]()
            b.record(stream)
            evs.append((a, b))
        for s in range(1, S):  # keep every hop's partial fresh for the merge
            hop_fwd(s)
        torch.cuda.synchronize()
        for n, (a, b) in zip(names, evs):
            times[n].append(a.elapsed_time(b))
    ms = {n: float(np.mean(t)) for n, t in times.items()}
    hop_flops = 4.0 * H * Nq * Ns * d
    rows = Nq * H
    merge_bytes = S * rows * (d * 2 + 4) + rows * (d * 2 + 4)
    out = {"mode": "ring", "shape": {"H": H, "d": d, "dtype": "bf16", "local_queries": Nq, "shards": S,
                                     "keys_per_shard": Ns, "causal": False},
           "steps": args.steps,
           "hop_fwd_ms": round(ms["hop_fwd"], 4), "hop_fwd_tflops": round(hop_flops / (ms["hop_fwd"] * 1e-3) / 1e12, 1),
           "hop_bwd_ms": round(ms["hop_bwd"], 4),
           "hop_bwd_tflops": round(2.5 * hop_flops / (ms["hop_bwd"] * 1e-3) / 1e12, 1),
           "merge_ms": round(ms["merge"], 4), "merge_bytes": merge_bytes,
           "merge_GBs": round(merge_bytes / (ms["merge"] * 1e-3) / 1e9, 1),
           "fwd_all_keys_ms": round(ms["fwd_all_keys"], 4),
           "ring_fwd_vs_one_call": round((S * ms["hop_fwd"] + ms["merge"]) / ms["fwd_all_keys"], 4),
           "xgmi_hop_bytes_per_head": 2 * Ns * d * 2}
    log(f"[bench] ring {out}")
    print(json.dumps(out), flush=True)


def reductions_main(args, dev):
    """The other streaming reductions: each case is timed with HIP events on
    the launch stream over `steps` launches; achieved = algorithmic bytes (read
    x and gamma / beta once, write y and the fp32 per-row statistics) over the
    average launch duration, against the 8 TB/s HBM peak.  Beside each case, a
    plain device copy of the same read + write volume (torch's copy_) is timed
    the same way, as the rate this GPU reaches in practice."""
    import numpy as np
    import torch

    from exact_io_aware_33_amd import fa_layernorm_rows, fa_softmax_rows

    calibration_copy(args, dev)
    g = torch.Generator(device="cpu").manual_seed(0)
    cases = [
        ("softmax_rows_16k_x_32k_bf16", "softmax", 16384, 32768, torch.bfloat16, 1, 1),
        ("softmax_rows_256k_x_64_f32", "softmax", 262144, 64, torch.float32, 1, 1),
        ("layernorm_64k_x_4096_bf16", "layernorm", 65536, 4096, torch.bfloat16, 1, 1),
        ("groupnorm_n32_c512_s4096_g32_bf16", "layernorm", 32 * 32, 16 * 4096, torch.bfloat16,
         32, 4096),
    ]
    rows_out = []
    stream = torch.cuda.current_stream(dev)
    for name, kind, R, L, dt, groups, inner in cases:
        x = torch.randn(R, L, generator=g, dtype=torch.float32).to(dt).to(dev)
        y = torch.empty_like(x)
        stat1 = torch.empty(R, dtype=torch.float32, device=dev)
        stat2 = torch.empty(R, dtype=torch.float32, device=dev)
        e = x.element_size()
        if kind == "softmax":
            def run():
                fa_softmax_rows(x, out=y, lse=stat1)
            nbytes = 2 * R * L * e + 4 * R
        else:
            nch = groups * (L // inner)
            gamma = torch.randn(nch, generator=g).to(dt).to(dev)
            beta = torch.randn(nch, generator=g).to(dt).to(dev)

            def run():
                fa_layernorm_rows(x, gamma, beta, groups=groups, inner=inner, out=y,
                                  mean=stat1, rstd=stat2)
            nbytes = 2 * R * L * e + 2 * nch * e + 8 * R
        warm_up(run, args.warmup)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            run()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        gbs = nbytes / (ms * 1e-3) / 1e9
        # the same read + write volume as a plain device copy: the practical ceiling
        for a, b in ev:
            a.record(stream)
            y.copy_(x)
            b.record(stream)
        torch.cuda.synchronize()
        copy_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        copy_gbs = 2 * R * L * e / (copy_ms * 1e-3) / 1e9
        rows_out.append({"case": name, "rows": R, "cols": L, "dtype": str(dt).split(".")[-1],
                         "groups": groups, "inner": inner, "avg_launch_ms": round(ms, 4),
                         "alg_bytes": nbytes, "achieved_GBs": round(gbs, 1),
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "device_copy_GBs": round(copy_gbs, 1),
                         "frac_of_copy": round(gbs / copy_gbs, 4)})
        log(f"[bench] {rows_out[-1]}")
        del x, y
    print(json.dumps({"metric": "streaming reductions, HBM GB/s of algorithmic bytes",
                      "unit": "GB/s", "peak": HBM_PEAK_GBS, "bound": "hbm", "steps": args.steps,
                      "warmup": args.warmup, "data": "synthetic", "cases": rows_out}), flush=True)


def standard_contrast_main(args, dev):
    """Standard attention next to this library's step on the same inputs:
    B=1, H=16, d=64, bf16, non-causal, N = 2K, 4K, 8K (or the one N of
    --contrast-n).  Standard attention here is the textbook sequence with
    every N x N matrix in HBM -- S = scale Q K^T and P = softmax(S) (fp32
    softmax, P stored in bf16), O = P V; backward dV = P^T dO, dP = dO V^T,
    dS = P (dP - D), dQ = dS K, dK = dS^T Q -- as plain torch batched
    products on contiguous operands.  Both run a fixed number of steps
    (warm-up + timed, printed), so a counter run of one N divides its HBM
    bytes by that count: the contrast the pages draw between standard and
    IO-aware attention, measured."""
    import numpy as np
    import torch

    from exact_io_aware_33_amd import fa_bwd, fa_fwd

    ns = (args.contrast_n,) if args.contrast_n else (2048, 4096, 8192)
    B, H, d = 1, 16, 64
    scale = 1.0 / math.sqrt(d)
    calibration_copy(args, dev)
    rows = []
    for N in ns:
        g = torch.Generator().manual_seed(N)
        q, k, v, do = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev) for _ in range(4))
        q3, k3, v3, do3 = (t.reshape(B * H, N, d).contiguous() for t in (q, k, v, do))

        def standard():
            s = torch.bmm(q3, k3.transpose(1, 2).contiguous()) * scale
            p = torch.softmax(s.float(), dim=-1).to(torch.bfloat16)
            o = torch.bmm(p, v3)
            dv = torch.bmm(p.transpose(1, 2).contiguous(), do3)
            dp = torch.bmm(do3, v3.transpose(1, 2).contiguous())
            dd = (do3.float() * o.float()).sum(-1, keepdim=True)
            ds = (p.float() * (dp.float() - dd) * scale).to(torch.bfloat16)
            dq = torch.bmm(ds, k3)
            dk = torch.bmm(ds.transpose(1, 2).contiguous(), q3)
            return o, dq, dk, dv

        def ours():
            o, lse = fa_fwd(q, k, v, scale=scale)
            return fa_bwd(q, k, v, o, lse, do, scale=scale)

        res = {"N": N}
        for name, fn in (("standard", standard), ("library", ours)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            res[f"{name}_ms"] = round(float(np.mean([a.elapsed_time(b) for a, b in ev])), 4)
        f = 3.5 * 4.0 * B * H * N * N * d
        res["standard_tflops"] = round(f / (res["standard_ms"] * 1e-3) / 1e12, 1)
        res["library_tflops"] = round(f / (res["library_ms"] * 1e-3) / 1e12, 1)
        res["nxn_bytes_per_matrix"] = B * H * N * N * 2
        res["steps_run_each"] = args.warmup + args.steps
        rows.append(res)
        log(f"[bench] contrast {res}")
        del q, k, v, do, q3, k3, v3, do3
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "standard_contrast", "B": B, "H": H, "d": d, "dtype": "bf16", "causal": False,
                      "rows": rows}), flush=True)


def scaling_main(args, dev):
    """One head count, growing N: B=1, H=16, d=64, bf16, non-causal, N = 2K,
    4K, 8K, 16K, 32K.  Each N has its own grid size, so a rocprofv3 counter
    run of this mode gives each kernel's HBM bytes as a function of N (the
    pages' claim: Theta(N^2 d^2 / M) for the tiled method, against N^2 for
    standard attention)."""
    from exact_io_aware_33_amd.inputs import Workload

    rows = []
    for N in (2048, 4096, 8192, 16384, 32768):
        w = Workload(f"scaling_n{N}", 1, 16, N, 64, "bf16")
        _, ms_step, fwd_ms, main_ms, dq_ms = time_attention(args, w, dev, args.steps,
                                                                    args.warmup)
        f_fwd = forward_flops(w, None)
        rows.append({"N": N, "fwd_bwd_tflops": round(3.5 * f_fwd / (ms_step * 1e-3) / 1e12, 1),
                     "kernel_ms": {"fwd": round(fwd_ms, 4), "bwd_main": round(main_ms, 4),
                                   "bwd_dq": round(dq_ms, 4)},
                     "grid_workgroups": 16 * (N // 128)})
        log(f"[bench] scaling {rows[-1]}")
    print(json.dumps({"mode": "scaling", "B": 1, "H": 16, "d": 64, "dtype": "bf16", "causal": False,
                      "rows": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the plain-GEMM rate reported beside the roofline")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="fused dropout probability (0 = none)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line, print the metric's N=1K-16K sweep "
                         "(bf16, d=64, H=16, B=16384/N, causal and not) as one JSON line")
    ap.add_argument("--cold", action="store_true",
                    help="also time steps that each follow a 512 MiB write (no input left in "
                         "the L2s or the MALL; reported as cold_ms_per_step; value stays warm)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed "
                         "(reported as graph_ms_per_step; value stays the eager step)")
    ap.add_argument("--standard-contrast", action="store_true",
                    help="instead of the headline line, time standard attention (every N x N matrix "
                         "in HBM, plain torch products) next to this library's step, N = 2K-8K")
    ap.add_argument("--contrast-n", type=int, default=0,
                    help="with --standard-contrast: only this N (for a counter run per N)")
    ap.add_argument("--scaling", action="store_true",
                    help="instead of the headline line, time fwd+bwd at B=1, H=16, d=64 bf16, "
                         "non-causal, N = 2K..32K (for HBM-byte scaling under rocprofv3 counters)")
    ap.add_argument("--query-tile", type=int, default=0,
                    help="queries per forward workgroup (0 = the library's choice; 64, 128, 256)")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="instead of the headline line, time the forward at B_r = 64 / 128 / 256 "
                         "(bf16, d=64, H=16, non-causal, N = 8K-32K; for FETCH_SIZE against B_r)")
    ap.add_argument("--ring", action="store_true",
                    help="instead of the headline line, time one device's hops of ring attention at the "
                         "per-hop shape (16K queries x 4 shards of 16K keys, bf16, d=64, H=16) and the "
                         "merge of their partial results")
    ap.add_argument("--reductions", action="store_true",
                    help="instead of the headline line, time the row softmax and LayerNorm / "
                         "GroupNorm kernels (HBM-bound) and print one JSON line")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(every (batch, head) is independent, so more GPUs would split B*H with no "
              "communication; that path is not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    from exact_io_aware_33_amd.inputs import WORKLOADS

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.sweep:
        return sweep_main(args, dev)
    if args.reductions:
        return reductions_main(args, dev)
    if args.tile_sweep:
        return tile_sweep_main(args, dev)
    if args.ring:
        return ring_main(args, dev)
    if args.standard_contrast:
        return standard_contrast_main(args, dev)
    if args.scaling:
        return scaling_main(args, dev)
    if not w.backward:
        return decode_main(args, w, dev)
    inputs, ms_step, fwd_ms, main_ms, dq_ms = time_attention(
        args, w, dev, args.steps, args.warmup)

    pairs = visible_pairs(w, None if inputs["key_lens"] is None else inputs["key_lens"].numpy(),
                          None if inputs["block_mask"] is None else inputs["block_mask"].numpy())
    f_fwd = forward_flops(w, pairs)
    f_step = 3.5 * f_fwd
    value = f_step / (ms_step * 1e-3) / 1e12
    # Algorithmic FLOPs per visible pair (the method's own matrix work): the
    # forward's S and PV (4d); the dK/dV kernel's S, dP, dV, dK (8d); the dQ
    # kernel's dQ product (2d).  The dQ kernel also recomputes S and dP (4d
    # more per pair, executed MFMA work but not the method's): reported apart.
    kernels = {
        "fwd_kernel": (fwd_ms, 4.0 * w.d * pairs, 4.0 * w.d * pairs),
        "bwd_main_kernel": (main_ms, 8.0 * w.d * pairs, 8.0 * w.d * pairs),
        "bwd_dq_kernel": (dq_ms, 2.0 * w.d * pairs, 6.0 * w.d * pairs),
    }
    name = max(kernels, key=lambda n: kernels[n][0])
    dur_ms, alg_flops, _ = kernels[name]
    achieved = alg_flops / (dur_ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    alg_step = 14.0 * w.d * pairs  # forward 4d + backward 10d per visible pair
    kernel_tflops = {n: {"algorithmic": round(a / (t * 1e-3) / 1e12, 1),
                         "executed_mfma": round(x / (t * 1e-3) / 1e12, 1)}
                     for n, (t, a, x) in kernels.items()}
    label = w.name if args.dropout == 0.0 else f"{w.name}_dropout{args.dropout:g}"
    traffic = traffic_from_profile(label, name)

    out = {
        "metric": "attention TFLOP/s fwd & fwd+bwd, N=1K-16K d=64 bf16; % of MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "N_k": w.Nk, "d": w.d,
                   "causal": w.causal, "mask_block": w.mb, "key_padding": w.lens is not None,
                   "dropout": args.dropout, "fwd_query_tile": args.query_tile or "library"},
        "flop_count": ("4 B H N^2 d (halved when causal); backward 2.5x" if headline_count(w)
                       else "4 d per visible (query, key) pair; backward 2.5x"),
        "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 3),
        "bwd_tflops": round(2.5 * f_fwd / ((main_ms + dq_ms) * 1e-3) / 1e12, 3),
        "mfma_peak_frac_step": round(alg_step / (ms_step * 1e-3) / 1e12 / peak, 4),
        "bwd_algorithmic_frac": round(10.0 * w.d * pairs / ((main_ms + dq_ms) * 1e-3)
                                      / 1e12 / peak, 4),
        "kernel_tflops": kernel_tflops,
        **({} if headline_count(w) else {"dense_equivalent_tflops": round(
            3.5 * dense_equivalent_flops(w) / (ms_step * 1e-3) / 1e12, 1)}),
        "warmup_extra_steps": time_attention.extra_warmup,
        **({"graph_ms_per_step": round(time_attention.graph_ms, 4),
            "graph_tflops": round(f_step / (time_attention.graph_ms * 1e-3) / 1e12, 3),
            "eager_ms_per_step_interleaved": round(time_attention.eager_alt_ms, 4)}
           if args.graph else {}),
        "kernel_ms": {"fwd": round(fwd_ms, 4), "bwd_main": round(main_ms, 4),
                      "bwd_dq": round(dq_ms, 4)},
        **time_attention.spread,
        **({"cold_ms_per_step": round(time_attention.cold_ms, 4),
            "cold_tflops": round(f_step / (time_attention.cold_ms * 1e-3) / 1e12, 3)}
           if getattr(args, "cold", False) else {}),
        "roofline": {"kernel": name, "bound": "mfma", "achieved": round(achieved, 3),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, "flops_per_launch": alg_flops,
                     "avg_launch_ms": round(dur_ms, 4),
                     **attainable(alg_flops, compulsory_bytes(w, name), peak, achieved)},
    }
    if not args.no_gemm_reference:
        ref = gemm_reference(w.dtype, dev)
        if ref is not None:
            ref["roofline_achieved_frac_of_gemm"] = round(achieved / ref["tflops"], 4)
            out["gemm_reference"] = ref
            log(f"[bench] gemm reference {ref}")
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (cpu_baseline)...")
        out["cpu_baseline"] = cpu_baseline(
            w, inputs, dropout=None if args.dropout == 0.0 else (args.dropout, drop_seed, 0))
        log(f"[bench] cpu_baseline done: {out['cpu_baseline']['value']} TFLOP/s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
