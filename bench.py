"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-naive]

With --workload decode_b8_h32_k16384_d128_bf16 a step is instead one
fa_forward_split call (a decode step: one query row per sequence and head),
and the roofline is HBM bandwidth.  With --workload bwd_b2_h16_n4096_d64_bf16
a step is one fa_backward call (gradients of all heads); with --workload
varlen_b16_h32_hkv8_n8192_d128_bf16 one fa_forward_varlen call over a packed
batch of 16 causal sequences with grouped key/value heads.

A step is one fa_forward call over the whole workload (every batch, head and
query row), with Q, K, V already resident in device memory.  Default
workload: 32 heads, N = 8192, d = 128, causal, bf16 (the shape the pages use
for the 4 GiB score-matrix example).  Prints one JSON line.

Throughput counts useful work only: 4*d flops per visible (query, key) pair
(two products of 2*d flops each); the masked half of a causal problem is
not counted.  `roofline` relates the fused kernel's average duration,
measured with HIP events on the stream it is launched on, to the bf16 dense
MFMA peak of MI355X.  `cpu_baseline` times the fp64 CPU oracle on a bounded
sample of query rows of the same workload on this host's cores.
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

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, 2.4 GHz
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "h32_n8192_d128_causal_bf16"
# Sources of the kernels each kind of workload runs (their hash tags stored
# counter readings, which are reported only for the source they were taken on).
HEADERS = ["fa_bf16_tiles.hpp", "fa_device.hpp", "fa_internal.hpp"]
KERNEL_SOURCES = {
    "forward": ["fa_fwd_bf16.hip", "fa_fwd_f32.hip"] + HEADERS,
    "split": ["fa_fwd_bf16.hip", "fa_merge.hip", "fa_decode.hip"] + HEADERS,
    "backward": ["fa_bwd_bf16.hip"] + HEADERS,
}


def kernel_hash(kind: str = "forward") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "io_aware_exact_forward_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kind: str = "forward"):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_hash") != kernel_hash(kind):
        return None
    return ent.get("hbm_bytes_per_launch")


def ceiling_record(dev, stream) -> dict:
    """What the device's matrix cores deliver under a sustained dense load, measured
    right after the timed steps: a pure-MFMA loop (lib/libfa_probe.so, bf16
    v_mfma_f32_32x32x16 back to back on every SIMD) and torch.matmul on
    8192 x 8192 x 8192 bf16 (the vendor GEMM).  Under such a load the engine
    clock settles near 1.75-1.8 GHz, so these rates, not the 2.4 GHz dense
    peak, are what an MFMA-bound kernel can approach on this machine.  Both
    follow the power controller: they vary by about 10 % from machine to
    machine and right after other heavy work."""
    import ctypes

    import torch

    from io_aware_exact_forward_amd import build as _b

    def timed(fn, reps):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    rec = {}
    path = _b.probe_lib_path()
    if os.path.exists(path):
        lib = ctypes.CDLL(path)
        lib.fa_probe_mfma_bf16.restype = ctypes.c_int
        lib.fa_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p]
        lib.fa_probe_mfma_flops.restype = ctypes.c_double
        lib.fa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        blocks = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
        iters = 1000
        buf = torch.empty(blocks * 512, dtype=torch.float32, device=dev)

        def probe():
            if lib.fa_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(buf.data_ptr()),
                                      ctypes.c_void_p(stream.cuda_stream)) != 0:
                raise RuntimeError("MFMA probe launch failed")
        sec = timed(probe, 30)
        rec["mfma_loop_tflops"] = lib.fa_probe_mfma_flops(blocks, iters) / sec / 1e12
        del buf
    g = torch.Generator(device=dev).manual_seed(11)
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(8192, 8192, device=dev, dtype=torch.bfloat16)
    with torch.cuda.stream(stream):
        sec = timed(lambda: torch.matmul(a, b, out=c), 20)
    rec["gemm_bf16_8192_tflops"] = 2.0 * 8192 ** 3 / sec / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return rec


def ceiling_with_fracs(dev, stream, tflops) -> dict:
    ceil = ceiling_record(dev, stream)
    return dict(ceil, **{"frac_of_" + k[:-len("_tflops")]: tflops / v for k, v in ceil.items()})


def stored_clock_cycles(workload: str, kind: str = "forward"):
    """GRBM_GUI_ACTIVE cycles per XCD per launch from the committed counter
    summary, if taken on the current kernel source; else None.  The count is
    the same for every launch of a kernel (it is the work, not the time), so
    dividing it by a launch's duration gives the engine clock of that run."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            ent = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not ent or ent.get("kernel_hash") != kernel_hash(kind):
        return None
    return ent.get("grbm_gui_active_per_xcd_per_launch")


def clock_record(workload: str, kind: str, ms: float, peak: float):
    """Engine clock of the timed steps and the dense peak at that clock."""
    cyc = stored_clock_cycles(workload, kind)
    if not cyc:
        return None
    ghz = cyc / (ms * 1e-3) / 1e9
    return {"engine_ghz": ghz, "peak_at_clock": peak * ghz / 2.4,
            "source": "GRBM_GUI_ACTIVE cycles per XCD per launch (profiles/traffic.json) / "
                      "event-timed launch duration"}


def timed_steps(step, args, stream):
    """Settle, then args.warmup untimed steps, then args.steps timed steps
    between two events on the launch stream.

    Settle: from idle, the power controller first lowers the engine clock
    under this load and then brings it back (launches 5-25 of the 32-head
    N = 8192 forward run up to 30 % slower than the steady state; the
    engine cycles per launch stay the same).  The bench measures the steady
    state: it runs the step until two consecutive blocks of 10 launches
    agree within 1 % (at least 60 launches, at most 2 s), timing each launch,
    and reports what launches 6-25 took, i.e. what 20 steps after 5 warm-ups
    from idle would have measured."""
    import torch
    ev = []
    t0 = time.perf_counter()
    n, prev, mean = 0, None, None
    while args.settle_max_s > 0:
        blk = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
        blk[0].record(stream)
        for i in range(10):
            step()
            blk[i + 1].record(stream)
        blk[-1].synchronize()
        d = [blk[i].elapsed_time(blk[i + 1]) for i in range(10)]
        ev += d
        n += 10
        mean = sum(d) / 10
        if (n >= 60 and prev is not None and abs(mean - prev) <= 0.01 * prev) or \
                time.perf_counter() - t0 > args.settle_max_s or n >= 2000:
            break
        prev = mean
    settle = {"launches": n, "seconds": time.perf_counter() - t0,
              "first_launches_ms": [round(x, 4) for x in ev[:30]],
              "launches_6_to_25_ms_per_step": (sum(ev[5:25]) / 20 if n >= 25 else None),
              "last_block_ms_per_step": mean}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    return start.elapsed_time(end) / args.steps, t_wall, settle


def kv_byte_model(wl, lens, esz):
    """HBM bytes of one forward if no key/value tile were shared between
    query tiles through L2: each query tile reads its rows of Q once and every
    key/value tile it sees (whole tiles, as the kernel loads them), and O and
    the LSE are written once.  The query/key tile sizes mirror the launch
    choice of the library (256 rows for large problems, 128 otherwise; 64 keys
    at d = 128, 128 at d = 64).  Beside the compulsory bytes (every tile read
    once) and the counters, it bounds how much L2 reuse the schedule gets."""
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    big = N >= 256 and B * H * ((N + 255) // 256) >= 512 and not (d == 64 and wl.ragged)
    bq = 256 if big and wl.dtype == "bf16" else 128
    bk = 64 if d == 128 else 128
    if wl.dtype != "bf16":
        bq, bk = 128, 64
    row = d * esz
    kv_tiles = 0
    q_rows = 0
    for L in lens:
        for q0 in range(0, N, bq):
            if q0 >= L:
                continue
            seen = min(L, q0 + bq) if wl.causal else L
            kv_tiles += (seen + bk - 1) // bk
            q_rows += min(bq, L - q0)
    no_reuse = H * (q_rows * row + kv_tiles * 2 * bk * row) + B * H * N * (row + 4)
    return {"query_tile_rows": bq, "key_tile_rows": bk, "kv_tile_loads": H * kv_tiles,
            "no_l2_reuse_bytes": no_reuse}


def to_device(inp, dev):
    import numpy as np
    import torch
    if inp.wl.dtype == "bf16":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    kl = None if inp.key_len is None else torch.from_numpy(inp.key_len).to(dev)
    return conv(inp.q), conv(inp.k), conv(inp.v), kl


def cpu_baseline(inp, wl, o_dev, lse_dev, target_s: float):
    """Time the fp64 oracle on a seeded sample of query rows (all heads)."""
    import numpy as np
    import oracle
    from io_aware_exact_forward_amd import workloads as W
    B, H, N, d = inp.q.shape
    qx, kx, vx = inp.exact("q"), inp.exact("k"), inp.exact("v")
    # calibrate: one small chunk to estimate the per-row cost
    rng = np.random.default_rng(4242)
    probe = np.sort(rng.choice(N, min(N, 64), replace=False))
    t0 = time.perf_counter()
    oracle.attention(qx[:1, :1], kx[:1, :1], vx[:1, :1], wl.scale, causal=wl.causal,
                     key_len=None if inp.key_len is None else inp.key_len[:1], rows=probe)
    per_row = (time.perf_counter() - t0) / len(probe)
    rows_per_head = int(max(8, min(N, target_s / max(per_row, 1e-9) / (B * H))))
    rows = np.stack([np.sort(rng.choice(N, rows_per_head, replace=False)) for _ in range(H)])
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention(qx, kx, vx, wl.scale, causal=wl.causal, key_len=inp.key_len,
                                      rows=rows)
    dt = time.perf_counter() - t0
    # useful flops in the sample: 4*d per visible pair
    lens = np.full(B, N) if inp.key_len is None else np.clip(inp.key_len, 0, N)
    pairs = 0
    for b in range(B):
        L = int(lens[b])
        for h in range(H):
            r = rows[h]
            r = r[r < L]
            pairs += int((r + 1).sum()) if wl.causal else len(r) * L
    flops = 4.0 * d * pairs
    # agreement of the device output on the sampled rows (context only)
    og = np.stack([o_dev[:, h, rows[h]] for h in range(H)], axis=1)
    err = float(np.nanmax(np.abs(og - o_ref))) if og.size else 0.0
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{rows_per_head} seeded query rows per head x {B * H} (batch, head) pairs "
                  f"({rows_per_head * B * H} rows of {B * H * N}); fp64 numpy, whole score rows "
                  f"materialised; {dt:.1f} s",
        "seconds": dt,
        "host_threads_available": len(os.sched_getaffinity(0)),
        "sample_rows_max_abs_err_vs_device": err,
    }


def bench_decode(args) -> int:
    """Decode: one query row per (sequence, head) against its key cache,
    through fa_forward_split with the library's own range count.  A step is
    one call (the range kernel and the merge).  Bound by HBM: the algorithmic
    bytes are each sequence's valid K and V rows read once plus q, o and LSE."""
    import numpy as np
    import torch

    import io_aware_exact_forward_amd as fa
    import oracle
    from io_aware_exact_forward_amd import workloads as W

    wl = W.DECODE_WORKLOADS[args.workload]
    inp = W.decode_inputs(wl)
    dev = torch.device("cuda:0")
    q, k, v, kl = to_device(inp, dev)
    B, H, Nk, d = wl.B, wl.H, wl.Nk, wl.d
    Hkv = wl.kv_heads
    lens = [int(x) for x in np.clip(inp.key_len, 0, Nk)]
    flops = 4.0 * d * H * sum(lens)
    # each valid K and V row of every key/value head read once; q, o, LSE
    algo_bytes = sum(Hkv * 2 * L * d * 2 + H * (2 * d * 2 + 4) for L in lens)
    ws_bytes = fa.fa_split_workspace_bytes(B, H, 1, Nk, d, 0)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, 1), dtype=torch.float32, device=dev)

    def step():
        fa.forward_split(q, k, v, scale=wl.scale, causal=True, key_len=kl, num_splits=0,
                         workspace=ws, out=out, lse=lse)

    stream = torch.cuda.current_stream(dev)
    ms, t_wall, settle = timed_steps(step, args, stream)
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "attention fwd TFLOP/s (bf16, 1 GPU); decode step, HBM-bound",
        "value": flops / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(wl.describe(), key_lens=lens, useful_flops=flops,
                       algorithmic_hbm_bytes=algo_bytes, workspace_bytes=ws_bytes,
                       parallelism="single GPU"),
        "roofline": {
            "bound": "hbm",
            "achieved": gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS,
            "traffic": stored_traffic(wl.name, "split"),
            "kernel": ("fa_decode_balanced_kernel + merge_kernel" if Hkv == H else
                       "fa_fwd_bf16_kernel (a key/value head's query heads as rows) + merge_kernel")
                      + " (one call; both inside the events)",
            "kernel_hash": kernel_hash("split"),
        },
        "wall_s_timed_region": t_wall,
        "settle": settle,
    }
    if not args.no_cpu_baseline:
        # the oracle on whole (sequence, head) rows, as many as fit the time budget
        qx, kx, vx = inp.exact("q"), inp.exact("k"), inp.exact("v")
        pairs, done, t0 = 0, 0, time.perf_counter()
        for b in range(B):
            for h in range(H):
                hk = h // (H // Hkv)  # the key/value head query head h reads
                oracle.attention(qx[b:b + 1, h:h + 1], kx[b:b + 1, hk:hk + 1],
                                 vx[b:b + 1, hk:hk + 1], wl.scale, causal=True,
                                 key_len=inp.key_len[b:b + 1], end_aligned=True)
                pairs += lens[b]
                done += 1
                if time.perf_counter() - t0 > args.cpu_seconds:
                    break
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            threads = len(os.sched_getaffinity(0))
        result["cpu_baseline"] = {
            "value": 4.0 * d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {B * H} (sequence, head) decode rows, fp64 numpy; {dt:.1f} s",
            "seconds": dt,
        }
    print(json.dumps(result), flush=True)
    return 0


def bench_backward(args) -> int:
    """Backward: one fa_backward call (the dQ and the dK/dV kernels) over the
    whole workload, with Q, K, V, O, LSE and dO resident.  Useful work is
    10*d flops per visible pair (the five products of the gradient: S, dV,
    dP, dQ, dK); the kernels also recompute S and dP once more."""
    import numpy as np
    import torch

    import io_aware_exact_forward_amd as fa
    import oracle
    from io_aware_exact_forward_amd import workloads as W

    wl = W.BWD_WORKLOADS[args.workload]
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    if args.n:
        N = args.n
    inp, do_bits = W.grad_inputs(B, H, N, d, wl.seed)
    dev = torch.device("cuda:0")
    q, k, v, _ = to_device(inp, dev)
    dout = torch.from_numpy(np.ascontiguousarray(do_bits).view(np.int16)).view(torch.bfloat16).to(dev)
    drop = args.dropout
    seed, offset = 2024, 1
    bias_t = None
    if args.bias:
        # an fp32 [N, N] additive mask shared by every batch entry and head
        bias_t = torch.randn((1, 1, N, (N + 3) // 4 * 4), device=dev, dtype=torch.float32,
                             generator=torch.Generator(device=dev).manual_seed(7))
        o, lse = fa.forward_bias(q, k, v, bias_t, scale=wl.scale, causal=wl.causal)
    elif drop > 0:
        # the forward with dropout, then its gradient with the same stream
        o, lse = fa.forward_dropout(q, k, v, p_drop=drop, seed=seed, offset=offset,
                                    scale=wl.scale, causal=wl.causal)
    else:
        o, lse = fa.forward(q, k, v, scale=wl.scale, causal=wl.causal)
    ws = torch.empty(fa.fa_backward_workspace_bytes(B, H, N, d, fa.FA_DTYPE_BF16), dtype=torch.uint8,
                     device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    pairs = W.valid_pairs(N, wl.causal, None, B) * H
    flops = 10.0 * d * pairs

    def step():
        if bias_t is not None:
            fa.backward_bias(q, k, v, o, lse, dout, bias_t, scale=wl.scale, causal=wl.causal,
                             workspace=ws, dq=dq, dk=dk, dv=dv)
        elif drop > 0:
            fa.backward_dropout(q, k, v, o, lse, dout, p_drop=drop, seed=seed, offset=offset,
                                scale=wl.scale, causal=wl.causal, workspace=ws, dq=dq, dk=dk,
                                dv=dv)
        else:
            fa.backward(q, k, v, o, lse, dout, scale=wl.scale, causal=wl.causal, workspace=ws,
                        dq=dq, dk=dk, dv=dv)

    stream = torch.cuda.current_stream(dev)
    ms, t_wall, settle = timed_steps(step, args, stream)
    tflops = flops / (ms * 1e-3) / 1e12
    ceil = ceiling_with_fracs(dev, stream, tflops)
    result = {
        "metric": "attention bwd TFLOP/s (bf16, 1 GPU; useful 10*d flops per visible pair)"
                  + (f"; dropout p={drop}" if drop > 0 else "")
                  + ("; additive mask fp32 [N, N]" if bias_t is not None else ""),
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(wl.describe(), N=N, useful_flops=flops,
                       workspace_bytes=ws.numel(), parallelism="single GPU"),
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / PEAK_BF16_TFLOPS,
            "traffic": (stored_traffic(wl.name, "backward")
                        if N == wl.N and drop == 0 and bias_t is None else None),
            "kernel": "fa_bwd_dq_kernel + fa_bwd_dkdv_kernel (one call; both inside the events)",
            "kernel_hash": kernel_hash("backward"),
        },
        "wall_s_timed_region": t_wall,
        "settle": settle,
    }
    # Stored-state comparison (the N x N matrices in HBM): latency and peak
    # allocated memory of both paths, each measured from the same resident
    # inputs and outputs.
    if not args.no_naive and drop == 0 and bias_t is None:
        def peak_of(fn, ws_bytes):
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats(dev)
            base = torch.cuda.memory_allocated(dev)
            w = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
            fn(w)
            torch.cuda.synchronize()
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for _ in range(args.steps):
                fn(w)
            s1.record(stream)
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated(dev) - base
            del w
            torch.cuda.empty_cache()
            return s0.elapsed_time(s1) / args.steps, peak
        fused_ms, fused_peak = peak_of(
            lambda w: fa.backward(q, k, v, o, lse, dout, scale=wl.scale, causal=wl.causal,
                                  workspace=w, dq=dq, dk=dk, dv=dv), ws.numel())
        need = fa.fa_naive_workspace_bytes(B, H, N, fa.FA_DTYPE_BF16)
        if need < 0.8 * torch.cuda.mem_get_info(dev)[0]:
            naive_ms, naive_peak = peak_of(
                lambda w: fa.naive_backward(q, k, v, o, lse, dout, scale=wl.scale,
                                            causal=wl.causal, workspace=w, dq=dq, dk=dk, dv=dv),
                need)
            resident = sum(t.numel() * t.element_size() for t in (q, k, v, o, lse, dout, dq, dk, dv))
            result["stored_state_comparison"] = {
                "recompute_ms": fused_ms, "stored_state_ms": naive_ms,
                "speedup_of_recompute": naive_ms / fused_ms,
                "resident_tensor_bytes": resident,
                "recompute_extra_peak_bytes": fused_peak, "stored_state_extra_peak_bytes": naive_peak,
                "note": "extra peak = allocation peak above the resident inputs and outputs "
                        "(the workspace: D per row, vs S/P and dP/dS matrices)",
            }
    if not args.no_cpu_baseline:
        qx, kx, vx = inp.exact("q"), inp.exact("k"), inp.exact("v")
        dox = W.bf16_decode(do_bits, np.float64)
        bias_np = None if bias_t is None else bias_t[0, 0, :, :N].double().cpu().numpy()
        t0, done = time.perf_counter(), 0
        for b in range(B):
            for h in range(H):
                sl = lambda x: x[b:b + 1, h:h + 1]
                if bias_t is not None:
                    oracle.attention_backward(sl(qx), sl(kx), sl(vx), sl(dox), wl.scale,
                                              causal=wl.causal, bias=bias_np)
                elif drop > 0:
                    oracle.dropout_attention_backward(sl(qx), sl(kx), sl(vx), sl(dox), wl.scale,
                                                      drop, seed, offset, causal=wl.causal,
                                                      head_ids=[h], H_all=H, batch_ids=[b])
                else:
                    oracle.attention_backward(sl(qx), sl(kx), sl(vx), sl(dox), wl.scale,
                                              causal=wl.causal)
                done += 1
                if time.perf_counter() - t0 > args.cpu_seconds:
                    break
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            threads = len(os.sched_getaffinity(0))
        result["cpu_baseline"] = {
            "value": flops / (B * H) * done / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {B * H} (batch, head) slices, fp64 numpy gradients with P "
                      f"materialised; {dt:.1f} s",
            "seconds": dt,
        }
    result["ceiling"] = ceil
    print(json.dumps(result), flush=True)
    return 0


def bench_varlen(args) -> int:
    """Packed variable-length causal batch with grouped key/value heads: one
    fa_forward_varlen call over the whole batch.  Useful work 4*d flops per
    visible pair, as for the square workloads.  With --backward: one
    fa_backward_varlen call (dQ, dK, dV of the same batch from its O and
    LSE), useful work 10*d flops per visible pair."""
    import numpy as np
    import torch

    import io_aware_exact_forward_amd as fa
    import oracle
    from io_aware_exact_forward_amd import workloads as W

    wl = W.VARLEN_WORKLOADS[args.workload]
    inp = W.varlen_inputs(wl)
    lens = np.diff(inp.cu_q).astype(np.int64)
    dev = torch.device("cuda:0")
    conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = conv(inp.q), conv(inp.k), conv(inp.v)
    cq = torch.from_numpy(inp.cu_q).to(dev)
    ck = torch.from_numpy(inp.cu_k).to(dev)
    mx = int(lens.max())
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], wl.H), dtype=torch.float32, device=dev)
    pairs_all = float(sum(L * (L + 1) // 2 for L in lens))
    flops = (10.0 if args.backward else 4.0) * wl.d * wl.H * pairs_all

    if args.backward:
        # upstream gradient: standard normal, bf16, drawn after the inputs
        rng = np.random.default_rng(wl.seed + 50)
        dout = conv(W.bf16_encode(rng.standard_normal(inp.q.shape, dtype=np.float32)))
        fa.forward_varlen(q, k, v, cq, ck, mx, mx, scale=wl.scale, causal=True, out=out, lse=lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(max(fa.fa_backward_workspace_bytes(1, wl.H, q.shape[0], wl.d,
                                                            fa.FA_DTYPE_BF16), 1),
                         dtype=torch.uint8, device=dev)

        def step():
            fa.backward_varlen(q, k, v, out, lse, dout, cq, ck, mx, mx, scale=wl.scale,
                               causal=True, workspace=ws, dq=dq, dk=dk, dv=dv)
    else:
        def step():
            fa.forward_varlen(q, k, v, cq, ck, mx, mx, scale=wl.scale, causal=True, out=out,
                              lse=lse)

    stream = torch.cuda.current_stream(dev)
    ms, t_wall, settle = timed_steps(step, args, stream)
    tflops = flops / (ms * 1e-3) / 1e12
    ceil = ceiling_with_fracs(dev, stream, tflops)
    kind = "backward" if args.backward else "forward"
    result = {
        "metric": ("attention bwd TFLOP/s (bf16, 1 GPU; useful 10*d flops per visible pair); "
                   "packed variable-length batch" if args.backward else
                   "attention fwd TFLOP/s (bf16, 1 GPU); packed variable-length batch"),
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": dict(wl.describe(), seq_lens=lens.tolist(), total_tokens=int(lens.sum()),
                       useful_flops=flops, parallelism="single GPU", **{"pass": kind}),
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                     "traffic": stored_traffic(wl.name + (":backward" if args.backward else ""),
                                               kind),
                     "kernel": ("fa_bwd_dq_kernel + fa_bwd_dkdv_kernel" if args.backward
                                else "fa_fwd_bf16_kernel"),
                     "kernel_hash": kernel_hash(kind)},
        "wall_s_timed_region": t_wall,
        "settle": settle,
    }
    if not args.no_cpu_baseline:
        # the oracle on whole sequences, shortest first, within the time budget
        qx, kx, vx = inp.exact("q"), inp.exact("k"), inp.exact("v")
        t0, done, pairs = time.perf_counter(), 0, 0
        dox = W.bf16_decode(dout.view(torch.int16).cpu().numpy().view(np.uint16), np.float64) \
            if args.backward else None
        for b in np.argsort(lens):
            a0, a1 = int(inp.cu_q[b]), int(inp.cu_q[b + 1])
            cu1 = np.array([0, a1 - a0])
            if args.backward:
                oracle.varlen_attention_backward(qx[a0:a1], kx[a0:a1], vx[a0:a1], dox[a0:a1],
                                                 cu1, cu1, wl.scale, True)
            else:
                oracle.varlen_attention(qx[a0:a1], kx[a0:a1], vx[a0:a1], cu1, cu1, wl.scale, True)
            done += 1
            pairs += (a1 - a0) * (a1 - a0 + 1) // 2
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            threads = len(os.sched_getaffinity(0))
        result["cpu_baseline"] = {
            "value": flops / pairs_all * pairs / dt / 1e12, "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {wl.B} sequences (shortest first), all heads, fp64; {dt:.1f} s",
            "seconds": dt,
        }
    result["ceiling"] = ceil
    print(json.dumps(result), flush=True)
    return 0


SWEEP_N = [256, 512, 1024, 2048, 4096, 8192, 16384, 32768]


def bench_sweep(args) -> int:
    """Sequence-length sweep of the forward, fused against the materialised
    three-pass baseline: for B = 1, H = 32, d = 128, causal, bf16 Q, K, V
    i.i.d. N(0, 1) (drawn on the device from a seeded generator), scale
    1/sqrt(128), and N from 256 to 32768: milliseconds per call (events on
    the launch stream, after the settle and warm-up of timed_steps), useful
    TFLOP/s, and the allocation peak of one call above the resident inputs
    (O and LSE for both; S and P for the naive path).  Prints one JSON line."""
    import torch

    import io_aware_exact_forward_amd as fa

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    H, d = 32, 128
    scale = 1.0 / math.sqrt(d)
    rows = []
    for N in SWEEP_N:
        g = torch.Generator(device=dev).manual_seed(5000 + N)
        q, k, v = (torch.randn(1, H, N, d, device=dev, dtype=torch.bfloat16, generator=g)
                   for _ in range(3))
        out = torch.empty_like(q)
        lse = torch.empty((1, H, N), dtype=torch.float32, device=dev)
        flops = 4.0 * d * H * N * (N + 1) / 2
        ms, _, _ = timed_steps(lambda: fa.forward(q, k, v, scale=scale, causal=True, out=out,
                                                  lse=lse), args, stream)

        def peak_of(fn):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats(dev)
            base = torch.cuda.memory_allocated(dev)
            r = fn()
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated(dev) - base
            del r
            torch.cuda.empty_cache()
            return peak
        row = {"N": N, "fused_ms": ms, "fused_tflops": flops / (ms * 1e-3) / 1e12,
               "fused_extra_peak_bytes": peak_of(lambda: fa.forward(q, k, v, scale=scale,
                                                                    causal=True)),
               "compulsory_bytes": 4 * H * N * d * 2 + H * N * 4,
               "naive_matrix_bytes": 2 * H * N * N * 2}
        need = fa.fa_naive_workspace_bytes(1, H, N, fa.FA_DTYPE_BF16)
        if not args.no_naive and need < 0.8 * torch.cuda.mem_get_info(dev)[0]:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            nrun = lambda: fa.naive_forward(q, k, v, scale=scale, causal=True, workspace=ws)
            nrun()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(3):
                nrun()
            e1.record(stream)
            torch.cuda.synchronize()
            del ws
            torch.cuda.empty_cache()
            nms = e0.elapsed_time(e1) / 3
            row.update(naive_ms=nms, naive_tflops=flops / (nms * 1e-3) / 1e12,
                       naive_extra_peak_bytes=peak_of(lambda: fa.naive_forward(
                           q, k, v, scale=scale, causal=True)),
                       speedup_of_fused=nms / ms)
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del q, k, v, out, lse
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "attention fwd sequence-length sweep (bf16, 1 GPU)",
                      "config": {"workload": "sweep_h32_d128_causal_bf16", "B": 1, "H": H,
                                 "d": d, "causal": True, "N": SWEEP_N},
                      "steps": args.steps, "warmup": args.warmup, "sweep": rows}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # after the settle (timed_steps) the warm-up steps only need to cover the
    # first launches' one-time costs
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="a square workload name, decode_b8_h32_k16384_d128_bf16 (one query "
                         "row per sequence and head against its key cache, split over key ranges) "
                         "bwd_b2_h16_n4096_d64_bf16 (the backward pass) or "
                         "varlen_b16_h32_hkv8_n8192_d128_bf16 (packed sequences, grouped heads)")
    ap.add_argument("--n", type=int, default=0,
                    help="backward workload only: another sequence length (512 .. 4096)")
    ap.add_argument("--bias", action="store_true",
                    help="square workloads: time fa_forward_bias with a random fp32 [N, N] "
                         "additive mask shared by all batches and heads; the backward "
                         "workload: fa_backward_bias of such a forward")
    ap.add_argument("--backward", action="store_true",
                    help="packed workload: time fa_backward_varlen on the batch instead")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="square workloads: time fa_forward_dropout at this rate instead; the "
                         "backward workload: fa_backward_dropout of such a forward")
    ap.add_argument("--settle-max-s", type=float, default=2.0,
                    help="upper bound on the settle before the warm-up (0: none, e.g. for "
                         "profiled runs that look at single launches)")
    ap.add_argument("--sweep", action="store_true",
                    help="sequence-length sweep (N = 256 .. 32768, 32 heads, d = 128, causal) "
                         "of the fused forward and the naive baseline: time and memory peak")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (calibrates "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the attention forward "
              f"shards by (batch, head) with no communication, so there is no multi-GPU step "
              f"to time here.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import io_aware_exact_forward_amd as fa
    from io_aware_exact_forward_amd import _lib
    from io_aware_exact_forward_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if not os.path.exists(_lib.lib_path()):
        from io_aware_exact_forward_amd import build as _b
        _b.build()
    fa.load()

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return 0

    if args.sweep:
        return bench_sweep(args)
    if args.workload in W.DECODE_WORKLOADS:
        return bench_decode(args)
    if args.workload in W.BWD_WORKLOADS:
        return bench_backward(args)
    if args.workload in W.VARLEN_WORKLOADS:
        return bench_varlen(args)
    wl = W.workload(args.workload)
    inp = W.make_inputs(wl)
    dev = torch.device("cuda:0")
    q, k, v, kl = to_device(inp, dev)
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    pairs = W.valid_pairs(N, wl.causal, inp.key_len, B) * H
    flops = 4.0 * d * pairs
    esz = 2 if wl.dtype == "bf16" else 4
    lens = [N] * B if inp.key_len is None else [max(0, min(int(x), N)) for x in inp.key_len]
    compulsory = sum(3 * H * L * d * esz for L in lens) + B * H * N * d * esz + B * H * N * 4

    stream = torch.cuda.current_stream(dev)
    if args.bias:
        bias_t = torch.randn((1, 1, N, (N + 3) // 4 * 4), device=dev, dtype=torch.float32,
                             generator=torch.Generator(device=dev).manual_seed(7))

        def fwd():
            fa.forward_bias(q, k, v, bias_t, scale=wl.scale, causal=wl.causal, key_len=kl,
                            out=out, lse=lse)
    elif args.dropout > 0:
        def fwd():
            fa.forward_dropout(q, k, v, p_drop=args.dropout, seed=2024, offset=0, scale=wl.scale,
                               causal=wl.causal, key_len=kl, out=out, lse=lse)
    else:
        def fwd():
            fa.forward(q, k, v, scale=wl.scale, causal=wl.causal, key_len=kl, out=out, lse=lse)
    ms, t_wall, settle = timed_steps(fwd, args, stream)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS

    result = {
        "metric": "attention fwd TFLOP/s (bf16, 1 GPU) and % of MFMA peak; HBM bytes vs N*d bound",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": dict(wl.describe(), useful_flops=flops, compulsory_hbm_bytes=compulsory,
                       parallelism="single GPU",
                       **({"dropout": args.dropout} if args.dropout > 0 else {}),
                       **({"bias": "fp32 [N, N] shared"} if args.bias else {})),
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": tflops / peak,
            "traffic": stored_traffic(wl.name) if args.dropout == 0 and not args.bias else None,
            "kernel": "fa_fwd_bf16_kernel" if wl.dtype == "bf16" else "fa_fwd_f32_kernel",
            "kernel_hash": kernel_hash(),
        },
        "wall_s_timed_region": t_wall,
        "settle": settle,
    }
    clk = clock_record(wl.name, "forward", ms, peak) if args.dropout == 0 and not args.bias \
        else None
    if clk:
        result["roofline"]["peak_at_measured_clock"] = clk["peak_at_clock"]
        result["roofline"]["frac_at_measured_clock"] = tflops / clk["peak_at_clock"]
        result["clock"] = clk

    if wl.dtype == "bf16":
        result["ceiling"] = ceiling_with_fracs(dev, stream, tflops)

    if args.dropout == 0 and not args.bias:
        model = kv_byte_model(wl, lens, esz)
        tr = result["roofline"]["traffic"]
        result["byte_model"] = dict(model, compulsory_bytes=compulsory, counter_bytes=tr,
                                    counters_over_compulsory=(tr / compulsory if tr else None))

    if not args.no_naive and args.dropout == 0 and not args.bias:
        need = fa.fa_naive_workspace_bytes(B, H, N, fa.FA_DTYPE_BF16 if wl.dtype == "bf16" else fa.FA_DTYPE_F32)
        free = torch.cuda.mem_get_info(dev)[0]
        if need < 0.8 * free:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            fa.naive_forward(q, k, v, scale=wl.scale, causal=wl.causal, key_len=kl, workspace=ws)
            torch.cuda.synchronize()
            nsteps = 3
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for _ in range(nsteps):
                fa.naive_forward(q, k, v, scale=wl.scale, causal=wl.causal, key_len=kl, workspace=ws)
            s1.record(stream)
            torch.cuda.synchronize()
            nms = s0.elapsed_time(s1) / nsteps
            result["naive_baseline"] = {"ms_per_step": nms, "tflops_useful": flops / (nms * 1e-3) / 1e12,
                                        "workspace_bytes": need, "speedup_of_fused": nms / ms}
            del ws
            torch.cuda.empty_cache()

            # allocation peak of one call above the resident inputs, each path
            # allocating what it needs (O and LSE; the naive path also S and P)
            def peak_of(fn):
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
                torch.cuda.reset_peak_memory_stats(dev)
                base = torch.cuda.memory_allocated(dev)
                r = fn()
                torch.cuda.synchronize()
                peak = torch.cuda.max_memory_allocated(dev) - base
                del r
                torch.cuda.empty_cache()
                return peak
            fused_peak = peak_of(lambda: fa.forward(q, k, v, scale=wl.scale, causal=wl.causal,
                                                    key_len=kl))
            naive_peak = peak_of(lambda: fa.naive_forward(q, k, v, scale=wl.scale,
                                                          causal=wl.causal, key_len=kl))
            result["peak_memory"] = {
                "fused_extra_peak_bytes": fused_peak, "naive_extra_peak_bytes": naive_peak,
                "naive_over_fused": naive_peak / fused_peak if fused_peak else None,
                "note": "allocation peak of one call above the resident Q, K, V (torch "
                        "allocator): O and LSE for both, plus S and P for the naive path"}

    if not args.no_cpu_baseline and args.dropout == 0 and not args.bias:
        o_host = out
        if wl.dtype == "bf16":
            o_np = W.bf16_decode(o_host.view(torch.int16).cpu().numpy().view(np.uint16))
        else:
            o_np = o_host.cpu().numpy().astype(np.float64)
        result["cpu_baseline"] = cpu_baseline(inp, wl, o_np, lse.cpu().numpy(), args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
