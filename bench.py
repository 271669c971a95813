#!/usr/bin/env python3
"""Benchmark: chunked causal linear-attention forward on one MI355X.

A step is one call of la_chunked_forward on one batch of synthetic input of
the headline workload: B=8, H=16, L=8192, d_k=d_v=128, bf16, identity feature
map, no normaliser, causal, chunk size C (default 64).  Inputs are resident in
HBM before the timed region; W untimed warmup steps, then exactly K timed
steps bracketed by device synchronisation, timed with HIP events on the
stream the kernels run on.

Prints one JSON line with the metric, the roofline of the dominant kernel and
the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk C] [--extra]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "chunked causal linear-attn forward tokens/sec and % MFMA peak, L=8192 d=128"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_I8_TOPS = 5000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_chunked_fwd_pipe_identity-L8192-d128-C64.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def lib_hash() -> str:
    """Hash of the kernel sources the library is built from (ties measured
    counters to the code they were taken on)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_causal_linear_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not os.path.isfile(os.path.join(csrc, f)):
            continue  # the measurement probe's sources are not the library's
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# the sources the dominant kernel (chunked_fwd_pipe at d_k = 64 and 128) is
# compiled from: its translation unit and the headers it includes
KERNEL_SOURCES = ("la_pipe.hip", "la_pipe.hpp", "la_fwd_pipe.hpp", "la_common.hpp", "la_kernels.hpp")


def kernel_hash() -> str:
    """Hash of the dominant kernel's sources (ties its traffic counters to the
    code they were taken on; other kernels' changes leave it alone)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_causal_linear_amd", "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """The `key: value` lines of the committed counter summary (or {})."""
    out = {}
    if not os.path.exists(TRAFFIC_FILE):
        return out
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                out[key.strip()] = val.strip()
    return out


def copy_calibration():
    """A plain device copy of 512 MiB, twice: under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE readings calibrate those counters."""
    import torch
    a = torch.empty(256 * 1024 * 1024, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def mfma_peak(kind: int, grid: int = 2048, iters: int = 1024):
    """Measured matrix-core rate (TFLOP/s for bf16, TOP/s for int8) of the probe
    loop in libla_probe.so (include/la_probe.h): median of five launches, each
    timed with an event pair on the current stream, after two untimed ones."""
    import ctypes

    import numpy as np
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "chunked_causal_linear_amd", "libla_probe.so"))
    lib.la_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.la_probe_mfma.restype = ctypes.c_int
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")

    def run():
        rc = lib.la_probe_mfma(kind, iters, grid, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"la_probe_mfma returned {rc}")
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    ms = float(np.median(per_launch_ms(run, 5)))
    per_inst = 16384 if kind == 0 else 32768
    return grid * 4 * iters * 8 * per_inst / (ms * 1e-3) / 1e12, ms


def memory_ceilings():
    """What plain streams get from this memory system, by access mix (GB/s,
    median of five launches each, after one untimed): reads only over 1 GiB
    and 2 GiB sets (libla_probe.so's la_probe_read, include/la_probe.h), the
    same probe re-reading a 128 MiB set four times per launch (the Infinity
    Cache), three reads and one write (torch.addcmul over 256 MiB operands) and
    one read and one write (a 512 MiB device copy)."""
    import ctypes

    import numpy as np
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "chunked_causal_linear_amd", "libla_probe.so"))
    lib.la_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.la_probe_read.restype = ctypes.c_int
    grid = 2048
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    buf = torch.ones(1 << 29, dtype=torch.float32, device="cuda")  # 2 GiB
    res = {}

    def rate(fn, nbytes):
        fn()
        torch.cuda.synchronize()
        return nbytes / (float(np.median(per_launch_ms(fn, 5))) * 1e-3) / 1e9

    def read(nbytes, reps):
        def run():
            rc = lib.la_probe_read(buf.data_ptr(), nbytes // 16, reps, grid, out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"la_probe_read returned {rc}")
        return rate(run, nbytes * reps)
    res["reads_1GiB"] = read(1 << 30, 1)
    res["reads_2GiB"] = read(1 << 31, 1)
    res["rereads_128MiB_x4"] = read(1 << 27, 4)
    del buf
    a, b, c, d = (torch.ones(1 << 27, dtype=torch.bfloat16, device="cuda") for _ in range(4))
    res["three_reads_one_write_1GiB"] = rate(lambda: torch.addcmul(a, b, c, out=d), 4 << 28)
    del a, b, c, d
    x = torch.ones(1 << 28, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    res["one_read_one_write_1GiB"] = rate(lambda: y.copy_(x), 2 << 29)
    del x, y
    torch.cuda.empty_cache()
    return {k: {"GB/s": v, "frac_of_8TBs": v / PEAK_HBM_GBS} for k, v in res.items()}


def cpu_info():
    """CPU model (from /proc/cpuinfo) and numpy's BLAS build and thread count."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = []
    try:
        import threadpoolctl
        for d in threadpoolctl.threadpool_info():
            if d.get("user_api") == "blas":
                blas.append({k: d.get(k) for k in ("internal_api", "version", "num_threads", "architecture",
                                                    "threading_layer")})
    except Exception as e:  # noqa: BLE001 - the record is informative only
        blas.append({"error": str(e)})
    return model, blas


def dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def time_steps(fn, steps: int, warmup: int):
    """Average ms per call over exactly `steps` calls (HIP events on the current stream)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_steps_each(fn, steps: int, warmup: int):
    """time_steps plus each call's own duration (an event pair around every
    call, all on the current stream inside the timed region)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, [a.elapsed_time(b) for a, b in evs]


def row_time(fn, steps: int = 20, spin_s: float = 0.15):
    """time_steps after running fn untimed for spin_s seconds (clock ramp)."""
    import torch
    t_end = time.perf_counter() + spin_s
    while time.perf_counter() < t_end:
        fn()
        torch.cuda.synchronize()
    return time_steps(fn, steps, 2)


def per_launch_ms(fn, steps: int):
    """Per-call durations (ms) with an event pair around each call."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(w, C: int, budget_s: float = 10.0):
    """The CPU oracle's chunked form, as it stands, on whole heads of the
    workload at full L, head after head until about `budget_s` seconds of CPU
    work; tokens/s extrapolated linearly over the heads."""
    import threadpoolctl

    import oracle
    import workloads as wl
    cores = len(os.sched_getaffinity(0))
    elapsed, heads = 0.0, 0
    # BLAS threads = the cores this process may run on, set explicitly
    with threadpoolctl.threadpool_limits(limits=cores, user_api="blas"):
        model, blas = cpu_info()
        while elapsed < budget_s and heads < w.BH:
            q, k, v = wl.head_inputs(w, heads)  # input generation is not timed
            t1 = time.perf_counter()
            oracle.chunked(q.exact, k.exact, v.exact, C, w.normalize)
            elapsed += time.perf_counter() - t1
            heads += 1
    per_head = elapsed / heads
    tokens_per_s = w.L / (w.H * per_head)  # B*L tokens take B*H head passes
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle.chunked (numpy float64, C={C}) on {heads} of {w.BH} heads at full L={w.L} "
                      f"({elapsed:.1f} s); {per_head:.3f} s per head, extrapolated over all heads",
            "cpu": model, "blas": blas, "blas_threads_set": cores}


def run_headline(args):
    import numpy as np
    import torch

    import chunked_causal_linear_amd as la
    import workloads as wl
    from chunked_causal_linear_amd.accounting import Work

    w = wl.WORKLOADS[3]
    C = args.chunk
    log(f"generating workload {w.name} (B={w.B} H={w.H} L={w.L} d={w.d_in})")
    q, k, v, _ = wl.workload_inputs(w, want_exact=False)
    qd, kd, vd = dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits)
    del q, k, v
    fwd = la.Forward(qd, kd, vd, C, causal=True, normalize=False, fmap="identity", group=args.group)
    G = la.forward_group(0, w.BH, w.L, w.d_in, w.d_v, C, True, False, "identity", 0, args.group)
    n_chunks = (w.L + C - 1) // C
    n_groups = (n_chunks + G - 1) // G
    torch.cuda.synchronize()
    # bring the GPU to its steady clock before the warmup steps (untimed)
    t_end = time.perf_counter() + args.spinup
    while time.perf_counter() < t_end:
        for _ in range(20):
            fwd.run()
        torch.cuda.synchronize()
    log(f"warmup {args.warmup}, timing {args.steps} steps, C={C}, group={G} ({n_groups} groups), "
        f"workspace {fwd.ws_bytes} B")
    # the timed region: exactly K steps, events only at its two ends
    ms = time_steps(fwd.run, args.steps, args.warmup)
    # then the same K steps again with an event pair around each, for the
    # kernel's own launch duration (those events would otherwise add their
    # own gaps between the timed steps)
    _, per_step = time_steps_each(fwd.run, args.steps, 0)

    # the phases one by one (same kernels the forward launches)
    S, _ = la.chunk_states(kd, vd, C * G)
    la.state_scan(S, None, want_final=False)
    o3 = torch.empty_like(fwd.o)
    ph3 = lambda: la.chunk_output(qd, kd, vd, C, G, P_prefix=S, out=o3)  # noqa: E731
    ph1 = lambda: la.chunk_states(kd, vd, C * G)  # noqa: E731
    S2 = S.clone()
    ph2 = lambda: la.state_scan(S2, None, want_final=False)  # noqa: E731
    for fn in (ph3, ph1, ph2):
        fn()
    torch.cuda.synchronize()
    if n_groups == 1:
        # the forward is the one phase-3 launch: its duration in the timed steps
        k3 = float(np.mean(per_step))
        k3_src = ("event pair around each of the K steps of a second pass right after the timed one "
                  "(the forward is this one launch)")
    else:
        k3 = float(np.mean(per_launch_ms(ph3, 20)))
        k3_src = "event pair around each of 20 la_chunk_output calls"
    k1 = float(np.mean(per_launch_ms(ph1, 10))) if n_groups > 1 else 0.0
    k2 = float(np.mean(per_launch_ms(ph2, 10))) if n_groups > 1 else 0.0
    assert torch.equal(o3, fwd.o), "phase 3 alone differs from the forward"
    # a plain streaming kernel with the same traffic (three reads and one write
    # of B*H*L*d bf16 each): the bandwidth this memory system gives that mix
    scratch = torch.empty_like(qd)
    ref = lambda: torch.addcmul(qd, kd, vd, out=scratch)  # noqa: E731
    ref()
    torch.cuda.synchronize()
    ref_ms = float(np.median(per_launch_ms(ref, 20)))
    ref_gbs = 4 * qd.numel() * 2 / (ref_ms * 1e-3) / 1e9
    del scratch

    # the matrix cores' attainable rate, measured in the same run
    peak_bf16, _ = mfma_peak(0)

    work = Work(w.BH, w.L, w.d_in, w.d_k, w.d_v, C)
    tokens = w.B * w.L
    flops = work.page_flops()
    useful = 2 * work.causal_useful_macs()
    prefix_bytes = w.BH * (n_groups - 1) * w.d_k * w.d_v * 4
    alg_bytes3 = work.fused_bytes() + prefix_bytes
    sec = ms * 1e-3
    achieved_gbs = alg_bytes3 / (k3 * 1e-3) / 1e9
    traffic = None
    tr = read_traffic()
    if tr.get("kernel_hash") == kernel_hash() and tr.get("chunk") == str(C) and tr.get("group") == str(G):
        traffic = float(tr["bytes_per_launch"])
    res = {
        "metric": METRIC,
        "value": tokens / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} L={w.L} d_k=d_v={w.d_in} bf16, identity map, "
                               f"no normaliser, causal, C={C}",
                   "B": w.B, "H": w.H, "L": w.L, "d": w.d_in, "C": C, "chunks_per_group": G,
                   "parallelism": "single-gpu"},
        "tflops_page_count": flops / sec / 1e12,
        "mfma_frac_page_count": flops / sec / 1e12 / PEAK_BF16_TFLOPS,
        "mfma_peak_measured_tflops": peak_bf16,
        "mfma_frac_page_count_of_measured_peak": flops / sec / 1e12 / peak_bf16,
        "tflops_causal_useful": useful / sec / 1e12,
        "head_tokens_per_s": w.BH * w.L / sec,
        "phases_ms": {"chunk_states": k1, "state_scan": k2, "chunk_output": k3},
        "step_ms_spread": {"from": "event pair around each of the K steps of the second pass",
                           "median": float(np.median(per_step)), "min": float(np.min(per_step)),
                           "max": float(np.max(per_step))},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "chunked_fwd_pipe" if C in (32, 64, 128) else "chunked_fwd_bf16",
                     "alg_bytes_per_launch": alg_bytes3,
                     "avg_launch_ms": k3,
                     "avg_launch_from": k3_src,
                     "mfma_frac_of_kernel": flops / (k3 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "stream_reference": {"kernel": "torch.addcmul over q, k, v into a scratch tensor "
                                                    "(three reads and one write of the same sizes)",
                                          "ms": ref_ms, "GB/s": ref_gbs, "frac": ref_gbs / PEAK_HBM_GBS}},
    }
    return res, fwd


def _oracle_time(fn, budget_s: float = 3.0):
    """Seconds per call of an oracle function, repeated until about budget_s."""
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 50:
            return el / n


def run_extras(args, out):
    """Every hot-path row measured on its own against its roofline, with the
    CPU oracle timed beside it on a bounded sample (not the headline line)."""
    import numpy as np
    import torch

    import chunked_causal_linear_amd as la
    import oracle
    import workloads as wl
    from chunked_causal_linear_amd.accounting import Work, decode_bytes, phase1_bytes, scan_bytes

    rows = {"memory_ceilings": memory_ceilings()}
    hbm = lambda b, ms: {"GB/s": b / (ms * 1e-3) / 1e9, "frac_of_8TBs": b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}  # noqa

    def med_ms(fn, n=10):
        fn()
        torch.cuda.synchronize()
        return float(np.median(per_launch_ms(fn, n)))

    # ---- a1: feature maps
    w4, w5 = wl.WORKLOADS[4], wl.WORKLOADS[5]
    x, _, _, _ = wl.workload_inputs(w4, want_exact=False)
    xd = dev_bf16(x.bits)
    x_sample = wl.bf16_bits_to_f64(x.bits[0, :4096])
    n_el = xd.numel()
    y = torch.empty_like(xd)
    ms = med_ms(lambda: la.feature_map(xd, "elu1", out=y))
    rows["a1_elu1"] = {"shape": f"[{w4.BH},{w4.L},{w4.d_in}] bf16 -> bf16", "ms": ms, **hbm(4 * n_el, ms),
                       "bound": "hbm", "oracle_s_per_row": _oracle_time(
                           lambda: oracle.phi_elu1(x_sample)) / 4096}
    del xd, y, x
    q5, _, _, W5 = wl.workload_inputs(w5, want_exact=False)
    qd = dev_bf16(q5.bits)
    Wd = dev_bf16(W5[0])
    yf = torch.empty(w5.BH, w5.L, w5.m, dtype=torch.bfloat16, device="cuda")
    ms = med_ms(lambda: la.feature_map(qd, "favor", W=Wd, out=yf))
    fl = 2.0 * w5.BH * w5.L * w5.m * w5.d_in
    byt = qd.numel() * 2 + yf.numel() * 2
    Wx = W5[1]
    q_sample = wl.bf16_bits_to_f64(q5.bits[0, :2048])
    rows["a1_favor"] = {"shape": f"[{w5.BH},{w5.L},{w5.d_in}] x W[{w5.m},{w5.d_in}] -> bf16 [..,{w5.m}]", "ms": ms,
                        **hbm(byt, ms), "TFLOP/s": fl / (ms * 1e-3) / 1e12,
                        "mfma_frac": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "bound": "hbm",
                        "oracle_s_per_row": _oracle_time(lambda: oracle.phi_favor(q_sample, Wx)) / 2048}
    del qd, yf, q5
    torch.cuda.empty_cache()

    # ---- a2, a3: per-chunk states and their scan at the headline shape, C = 64
    w3 = wl.WORKLOADS[3]
    q, k, v, _ = wl.workload_inputs(w3, want_exact=False)
    kd, vd = dev_bf16(k.bits), dev_bf16(v.bits)
    C = 64
    N = w3.L // C
    S, _ = la.chunk_states(kd, vd, C)
    ms = med_ms(lambda: la.chunk_states(kd, vd, C, out=S))
    kh = wl.bf16_bits_to_f64(k.bits[0])
    vh = wl.bf16_bits_to_f64(v.bits[0])
    rows["a2_chunk_states"] = {"shape": f"BH={w3.BH} L={w3.L} d={w3.d_in} C={C}", "ms": ms,
                               **hbm(phase1_bytes(w3.BH, w3.L, w3.d_k, w3.d_v, C, False), ms), "bound": "hbm",
                               "oracle_s_per_head": _oracle_time(lambda: oracle.chunk_states(kh, vh, C))}
    S2 = S.clone()
    ms = med_ms(lambda: la.state_scan(S2, None, want_final=False))
    Sh = np.asarray(S[0].float().cpu(), dtype=np.float64)
    rows["a3_state_scan"] = {"shape": f"BH={w3.BH} N={N} d={w3.d_k}x{w3.d_v} fp32", "ms": ms,
                             **hbm(scan_bytes(w3.BH, N, w3.d_k, w3.d_v, False, False), ms), "bound": "hbm",
                             "oracle_s_per_head": _oracle_time(lambda: oracle.exclusive_scan(Sh))}
    del S, S2, Sh
    torch.cuda.empty_cache()

    # ---- a4: the forward at every workload and chunk size
    qd = dev_bf16(q.bits)
    qh3, kh3, vh3 = (wl.bf16_bits_to_f64(t.bits[0][:1024]) for t in (q, k, v))  # oracle sample (one head)
    del q, k, v
    fwd = {}
    for C in (32, 64, 128):
        f = la.Forward(qd, kd, vd, C)
        ms = row_time(f.run)
        wk = Work(w3.BH, w3.L, w3.d_in, w3.d_k, w3.d_v, C)
        fwd[f"w3_C{C}"] = {"ms": ms, "tokens_per_s": w3.B * w3.L / (ms * 1e-3), **hbm(wk.fused_bytes(), ms),
                           "TFLOP/s_page": wk.page_flops() / (ms * 1e-3) / 1e12}
        del f
    # the decayed recurrence (next row: Retention), headline shape, C = 64
    decay = {}
    f = la.Forward(qd, kd, vd, 64, gamma=0.99)
    ms = row_time(f.run)
    wk = Work(w3.BH, w3.L, w3.d_in, w3.d_k, w3.d_v, 64)
    decay["w3_C64_gamma0.99"] = {"ms": ms, "tokens_per_s": w3.B * w3.L / (ms * 1e-3), **hbm(wk.fused_bytes(), ms),
                                 "vs_no_decay": fwd["w3_C64"]["ms"] / ms,
                                 "oracle_s_per_head": _oracle_time(
                                     lambda: oracle.decay_chunked(qh3, kh3, vh3, 64, 0.99)) * w3.L / 1024,
                                 "oracle_sample": "oracle.decay_chunked on 1024 rows of one head, scaled to L"}
    del f
    qi, ki, vi = wl.random_case(33, w3.BH, w3.L, 128, 128, "i8")
    tq, tk, tv = (torch.from_numpy(t.bits).cuda() for t in (qi, ki, vi))
    del qi, ki, vi
    f = la.Forward(tq, tk, tv, 64)
    ms = row_time(f.run)
    wk = Work(w3.BH, w3.L, 128, 128, 128, 64, in_bytes=1, out_bytes=4)
    fwd["w3_int8_C64"] = {"ms": ms, "tokens_per_s": w3.B * w3.L / (ms * 1e-3), **hbm(wk.fused_bytes(), ms),
                          "TOP/s_page": wk.page_flops() / (ms * 1e-3) / 1e12}
    del f, tq, tk, tv, qd, kd, vd
    torch.cuda.empty_cache()
    decode = None
    for wid in (2, 4, 5):
        w = wl.WORKLOADS[wid]
        q, k, v, W = wl.workload_inputs(w, want_exact=False)
        qd, kd, vd = dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits)
        del q, k, v
        Wd = dev_bf16(W[0]) if W is not None else None
        C = w.chunks[0]
        f = la.Forward(qd, kd, vd, C, normalize=w.normalize, fmap=w.fmap, W=Wd, return_state=w.return_state)
        ms = row_time(f.run)
        wk = Work(w.BH, w.L, w.d_in, w.d_k, w.d_v, C, w.normalize, w.fmap)
        fwd[f"w{wid}"] = {"workload": w.name, "ms": ms, "tokens_per_s": w.B * w.L / (ms * 1e-3),
                          **hbm(wk.fused_bytes(w.return_state), ms),
                          "TFLOP/s_page": wk.page_flops() / (ms * 1e-3) / 1e12}
        if wid == 4:
            del f
            f = la.Forward(qd, kd, vd, C, normalize=w.normalize, fmap=w.fmap, W=Wd, return_state=w.return_state,
                           gamma=0.999)
            ms_d = row_time(f.run)
            decay["w4_gamma0.999"] = {"workload": w.name, "ms": ms_d, "tokens_per_s": w.B * w.L / (ms_d * 1e-3),
                                      **hbm(wk.fused_bytes(w.return_state), ms_d), "vs_no_decay": ms / ms_d}
        if wid == 5:
            # ---- a5: decode on 256 streams x 12 heads of 256 x 64 fp32 states
            n = wl.DECODE_STREAMS * w.H
            idx = torch.tensor([(s_ % w.B) * w.H + h for s_ in range(wl.DECODE_STREAMS) for h in range(w.H)],
                               device="cuda")
            S = f.S_final[idx].contiguous()
            z = f.z_final[idx].contiguous()
            pq, pk, pv = wl.decode_pool(w, n, pool=wl.DECODE_POOL)
            dq, dk_, dv_ = dev_bf16(pq.bits), dev_bf16(pk.bits), dev_bf16(pv.bits)
            o = torch.empty(n, w.d_v, dtype=torch.float32, device="cuda")
            state = {"t": 0}

            def step():
                t = state["t"] % wl.DECODE_POOL
                la.recurrent_step(dq[t], dk_[t], dv_[t], S, z, fmap="favor", W=Wd, normalize=True, out=o)
                state["t"] += 1
            ms_d = time_steps(step, args.decode_steps, 8)
            db = decode_bytes(n, w.d_in, w.d_k, w.d_v, True, m_proj=w.m)
            Sh = np.asarray(S[:64].cpu(), dtype=np.float64)
            zh = np.asarray(z[:64].cpu(), dtype=np.float64)
            Wx = W[1]
            qh = oracle.phi_favor(wl.bf16_bits_to_f64(pq.bits[0][:64]), Wx)
            kh = oracle.phi_favor(wl.bf16_bits_to_f64(pk.bits[0][:64]), Wx)
            vh = wl.bf16_bits_to_f64(pv.bits[0][:64])

            def oracle_step():
                for i in range(64):
                    oracle.recurrent_step(Sh[i], zh[i], qh[i], kh[i], vh[i], True)
            decode = {"states": n, "steps": args.decode_steps, "ms_per_step": ms_d,
                      "tokens_per_s": wl.DECODE_STREAMS / (ms_d * 1e-3), **hbm(db, ms_d), "bound": "hbm",
                      "note": "the 201 MB state set fits the 256 MB Infinity Cache: an effective rate",
                      "oracle_s_per_state_step": _oracle_time(oracle_step) / 64}
        del f, qd, kd, vd
        torch.cuda.empty_cache()
    rows["a4_forward"] = fwd
    rows["next_decay"] = decay
    # ---- next: log-linear attention at the headline shape (chunks of 64, random level weights)
    qd = dev_bf16(wl.full_tensor(3, wl.TENSOR_Q, w3.BH, w3.L, w3.d_in, "bf16", 1.0 / np.sqrt(w3.d_in), False).bits)
    kd = dev_bf16(wl.full_tensor(3, wl.TENSOR_K, w3.BH, w3.L, w3.d_in, "bf16", 1.0 / np.sqrt(w3.d_in), False).bits)
    vd = dev_bf16(wl.full_tensor(3, wl.TENSOR_V, w3.BH, w3.L, w3.d_v, "bf16", 1.0 / np.sqrt(w3.d_in), False).bits)
    nl = la.loglinear_levels(w3.L)
    lamd = torch.from_numpy(wl.loglinear_weights(3, w3.BH, w3.L, nl)).cuda()
    f = la.LogLinearForward(qd, kd, vd, lamd)
    ms = row_time(f.run)
    N = w3.L // 64
    pops = sum(bin(n).count("1") for n in range(N))
    state = w3.d_k * w3.d_v * 4
    wk3 = Work(w3.BH, w3.L, w3.d_in, w3.d_k, w3.d_v, 64)
    ll_bytes = (wk3.fused_bytes() + w3.BH * w3.L * nl * 4           # q, k, v, o and the level weights
                + w3.BH * w3.L * (w3.d_k + w3.d_v) * 2                # phase 1 reads k, v
                + w3.BH * N * state * 2                              # it writes N fp32 states, the pyramid reads them
                + w3.BH * (N - 1) * state // 2                       # and writes N - 1 bf16 nodes
                + w3.BH * (N // 2) * state                           # odd chunks read a level-1 bucket (fp32)
                + w3.BH * (pops - N // 2) * state // 2)              # and every chunk one bf16 node per higher set bit
    lq, lk, lv = (wl.head_tensor(3, t, 0, 1024, w3.d_in, "bf16", 1.0 / np.sqrt(w3.d_in)).exact for t in
                  (wl.TENSOR_Q, wl.TENSOR_K, wl.TENSOR_V))
    lam_h = wl.loglinear_weights(3, 1, 1024, oracle.loglinear_levels(1024))[0].astype(np.float64)
    rows["next_loglinear"] = {
        "shape": f"BH={w3.BH} L={w3.L} d={w3.d_in} C=64, {nl} levels", "ms": ms,
        "tokens_per_s": w3.B * w3.L / (ms * 1e-3), "vs_linear_forward": fwd["w3_C64"]["ms"] / ms,
        **hbm(ll_bytes, ms), "bytes": ll_bytes,
        "oracle_s_per_head": _oracle_time(lambda: oracle.loglinear_chunked(lq, lk, lv, lam_h, 64)) * w3.L / 1024,
        "oracle_sample": "oracle.loglinear_chunked on 1024 rows of one head, scaled to L"}
    # one decode step per head at position L - 1 = 8191 (twelve levels above
    # level 0 hold keys: the step reads thirteen level states and writes two)
    t_step = w3.L - 1
    qs_, ks_, vs_ = (x[:, t_step].contiguous() for x in (qd, kd, vd))
    lam_s = lamd[:, t_step].contiguous()
    S_ll = torch.randn(w3.BH, nl, w3.d_k, w3.d_v, device="cuda")
    o_ll = torch.empty(w3.BH, w3.d_v, device="cuda")
    step = lambda: la.recurrent_step_loglinear(qs_, ks_, vs_, lam_s, S_ll, t_step, out=o_ll)  # noqa: E731
    ms_step = med_ms(step, 20)
    n_read = 1 + bin(t_step >> 1).count("1")  # level 0 (merged into level 1) and the set bits above
    step_bytes = w3.BH * (n_read + 2) * w3.d_k * w3.d_v * 4
    lq1, lk1, lv1 = (x.exact for x in wl.head_inputs(w3, 0, 64))
    lam1 = wl.loglinear_weights(3, 1, 64, oracle.loglinear_levels(64))[0].astype(np.float64)
    rows["next_loglinear"]["decode_step"] = {
        "states": w3.BH, "position": t_step, "levels_read": n_read, "ms": ms_step, **hbm(step_bytes, ms_step),
        "bytes": step_bytes,
        "oracle_s_per_state_step": _oracle_time(lambda: oracle.loglinear_recurrent(lq1, lk1, lv1, lam1)) / 64,
        "oracle_sample": "oracle.loglinear_recurrent over 64 positions of one head (d = 128)"}
    # the level states after the whole sequence (a prefill for the decode)
    ms_pre = med_ms(lambda: la.loglinear_prefix_levels(kd, vd, nl), 10)
    n_ch = (w3.L - 1) // 64
    pre_bytes = (w3.BH * w3.L * (w3.d_k + w3.d_v) * 2 + 2 * w3.BH * n_ch * w3.d_k * w3.d_v * 4
                 + w3.BH * nl * w3.d_k * w3.d_v * 4)
    rows["next_loglinear"]["prefix_levels"] = {
        "heads": w3.BH, "L": w3.L, "levels": nl, "ms": ms_pre, **hbm(pre_bytes, ms_pre), "bytes": pre_bytes,
        "note": "k, v read by phase 1 (chunks of 64), chunk states written and read once, the levels written"}
    # the forward that also leaves the level states (one pyramid node per level of 2 chunks or more)
    fl = la.LogLinearForward(qd, kd, vd, lamd, state_levels=nl)
    ms_fl = row_time(fl.run)
    rows["next_loglinear"]["forward_with_levels"] = {
        "ms": ms_fl, "extra_ms_over_forward": ms_fl - ms,
        "saved_ms_vs_forward_then_prefix_levels": ms + ms_pre - ms_fl,
        "note": "the levels gathered from the forward's own chunk states and pyramid (no second pass over k, v)"}
    del f, fl, qd, kd, vd, lamd, S_ll
    torch.cuda.empty_cache()
    # ---- next: the delta rule and its gated form at the headline shape (chunks of 64)
    delta = {}
    C = 64
    n_ch = (w3.L + C - 1) // C
    # matrix-core work per chunk and head: K K^T, Q K^T, T R, the intra product
    # (4 C^2 d), K P, Q P, K^T U (3 C d^2) and the substitution (C^3 / 2)
    d_flops = 2 * (4 * C * C * w3.d_k + 3 * C * w3.d_k * w3.d_v + C ** 3 // 2) * n_ch * w3.BH
    # bytes: q, k, v, o; k again for the transform; T written once and read by each value
    # tile; the gate logs written and read by each value tile; beta (and alpha) read once
    n_vt = w3.d_v // 64
    d_bytes = w3.BH * (w3.L * (3 * w3.d_k + 2 * w3.d_v) * 2 + n_ch * C * C * 2 * (1 + n_vt)
                       + n_ch * C * 4 * (1 + n_vt))
    for gated in (False, True):
        q, k, v, beta, alpha = wl.delta_inputs(3, w3.BH, w3.L, w3.d_k, w3.d_v, gated, want_exact=False)
        bd = torch.from_numpy(beta).cuda()
        ad = torch.from_numpy(alpha).cuda() if gated else None
        qd, kd, vd = dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits)
        del q, k, v
        f = la.DeltaForward(qd, kd, vd, bd, ad, return_state=True)
        ms = row_time(f.run)
        nb = d_bytes + w3.BH * w3.L * 4 * (2 if gated else 1)
        ent = {"ms": ms, "tokens_per_s": w3.B * w3.L / (ms * 1e-3), **hbm(nb, ms),
               "TFLOP/s": d_flops / (ms * 1e-3) / 1e12, "vs_linear_forward": fwd["w3_C64"]["ms"] / ms}
        if gated:
            # one decode step on the 128 final states (128 x 128 fp32), from the forward's last token
            S, t0 = f.S_final, w3.L - 1
            o = torch.empty(w3.BH, w3.d_v, dtype=torch.float32, device="cuda")
            qs, ks, vs = (x[:, t0].contiguous() for x in (qd, kd, vd))
            bs, as_ = bd[:, t0].contiguous(), ad[:, t0].contiguous()
            ms_d = row_time(lambda: la.recurrent_step_delta(qs, ks, vs, S, bs, as_, out=o))
            delta["decode_128_states"] = {"ms": ms_d, **hbm(w3.BH * w3.d_k * w3.d_v * 4 * 2, ms_d)}
            qh_, kh_, vh_, bh_, ah_ = wl.delta_head_inputs(3, 0, 1024, w3.d_k, w3.d_v, True)
            ent["oracle_s_per_head"] = _oracle_time(
                lambda: oracle.delta_chunked(qh_, kh_, vh_, bh_.astype(np.float64), ah_.astype(np.float64), C)) \
                * w3.L / 1024
            ent["oracle_sample"] = "oracle.delta_chunked on 1024 rows of one head, scaled to L"
        delta["w3_gated" if gated else "w3"] = ent
        del f, qd, kd, vd, bd, ad
        torch.cuda.empty_cache()
    rows["next_delta"] = delta
    # ---- next: FAVOR+ against exact softmax (the linear-attention page's error study)
    qf, kf, vf = wl.favor_study_inputs()
    dd = qf.exact.shape[2]
    ref = oracle.softmax_attention(qf.exact[0], kf.exact[0], vf.exact[0], False)
    study = {}
    for m in (16, 32, 64, 128, 256):
        errs = []
        for t in range(4):
            Wb, _ = wl.orthogonal_random_features(m, dd, [70, m, t])
            fo = la.chunked_forward(dev_bf16(qf.bits), dev_bf16(kf.bits), dev_bf16(vf.bits), 64, causal=False,
                                    normalize=True, fmap="favor", W=dev_bf16(Wb), in_scale=dd ** -0.25)
            errs.append(float(np.mean((fo.float().cpu().numpy()[0].astype(np.float64) - ref) ** 2)))
        study[str(m)] = float(np.mean(errs))
    ms_ = [int(m) for m in study]
    rows["next_favor_vs_softmax"] = {
        "inputs": "one head, n=128, d=64, N(0,1)*0.4 (the page's study shape), bf16; non-causal, normalised",
        "mse_by_m": study, "trials": 4,
        "loglog_slope": float(np.polyfit(np.log(ms_), np.log([study[str(m)] for m in ms_]), 1)[0]),
        "oracle_softmax_s": _oracle_time(lambda: oracle.softmax_attention(qf.exact[0], kf.exact[0], vf.exact[0]))}
    rows["a5_decode"] = decode
    out["rows"] = rows


ROWS = ("fwd_w3_C32", "fwd_w3_C64", "fwd_w3_C128", "fwd_w3_int8_C64", "states_w3_C64", "states_w3_C1024",
        "scan_w3_C64", "fmap_favor_w5", "fwd_w2", "fwd_w4", "fwd_w5", "decode_w5", "mfma_peak_bf16", "mfma_peak_i8",
        "copy_512MiB", "memory_ceilings", "delta_w3", "delta_w3_gated", "delta_decode_w3", "loglinear_w3",
        "loglinear_w3_levels")


def run_row(name: str, reps: int):
    """Run one hot-path row `reps` times after one untimed call, and nothing else
    (for rocprofv3 counter passes over a short program)."""
    import numpy as np
    import torch

    import chunked_causal_linear_amd as la
    import workloads as wl

    if name not in ROWS:
        raise SystemExit(f"unknown row {name}; one of {', '.join(ROWS)}")
    fn = None
    if name.startswith("mfma_peak"):
        for _ in range(reps):
            tf, ms = mfma_peak(0 if name.endswith("bf16") else 1)
        log(f"{name}: {tf:.1f} T(FL)OP/s, {ms:.3f} ms per probe launch")
        return
    if name == "copy_512MiB":
        copy_calibration()
        log(f"{name}: two 512 MiB device copies")
        return
    if name == "memory_ceilings":
        for _ in range(reps):
            log(json.dumps(memory_ceilings()))
        return
    w3 = wl.WORKLOADS[3]
    if name.startswith(("fwd_w3_C", "states_w3", "scan_w3")):
        q, k, v, _ = wl.workload_inputs(w3, want_exact=False)
        qd, kd, vd = dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits)
        del q, k, v
        if name.startswith("fwd_w3_C"):
            fn = la.Forward(qd, kd, vd, int(name.split("C")[-1])).run
        elif name.startswith("states_w3"):
            C = int(name.split("C")[-1])
            S, _ = la.chunk_states(kd, vd, C)
            fn = lambda: la.chunk_states(kd, vd, C, out=S)  # noqa: E731
        else:
            S, _ = la.chunk_states(kd, vd, 64)
            fn = lambda: la.state_scan(S, None, want_final=False)  # noqa: E731
    elif name.startswith("delta"):
        gated = name != "delta_w3"
        q, k, v, beta, alpha = wl.delta_inputs(3, w3.BH, w3.L, w3.d_k, w3.d_v, gated, want_exact=False)
        bd = torch.from_numpy(beta).cuda()
        ad = torch.from_numpy(alpha).cuda() if gated else None
        qd, kd, vd = dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits)
        del q, k, v
        if name == "delta_decode_w3":
            # one decode step on every head's final state of the forward (128 states of 128 x 128)
            f = la.DeltaForward(qd, kd, vd, bd, ad, return_state=True)
            f.run()
            S, t0 = f.S_final, w3.L - 1
            o = torch.empty(w3.BH, w3.d_v, dtype=torch.float32, device="cuda")
            qs, ks, vs = (x[:, t0].contiguous() for x in (qd, kd, vd))
            bs, as_ = bd[:, t0].contiguous(), ad[:, t0].contiguous()
            fn = lambda: la.recurrent_step_delta(qs, ks, vs, S, bs, as_, out=o)  # noqa: E731
        else:
            fn = la.DeltaForward(qd, kd, vd, bd, ad).run
    elif name.startswith("loglinear_w3"):
        # log-linear attention at the headline shape (chunks of 64, seeded level weights),
        # optionally also writing the level states after the last token
        q, k, v, _ = wl.workload_inputs(w3, want_exact=False)
        qd, kd, vd = dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits)
        del q, k, v
        nl = la.loglinear_levels(w3.L)
        lamd = torch.from_numpy(wl.loglinear_weights(3, w3.BH, w3.L, nl)).cuda()
        fn = la.LogLinearForward(qd, kd, vd, lamd, state_levels=nl if name.endswith("levels") else None).run
    elif name == "fwd_w3_int8_C64":
        qi, ki, vi = wl.random_case(33, w3.BH, w3.L, 128, 128, "i8")
        tq, tk, tv = (torch.from_numpy(t.bits).cuda() for t in (qi, ki, vi))
        fn = la.Forward(tq, tk, tv, 64).run
    elif name == "fmap_favor_w5":
        w5 = wl.WORKLOADS[5]
        q5, _, _, W5 = wl.workload_inputs(w5, want_exact=False)
        qd, Wd = dev_bf16(q5.bits), dev_bf16(W5[0])
        yf = torch.empty(w5.BH, w5.L, w5.m, dtype=torch.bfloat16, device="cuda")
        fn = lambda: la.feature_map(qd, "favor", W=Wd, out=yf)  # noqa: E731
    elif name in ("fwd_w2", "fwd_w4", "fwd_w5", "decode_w5"):
        w = wl.WORKLOADS[int(name[-1])]
        q, k, v, W = wl.workload_inputs(w, want_exact=False)
        qd, kd, vd = dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits)
        del q, k, v
        Wd = dev_bf16(W[0]) if W is not None else None
        f = la.Forward(qd, kd, vd, w.chunks[0], normalize=w.normalize, fmap=w.fmap, W=Wd,
                       return_state=w.return_state)
        fn = f.run
        if name == "decode_w5":
            f.run()
            n = wl.DECODE_STREAMS * w.H
            idx = torch.tensor([(s_ % w.B) * w.H + h for s_ in range(wl.DECODE_STREAMS) for h in range(w.H)],
                               device="cuda")
            S = f.S_final[idx].contiguous()
            z = f.z_final[idx].contiguous()
            pq, pk, pv = wl.decode_pool(w, n, pool=wl.DECODE_POOL)
            dq, dk_, dv_ = dev_bf16(pq.bits), dev_bf16(pk.bits), dev_bf16(pv.bits)
            o = torch.empty(n, w.d_v, dtype=torch.float32, device="cuda")
            state = {"t": 0}

            def fn():
                t = state["t"] % wl.DECODE_POOL
                la.recurrent_step(dq[t], dk_[t], dv_[t], S, z, fmap="favor", W=Wd, normalize=True, out=o)
                state["t"] += 1
    fn()
    torch.cuda.synchronize()
    ms = per_launch_ms(fn, reps)
    log(f"{name}: {reps} calls, median {float(np.median(ms)):.4f} ms per call")


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_I8",
                 "SQ_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE", "GRBM_COUNT")
N_XCD, N_SIMD = 8, 1024  # MI355X: GRBM_GUI_ACTIVE is summed over the 8 XCDs; 256 CUs x 4 SIMDs


def pmc_summary(dirs):
    """Per-kernel table from rocprofv3 --pmc counter_collection.csv files (one
    directory per --row run): mean over dispatches of the kernel duration, the
    matrix-core busy fraction SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x
    1024 SIMDs) and the executed matrix-core work (SQ_INSTS_VALU_MFMA_MOPS_* x 512)."""
    import csv
    import glob
    from collections import defaultdict
    lines = [f"{'row':18s} {'kernel':62s} {'disp':>4s} {'avg_us':>8s} {'clk_GHz':>7s} {'mfma_busy':>9s} "
             f"{'bf16_GFLOP':>10s} {'i8_GOP':>8s} {'exec_TFLOP/s':>12s}"]
    for d in dirs:
        row = os.path.basename(os.path.normpath(d))
        row = row[4:] if row.startswith("pmc_") else row
        files = glob.glob(os.path.join(d, "*counter_collection.csv"))
        if not files:
            continue
        vals = defaultdict(lambda: defaultdict(list))
        dur = defaultdict(dict)
        for r in csv.DictReader(open(files[0])):
            name = r["Kernel_Name"].replace("void ", "")
            k = name[:name.rfind("(")] if name.endswith(")") else name
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[k][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for k, c in vals.items():
            mean = lambda n: sum(c[n]) / len(c[n]) if c[n] else 0.0  # noqa: E731
            t_ns = sum(dur[k].values()) / len(dur[k])
            gui = mean("GRBM_GUI_ACTIVE") / N_XCD
            busy = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (gui * N_SIMD) if gui else 0.0
            bf = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
            i8 = mean("SQ_INSTS_VALU_MFMA_MOPS_I8") * 512
            lines.append(f"{row:18s} {k[:62]:62s} {len(dur[k]):4d} {t_ns / 1e3:8.1f} {gui / t_ns:7.2f} "
                         f"{busy:9.3f} {bf / 1e9:10.2f} {i8 / 1e9:8.2f} {(bf + i8) / t_ns / 1e3:12.1f}")
    return "\n".join(lines)


def traffic_summary(fetch_dir: str, write_dir: str, chunk: int, group: int, commands: list) -> str:
    """The HBM traffic file of the dominant kernel from two rocprofv3 --pmc runs
    of `bench.py --copy-calibration` (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch).  Each counter is scaled by what it reads for the run's last two
    dispatches of the runtime's copy kernel: the two plain 512 MiB copies that
    end the program, factor = 524288 KiB / their mean reading."""
    import csv
    import glob

    def read(d, counter):
        f = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
        kern, copies, name = [], [], None
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            if "chunked_fwd_pipe" in r["Kernel_Name"]:
                kern.append(float(r["Counter_Value"]))
                name = r["Kernel_Name"].replace("void ", "").split("(")[0]
            elif "copyBuffer" in r["Kernel_Name"]:
                copies.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        copies.sort()
        cal = [v for _, v in copies[-2:]]
        return name, kern, sum(cal) / len(cal)

    name, kf, cf = read(fetch_dir, "FETCH_SIZE")
    _, kw, cw = read(write_dir, "WRITE_SIZE")
    ff, wf = 524288.0 / cf, 524288.0 / cw
    fetch, write = sum(kf) / len(kf), sum(kw) / len(kw)
    per_launch = (fetch * ff + write * wf) * 1024
    alg = 1073741824  # q, k, v read and o written once: 4 x 8 x 16 x 8192 x 128 x 2 B
    lines = ["# HBM traffic of chunked_fwd_pipe (phase 3), bench.py headline: identity map, "
             "B=8 H=16 L=8192 d=128, bf16",
             "# commands (repo root; each pass its own run):"]
    lines += [f"#   {c}" for c in commands]
    lines += ["# calibration: the same runs end with a plain device copy of 512 MiB (bench.py --copy-calibration);",
              "# factor = 524288 KiB / what the counter reads for that copy.",
              "# bytes_per_launch = (FETCH_SIZE * fetch_factor + WRITE_SIZE * write_factor) * 1024, "
              "mean over dispatches.",
              "# written by: python3 bench.py --traffic-summary <fetch dir> <write dir>",
              f"kernel: {name}", f"kernel_hash: {kernel_hash()}",
              f"chunk: {chunk}", f"group: {group}",
              f"dispatches_fetch: {len(kf)}", f"dispatches_write: {len(kw)}",
              f"fetch_kib_per_dispatch: {fetch:.1f}", f"write_kib_per_dispatch: {write:.1f}",
              f"copy_fetch_kib: {cf:.1f}", f"copy_write_kib: {cw:.1f}",
              f"fetch_factor: {ff:.4f}", f"write_factor: {wf:.4f}",
              f"bytes_per_launch: {per_launch:.0f}", f"algorithmic_bytes_per_launch: {alg}",
              f"traffic_over_algorithmic: {per_launch / alg:.4f}"]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=64)
    ap.add_argument("--group", type=int, default=0)
    ap.add_argument("--extra", action="store_true", help="also time the other workloads and chunk sizes")
    ap.add_argument("--decode-steps", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--spinup", type=float, default=0.5,
                    help="seconds of untimed forward calls before the warmup steps (GPU clock ramp)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with a plain 512 MiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--row", default=None,
                    help="run only this row REPS times (for counter passes): " + ", ".join(ROWS))
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--pmc-summary", nargs="+", default=None, metavar="DIR",
                    help="print the matrix-core counter table of rocprofv3 --pmc runs of --row (no GPU needed)")
    ap.add_argument("--traffic-summary", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the headline kernel's HBM traffic file from rocprofv3 --pmc FETCH_SIZE and "
                         "WRITE_SIZE runs of bench.py --copy-calibration (no GPU needed)")
    args = ap.parse_args()
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary))
        return
    if args.traffic_summary:
        fetch_dir, write_dir = (os.path.relpath(d, ROOT) for d in args.traffic_summary)
        cmd = ("rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python3 bench.py "
               "--steps 3 --warmup 1 --no-cpu-baseline --copy-calibration")
        text = traffic_summary(*args.traffic_summary, args.chunk, 8192 // args.chunk,
                               [cmd.format(c="FETCH_SIZE", d=fetch_dir), cmd.format(c="WRITE_SIZE", d=write_dir)])
        with open(TRAFFIC_FILE, "w") as fh:
            fh.write(text)
        print(text, end="")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.row is not None:
        run_row(args.row, args.reps)
        return
    res, fwd = run_headline(args)
    del fwd
    torch.cuda.empty_cache()
    if args.extra:
        run_extras(args, res)
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        import workloads as wl
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(wl.WORKLOADS[3], args.chunk)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
