"""Benchmark of the SVDQuant W4A4 + rank-r linear layer on one MI355X.

One step = one call of svdq_linear (smoothing + quantization + down-projection
kernel, then the W4A4 GEMM with the low-rank/bias/activation epilogue) on one
batch of synthetic, seeded DiT-shaped inputs already resident in HBM.  The
weights are packed once beforehand (offline, not timed).

Prints one JSON line.  value = effective TOPS = 2 M N K / t_step.
The roofline object describes the dominant kernel (the GEMM), timed with
HIP events over its own timed loop on the stream it runs on; the
cpu_baseline object times the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense 8-bit MFMA: INT8 5.0 POP/s, FP8 5.0 PFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense FP4 (and FP6) MFMA, 10.1 PFLOP/s
# The INT4 GEMM's group sums run on the FP6 (E2M3) form of the scaled matrix
# instruction, so its roofline is the FP6 peak; the fraction of the 8-bit peak
# (the reference the metric's name gives) is reported beside it.
PEAK_FP6_TFLOPS = PEAK_FP4_TFLOPS
# fp32 FMA lane-operations per second, from the published fp32 vector peak (157.3 TFLOP/s =
# 256 CUs x 4 SIMDs x 32 lanes x 2 flops x 2.4 GHz); two waves of a SIMD were measured
# issuing about 28 lanes of fp32 FMA per cycle together, so 16 lanes is not the ceiling
PEAK_VALU_TOPS = 256 * 4 * 32 * 2.4e9 / 1e12
CACHE_BYTES = 256 << 20      # Infinity Cache; rotating input sets exceed 2x this
METRIC = "effective TOPS (2MNK/t) of W4A4+rank-32 linear; % of INT8 MFMA / HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 50, or enough for ~20 ms of a short workload)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: about 0.1 s of the "
                         "workload's steps; the GPU clocks take 25-70 ms to settle after idle)")
    ap.add_argument("--workload", default="mlp_up",
                    choices=["tiny", "qkv", "mlp_up", "mlp_down", "awq_mod", "awq_mod_single",
                             "qkv_fused", "mlp_chain", "block", "mx_qkv", "mx_mlp_up",
                             "mx_mlp_down"])
    ap.add_argument("--M", type=int, default=None, help="override the token count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rank-overhead", action="store_true",
                    help="skip the r = 0 timing loops (cleaner kernel traces)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of a known size (counter calibration)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-small-m", action="store_true",
                    help="skip the 256-token case of the default line's layer shape")
    args = ap.parse_args()
    if args.warmup is None:
        # about 0.1 s of steps, so that the clocks have settled when the timed steps start
        args.warmup = WARMUP_STEPS.get(args.workload, 300)
    if args.steps is None:
        # short steps: enough of them that the host's start and stop cost little
        args.steps = TIMED_STEPS.get(args.workload, 50)
    return args


# Default warm-up steps per workload (≈ 0.1 s each at the measured step times).
WARMUP_STEPS = {"tiny": 3000, "qkv": 300, "mlp_up": 300, "mlp_down": 300, "awq_mod": 10000,
                "awq_mod_single": 10000, "qkv_fused": 300, "mlp_chain": 150, "block": 100,
                "mx_qkv": 600, "mx_mlp_up": 600, "mx_mlp_down": 600}
TIMED_STEPS = {"tiny": 1000, "awq_mod": 2000, "awq_mod_single": 2000}
SETTLE_S = 0.1               # untimed calls before each per-kernel timing loop (seconds)


def settle(fn, seconds=SETTLE_S):
    """Untimed calls of fn(i) for at least `seconds` of wall time: the GPU clocks take
    25-70 ms of load to settle after idle or after a lighter kernel."""
    import torch
    t0 = time.perf_counter()
    for i in range(4):
        fn(i)
    torch.cuda.synchronize()
    per = max((time.perf_counter() - t0) / 4, 1e-6)
    n = int(np.ceil(max(seconds - (time.perf_counter() - t0), 0.0) / per))
    for i in range(n):
        fn(4 + i)
    torch.cuda.synchronize()


def event_loop(fn, stream, n):
    """Seconds per call of fn over n back-to-back calls, HIP events on `stream` (the
    stream the kernels are launched on)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / n


def time_calls(fns, stream, n, reps=3):
    """Seconds per call of each fn in the dict `fns`: `reps` rounds in which every fn in
    turn is settled (SETTLE_S of untimed calls) and then timed over n calls; the median of
    its rounds.  Interleaving the rounds keeps one fn's figure from depending on the
    clocks left behind by the previous one."""
    got = {k: [] for k in fns}
    for _ in range(reps):
        for k, fn in fns.items():
            settle(fn)
            got[k].append(event_loop(fn, stream, n))
    return {k: float(np.median(v)) for k, v in got.items()}


def k1_bytes(M, K, r):
    G = K // 64
    return 2 * M * K + 4 * K + 2 * K * r + M * K // 2 + 4 * M * G + 4 * M * r


def k2_bytes(M, N, K, r):
    G = K // 64
    return (M * K // 2 + 4 * M * G + N * K // 2 + 4 * N * G + 4 * M * r + 2 * r * N + 2 * N
            + 2 * M * N)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a4_lr_gemm_qkv_traffic.txt")
_CSRC = os.path.join(ROOT, "bit_diffusion_transformer_amd", "csrc")
GEMM_SOURCE = tuple(os.path.join(_CSRC, f) for f in
                    ("w4a4_tile.h", "w4a4_gemm.hip", "svdq_device.h", "svdq_internal.h"))
K1_SOURCE = tuple(os.path.join(_CSRC, f) for f in
                  ("quant_down.hip", "svdq_device.h", "svdq_internal.h"))
# counter summaries of the default line's other kernels: K1 at the line's size, the
# GEMM at 256 tokens
K1_TRAFFIC = (os.path.join(ROOT, "profiles", "quantize_act_down_mlp_up_traffic.txt"), K1_SOURCE)
M256_TRAFFIC = (os.path.join(ROOT, "profiles", "w4a4_lr_gemm_quarter_mlp_up_m256_traffic.txt"),
                GEMM_SOURCE)


# workload -> (committed counter summary, kernel source it was taken with)
TRAFFIC = {
    "qkv": (None, None),
    "mlp_up": (os.path.join(ROOT, "profiles", "w4a4_lr_gemm_mlp_up_traffic.txt"), GEMM_SOURCE),
    "awq_mod": (os.path.join(ROOT, "profiles", "awq_w4a16_linear_mod_traffic.txt"),
                (os.path.join(_CSRC, "awq_w4a16.hip"),)),
    "mx_qkv": (os.path.join(ROOT, "profiles", "w4a4_mx_lr_gemm_qkv_traffic.txt"),
               (os.path.join(_CSRC, "w4a4_tile.h"), os.path.join(_CSRC, "w4a4_mx_gemm.hip"))),
}


def source_sha256(paths):
    """SHA-256 of the kernel's source files, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per call of the dominant kernel from the committed counter
    summary, if it was taken on this workload with the current kernel source;
    else None."""
    if workload not in TRAFFIC:
        return None
    path, source = TRAFFIC[workload]
    if path is None:
        path, source = TRAFFIC_FILE, GEMM_SOURCE
    return traffic_from(path, source)


def traffic_from(path, source):
    """traffic_bytes_per_call of a committed counter summary whose kernel_source_sha256
    matches the current source files; else None."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != source_sha256(source) or "traffic_bytes_per_call" not in kv:
        return None
    return int(float(kv["traffic_bytes_per_call"]))


def calibrate_copy():
    """A plain device-to-device copy of a known size, for scaling FETCH_SIZE and
    WRITE_SIZE counter readings to bytes."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}), flush=True)


def bench_awq(args):
    """The W4A16 (awq_w4a16) modulation projection: one step = one svdq_awq_w4a16_linear
    call; HBM-bound, so the metric is GB/s of its algorithmic bytes."""
    import torch

    import bit_diffusion_transformer_amd as bdt
    from synth import AWQ_CONFIGS, make_awq_layer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    spec = AWQ_CONFIGS[args.workload]
    L = make_awq_layer(spec, seed=0, M=args.M)
    M, K, N = L.spec.M, L.spec.K, L.spec.N
    W = torch.from_numpy(L.W).to(dev)
    packed = bdt.awq_pack_weights(W)
    del W
    X = torch.from_numpy(L.X.view(np.int16).copy()).to(dev)
    bias = torch.from_numpy(L.bias.view(np.int16).copy()).to(dev) if L.bias is not None else None
    nbytes = 2 * M * K + packed.numel() + (2 * N if bias is not None else 0) + 2 * M * N
    nsets = max(2, int(np.ceil(2 * CACHE_BYTES / nbytes)))
    sets = [(X.clone(), packed.clone(), bias.clone() if bias is not None else None,
             torch.empty((M, N), dtype=torch.int16, device=dev)) for _ in range(nsets)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(i):
        x, p, b, y = sets[i % nsets]
        bdt.svdq_awq_w4a16_linear(x, p, b, M, N, K, y, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    n_k = max(args.steps, 50)
    settle(step)
    t_k = event_loop(step, stream, n_k)
    gbs = nbytes / t_step / 1e9
    out = {
        "metric": "GB/s (algorithmic bytes / t) of the W4A16 modulation projection",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded conditioning vectors and random weights of the stated shape)",
        "config": {"workload": "%s: M=%d K=%d N=%d group=64 bias=%s (W4A16 records, %d B)"
                               % (spec.name, M, K, N, bias is not None, packed.numel()),
                   "global_batch": M, "input_sets_rotated": nsets},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / t_k / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / t_k / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(args.workload),
                     "kernel": "awq_linear_kernel", "avg_launch_us": round(t_k * 1e6, 2),
                     "algorithmic_bytes": nbytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        oracle.set_threads(cores)
        q, s_, z = oracle.awq_quantize(L.W)
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 2.0:    # whole layer, repeated ~2 s
            oracle.awq_linear(L.X, q, s_, z, L.bias)
            reps += 1
        tc = (time.perf_counter() - t0) / reps
        out["cpu_baseline"] = {"value": round(nbytes / tc / 1e9, 3), "unit": "GB/s",
                               "cores": cores, "kind": "oracle",
                               "sample": "the whole layer (all %d rows) x %d, %.3f s each"
                                         % (M, reps, tc)}
    print(json.dumps(out), flush=True)


def bench_qkv_fused(args):
    """The qkv projection with the fused QKV epilogue (per-head RMS norm + rotary turn of Q
    and K, [B, H, S, D] outputs): one step = one svdq_linear_qkv call.  Same metric as the
    default line (2MNK/t); the plain svdq_linear on the same inputs is timed beside it."""
    import torch

    import bit_diffusion_transformer_amd as bdt
    from synth import CONFIGS, make_layer, make_qkv_epilogue

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    spec = CONFIGS["qkv"]
    L = make_layer(spec, seed=0, M=args.M)
    M, K, N, r = L.spec.M, L.spec.K, L.spec.N, L.spec.r
    H, D = 24, 128
    assert N == 3 * H * D
    S = M                                   # one sequence of M tokens
    E = make_qkv_epilogue(H, D, S, cfg_id=40)

    def d(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    qw, sw = bdt.pack_weights(d(L.R))
    base = dict(X=d(L.X), lam=d(L.lam), L1=d(L.L1), L2=d(L.L2), bias=d(L.bias), qw=qw, sw=sw,
                gq=d(E.gamma_q), gk=d(E.gamma_k), cos=d(E.cos_t), sin=d(E.sin_t))
    ws_bytes = bdt.svdq_linear_workspace_bytes(M, K, r)
    set_bytes = (2 * M * K + qw.numel() + sw.numel() * 4 + 2 * M * N + ws_bytes
                 + 4 * K + 2 * K * r + 2 * r * N + 2 * N + 8 * S * (D // 2))
    nsets = max(2, int(np.ceil(2 * CACHE_BYTES / set_bytes)))
    bits = bdt._bits
    sets = []
    for _ in range(nsets):
        st = {k: v.clone() for k, v in base.items()}
        st["Q"], st["K"], st["V"] = (torch.empty((M // S, H, S, D), dtype=torch.bfloat16,
                                                 device=dev) for _ in range(3))
        st["Y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        st["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        st["epi"] = bdt.qkv_epilogue(H, D, S, bits(st["gq"]), bits(st["gk"]), E.eps, st["cos"],
                                     st["sin"], bits(st["Q"]), bits(st["K"]), bits(st["V"]))
        sets.append(st)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(i):
        st = sets[i % nsets]
        bdt.svdq_linear_qkv(bits(st["X"]), st["lam"], bits(st["L1"]), st["qw"], st["sw"],
                            bits(st["L2"]), bits(st["bias"]), M, K, r, st["epi"], st["ws"],
                            ws_bytes, stream)

    def plain(i):
        st = sets[i % nsets]
        bdt.svdq_linear(bits(st["X"]), st["lam"], bits(st["L1"]), st["qw"], st["sw"],
                        bits(st["L2"]), bits(st["bias"]), 0, M, N, K, r, bits(st["Y"]),
                        st["ws"], ws_bytes, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    ops = 2.0 * M * N * K

    carved = [bdt.quantize_act_down(st["X"], st["lam"], st["L1"]) for st in sets]
    torch.cuda.synchronize()

    def gemm_qkv(i):
        st, (qa, sa, xl1) = sets[i % nsets], carved[i % nsets]
        bdt.svdq_w4a4_lr_gemm_qkv(qa, sa, st["qw"], st["sw"], xl1, bits(st["L2"]),
                                  bits(st["bias"]), M, K, r, st["epi"], stream)

    def time_loop(fn, n):
        settle(fn)
        return event_loop(fn, stream, n)

    n_k = max(args.steps, 20)
    t_gq = time_loop(gemm_qkv, n_k)
    t_lin = time_loop(step, n_k)
    t_plain = time_loop(plain, n_k)
    gemm_tops = ops / t_gq / 1e12
    out = {
        "metric": METRIC, "value": round(ops / t_step / 1e12, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp6",
        "data": "synthetic (seeded DiT-shaped inputs, random weights of the stated shapes)",
        "config": {"workload": "qkv_fused: M=%d K=%d N=%d r=%d group=64 heads=%d head_dim=%d "
                               "seq=%d, Q/K RMS norm + rotary, [B,H,S,D] bf16 out"
                               % (M, K, N, r, H, D, S),
                   "global_batch": M, "input_sets_rotated": nsets},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_FP6_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_FP6_TFLOPS, 4),
                     "frac_of_int8_peak": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": None,
                     "kernel": "w4a4_lr_gemm_qkv_kernel (one launch per svdq_w4a4_lr_gemm_qkv call)",
                     "avg_launch_us": round(t_gq * 1e6, 2), "algorithmic_ops": ops},
        "fused_vs_plain": {"linear_qkv_us": round(t_lin * 1e6, 2),
                           "linear_plain_us": round(t_plain * 1e6, 2),
                           "epilogue_overhead": round(t_lin / t_plain - 1.0, 4)},
    }
    print(json.dumps(out), flush=True)


def mx_gemm_bytes(M, N, K, r):
    """Algorithmic bytes of one MXFP4 GEMM call: codes and E8M0 bytes of both
    operands, xl1, L2, bias once, Y once."""
    return (M * K // 2 + M * K // 32 + N * K // 2 + N * K // 32 + 4 * M * r + 2 * r * N + 2 * N
            + 2 * M * N)


def bench_mx(args):
    """The MXFP4 (4-bit float) variant of the layer: one step = one svdq_mx_linear call on
    the named workload's shapes.  Metric 2MNK/t as the default line; the INT4 svdq_linear
    on the same inputs is timed beside it."""
    import torch

    import bit_diffusion_transformer_amd as bdt
    from synth import CONFIGS, make_layer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    spec = CONFIGS[args.workload[3:]]
    L = make_layer(spec, seed=0, M=args.M)
    M, K, N, r, act = L.spec.M, L.spec.K, L.spec.N, L.spec.r, L.spec.act

    def d(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    R = d(L.R)
    qw, sw = bdt.mx_pack_weights(R)
    qw4, sw4 = bdt.pack_weights(R)
    del R
    base = dict(X=d(L.X), lam=d(L.lam), L1=d(L.L1), L2=d(L.L2), bias=d(L.bias), qw=qw, sw=sw,
                qw4=qw4, sw4=sw4)
    ws_bytes = max(bdt.svdq_mx_linear_workspace_bytes(M, K, r),
                   bdt.svdq_linear_workspace_bytes(M, K, r))
    set_bytes = (2 * M * K + qw.numel() + sw.numel() + 2 * M * N + ws_bytes
                 + 4 * K + 2 * K * r + 2 * r * N + 2 * N)
    nsets = max(2, int(np.ceil(2 * CACHE_BYTES / set_bytes)))
    bits = bdt._bits
    sets = []
    for _ in range(nsets):
        st = {k: (v.clone() if v is not None else None) for k, v in base.items()}
        st["Y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        st["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        sets.append(st)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(i):
        st = sets[i % nsets]
        bdt.svdq_mx_linear(bits(st["X"]), st["lam"], bits(st["L1"]), st["qw"], st["sw"],
                           bits(st["L2"]), bits(st["bias"]), act, M, N, K, r, bits(st["Y"]),
                           st["ws"], ws_bytes, stream)

    def int4(i):
        st = sets[i % nsets]
        bdt.svdq_linear(bits(st["X"]), st["lam"], bits(st["L1"]), st["qw4"], st["sw4"],
                        bits(st["L2"]), bits(st["bias"]), act, M, N, K, r, bits(st["Y"]),
                        st["ws"], ws_bytes, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    ops = 2.0 * M * N * K

    carved = [bdt.mx_quantize_act_down(st["X"], st["lam"], st["L1"]) for st in sets]
    down_ws = bdt.svdq_quantize_act_down_workspace_bytes(M, K, r)
    for st in sets:
        st["ws_down"] = torch.empty(max(down_ws, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def gemm(i):
        st, (qa, sa, xl1) = sets[i % nsets], carved[i % nsets]
        bdt.svdq_mx_lr_gemm(qa, sa, st["qw"], st["sw"], xl1, bits(st["L2"]), bits(st["bias"]),
                            act, M, N, K, r, bits(st["Y"]), stream)

    def quant(i):
        st, (qa, sa, xl1) = sets[i % nsets], carved[i % nsets]
        bdt.svdq_mx_quantize_act_down(bits(st["X"]), st["lam"], bits(st["L1"]), M, K, r, qa, sa,
                                      xl1, st["ws_down"], down_ws, stream)

    def time_loop(fn, n):
        settle(fn)
        return event_loop(fn, stream, n)

    n_k = max(args.steps, 20)
    t_gemm = time_loop(gemm, n_k)
    t_quant = time_loop(quant, n_k)
    t_lin = time_loop(step, n_k)
    t_int4 = time_loop(int4, n_k)
    gemm_tflops = ops / t_gemm / 1e12
    out = {
        "metric": METRIC, "value": round(ops / t_step / 1e12, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp4",
        "data": "synthetic (seeded DiT-shaped inputs, random weights of the stated shapes)",
        "config": {"workload": "%s: MXFP4 (E2M1, E8M0 per 32) M=%d K=%d N=%d r=%d act=%s "
                               "bias=%s" % (args.workload, M, K, N, r, "gelu" if act else "none",
                                            L.bias is not None),
                   "global_batch": M, "input_sets_rotated": nsets},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload) if args.M is None else None,
                     "kernel": "w4a4_mx_lr_gemm_kernel (one launch per svdq_mx_lr_gemm call)",
                     "avg_launch_us": round(t_gemm * 1e6, 2), "algorithmic_ops": ops,
                     "algorithmic_bytes": mx_gemm_bytes(M, N, K, r)},
        "quantize_act_down": {"us": round(t_quant * 1e6, 2)},
        "vs_int4": {"mx_linear_us": round(t_lin * 1e6, 2), "int4_linear_us": round(t_int4 * 1e6, 2),
                    "speedup": round(t_int4 / t_lin, 3)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_mx(L, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def _sized_run(run, M, target_s):
    """Rows of X (and whole-layer repeats) for about target_s seconds of oracle work.
    A call has a fixed part (the oracle unpacks the weight codes every call), so the
    row count is extrapolated from the marginal time per row of the last two runs;
    when the whole layer takes less than half the target it is repeated.  Returns
    (rows, repeats, seconds of the timed repeats)."""
    rows, prev = min(M, 16), None
    t = run(rows)
    for _ in range(3):
        if t >= target_s / 2 or rows >= M:
            break
        per_row = (t - prev[1]) / (rows - prev[0]) if prev and rows > prev[0] else t / rows
        nxt = int(min(M, max(rows + 1, rows + (target_s - t) / max(per_row, 1e-6))))
        prev = (rows, t)
        rows, t = nxt, run(nxt)
    reps = 1
    if rows >= M and t < target_s / 2:
        reps = max(1, int(round(target_s / max(t, 1e-3))))
        t = sum(run(rows) for _ in range(reps))
    return rows, reps, t


def cpu_baseline_mx(L, target_s):
    """The CPU oracle of the MXFP4 layer on a bounded sample (rows of X)."""
    import oracle
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    M, K, N, act = L.spec.M, L.spec.K, L.spec.N, L.spec.act
    qw, sw = oracle.mx_quantize(L.R)              # offline, not timed

    def run(rows):
        X = np.ascontiguousarray(L.X[:rows])
        t0 = time.perf_counter()
        oracle.mx_linear(X, L.lam, L.L1, qw, sw, L.L2, L.bias, act)
        return time.perf_counter() - t0

    rows, reps, t = _sized_run(run, M, target_s)
    return {"value": round(2.0 * rows * N * K * reps / t / 1e12, 5), "unit": "TOPS",
            "cores": cores, "kind": "oracle",
            "sample": "first %d of %d token rows of the same MXFP4 layer%s, %.1f s"
                      % (rows, M, " (%d runs)" % reps if reps > 1 else "", t)}


def bench_block(args):
    """One DiT block's four linears back to back (QKV 3072 -> 9216, out 3072 -> 3072, MLP up
    3072 -> 12288 with GELU, MLP down 12288 -> 3072; rank 32; 4608 tokens, or --M): one step =
    four svdq_linear calls on one stream, each layer on its own seeded inputs (not chained).
    Metric: the block's sum of 2 M N K over the step time; each layer's GEMM is also timed alone
    with HIP events, and the roofline line is the four GEMMs together against the 8-bit peak."""
    import torch

    import bit_diffusion_transformer_amd as bdt
    from synth import DIT_CHAIN, make_layer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    M = DIT_CHAIN[0].M if args.M is None else args.M
    specs = [s.with_M(M) for s in DIT_CHAIN]

    def d(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    layers = []
    for spec in specs:
        L = make_layer(spec, seed=0, M=M)
        qw, sw = bdt.pack_weights(d(L.R))
        layers.append(dict(spec=spec, X=d(L.X), lam=d(L.lam), L1=d(L.L1), L2=d(L.L2),
                           bias=d(L.bias), qw=qw, sw=sw))
        del L
    torch.cuda.synchronize()
    ws_bytes = max(bdt.svdq_linear_workspace_bytes(M, l["spec"].K, l["spec"].r) for l in layers)
    set_bytes = sum(sum(v.numel() * v.element_size() for k, v in l.items()
                        if k != "spec" and v is not None) + 2 * M * l["spec"].N for l in layers)
    nsets = max(2, int(np.ceil(2 * CACHE_BYTES / (set_bytes + ws_bytes))))
    bits = bdt._bits
    sets = []
    for _ in range(nsets):
        sets.append(dict(
            L=[{k: (v.clone() if (k != "spec" and v is not None) else v) for k, v in l.items()}
               for l in layers],
            Y=[torch.empty((M, l["spec"].N), dtype=torch.bfloat16, device=dev) for l in layers],
            ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def linear(st, j):
        l, sp = st["L"][j], st["L"][j]["spec"]
        bdt.svdq_linear(bits(l["X"]), l["lam"], bits(l["L1"]), l["qw"], l["sw"], bits(l["L2"]),
                        bits(l["bias"]), sp.act, M, sp.N, sp.K, sp.r, bits(st["Y"][j]), st["ws"],
                        ws_bytes, stream)

    def step(i):
        st = sets[i % nsets]
        for j in range(len(layers)):
            linear(st, j)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    ops = [2.0 * M * l["spec"].N * l["spec"].K for l in layers]

    # each layer's GEMM alone (inputs from one K1 per set), HIP events on the stream
    carved = [[bdt.quantize_act_down(l["X"], l["lam"], l["L1"]) for l in st["L"]] for st in sets]
    torch.cuda.synchronize()
    n_k = max(args.steps, 20)
    per = []
    for j, l0 in enumerate(layers):
        sp = l0["spec"]

        def gemm(i):
            st = sets[i % nsets]
            l, (qa, sa, xl1) = st["L"][j], carved[i % nsets][j]
            bdt.svdq_w4a4_lr_gemm(qa, sa, l["qw"], l["sw"], xl1, bits(l["L2"]), bits(l["bias"]),
                                  sp.act, M, sp.N, sp.K, sp.r, bits(st["Y"][j]), stream)

        settle(gemm)
        t = event_loop(gemm, stream, n_k)
        per.append({"layer": sp.name.replace("chain_", ""), "M": M, "K": sp.K, "N": sp.N,
                    "gemm_us": round(t * 1e6, 2), "gemm_tops": round(ops[j] / t / 1e12, 1)})
    t_gemms = sum(p["gemm_us"] for p in per) / 1e6
    achieved = sum(ops) / t_gemms / 1e12
    out = {
        "metric": "effective TOPS (sum of 2MNK / t) of one DiT block's four W4A4+rank-32 linears",
        "value": round(sum(ops) / t_step / 1e12, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp6",
        "data": "synthetic (seeded DiT-shaped inputs, random weights of the stated shapes)",
        "config": {"workload": "block: qkv 3072->9216, out 3072->3072, up 3072->12288 (GELU), "
                               "down 12288->3072; M=%d r=32 group=64" % M,
                   "global_batch": M, "input_sets_rotated": nsets},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP6_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP6_TFLOPS, 4),
                     "frac_of_int8_peak": round(achieved / PEAK_INT8_TOPS, 4),
                     "traffic": None,
                     "kernel": "w4a4_lr_gemm_kernel, the four layers' calls together",
                     "avg_launch_us": round(t_gemms * 1e6, 2), "algorithmic_ops": sum(ops)},
        "per_layer": per,
    }
    print(json.dumps(out), flush=True)


def bench_mlp_chain(args):
    """One DiT block's MLP (3072 -> 12288 GELU -> 3072, rank 32, 4608 tokens): one step =
    one svdq_mlp call (the up GEMM runs the down layer's activation step in its epilogue).
    Metric 2 M (K Nh + Nh K) / t; the unfused chain (svdq_linear twice, through the bf16
    intermediate) is timed beside it on the same inputs."""
    import torch

    import bit_diffusion_transformer_amd as bdt
    from synth import DIT_CHAIN, make_layer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    up_s, dn_s = DIT_CHAIN[2], DIT_CHAIN[3]
    M = up_s.M if args.M is None else args.M
    up, dn = make_layer(up_s, seed=0, M=M), make_layer(dn_s, seed=0, M=M)
    K, Nh, ru, rd = up_s.K, up_s.N, up_s.r, dn_s.r

    def d(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def layer(L):
        qw, sw = bdt.pack_weights(d(L.R))
        return dict(lam=d(L.lam), L1=d(L.L1), L2=d(L.L2), bias=d(L.bias), qw=qw, sw=sw)

    U0, D0 = layer(up), layer(dn)
    ws_mlp = bdt.svdq_mlp_workspace_bytes(M, K, Nh, ru, rd)
    ws_up = bdt.svdq_linear_workspace_bytes(M, K, ru)
    ws_dn = bdt.svdq_linear_workspace_bytes(M, Nh, rd)
    wbytes = sum(v.numel() * v.element_size() for L in (U0, D0) for v in L.values()
                 if v is not None)
    set_bytes = wbytes + 2 * M * K * 2 + 2 * M * Nh + max(ws_mlp, ws_up + ws_dn)
    nsets = max(2, int(np.ceil(2 * CACHE_BYTES / set_bytes)))
    bits = bdt._bits
    sets = []
    for _ in range(nsets):
        st = dict(U={k: (v.clone() if v is not None else None) for k, v in U0.items()},
                  D={k: (v.clone() if v is not None else None) for k, v in D0.items()},
                  X=d(up.X).clone(), Y=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
                  H=torch.empty((M, Nh), dtype=torch.bfloat16, device=dev),
                  ws=torch.empty(max(ws_mlp, ws_up, ws_dn), dtype=torch.uint8, device=dev))
        sets.append(st)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def fused(i):
        st = sets[i % nsets]
        U, D = st["U"], st["D"]
        bdt.svdq_mlp(bits(st["X"]), U["lam"], bits(U["L1"]), U["qw"], U["sw"], bits(U["L2"]),
                     bits(U["bias"]), D["lam"], bits(D["L1"]), D["qw"], D["sw"], bits(D["L2"]),
                     bits(D["bias"]), 1, M, K, Nh, ru, rd, bits(st["Y"]), st["ws"], ws_mlp,
                     stream)

    def unfused(i):
        st = sets[i % nsets]
        U, D = st["U"], st["D"]
        bdt.svdq_linear(bits(st["X"]), U["lam"], bits(U["L1"]), U["qw"], U["sw"], bits(U["L2"]),
                        bits(U["bias"]), 1, M, Nh, K, ru, bits(st["H"]), st["ws"], ws_up, stream)
        bdt.svdq_linear(bits(st["H"]), D["lam"], bits(D["L1"]), D["qw"], D["sw"], bits(D["L2"]),
                        bits(D["bias"]), 0, M, K, Nh, rd, bits(st["Y"]), st["ws"], ws_dn, stream)

    for i in range(args.warmup):
        fused(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fused(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    ops = 2.0 * M * K * Nh * 2

    def time_loop(fn, n):
        settle(fn)
        return event_loop(fn, stream, n)

    n_k = max(args.steps, 20)
    # the fused up GEMM alone (its inputs from one K1 per set)
    carved = [bdt.quantize_act_down(st["X"], st["U"]["lam"], st["U"]["L1"]) for st in sets]
    outs = [(torch.empty((bdt.pair_rows(M), Nh), dtype=torch.uint8, device=dev),
             torch.empty((M, Nh // 64), dtype=torch.float32, device=dev),
             torch.empty((M, rd), dtype=torch.float32, device=dev)) for _ in sets]
    ws_g = bdt.svdq_w4a4_lr_gemm_quant_down_workspace_bytes(M, Nh, rd)
    torch.cuda.synchronize()

    def up_fused(i):
        st, (qa, sa, xl1), (qn, sn, xn) = sets[i % nsets], carved[i % nsets], outs[i % nsets]
        U, D = st["U"], st["D"]
        bdt.svdq_w4a4_lr_gemm_quant_down(qa, sa, U["qw"], U["sw"], xl1, bits(U["L2"]),
                                         bits(U["bias"]), 1, M, Nh, K, ru, D["lam"],
                                         bits(D["L1"]), rd, qn, sn, xn, st["ws"], ws_g, stream)

    def up_plain(i):
        st, (qa, sa, xl1) = sets[i % nsets], carved[i % nsets]
        U = st["U"]
        bdt.svdq_w4a4_lr_gemm(qa, sa, U["qw"], U["sw"], xl1, bits(U["L2"]), bits(U["bias"]), 1,
                              M, Nh, K, ru, bits(st["H"]), stream)

    t_f = time_loop(fused, n_k)
    t_u = time_loop(unfused, n_k)
    t_gf = time_loop(up_fused, n_k)
    t_gp = time_loop(up_plain, n_k)
    ops_up = 2.0 * M * Nh * K
    out = {
        "metric": METRIC, "value": round(ops / t_step / 1e12, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp6",
        "data": "synthetic (seeded DiT-shaped inputs, random weights of the stated shapes)",
        "config": {"workload": "mlp_chain: M=%d %d -> %d (GELU) -> %d, r=%d/%d group=64"
                               % (M, K, Nh, K, ru, rd),
                   "global_batch": M, "input_sets_rotated": nsets},
        "roofline": {"bound": "mfma", "achieved": round(ops_up / t_gf / 1e12, 2),
                     "peak": PEAK_FP6_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ops_up / t_gf / 1e12 / PEAK_FP6_TFLOPS, 4),
                     "frac_of_int8_peak": round(ops_up / t_gf / 1e12 / PEAK_INT8_TOPS, 4), "traffic": None,
                     "kernel": "w4a4_lr_gemm_mlp_kernel + xl1 reduce (one "
                               "svdq_w4a4_lr_gemm_quant_down call)",
                     "avg_launch_us": round(t_gf * 1e6, 2), "algorithmic_ops": ops_up},
        "fused_vs_unfused": {"mlp_fused_us": round(t_f * 1e6, 2),
                             "mlp_unfused_us": round(t_u * 1e6, 2),
                             "speedup": round(t_u / t_f, 4),
                             "up_gemm_fused_us": round(t_gf * 1e6, 2),
                             "up_gemm_plain_us": round(t_gp * 1e6, 2)},
    }
    print(json.dumps(out), flush=True)


class LayerBench:
    """One layer's device inputs for bench.py: weights packed once (offline, not timed), and
    enough rotated copies of every input and output (> 2 x the 256 MB Infinity Cache in
    total) that no call is served its own inputs from the cache."""

    def __init__(self, L, dev):
        import torch

        import bit_diffusion_transformer_amd as bdt
        self.bdt, self.L = bdt, L
        M, K, N, r = L.spec.M, L.spec.K, L.spec.N, L.spec.r
        self.M, self.K, self.N, self.r, self.act = M, K, N, r, L.spec.act

        def d(a):
            if a is None:
                return None
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16).copy()).to(dev).view(torch.bfloat16)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        base = dict(X=d(L.X), lam=d(L.lam), L1=d(L.L1), L2=d(L.L2), bias=d(L.bias))
        qw, sw = bdt.pack_weights(d(L.R))
        torch.cuda.synchronize()
        base.update(qw=qw, sw=sw)
        self.ws_bytes = bdt.svdq_linear_workspace_bytes(M, K, r)
        self.down_ws = bdt.svdq_quantize_act_down_workspace_bytes(M, K, r)
        set_bytes = (2 * M * K + qw.numel() + sw.numel() * 4 + 2 * M * N + self.ws_bytes
                     + 4 * K + 2 * K * r + 2 * r * N + 2 * N)
        self.nsets = max(2, int(np.ceil(2 * CACHE_BYTES / set_bytes)))
        self.sets = []
        for _ in range(self.nsets):
            st = {k: (v.clone() if v is not None else None) for k, v in base.items()}
            st["Y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            st["ws"] = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
            st["ws_down"] = torch.empty(max(self.down_ws, 1), dtype=torch.uint8, device=dev)
            st["carved"] = bdt.quantize_act_down(st["X"], st["lam"], st["L1"] if r else None)
            self.sets.append(st)
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()

    def linear(self, i, rank=None):
        """One svdq_linear call on input set i (rank 0: the W4A4 layer without the branch)."""
        bits, st, r = self.bdt._bits, self.sets[i % self.nsets], self.r if rank is None else rank
        self.bdt.svdq_linear(bits(st["X"]), st["lam"], bits(st["L1"]) if r else None, st["qw"],
                             st["sw"], bits(st["L2"]) if r else None, bits(st["bias"]), self.act,
                             self.M, self.N, self.K, r, bits(st["Y"]), st["ws"], self.ws_bytes,
                             self.stream)

    def quant(self, i):
        """One svdq_quantize_act_down call (K1) on input set i."""
        bits, st, r = self.bdt._bits, self.sets[i % self.nsets], self.r
        qa, sa, xl1 = st["carved"]
        self.bdt.svdq_quantize_act_down(bits(st["X"]), st["lam"], bits(st["L1"]) if r else None,
                                        self.M, self.K, r, qa, sa, xl1, st["ws_down"],
                                        self.down_ws, self.stream)

    def gemm(self, i, rank=None):
        """One svdq_w4a4_lr_gemm call (K2) on input set i's K1 outputs."""
        bits, st, r = self.bdt._bits, self.sets[i % self.nsets], self.r if rank is None else rank
        qa, sa, xl1 = st["carved"]
        self.bdt.svdq_w4a4_lr_gemm(qa, sa, st["qw"], st["sw"], xl1 if r else None,
                                   bits(st["L2"]) if r else None, bits(st["bias"]), self.act,
                                   self.M, self.N, self.K, r, bits(st["Y"]), self.stream)

    def per_kernel(self, n, rank_loops):
        """Per-call seconds of K1, K2 and the whole layer (and, with rank_loops, of K2 and the
        layer at r = 0), each settled and timed with HIP events, rounds interleaved."""
        fns = {"gemm": self.gemm, "quant": self.quant, "linear": self.linear}
        if rank_loops and self.r > 0:
            fns["gemm_r0"] = lambda i: self.gemm(i, 0)
            fns["linear_r0"] = lambda i: self.linear(i, 0)
        return time_calls(fns, self.stream, n)


def small_m_line(spec, dev, n):
    """The same layer shape at 256 tokens: K1, K2 and the whole layer per call; K2 against
    both rooflines (HBM bytes and FP6 MFMA ops), since 256 tokens sit near the ridge."""
    from synth import make_layer
    L = make_layer(spec, seed=0, M=256)
    lb = LayerBench(L, dev)
    t = lb.per_kernel(n, False)
    M, K, N, r = lb.M, lb.K, lb.N, lb.r
    ops, b2 = 2.0 * M * N * K, k2_bytes(M, N, K, r)
    t_hbm, t_mfma = b2 / (PEAK_HBM_GBS * 1e9), ops / (PEAK_FP6_TFLOPS * 1e12)
    out = {"M": M, "K": K, "N": N, "r": r, "input_sets_rotated": lb.nsets,
           "gemm_us": round(t["gemm"] * 1e6, 2),
           "gemm_algorithmic_bytes": b2,
           "gemm_GB/s": round(b2 / t["gemm"] / 1e9, 1),
           "gemm_hbm_frac": round(t_hbm / t["gemm"], 4),
           "gemm_mfma_frac": round(t_mfma / t["gemm"], 4),
           "gemm_roofline_us": round(max(t_hbm, t_mfma) * 1e6, 2),
           "gemm_roofline_frac": round(max(t_hbm, t_mfma) / t["gemm"], 4),
           "quantize_act_down_us": round(t["quant"] * 1e6, 2),
           "quantize_act_down_hbm_frac": round(k1_bytes(M, K, r) / t["quant"] / 1e9
                                               / PEAK_HBM_GBS, 4),
           "linear_us": round(t["linear"] * 1e6, 2),
           "linear_tops": round(ops / t["linear"] / 1e12, 2),
           "kernel": "w4a4_lr_gemm_quarter_kernel (64 x 64 tiles, the tile policy's choice "
                     "at this size)",
           "gemm_traffic": traffic_from(*M256_TRAFFIC) if spec.name == "mlp_up" else None}
    del lb
    return out


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    extra = {"qkv_fused": bench_qkv_fused, "mlp_chain": bench_mlp_chain, "block": bench_block,
             "mx_qkv": bench_mx,
             "mx_mlp_up": bench_mx, "mx_mlp_down": bench_mx}
    if args.workload.startswith("awq") or args.workload in extra:
        if args.gpus != 1:
            print("bench.py runs on one GPU only (--gpus %d requested)" % args.gpus,
                  file=sys.stderr)
            sys.exit(2)
        (bench_awq if args.workload.startswith("awq") else extra[args.workload])(args)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the layer has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import CONFIGS, make_layer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    spec = CONFIGS[args.workload]
    L = make_layer(spec, seed=0, M=args.M)
    lb = LayerBench(L, dev)
    M, K, N, r, act = lb.M, lb.K, lb.N, lb.r, lb.act

    # ---------------- each kernel alone, HIP events on the stream they run on.  This runs
    # first, so the timed steps below also start on settled clocks.
    n_k = max(args.steps, 20)
    rank_loops = r > 0 and not args.no_rank_overhead
    t = lb.per_kernel(n_k, rank_loops)

    # ---------------- timed region: `warmup` untimed steps, then exactly `steps` steps
    for i in range(args.warmup):
        lb.linear(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        lb.linear(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    ops = 2.0 * M * N * K
    value = ops / t_step / 1e12

    t_gemm, t_quant, t_lin = t["gemm"], t["quant"], t["linear"]
    gemm_tops = ops / t_gemm / 1e12
    gemm_gbs = k2_bytes(M, N, K, r) / t_gemm / 1e9
    bound_mfma = ops / (PEAK_FP6_TFLOPS * 1e12) >= k2_bytes(M, N, K, r) / (PEAK_HBM_GBS * 1e9)
    if bound_mfma:
        roof = {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_FP6_TFLOPS,
                "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_FP6_TFLOPS, 4),
                "frac_of_int8_peak": round(gemm_tops / PEAK_INT8_TOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gemm_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gemm_gbs / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(args.workload) if args.M is None else None
    roof["kernel"] = "w4a4_lr_gemm_kernel (one launch per svdq_w4a4_lr_gemm call)"
    # the co-bound: the per-group rescale is one fp32 fma per output and group of 64 on the
    # VALU (the group sums leave the matrix unit as fp32, so there is no convert)
    valu_ops = 1.0 * M * N * (K // 64)
    roof["valu_rescale"] = {"lane_ops": valu_ops, "achieved": round(valu_ops / t_gemm / 1e12, 2),
                            "peak": round(PEAK_VALU_TOPS, 2), "unit": "Tops",
                            "frac": round(valu_ops / t_gemm / 1e12 / PEAK_VALU_TOPS, 4)}
    roof["avg_launch_us"] = round(t_gemm * 1e6, 2)
    roof["algorithmic_ops"] = ops
    roof["algorithmic_bytes"] = k2_bytes(M, N, K, r)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6",
        "data": "synthetic (seeded DiT-shaped inputs, random weights of the stated shapes)",
        "config": {"workload": "%s: M=%d K=%d N=%d r=%d group=64 act=%s bias=%s"
                               % (spec.name, M, K, N, r, "gelu" if act else "none",
                                  L.bias is not None),
                   "global_batch": M, "input_sets_rotated": lb.nsets},
        "roofline": roof,
        "rank_branch_overhead": None if "gemm_r0" not in t else {
            "gemm_r%d_us" % r: round(t_gemm * 1e6, 2), "gemm_r0_us": round(t["gemm_r0"] * 1e6, 2),
            "gemm_frac": round(t_gemm / t["gemm_r0"] - 1, 4),
            "linear_r%d_us" % r: round(t_lin * 1e6, 2),
            "linear_r0_us": round(t["linear_r0"] * 1e6, 2),
            "linear_frac": round(t_lin / t["linear_r0"] - 1, 4)},
        "quantize_act_down": {"us": round(t_quant * 1e6, 2),
                              "algorithmic_bytes": k1_bytes(M, K, r),
                              "GB/s": round(k1_bytes(M, K, r) / t_quant / 1e9, 1),
                              "hbm_frac": round(k1_bytes(M, K, r) / t_quant / 1e9 / PEAK_HBM_GBS, 4),
                              "traffic": (traffic_from(*K1_TRAFFIC)
                                          if args.workload == "mlp_up" and args.M is None
                                          else None)},
        "timing": {"linear_us": round(t_lin * 1e6, 2),
                   "per_kernel": "median of 3 interleaved rounds; each round %.1f s of untimed "
                                 "calls, then %d calls between HIP events" % (SETTLE_S, n_k),
                   # K1 + K2 back to back cannot take less than K2 alone
                   "consistent": bool(t_lin >= t_gemm)},
    }
    del lb
    torch.cuda.empty_cache()
    if args.M is None and not args.no_small_m and M > 256:
        out["m256"] = small_m_line(spec, dev, n_k)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(L, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline(L, target_s):
    """The CPU oracle on a bounded sample of the same layer (rows of X)."""
    import oracle
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    M, K, N, r, act = L.spec.M, L.spec.K, L.spec.N, L.spec.r, L.spec.act
    qw, sw = oracle.pack_weights(L.R)             # offline, not timed

    def run(rows):
        X = np.ascontiguousarray(L.X[:rows])
        t0 = time.perf_counter()
        oracle.linear(X, L.lam, L.L1, qw, sw, L.L2, L.bias, act)
        return time.perf_counter() - t0

    rows, reps, t = _sized_run(run, M, target_s)
    tops = 2.0 * rows * N * K * reps / t / 1e12
    return {"value": round(tops, 5), "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": "first %d of %d token rows of the same layer%s (whole layer per row: "
                      "smoothing, quantization, down-projection, W4A4 product, low-rank, "
                      "bias, act), %.1f s" % (rows, M, " (%d runs)" % reps if reps > 1 else "", t)}


if __name__ == "__main__":
    main()
