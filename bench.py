"""Benchmark of the MI355X MoE block forward (one JSON line on stdout).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5] [--decode-workload c2]
                    [--no-cpu-baseline]

A step is one whole moe_forward (router + top-k + permutation + gate_up/GLU +
down + combine) over one batch of seeded synthetic input already resident in
HBM.  The headline workload is the largest single-GPU one: the
gpt-oss-120b-shaped MoE block at prefill, T = 16384 tokens, H = I = 2880,
E = 128 experts, top-4, bf16 weights N(0, 0.02), biases N(0, 0.01), x scaled
so ~5% of gate/up pre-activations hit the clamp, router bias drawn Zipf(1.1)
over the experts (skewed loads, the hottest expert > 10x the mean), seed 0.
`value` is tokens per second of the whole job, from K steps run back to back
(warm caches) between two HIP events on the launch stream; `ms_per_step` is
that time / K.  The same workload's per-step p50 with the caches flushed
before every step is reported beside it (`cold_latency_us`).

Extra objects:
  roofline      the dominant kernel (the gate_up expert kernel, two thirds of
                the flops and bytes): algorithmic flops (prefill) or bytes
                (decode) per launch / its mean launch time, timed with HIP
                events on the stream it runs on;
  decode        the same measurement, compactly, for the decode batch
                (gpt-oss-20b block, T = 64, E = 32): tokens/s, the gate_up
                kernel's HBM roofline and the whole layer's;
  cpu_baseline  the float64 oracle timed on the host cores over the whole
                headline batch (a baseline, not the target).
Context fields: per-step latency percentiles with warm and with cold caches
(a 512 MiB buffer written before each cold step, outside its events), the
time per step of a HIP graph replaying one captured step, and what a plain
1 GiB copy and a bf16 8192^3 hipBLASLt GEMM reach on the same GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
METRIC = "MoE-layer tokens/sec + % of HBM or bf16 MFMA roofline on 1 MI355X"


def _alg_bytes_layer(cfg, D):
    """Bytes the method must move: weights and biases of the D live experts,
    the router, x read once and y written once."""
    H, I, E, T = cfg.H, cfg.I, cfg.E, cfg.T
    per_expert = H * 2 * I * 2 + I * H * 2 + 2 * I * 2 + H * 2
    return D * per_expert + E * H * 2 + E * 2 + 2 * T * H * 2


def _alg_bytes_gate_up(cfg, D):
    """gate_up launch: live experts' Wgu and bgu, x read once, h written once."""
    H, I, T, k = cfg.H, cfg.I, cfg.T, cfg.k
    return D * (H * 2 * I * 2 + 2 * I * 2) + T * H * 2 + T * k * I * 2


def _mx_bytes(K, N):
    """One MXFP4 weight [N][K]: 4-bit codes plus one scale byte per 32 values."""
    return N * K // 2 + N * K // 32


def _alg_bytes_layer_mxfp4(cfg, D):
    H, I, E, T = cfg.H, cfg.I, cfg.E, cfg.T
    per_expert = _mx_bytes(H, 2 * I) + _mx_bytes(I, H) + 2 * I * 2 + H * 2
    return D * per_expert + E * H * 2 + E * 2 + 2 * T * H * 2


def _alg_bytes_gate_up_mxfp4(cfg, D):
    H, I, T, k = cfg.H, cfg.I, cfg.T, cfg.k
    return D * (_mx_bytes(H, 2 * I) + 2 * I * 2) + T * H * 2 + T * k * I * 2


def _f8_bytes(K, N):
    """One FP8 weight [N][K]: one byte per value plus its float32 scale."""
    return N * K + 4


def _alg_bytes_layer_fp8(cfg, D):
    H, I, E, T = cfg.H, cfg.I, cfg.E, cfg.T
    per_expert = _f8_bytes(H, 2 * I) + _f8_bytes(I, H) + 2 * I * 2 + H * 2
    return D * per_expert + E * H * 2 + E * 2 + 2 * T * H * 2


def _alg_bytes_gate_up_fp8(cfg, D):
    H, I, T, k = cfg.H, cfg.I, cfg.T, cfg.k
    return D * (_f8_bytes(H, 2 * I) + 2 * I * 2) + T * H * 2 + T * k * I * 2


def _alg_flops_layer(cfg):
    H, I, E, T, k = cfg.H, cfg.I, cfg.E, cfg.T, cfg.k
    return T * (2 * H * E + k * (2 * H * 2 * I + 2 * I * H))


def _source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel_file, workload, stem=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken.
    stem names the summary when one source file holds several kernels."""
    stem = stem or kernel_file.split('/')[-1].split('.')[0]
    path = os.path.join(ROOT, "profiles", f"counters_{stem}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_digest") != _source_digest([kernel_file, "moe_layer_route_amd/csrc/device_common.h"]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, k, min_seconds=10.0, max_reps=3, mx_arrays=None, f8_arrays=None):
    """The float64 oracle on the host cores over the whole workload, repeated
    until about min_seconds of CPU time (at most max_reps runs).  mx_arrays /
    f8_arrays: the MXFP4 or FP8 inputs, timed through the oracle's forward for
    that format instead."""
    import numpy as np
    import oracle.moe_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas_pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max([i.get("num_threads", 1) for i in blas_pools] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in blas_pools})) or "unknown"
    except Exception:  # pragma: no cover
        cores, blas = 1, "unknown"
    times = []
    t_all = time.perf_counter()
    while len(times) < max_reps and (time.perf_counter() - t_all) < min_seconds:
        t0 = time.perf_counter()
        if mx_arrays is not None:
            orc.moe_forward_mxfp4(*mx_arrays, k=k)
        elif f8_arrays is not None:
            orc.moe_forward_fp8(*f8_arrays, k=k)
        else:
            orc.moe_forward(*inp.arrays(), k=k)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": inp.cfg.T / t, "unit": "tokens/s", "cores": int(cores), "kind": "oracle", "blas": blas,
            "sample": f"whole {inp.cfg.name} batch (T={inp.cfg.T}) through the float64 numpy oracle"
                      f"{' (MXFP4 weights)' if mx_arrays is not None else ''}"
                      f"{' (FP8 W8A8)' if f8_arrays is not None else ''}, "
                      f"median of {len(times)} runs of {t:.2f} s"}


def _per_step_us(torch, step, stream, n, before=None):
    """p10 / p50 / p90 of single steps, each between its own pair of events."""
    import numpy as np
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        if before is not None:
            before()
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return {"p10": float(np.percentile(us, 10)), "p50": float(np.percentile(us, 50)),
            "p90": float(np.percentile(us, 90)), "n": n}


def _achievable(torch):
    """What plain kernels reach on this GPU right now, as context for the
    roofline fractions (which use the published peaks): the library's
    hand-written streaming-read and MFMA probes, a 1 GiB device-to-device
    copy and a bf16 8192^3 torch.matmul (hipBLASLt)."""
    import numpy as np

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts))

    from moe_layer_route_amd import binding

    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    # hand-written streaming-read probe over the same 1 GiB (8192 workgroups of 128 KiB)
    rd = torch.empty(8192 * 4, dtype=torch.int32, device="cuda")
    t_read = timed(lambda: binding.probe_read(src, 8192, out=rd))
    del src, dst, rd
    # hand-written MFMA probe: 1024 workgroups x 4 waves x 4096 x 8 MFMAs 32x32x16 bf16
    mo = torch.empty(1024 * 4, dtype=torch.float32, device="cuda")
    t_mfma = timed(lambda: binding.probe_mfma_bf16(4096, 1024, out=mo))
    mfma_ok = bool((mo == 2048.0 * 4096).all().item())
    del mo
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    t_mm = timed(lambda: torch.matmul(a, b))
    del a, b
    return {"copy_1GiB_GBs": 2 * (1 << 30) / t_copy / 1e9, "matmul_bf16_8192_TFLOPs": 2 * n ** 3 / t_mm / 1e12,
            "probe_read_1GiB_GBs": (1 << 30) / t_read / 1e9,
            "probe_mfma_bf16_TFLOPs": 1024 * 4 * 4096 * 8 * 32768 / t_mfma / 1e12, "probe_mfma_check": mfma_ok}


def _timed_steps(torch, step, stream, steps):
    """Mean time of `steps` back-to-back steps between two events on `stream` (ms)."""
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def measure(args, name, headline=True):
    """Time one workload: the whole step, its latency percentiles (warm, cold,
    graph replay) and the dominant kernel.  Returns (record, inputs, format
    arrays for the oracle)."""
    import numpy as np
    import torch
    from moe_layer_route_amd import binding, datagen as d

    cfg = d.CONFIGS[name]
    inp = d.make_inputs(cfg, seed=0)
    print(f"[bench] inputs ready: {cfg.name} T={cfg.T} E={cfg.E}", file=sys.stderr, flush=True)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    x, Wr, br, Wgu, bgu, Wd, bd = [dev(a) for a in inp.arrays()]
    mx = args.weights == "mxfp4"
    f8 = args.weights == "fp8"
    mx_arrays = f8_arrays = None
    if f8:
        gq, gs, bgu_f, dq, ds, bd_f = d.make_experts_fp8(cfg, seed=0)
        f8_arrays = (inp.x, inp.Wr, inp.br, gq, gs, bgu_f, dq, ds, bd_f)
        Wgu_q, Wgu_s, Wd_q, Wd_s = [torch.from_numpy(a).cuda() for a in (gq, gs, dq, ds)]
        bgu, bd = dev(bgu_f), dev(bd_f)
        del Wgu, Wd
        print("[bench] FP8 expert weights ready", file=sys.stderr, flush=True)
    if mx:
        gq, gs, bgu_m, dq, ds, bd_m = d.make_experts_mxfp4(cfg, seed=0)
        mx_arrays = (inp.x, inp.Wr, inp.br, gq, gs, bgu_m, dq, ds, bd_m)
        Wgu_q, Wgu_s, Wd_q, Wd_s = [torch.from_numpy(a).cuda() for a in (gq, gs, dq, ds)]
        bgu, bd = dev(bgu_m), dev(bd_m)
        del Wgu, Wd
        print("[bench] MXFP4 expert weights ready", file=sys.stderr, flush=True)
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    ws = binding.alloc_workspace_fp8(T, H, E, k, I) if f8 else binding.alloc_workspace(T, H, E, k, I)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(st=None):
        if f8:
            binding.moe_forward_fp8(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k=k, y=y, workspace=ws,
                                    topk_ids=ids, topk_w=w, path=args.path,
                                    stream=st if st is not None else stream)
        elif mx:
            binding.moe_forward_mxfp4(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k=k, y=y, workspace=ws,
                                      topk_ids=ids, topk_w=w, path=args.path,
                                      stream=st if st is not None else stream)
        else:
            binding.moe_forward(x, Wr, br, Wgu, bgu, Wd, bd, k=k, y=y, workspace=ws, topk_ids=ids, topk_w=w,
                                path=args.path, stream=st if st is not None else stream)

    for _ in range(args.warmup):
        step()
    ms_per_step = _timed_steps(torch, step, stream, args.steps)
    print(f"[bench] {name}: timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    # Per-step latency: every step between its own pair of events, warm caches.
    lat = _per_step_us(torch, step, stream, args.steps)
    # Cold caches: a 512 MiB buffer is written before every step (outside the
    # events), which evicts the L2s and most of the MALL.
    flush = torch.empty(1 << 27, dtype=torch.float32, device="cuda")
    cold = _per_step_us(torch, step, stream, min(args.steps, 20), before=lambda: flush.fill_(1.0))
    del flush
    # One step captured in a HIP graph and replayed (the verify-pass setting).
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(side)
    stream.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    graph.replay()
    graph_ms = _timed_steps(torch, graph.replay, stream, args.steps)
    del graph
    # Four steps captured in one graph: the graph launch's fixed cost (about
    # 9 us before its first kernel) is paid once per four steps.
    graph4 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph4):
        for _ in range(4):
            step(torch.cuda.current_stream())
    graph4.replay()
    graph4_ms = _timed_steps(torch, graph4.replay, stream, max(1, args.steps // 4)) / 4
    del graph4
    print(f"[bench] {name}: per-step p50 {lat['p50']:.1f} us, cold p50 {cold['p50']:.1f} us, "
          f"graph replay {graph_ms * 1e3:.1f} us/step (4 steps per graph: {graph4_ms * 1e3:.1f})", file=sys.stderr,
          flush=True)

    # Dominant kernel: the same pipeline through the stage calls, with events
    # around every gate_up launch on the stream it is launched on.
    cnt, off, rows, pos = binding.moe_permute(ids, E, stream=stream)
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T * k, H), dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    if f8:
        xq = torch.empty((T, H), dtype=torch.uint8, device="cuda")
        sx = torch.empty((T,), dtype=torch.float32, device="cuda")
        hq = torch.empty((T * k, I), dtype=torch.uint8, device="cuda")
        sh = torch.empty((T * k,), dtype=torch.float32, device="cuda")

    def stage_step(ev=None):
        binding.moe_route(x, Wr, br, k, topk_ids=ids, topk_w=w, stream=stream)
        st = binding.library().moe_permute(binding._ptr(ids), T, E, k, binding._ptr(cnt), binding._ptr(off),
                                           binding._ptr(rows), binding._ptr(pos), binding._stream(stream))
        binding._check(st, "moe_permute")
        if f8:
            binding.moe_quantize_rows_fp8(x, codes=xq, scales=sx, stream=stream)
        if ev:
            ev[0].record(stream)
        if f8:
            binding.moe_gate_up_fp8(xq, sx, Wgu_q, Wgu_s, bgu, cnt, off, rows, k, h=h, path=args.path, stream=stream)
        elif mx:
            binding.moe_gate_up_mxfp4(x, Wgu_q, Wgu_s, bgu, cnt, off, rows, k, h=h, path=args.path, stream=stream)
        else:
            binding.moe_gate_up(x, Wgu, bgu, cnt, off, rows, k, path=args.path, h=h, stream=stream)
        if ev:
            ev[1].record(stream)
        if f8:
            binding.moe_quantize_rows_fp8(h, codes=hq, scales=sh, stream=stream)
            binding.moe_down_fp8(hq, sh, Wd_q, Wd_s, bd, cnt, off, T, k, o=o, path=args.path, stream=stream)
        elif mx:
            binding.moe_down_mxfp4(h, Wd_q, Wd_s, bd, cnt, off, T, k, o=o, path=args.path, stream=stream)
        else:
            binding.moe_down(h, Wd, bd, cnt, off, T, k, path=args.path, o=o, stream=stream)
        binding.moe_combine(o, pos, w, y=y, stream=stream)

    for _ in range(max(2, args.warmup // 2)):
        stage_step()
    torch.cuda.synchronize()
    for ev in evs:
        stage_step(ev)
    torch.cuda.synchronize()
    gate_up_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    D = int((torch.bincount(ids.reshape(-1).long(), minlength=E) > 0).sum().item())
    path = args.path if args.path != "auto" else binding.expert_path(T, E, k)
    gu_bytes = (_alg_bytes_gate_up_mxfp4(cfg, D) if mx else _alg_bytes_gate_up_fp8(cfg, D) if f8
                else _alg_bytes_gate_up(cfg, D))
    gu_flops = 2 * T * k * H * 2 * I
    gu_file = (f"moe_layer_route_amd/csrc/{'mxfp4' if path == 'gemv' else 'mxfp4_gemm'}.hip" if mx else
               f"moe_layer_route_amd/csrc/{'fp8' if path == 'gemv' else 'fp8_gemm'}.hip" if f8 else
               f"moe_layer_route_amd/csrc/{path}.hip")
    gu_stem = "fp8_gemv" if f8 and path == "gemv" else "fp8_gemm" if f8 else None
    traffic = _traffic(gu_file, cfg.name, stem=gu_stem)
    kernel = {("fp8", "gemv"): "gemv_fp8_kernel<gate_up>", ("fp8", "gemm"): "gemm_fp8_lds_kernel<gate_up>",
              ("mxfp4", "gemv"): "gemv_mxfp4_kernel<gate_up>", ("mxfp4", "gemm"): "gemm_mxfp4_kernel<gate_up>",
              ("bf16", "gemv"): "gemv_expert_kernel<gate_up>",
              ("bf16", "gemm"): "gemm_expert_kernel<gate_up>"}[(args.weights, path)]
    if path == "gemv":
        roofline = {"bound": "hbm", "kernel": kernel, "achieved": gu_bytes / (gate_up_ms * 1e-3) / 1e9,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roofline = {"bound": "mfma", "kernel": kernel, "achieved": gu_flops / (gate_up_ms * 1e-3) / 1e12,
                    "peak": FP8_PEAK_TFLOPS if f8 else BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roofline.update(frac=roofline["achieved"] / roofline["peak"], traffic=traffic,
                    alg_bytes_per_launch=gu_bytes, alg_flops_per_launch=gu_flops, launch_us=gate_up_ms * 1e3)
    layer_bytes = (_alg_bytes_layer_mxfp4(cfg, D) if mx else _alg_bytes_layer_fp8(cfg, D) if f8
                   else _alg_bytes_layer(cfg, D))
    mfma_peak = FP8_PEAK_TFLOPS if f8 else BF16_PEAK_TFLOPS
    layer_flops = _alg_flops_layer(cfg)
    step_s = ms_per_step * 1e-3
    rec = {
        "workload": f"{cfg.name}: {cfg.description}",
        "T": T, "H": H, "I": I, "E": E, "k": k, "seed": 0, "path": path, "live_experts": D,
        "weights": args.weights,
        "ms_per_step": ms_per_step,
        "tokens_per_s": T / step_s,
        "roofline": roofline,
        "layer": {"alg_bytes": layer_bytes, "alg_flops": layer_flops,
                  "hbm_GBs": layer_bytes / step_s / 1e9, "hbm_frac": layer_bytes / step_s / 1e9 / HBM_PEAK_GBS,
                  "tflops": layer_flops / step_s / 1e12,
                  "mfma_frac": layer_flops / step_s / 1e12 / mfma_peak},
        "latency_us": lat,
        "cold_latency_us": cold,
        "graph_ms_per_step": graph_ms,
        "graph4_ms_per_step": graph4_ms,
    }
    if not headline:
        return rec, None, None

    padded = None
    if args.n_valid is not None:
        nv_t = torch.tensor([args.n_valid], dtype=torch.int32, device="cuda")
        counts = torch.empty((E,), dtype=torch.int32, device="cuda")

        def pad_step():
            if mx or f8:
                (binding.moe_forward_padded_mxfp4 if mx else binding.moe_forward_padded_fp8)(
                    x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k=k, n_valid=nv_t, y=y, workspace=ws,
                    topk_ids=ids, topk_w=w, expert_counts=counts, path=args.path, stream=stream)
            else:
                binding.moe_forward_padded(x, Wr, br, Wgu, bgu, Wd, bd, k=k, n_valid=nv_t, y=y, workspace=ws,
                                           topk_ids=ids, topk_w=w, expert_counts=counts, path=args.path,
                                           stream=stream)

        for _ in range(args.warmup):
            pad_step()
        pad_ms = _timed_steps(torch, pad_step, stream, args.steps)
        nv = min(max(args.n_valid, 0), T)
        padded = {"n_valid": nv, "ms_per_step": pad_ms, "valid_tokens_per_s": nv / (pad_ms * 1e-3),
                  "live_experts": int((counts > 0).sum().item()), "max_expert_load": int(counts.max().item())}
        print(f"[bench] padded batch ({nv} of {T} rows valid): {pad_ms * 1e3:.1f} us/step", file=sys.stderr,
              flush=True)
    rec["padded"] = padded

    ep_share = None
    if args.ep > 1:
        nl = E // args.ep
        y_part = torch.empty((T, H), dtype=torch.float32, device="cuda")
        if mx or f8:
            local = [t[:nl] for t in (Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd)]
            ep_call = binding.moe_forward_ep_mxfp4 if mx else binding.moe_forward_ep_fp8
        else:
            local = [t[:nl] for t in (Wgu, bgu, Wd, bd)]
            ep_call = binding.moe_forward_ep

        def ep_step():
            ep_call(x, Wr, br, *local, 0, k=k, y_partial=y_part, workspace=ws, path=args.path, stream=stream)

        for _ in range(args.warmup):
            ep_step()
        ep_ms = _timed_steps(torch, ep_step, stream, args.steps)
        local_slots = int(((ids >= 0) & (ids < nl)).sum().item())
        ep_share = {"ranks": args.ep, "local_experts": nl, "local_slots": local_slots, "ms_per_step": ep_ms,
                    "tokens_per_s_per_rank": T / (ep_ms * 1e-3)}
        print(f"[bench] expert-parallel rank share ({nl} of {E} experts): {ep_ms * 1e3:.1f} us/step",
              file=sys.stderr, flush=True)
    rec["ep_rank_share"] = ep_share
    return rec, inp, (mx_arrays, f8_arrays)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5"],
                    help="headline workload (default c5, the largest single-GPU configuration)")
    ap.add_argument("--decode-workload", default="c2", choices=["none", "c1", "c2", "c3", "c4", "c5"],
                    help="second workload reported in the `decode` key (default c2, the decode batch)")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "gemm"])
    ap.add_argument("--weights", default="bf16", choices=["bf16", "mxfp4", "fp8"],
                    help="expert weight format: bf16 (moe_forward), MXFP4 W4A16 (moe_forward_mxfp4) or FP8 "
                         "W8A8 (moe_forward_fp8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-achievable", action="store_true", help="skip the copy / probe / hipBLASLt context")
    ap.add_argument("--ep", type=int, default=1,
                    help="also time one expert-parallel rank's share of W ranks: experts [0, E/W), "
                         "all tokens routed (reported in ep_rank_share, not in value)")
    ap.add_argument("--n-valid", type=int, default=None,
                    help="also time the padded forward (moe_forward_padded and its MXFP4 / FP8 forms) with this many "
                         "valid rows, the rest padding")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy, the reference kernel "
                         "that scales the rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    from moe_layer_route_amd import datagen as d

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.ep > 1 and d.CONFIGS[args.workload].E % args.ep:
        print(f"bench.py: E={d.CONFIGS[args.workload].E} is not divisible by --ep {args.ep}", file=sys.stderr)
        return 2

    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] copy probe: 1 GiB read + 1 GiB written", file=sys.stderr, flush=True)

    rec, inp, (mx_arrays, f8_arrays) = measure(args, args.workload, headline=True)
    torch.cuda.empty_cache()
    decode = None
    if args.decode_workload not in ("none", args.workload):
        decode, _, _ = measure(args, args.decode_workload, headline=False)
        torch.cuda.empty_cache()

    cfg = inp.cfg
    out = {
        "metric": METRIC,
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if args.weights == "fp8" else "bf16",
        "data": "synthetic (seeded normal bf16 inputs of the gpt-oss MoE block shapes; random-init weights)",
        "timing": "value and ms_per_step: K steps back to back (warm caches) between two HIP events on the "
                  "launch stream; cold_latency_us: per-step percentiles with a 512 MiB write before each step",
        "config": {k: rec[k] for k in ("workload", "T", "H", "I", "E", "k", "seed", "path", "live_experts",
                                        "weights")},
        "roofline": rec["roofline"],
        "layer": rec["layer"],
        "latency_us": rec["latency_us"],
        "cold_latency_us": rec["cold_latency_us"],
        "graph_ms_per_step": rec["graph_ms_per_step"],
        "graph4_ms_per_step": rec["graph4_ms_per_step"],
        "decode": decode,
        "achievable": None if args.no_achievable else _achievable(torch),
        "ep_rank_share": rec["ep_rank_share"],
        "padded": rec["padded"],
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, cfg.k, mx_arrays=mx_arrays, f8_arrays=f8_arrays)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
