#!/usr/bin/env python3
"""Benchmark of the masked-attention forward hot path on one MI355X.

One step = the whole path over one batch already resident in HBM:
  rk_mask_plan        (tile plan + launch schedule)
  rk_time_rope        (K rotated by time RoPE)
  rk_masked_attn_fwd  (Q rotated while staged; masked flash attention)
Steps are independent batches.  With --pipeline on the next step's plan
and K rotation run on a second stream while this step's attention runs
(double-buffered plan workspace and rotated keys); off runs each step's
three stages back to back on one stream; auto (default) pipelines when a
serial warmup step takes more than 1 ms.
The default workload is the TM20K-shaped batch (8 users x (20000 history +
1 target), causal, H = 8, d_head = 64, bf16, time RoPE).

Prints ONE JSON line.  `value` is the effective attention throughput of the
whole step: 4 * d_head * heads * (visible pairs) / step time.  The roofline
object is for the dominant kernel (the attention kernel), timed with HIP
events on the stream it runs on.  The CPU baseline times the fp64 oracle on a
bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import contextlib
import ctypes as C
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "masked-attn fwd effective TFLOP/s (visible pairs) + % bf16 MFMA peak; candidates/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ATTN_SRC = os.path.join(ROOT, "masked_attention_amd", "csrc", "attn_mfma.hip")
ATTN_KERNEL = "attn_mfma_bf16_kernel"



@contextlib.contextmanager
def _gc_paused():
    """Python's cyclic garbage collector held off over a timed region (as
    timeit does): a full pass over torch's object graph stalls the host for
    tens of milliseconds, which a step of a fraction of a millisecond cannot
    hide behind queued GPU work.  The collection itself runs before the
    warmup steps (_gc_before_warmup), so that the GPU is not left idle, and
    its clock low, just before the first timed step."""
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


def _gc_before_warmup():
    """One full collection ahead of the warmup steps (see _gc_paused)."""
    gc.collect()


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, help="named workload 1..5 (default 5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=4,
                    help="oracle sample: request 0 with this many heads")
    ap.add_argument("--candidates-only", action="store_true",
                    help="serving step: the history keys are rotated once before timing; each "
                         "step plans the candidates' query tiles only, rotates the candidate "
                         "keys into the key cache and runs the attention for those tiles")
    ap.add_argument("--qk-norm", action="store_true",
                    help="with QK Norm (RMSNorm of Q and K rows before the rotation): forward "
                         "with gains 1 (K normalised in its rotation pass, Q while staged); "
                         "with --backward, random gains and their gradients")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward step instead: the forward runs once (untimed) for "
                         "O and LSE; each step plans with the key-major tables and runs "
                         "rk_masked_attn_bwd (Q/K rotation, dQ kernel, dK/dV kernel)")
    ap.add_argument("--pointwise", action="store_true",
                    help="time HSTU pointwise attention (SiLU, rab tables of 128 position and 32 "
                         "time buckets, scale 1/sqrt(d)) on the workload instead: plan + "
                         "rk_pointwise_attn_fwd")
    ap.add_argument("--lazformer", action="store_true",
                    help="time LazFormer's attention stack instead: group-sum compression of "
                         "Q/K/V (2048 -> 1152), then per layer the pruned input gathered, "
                         "planned (window = global tail = 128) and attended, 5 layers")
    ap.add_argument("--pipeline", choices=("auto", "on", "off"), default="auto",
                    help="on: the next batch's plan and K rotation (double-buffered workspace "
                         "and rotated keys) run on a second stream while this batch's "
                         "attention runs; off: the three stages of a step run back to back on "
                         "one stream; auto (default): on when a serial warmup step takes more "
                         "than 1 ms (the cross-stream synchronisation costs more than the "
                         "overlap gains on shorter steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="no GPU work: print a summary of the rocprofv3 --kernel-trace --stats "
                         "output in DIR (needs --bench-line: the JSON line the profiled run "
                         "printed); the attention kernel is summarised over the timed launches")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "MFMA_DIR"),
                    help="no GPU work: write the attention kernel's calibrated HBM traffic and "
                         "MFMA-utilisation summaries under profiles/ from three rocprofv3 --pmc "
                         "runs (FETCH_SIZE; WRITE_SIZE; MFMA counters), each of a bench.py run "
                         "with --copy-calibration (needs --bench-line)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="measure the chip's sustained bf16 MFMA rate instead (a whole-chip loop "
                         "of v_mfma_f32_32x32x16_bf16 at 8 waves per SIMD, on constant and on "
                         "random operands; built with hipcc at run time)")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="matrix-core counters of every kernel in a rocprofv3 --pmc run "
                         "(GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES, SQ_WAVE_CYCLES, ...): "
                         "busy share, resident waves per SIMD and clock per kernel")
    ap.add_argument("--bench-line", metavar="FILE", help="file whose last line is a bench JSON line")
    ap.add_argument("--profile-cmd", action="append", default=[],
                    help="profiler command to record in a summary (repeatable)")
    return ap.parse_args()


def _profile_kv(kind: str, workload: str):
    """Key/value lines of profiles/attn_fwd_<kind>_<workload>.txt if that
    summary was taken on the current attention kernel source, else None."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{kind}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    return kv if kv.get("attn_source_sha256") == sha else None


def _traffic_from_profile(workload: str):
    """HBM bytes per attention launch from the committed PMC summary, if it
    was taken on the current kernel source; otherwise None."""
    kv = _profile_kv("hbm_traffic", workload)
    try:
        return float(kv["hbm_bytes_per_launch"]) if kv else None
    except (KeyError, ValueError):
        return None


def _mfma_util_from_profile(workload: str, attn_ms: float, achieved: float, flops: float):
    """MFMA busy share and the clock-adjusted peak fraction from the committed
    counter summary (current kernel source only): the kernel's active GPU
    cycles divided by this run's launch time give the clock it ran at."""
    kv = _profile_kv("mfma_util", workload)
    if not kv:
        return None
    try:
        cycles = float(kv["active_cycles_per_xcd"])
        clock_ghz = cycles / (attn_ms * 1e-3) / 1e9
        return {"mfma_busy_frac": float(kv["mfma_busy_frac"]),
                "useful_of_issued_flops": round(flops / float(kv["issued_flops"]), 4),
                "clock_ghz": round(clock_ghz, 3),
                "frac_clock_adjusted": round(achieved / (PEAK_BF16_TFLOPS * clock_ghz / 2.4), 4)}
    except (KeyError, ValueError):
        return None


PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector


def _roofline(dtype: str, flops: float, alg_bytes: int, ms: float, traffic):
    """Roofline of the attention kernel: the bound is whichever of the matrix
    cores (visible-pair FLOPs at the dense bf16 MFMA peak) and HBM (the
    algorithmic bytes at 8 TB/s) needs more time; the fp32 path runs on the
    vector ALUs.  The other bound's figures ride along under `other`."""
    sec = ms * 1e-3
    tf = flops / sec / 1e12
    gbs = alg_bytes / sec / 1e9
    peak_c = PEAK_FP32_TFLOPS if dtype == "f32" else PEAK_BF16_TFLOPS
    if dtype == "f32":
        main = {"bound": "alu", "kernel": "attn_ref_kernel", "achieved": round(tf, 3),
                "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_TFLOPS, 5)}
        other = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(gbs / PEAK_HBM_GBS, 5)}
    else:
        mf = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
              "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        hb = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": round(gbs / PEAK_HBM_GBS, 4)}
        hbm_first = alg_bytes / (PEAK_HBM_GBS * 1e9) > flops / (PEAK_BF16_TFLOPS * 1e12)
        main, other = (hb, mf) if hbm_first else (mf, hb)
        main = {"bound": main["bound"], "kernel": ATTN_KERNEL,
                **{k: v for k, v in main.items() if k != "bound"}}
    main.update({"traffic": traffic, "alg_bytes": alg_bytes,
                 "bound_time_us": {"alu" if dtype == "f32" else "mfma":
                                   round(flops / (peak_c * 1e12) * 1e6, 2),
                                   "hbm": round(alg_bytes / (PEAK_HBM_GBS * 1e9) * 1e6, 2)},
                 "other": other})
    return main


def _cpu_baseline(wl, n_heads: int):
    """Time the fp64 oracle, as it stands, on request 0 and heads 0..n_heads-1."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max(int(i.get("num_threads", 1)) for i in info) if info else 1
    except Exception:
        cores = len(os.sched_getaffinity(0))
    a, b = wl.request(0)
    pairs = oracle.count_visible(wl.seg_kind[a:b], wl.timestamps[a:b], delay=wl.delay,
                                 window=wl.window, static_bidirectional=wl.static_bidirectional)
    heads = list(range(min(n_heads, wl.heads)))
    rope = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)
    t0 = time.perf_counter()
    oracle.attention_forward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k, wl.v,
                             delay=wl.delay, window=wl.window,
                             static_bidirectional=wl.static_bidirectional, rope=rope,
                             heads=heads, requests=[0])
    dt = time.perf_counter() - t0
    flops = 4.0 * wl.d_head * pairs * len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"request 0 ({b - a} tokens, {pairs} visible pairs per head), heads "
                      f"0-{len(heads) - 1}, fp64 NumPy with explicit mask, {dt:.2f} s wall"}


def _cpu_baseline_bwd(wl, n_heads: int):
    """Time the fp64 oracle backward, as it stands, on request 0 and heads
    0..n_heads-1 (its forward statistics included)."""
    import oracle
    from rk_workloads import draw_grad
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max(int(i.get("num_threads", 1)) for i in info) if info else 1
    except Exception:
        cores = len(os.sched_getaffinity(0))
    a, b = wl.request(0)
    pairs = oracle.count_visible(wl.seg_kind[a:b], wl.timestamps[a:b], delay=wl.delay,
                                 window=wl.window, static_bidirectional=wl.static_bidirectional)
    heads = list(range(min(n_heads, wl.heads)))
    rope = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)
    do = draw_grad(wl)
    t0 = time.perf_counter()
    oracle.attention_backward(wl.req_offsets, wl.seg_kind, wl.timestamps, wl.q, wl.k, wl.v, do,
                              delay=wl.delay, window=wl.window,
                              static_bidirectional=wl.static_bidirectional, rope=rope,
                              heads=heads, requests=[0])
    dt = time.perf_counter() - t0
    flops = 10.0 * wl.d_head * pairs * len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"request 0 ({b - a} tokens, {pairs} visible pairs per head), heads "
                      f"0-{len(heads) - 1}, fp64 NumPy backward with explicit mask, "
                      f"{dt:.2f} s wall"}


def backward_main(args) -> int:
    """One JSON line for the backward step (effective FLOPs = 10 d per
    visible pair and head: the five d-wide products of the backward)."""
    import numpy as np
    import torch

    import masked_attention_amd as rk
    from rk_workloads import draw_grad, make_config

    torch.cuda.init()
    dev = torch.device("cuda:0")
    wl = make_config(args.config)
    H, d = wl.heads, wl.d_head
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    batch = rk.Batch.from_workload(wl, device=dev)
    q, k, v = (torch.from_numpy(x).to(dev).to(tdt) for x in (wl.q, wl.k, wl.v))
    do = torch.from_numpy(draw_grad(wl)).to(dev).to(tdt)
    rope = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)
    ws = torch.empty(rk.rk_plan_workspace_size(batch, H), dtype=torch.uint8, device=dev)
    mk = dict(delay=wl.delay, window=wl.window, static_bidirectional=wl.static_bidirectional,
              num_heads=H, backward=True, workspace=ws)
    plan = rk.Plan(batch, **mk)
    pairs = plan.stats()["visible_pairs"]
    norm = None
    if args.qk_norm:
        # QK Norm with gains (their gradients are part of the step)
        g = torch.Generator().manual_seed(11)
        norm = dict(eps=1e-6, gamma_q=(0.5 + torch.rand(d, generator=g)).to(dev),
                    gamma_k=(0.5 + torch.rand(d, generator=g)).to(dev))
    o, lse = rk.rk_masked_attn_fwd(plan, q, k, v, rope=rope, want_lse=True, qk_norm=norm)
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    bws = None
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        p = rk.Plan(batch, **mk)
        if ev: ev[1].record(stream)
        rk.rk_masked_attn_bwd(p, q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, rope=rope,
                              workspace=bws, qk_norm=norm)
        if ev: ev[2].record(stream)
        return p

    plans = [step()]
    from masked_attention_amd import _rk
    import ctypes as C
    a = rk.binding._bwd_args(q, k, v, o, do, lse, dq, dk, dv, 0.0,
                             rk.binding.rope_params(**rope), False, False, None)
    if norm is not None:
        nq = rk.binding.qk_norm_params(**norm)
        a.qk_norm = C.cast(C.pointer(nq), C.c_void_p)
        dgs = torch.empty(2 * d, dtype=torch.float32, device=dev)
        a.dgamma_q, a.dgamma_k = dgs.data_ptr(), dgs[d:].data_ptr()
    n = C.c_size_t()
    _rk.check(_rk.lib().rk_attn_bwd_workspace_size(plan.handle, C.byref(a), C.byref(n)), "ws")
    bws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
    _gc_before_warmup()
    for _ in range(args.warmup):
        plans.append(step())
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    with _gc_paused():
        t0 = time.perf_counter()
        for i in range(args.steps):
            plans.append(step(evs[i]))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    for p in plans:
        p.close()
    ms_step = (t1 - t0) * 1e3 / args.steps
    plan_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    flops = 10.0 * d * H * pairs
    achieved = flops / (bwd_ms * 1e-3) / 1e12
    out = {
        "metric": "masked-attn bwd effective TFLOP/s (visible pairs, 10 d FLOPs per pair and head)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded generator with the workload's shapes and time law)",
        "config": {"workload": wl.name + " backward" + (" qk-norm" if args.qk_norm else ""),
                   "requests": wl.num_requests,
                   "tokens": wl.total_tokens, "heads": H, "d_head": d,
                   "visible_pairs_per_head": pairs},
        "pct_bf16_peak": round(100.0 * flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "stage_ms": {"plan": round(plan_ms, 4), "backward": round(bwd_ms, 4)},
        "roofline": {"bound": "mfma", "kernel": "rk_masked_attn_bwd (Q/K rotation" + (
                     " with QK Norm, dq and dkdv kernels, QK Norm backward)" if args.qk_norm
                     else ", dq and dkdv kernels)"), "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline_bwd(wl, args.cpu_heads)
    print(json.dumps(out), flush=True)
    return 0


def pointwise_main(args) -> int:
    """One JSON line for HSTU pointwise attention over a named workload (the
    same visible pairs; FLOPs counted as 4 d per visible pair and head)."""
    import numpy as np
    import torch

    import masked_attention_amd as rk
    from rk_workloads import make_config

    torch.cuda.init()
    dev = torch.device("cuda:0")
    wl = make_config(args.config)
    H, d = wl.heads, wl.d_head
    batch = rk.Batch.from_workload(wl, device=dev)
    q, k, v = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (wl.q, wl.k, wl.v))
    rng = np.random.default_rng(77)
    pb = torch.from_numpy((rng.standard_normal(128) * 0.3).astype(np.float32)).to(dev)
    tb = torch.from_numpy((rng.standard_normal(32) * 0.3).astype(np.float32)).to(dev)
    ws = torch.empty(rk.rk_plan_workspace_size(batch, H), dtype=torch.uint8, device=dev)
    mk = dict(delay=wl.delay, window=wl.window, static_bidirectional=wl.static_bidirectional,
              num_heads=H, workspace=ws)
    p0 = rk.Plan(batch, **mk)
    pairs = p0.stats()["visible_pairs"]
    p0.close()
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    plans = []

    def step(ev=None):
        if ev: ev[0].record(stream)
        p = rk.Plan(batch, **mk)
        if ev: ev[1].record(stream)
        rk.rk_pointwise_attn_fwd(p, q, k, v, out=o, scale=1.0 / np.sqrt(d), pos_bias=pb,
                                 time_bias=tb)
        if ev: ev[2].record(stream)
        plans.append(p)

    _gc_before_warmup()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    with _gc_paused():
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    for p in plans:
        p.close()
    ms_step = (t1 - t0) * 1e3 / args.steps
    plan_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    attn_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    flops = 4.0 * d * H * pairs
    achieved = flops / (attn_ms * 1e-3) / 1e12
    out = {
        "metric": "HSTU pointwise attention effective TFLOP/s (visible pairs)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generator with the workload's shapes and time law)",
        "config": {"workload": wl.name + " pointwise", "requests": wl.num_requests,
                   "tokens": wl.total_tokens, "heads": H, "d_head": d,
                   "visible_pairs_per_head": pairs, "pos_buckets": 128, "time_buckets": 32},
        "stage_ms": {"plan": round(plan_ms, 4), "attention": round(attn_ms, 4)},
        "roofline": {"bound": "mfma", "kernel": "pw_mfma_bf16_d64_kernel",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def lazformer_main(args) -> int:
    """One JSON line for LazFormer's attention stack (section 2.3): per
    step, compression of Q, K, V (rk_gather_sum over rk_compress_layout's
    ranges) and, for each of the 5 layers, the pruned layer input gathered,
    planned and attended.  Layouts are host work done once before timing."""
    import numpy as np
    import torch

    import masked_attention_amd as rk
    from rk_workloads import CANDIDATE, HISTORY, NOW, history_span, make_custom

    torch.cuda.init()
    dev = torch.device("cuda:0")
    R, L_hist, n_cand, H, d = 64, 2048, 32, 4, 64
    keep, group, W, G, n_min, n_layers = 1024, 8, 128, 128, 128, 5
    rng = np.random.default_rng(1006)
    reqs = [[(HISTORY, history_span(rng, L_hist, NOW - 60)),
             (CANDIDATE, np.full(n_cand, NOW, np.int64))] for _ in range(R)]
    wl = make_custom(reqs, heads=H, d_head=d, dtype="bf16", seed=1006,
                     name=f"lazformer-{R}x({L_hist}+{n_cand})-keep{keep}-g{group}-W{W}-G{G}-5layers")
    rope = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)
    t0 = time.perf_counter()
    lay = rk.Layout.from_workload(wl)
    comp = rk.rk_compress_layout(lay, keep=keep, group=group)
    lt = comp.history_lengths()
    layers = [rk.rk_prune_layout(comp, l_tilde=lt, n_min=n_min, layer=l, num_layers=n_layers)
              for l in range(1, n_layers + 1)]
    host_ms = (time.perf_counter() - t0) * 1e3
    qkv = [torch.from_numpy(a).to(dev).to(torch.bfloat16) for a in (wl.q, wl.k, wl.v)]
    rg_c = torch.from_numpy(comp.ranges.copy()).to(dev)
    comp_t = [torch.empty((comp.T, H, d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    per = []
    for lay_l in layers:
        anchors = np.full(lay_l.R, NOW, np.int64)
        batch = rk.Batch(lay_l.req_offsets, lay_l.seg_kind, lay_l.timestamps, anchors, device=dev)
        ws = torch.empty(rk.rk_plan_workspace_size(batch, H), dtype=torch.uint8, device=dev)
        per.append(dict(batch=batch, ws=ws, rg=torch.from_numpy(lay_l.ranges.copy()).to(dev),
                        t=[torch.empty((lay_l.T, H, d), dtype=torch.bfloat16, device=dev)
                           for _ in range(3)],
                        o=torch.empty((lay_l.T, H, d), dtype=torch.bfloat16, device=dev)))
    # visible pairs of every layer (from the plans)
    pairs = []
    for pl in per:
        p = rk.Plan(pl["batch"], window=W, global_tail=G, num_heads=H, workspace=pl["ws"])
        pairs.append(p.stats()["visible_pairs"])
        p.close()
    stream = torch.cuda.current_stream()
    plans = []

    def step(ev=None):
        if ev: ev[0].record(stream)
        for src, dst in zip(qkv, comp_t):
            rk.rk_gather_sum(rg_c, src, out=dst)
        if ev: ev[1].record(stream)
        for pl in per:
            for src, dst in zip(comp_t, pl["t"]):
                rk.rk_gather_sum(pl["rg"], src, out=dst)
            p = rk.Plan(pl["batch"], window=W, global_tail=G, num_heads=H, workspace=pl["ws"])
            rk.rk_masked_attn_fwd(p, *pl["t"], out=pl["o"], rope=rope)
            plans.append(p)
        if ev: ev[2].record(stream)

    _gc_before_warmup()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    with _gc_paused():
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    for p in plans:
        p.close()
    ms_step = (t1 - t0) * 1e3 / args.steps
    comp_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    layers_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    flops = 4.0 * d * H * float(sum(pairs))
    comp_bytes = 3 * (wl.total_tokens + comp.T) * H * d * 2 + comp.T * 8
    out = {
        "metric": "LazFormer attention stack: effective TFLOP/s over the visible pairs of all "
                  "layers",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; history spans 1 yr)",
        "config": {"workload": wl.name, "requests": R, "tokens": wl.total_tokens,
                   "compressed_tokens": comp.T, "layer_tokens": [x.T for x in layers],
                   "heads": H, "d_head": d, "visible_pairs_per_head": pairs},
        "stage_ms": {"compress": round(comp_ms, 4), "layers": round(layers_ms, 4),
                     "host_layouts_once": round(host_ms, 2)},
        "stage_hbm_gbs": {"compress": round(comp_bytes / (comp_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "kernel": "gather_sum_kernel (compression of Q, K, V)",
                     "achieved": round(comp_bytes / (comp_ms * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(comp_bytes / (comp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": None, "alg_bytes": comp_bytes},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


def _short_kernel(name: str) -> str:
    import re
    if "elementwise" in name:
        return "torch elementwise (input upload)"
    m = re.search(r"(\w+_kernel(<[^>(]*>)?)", name)
    if m:
        return m.group(1).replace("__hip_bfloat16", "bf16")
    return name.split("(")[0][:44]


def _csv_rows(path: str):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath: str, suffix: str) -> str:
    for root, _, files in os.walk(dirpath):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def _bench_line(path: str) -> dict:
    lines = [ln for ln in open(path).read().splitlines() if ln.strip().startswith("{")]
    return json.loads(lines[-1])


def _header(title: str, args) -> list:
    out = [f"# {title}", "# commands (on the MI355X box, from the repository root):"]
    out += [f"#   {c}" for c in args.profile_cmd]
    argv = " ".join(a if " " not in a and "(" not in a else repr(a) for a in sys.argv[1:])
    out.append(f"#   python3 bench.py {argv}")
    return out


def summarize_trace(args) -> int:
    """Kernel-trace summary of a profiled bench run: every kernel over all its
    launches (from the stats CSV), then the attention kernel over the timed
    launches only (the bench line says where they are in launch order) and
    the planner / rotation kernels over the serial steps at the end."""
    import statistics
    b = _bench_line(args.bench_line)
    wl = b["config"]["workload"]
    out = _header(f"rocprofv3 kernel-trace summary: {wl}", args)
    stats = _csv_rows(_find(args.summarize_trace, "kernel_stats.csv"))
    trace = _csv_rows(_find(args.summarize_trace, "kernel_trace.csv"))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    out += ["", "All launches (kernel_stats.csv; microseconds):",
            f"{'kernel':<44s} {'calls':>6s} {'total_us':>12s} {'avg_us':>10s} {'pct':>7s}"]
    for r in stats:
        out.append(f"{_short_kernel(r['Name']):<44s} {int(r['Calls']):>6d} "
                   f"{float(r['TotalDurationNs']) / 1e3:>12.1f} {float(r['AverageNs']) / 1e3:>10.1f} "
                   f"{float(r['Percentage']):>7.2f}")
    by = {}
    for r in trace:
        by.setdefault(_short_kernel(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if "launches" not in b:
        # the backward, pointwise and LazFormer lines: per-launch medians of
        # every kernel launched at least ten times, and the line itself
        out += ["", "Per-launch medians (kernel_trace.csv; microseconds):"]
        for k, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            if len(d) >= 10:
                out.append(f"  {k:<42s} {statistics.median(d):>9.1f}  ({len(d)} launches)")
        out += ["", "bench.py line of the same run: " + json.dumps(
                    {k: b[k] for k in ("metric", "value", "unit", "ms_per_step")}),
                "  stage_ms: " + json.dumps(b.get("stage_ms"))
                + (f"; roofline frac: {b['roofline']['frac']}" if "roofline" in b else "")]
        print("\n".join(out))
        return 0
    la = b["launches"]
    attn_key = [k for k in by if k.startswith("attn_mfma") or k.startswith("attn_ref")]
    out += ["", "Attention kernel over the timed launches (kernel_trace.csv, in launch order: "
            f"{la['attention_before_timed']} before, {la['attention_timed']} timed, "
            f"{la['serial_after']} serial after):"]
    flops = 4.0 * b["config"]["d_head"] * b["config"]["heads"] * b["config"]["visible_pairs_per_head"]
    for k in attn_key:
        d = by[k]
        t0 = la["attention_before_timed"]
        timed = d[t0:t0 + la["attention_timed"]]
        if len(timed) != la["attention_timed"]:
            out.append(f"  {k}: {len(d)} launches, fewer than the bench line implies")
            continue
        mean, med = statistics.mean(timed), statistics.median(timed)
        peak = b["roofline"]["peak"] if b["roofline"]["unit"] == "TFLOP/s" else PEAK_BF16_TFLOPS
        out += [f"  {k}: {len(timed)} launches: mean {mean:.1f} us, median {med:.1f} us, "
                f"min {min(timed):.1f} us, max {max(timed):.1f} us",
                f"  effective TFLOP/s from the trace mean: {flops / (mean * 1e-6) / 1e12:.1f} "
                f"({flops / (mean * 1e-6) / 1e12 / peak:.4f} of {peak:.0f}); bench line: "
                f"{b['ms_per_step'] * 1e3:.1f} us per step, attention events median "
                f"{b['stage_ms']['attention'] * 1e3:.1f} us, mean "
                f"{b.get('attention_mean_ms', float('nan')) * 1e3:.1f} us"]
    ns = la["serial_after"]
    out += ["", f"Planner and rotation kernels over the {ns} serial steps at the end (median us "
            "per launch; each stage alone on the GPU):"]
    tot = 0.0
    for k, d in by.items():
        if k.startswith("plan_") or k.startswith("rope"):
            m = statistics.median(d[-ns:])
            tot += m if k.startswith("plan_") else 0.0
            out.append(f"  {k:<42s} {m:>9.1f}")
    out.append(f"  planner kernels per step {tot:.1f} us; bench line serial stages: "
               f"{json.dumps(b.get('stage_ms_serial'))} ms")
    print("\n".join(out))
    return 0


def summarize_pmc(args) -> int:
    """Calibrated HBM traffic and MFMA utilisation of the attention kernel
    from three counter runs, written to the two profiles/ files bench.py
    reads (with the kernel source hash they were taken on)."""
    import statistics
    b = _bench_line(args.bench_line)
    wl = b["config"]["workload"]
    alg = b["roofline"]["alg_bytes"]
    fetch_dir, write_dir, mfma_dir = args.summarize_pmc
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()

    def per(path, counter):
        out = {}
        for r in _csv_rows(path):
            if r["Counter_Name"] == counter:
                out.setdefault((r["Kernel_Name"], int(r["Grid_Size"])), []).append(
                    float(r["Counter_Value"]))
        return out

    f = per(_find(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    w = per(_find(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    cf = max(v for (k, g), vs in f.items() if "copyBuffer" in k for v in vs)
    cw = max(v for (k, g), vs in w.items() if "copyBuffer" in k for v in vs)
    af = [v for (k, g), vs in f.items() if ATTN_KERNEL in k for v in vs]
    aw = [v for (k, g), vs in w.items() if ATTN_KERNEL in k for v in vs]
    sf, sw = 1048576.0 / cf, 1048576.0 / cw  # the 1 GiB copy moves 1048576 KiB each way
    fb = statistics.mean(af) * sf * 1024
    wb = statistics.mean(aw) * sw * 1024
    head = _header(f"HBM traffic of the attention kernel, {wl}", args)
    txt = head + [
        "# Counters are KiB per dispatch.  Calibration: the 1 GiB device copy (--copy-calibration,",
        f"# __amd_rocclr_copyBuffer) reads {cf:.1f} KiB by FETCH_SIZE and writes {cw:.1f} KiB by",
        f"# WRITE_SIZE for 1048576 KiB moved each way, so FETCH_SIZE is scaled by {sf:.4f} and",
        f"# WRITE_SIZE by {sw:.4f}.",
        f"# Attention FETCH_SIZE per launch ({len(af)} launches): "
        + ", ".join(f"{x:.1f}" for x in af) + " KiB",
        f"# Attention WRITE_SIZE per launch ({len(aw)} launches): "
        + ", ".join(f"{x:.1f}" for x in aw) + " KiB",
        f"# Algorithmic bytes per launch (Q, K, V read once, O written once, timestamps): {alg}",
        f"attn_source_sha256: {sha}",
        f"fetch_bytes_per_launch: {fb:.0f}",
        f"write_bytes_per_launch: {wb:.0f}",
        f"hbm_bytes_per_launch: {fb + wb:.0f}",
        f"traffic_over_algorithmic: {(fb + wb) / alg:.3f}"]
    path = os.path.join(ROOT, "profiles", f"attn_fwd_hbm_traffic_{wl}.txt")
    open(path, "w").write("\n".join(txt) + "\n")
    m, dur = {}, []
    for r in _csv_rows(_find(mfma_dir, "counter_collection.csv")):
        if ATTN_KERNEL in r["Kernel_Name"]:
            m.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                dur.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    mean = {k: statistics.mean(v) for k, v in m.items()}
    act = mean["GRBM_GUI_ACTIVE"] / 8           # summed over the 8 XCDs
    busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024  # summed over the 1024 SIMDs
    issued = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    d = statistics.mean(dur)
    waves = ""
    if "SQ_WAVE_CYCLES" in mean and "SQ_BUSY_CYCLES" in mean:
        # resident wave-cycles, counted in units of 4 cycles and summed over
        # the chip, per SIMD and active cycle
        waves = f"waves_per_simd: {mean['SQ_WAVE_CYCLES'] * 4 / (act * 1024):.3f}"
    txt = _header(f"MFMA utilisation of the attention kernel, {wl}", args) + [
        f"# Means over {len(dur)} attention dispatches.  GRBM_GUI_ACTIVE is summed over the 8 XCDs",
        "# and SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs; one v_mfma_f32_32x32x16_bf16 counts",
        "# 32 busy cycles and 64 bf16 MOPs (512 FLOPs each).  waves_per_simd = SQ_WAVE_CYCLES",
        "# * 4 / (active cycles per XCD * 1024 SIMDs): resident waves per SIMD (3 at most here).",
        *[f"#   {k:<29s} {v:.4e}" for k, v in sorted(mean.items())],
        f"#   dispatch duration (ns)        {d:.4e}",
        "# mfma_busy_frac = MFMA busy cycles per SIMD / active cycles per XCD: the share of the",
        "# kernel's cycles in which a SIMD's matrix core was busy, independent of the clock.",
        "# issued_flops counts the MFMA work issued (whole tiles, masked parts of PARTIAL tiles",
        "# included); bench.py divides the visible-pair FLOPs by it.",
        f"attn_source_sha256: {sha}",
        f"active_cycles_per_xcd: {act:.0f}",
        f"mfma_busy_cycles_per_simd: {busy:.0f}",
        f"mfma_busy_frac: {busy / act:.4f}",
        f"issued_flops: {issued:.6e}",
        f"clock_ghz_under_profiler: {act / d:.3f}"] + ([waves] if waves else [])
    path2 = os.path.join(ROOT, "profiles", f"attn_fwd_mfma_util_{wl}.txt")
    open(path2, "w").write("\n".join(txt) + "\n")
    print(path)
    print(path2)
    return 0


def summarize_mfma(args) -> int:
    """Per-kernel matrix-core counters of a --pmc run: means over each
    kernel's dispatches of the MFMA busy share of its active cycles, the
    resident waves per SIMD and the clock under the profiler."""
    import statistics
    b = _bench_line(args.bench_line)
    out = _header(f"MFMA utilisation per kernel, {b['config']['workload']} ({b['metric']})", args)
    m, dur = {}, {}
    for r in _csv_rows(_find(args.summarize_mfma, "counter_collection.csv")):
        k = _short_kernel(r["Kernel_Name"])
        m.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            dur.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out += ["# GRBM_GUI_ACTIVE is summed over the 8 XCDs, SQ_VALU_MFMA_BUSY_CYCLES over the 1024",
            "# SIMDs (one v_mfma_f32_32x32x16_bf16 counts 32 busy cycles), SQ_WAVE_CYCLES in units",
            "# of 4 cycles over the chip.  Means over each kernel's dispatches.",
            f"{'kernel':<44s} {'launches':>8s} {'us':>9s} {'mfma_busy':>9s} {'waves/SIMD':>10s} "
            f"{'GHz':>6s} {'MFMA TFLOP/s':>12s}"]
    for k, c in sorted(m.items(), key=lambda kv: -sum(dur.get(kv[0], [0]))):
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in c or "GRBM_GUI_ACTIVE" not in c:
            continue
        mean = {n: statistics.mean(v) for n, v in c.items()}
        act = mean["GRBM_GUI_ACTIVE"] / 8
        if act <= 0:
            continue
        d = statistics.mean(dur[k])
        busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / act
        waves = mean.get("SQ_WAVE_CYCLES", 0.0) * 4 / (act * 1024)
        flops = mean.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        out.append(f"{k:<44s} {len(dur[k]):>8d} {d / 1e3:>9.1f} {busy:>9.4f} {waves:>10.3f} "
                   f"{act / d:>6.3f} {flops / d / 1e3:>12.1f}")
    print("\n".join(out))
    return 0


# Whole-chip MFMA loop: 2048 workgroups of 4 waves (8 waves per SIMD), each
# wave issuing 8 independent-accumulator-pair v_mfma_f32_32x32x16_bf16 per
# iteration on operands that are either constant or random bf16 values that
# rotate between instructions.  The rate comes from HIP events around the
# second launch of each kind (the first warms the clock up).
_CEILING_SRC = r"""
#include <hip/hip_runtime.h>
#include <cstdio>
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
template <int RANDOM>
__global__ __launch_bounds__(256) void mfma_loop(float* out, long long* cyc, int iters,
                                                 unsigned seed) {
  const int t = threadIdx.x;
  bf16x8 fa[4], fb[4];
  unsigned x = seed ^ (t * 2654435761u) ^ (blockIdx.x * 40503u);
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 8; ++i) {
      x = x * 1664525u + 1013904223u;
      fa[j][i] = (__bf16)(RANDOM ? (float)((x >> 9) & 0xffff) / 65536.f - 0.5f : 0.25f);
      x = x * 1664525u + 1013904223u;
      fb[j][i] = (__bf16)(RANDOM ? (float)((x >> 9) & 0xffff) / 65536.f - 0.5f : 0.5f);
    }
  f32x16 a0 = {}, a1 = {};
  const long long c0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j], fb[j], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[(j + 1) & 3], fa[(j + 2) & 3], a1, 0, 0, 0);
    }
  }
  const long long c1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += a0[i] + a1[i];
  out[blockIdx.x * blockDim.x + t] = s;
  if (t == 0) cyc[blockIdx.x] = c1 - c0;
}
template <int R>
static void run(const char* name, float* out, long long* cyc, int iters) {
  hipLaunchKernelGGL(mfma_loop<R>, dim3(2048), dim3(256), 0, 0, out, cyc, iters, 7u);
  (void)hipDeviceSynchronize();
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  (void)hipEventRecord(e0);
  hipLaunchKernelGGL(mfma_loop<R>, dim3(2048), dim3(256), 0, 0, out, cyc, iters, 9u);
  (void)hipEventRecord(e1);
  (void)hipEventSynchronize(e1);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  static long long h[2048];
  (void)hipMemcpy(h, cyc, sizeof(h), hipMemcpyDeviceToHost);
  long long mx = 0;
  for (long long v : h) mx = v > mx ? v : mx;
  const double flops = 2048.0 * 4 * iters * 8 * 32768.0;
  printf("%s %.4f %.6e %.6e\n", name, ms, flops, (double)mx);
}
int main() {
  float* out;
  long long* cyc;
  if (hipMalloc(&out, 2048 * 256 * sizeof(float)) != hipSuccess) return 1;
  if (hipMalloc(&cyc, 2048 * sizeof(long long)) != hipSuccess) return 1;
  for (int rep = 0; rep < 2; ++rep) {
    run<0>("constant", out, cyc, 20000);
    run<1>("random", out, cyc, 20000);
  }
  return 0;
}
"""


def mfma_ceiling_main(args) -> int:
    """One JSON line: the sustained bf16 MFMA rate of a whole-chip
    v_mfma_f32_32x32x16_bf16 loop on constant and on random operands."""
    import shutil
    import subprocess
    import tempfile
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "ceiling.hip"), os.path.join(d, "ceiling")
        open(src, "w").write(_CEILING_SRC)
        subprocess.run([hipcc, "-O3", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-o", exe, src], check=True,
                       capture_output=True)
        res = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    runs = []
    for line in res.splitlines():
        name, ms, flops, cyc = line.split()
        ms, flops, cyc = float(ms), float(flops), float(cyc)
        runs.append({"operands": name, "ms": round(ms, 3),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                     "frac_of_2500": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
    print(json.dumps({"metric": "sustained bf16 MFMA rate, whole-chip v_mfma_f32_32x32x16_bf16 "
                                "loop (2048 workgroups x 4 waves)", "runs": runs}), flush=True)
    return 0


def main() -> int:
    args = _parse()
    if args.mfma_ceiling:
        return mfma_ceiling_main(args)
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.summarize_mfma:
        return summarize_mfma(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the masked-attention path is built and "
              "measured on a single MI355X (requests and heads shard across GPUs without "
              "communication; see the design notes). Use --gpus 1.", file=sys.stderr)
        return 2
    if args.backward:
        return backward_main(args)
    if args.lazformer:
        return lazformer_main(args)
    if args.pointwise:
        return pointwise_main(args)

    import numpy as np
    import torch

    import masked_attention_amd as rk
    from masked_attention_amd import _rk
    from rk_workloads import make_config

    lib = _rk.lib()
    torch.cuda.init()
    dev = torch.device("cuda:0")
    wl = make_config(args.config)
    H, d = wl.heads, wl.d_head
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    batch = rk.Batch.from_workload(wl, device=dev)
    q, k, v = (torch.from_numpy(x).to(dev).to(tdt) for x in (wl.q, wl.k, wl.v))
    krot = torch.empty_like(k)
    o = torch.empty_like(q)
    rope = dict(phi_min=wl.phi_min, dt_max=wl.dt_max, base=wl.base)
    ws = torch.empty(rk.rk_plan_workspace_size(batch, H), dtype=torch.uint8, device=dev)
    ref_plan = rk.Plan(batch, delay=wl.delay, window=wl.window,
                       static_bidirectional=wl.static_bidirectional, num_heads=H, workspace=ws)
    stats = ref_plan.stats()
    pairs = stats["visible_pairs"]
    if args.candidates_only:
        # useful work of a serving step: the candidate rows' visible pairs
        rd = ref_plan.row_desc().to(torch.int64)
        lo, hi_raw = rd[:, 0], rd[:, 1]
        self_bit = hi_raw < 0
        hi = hi_raw & 0x7FFFFFFF
        cand = batch.seg_kind == _rk.RK_SEG_CANDIDATE
        pairs = int(((hi - lo).clamp(min=0) + self_bit.to(torch.int64))[cand].sum().item())
        # history (and profile / real-time) keys rotated once, outside the timed steps
        if args.qk_norm:
            rk.rk_qk_norm_rope(batch, k, eps=1e-6, rope=rope, out=krot)
        else:
            rk.rk_time_rope(batch, k, out=krot, **rope)
    flops = 4.0 * d * H * pairs

    # raw C arguments, built once
    mp = _rk.sized(_rk.rk_mask_params, delay=wl.delay, window=wl.window,
                   flags=(_rk.RK_STATIC_BIDIRECTIONAL if wl.static_bidirectional else 0) | (
                       _rk.RK_QUERY_CANDIDATES_ONLY if args.candidates_only else 0))
    rp = rk.binding.rope_params(**rope)
    # the step's rotation: every key, or only the candidate keys into the cache
    rp_step = rk.binding.rope_params(
        **rope, kinds=(1 << _rk.RK_SEG_CANDIDATE) if args.candidates_only else 0)
    nq = rk.binding.qk_norm_params(1e-6) if args.qk_norm else None
    stream = torch.cuda.current_stream()
    sp = C.c_void_p(stream.cuda_stream)
    dcode = _rk.RK_BF16 if wl.dtype == "bf16" else _rk.RK_F32
    attn = _rk.sized(_rk.rk_attn_args, flags=_rk.RK_ATTN_K_PREROTATED, dtype=dcode, num_heads=H,
                     d_head=d, q=q.data_ptr(), k=krot.data_ptr(), v=v.data_ptr(), o=o.data_ptr(),
                     q_stride_tok=H * d, q_stride_head=d, k_stride_tok=H * d, k_stride_head=d,
                     v_stride_tok=H * d, v_stride_head=d, o_stride_tok=H * d, o_stride_head=d,
                     scale=0.0)
    attn.rope = C.cast(C.pointer(rp), C.c_void_p)
    if nq is not None:
        attn.qk_norm = C.cast(C.pointer(nq), C.c_void_p)
    attn_ws = None
    if args.candidates_only:
        # partial results of split items live in the attention workspace
        size_plan = rk.Plan(batch, delay=wl.delay, window=wl.window,
                            static_bidirectional=wl.static_bidirectional, num_heads=H,
                            candidates_only=True)
        n_ws = C.c_size_t()
        _rk.check(lib.rk_attn_workspace_size(size_plan.handle, C.byref(attn), C.byref(n_ws)),
                  "rk_attn_workspace_size")
        split_stats = size_plan.stats()
        size_plan.close()
        if n_ws.value:
            attn_ws = torch.empty(n_ws.value, dtype=torch.uint8, device=dev)
            attn.workspace = attn_ws.data_ptr()
            attn.workspace_bytes = n_ws.value
    handles = []
    # Consecutive batches are independent: unless --serial, batch i+1's plan
    # and K rotation run on a second stream (default priority) into the other
    # half of a double buffer while batch i's attention runs; events order
    # every reuse of a buffer after the attention that read it.
    krots, wss, attns = [krot, krot.clone()], [ws, torch.empty_like(ws)], [attn]
    a2 = _rk.rk_attn_args.from_buffer_copy(attn)
    a2.k = krots[1].data_ptr()  # the second buffer (cached history keys copied)
    attns.append(a2)
    side_stream = torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in range(2)]  # plan + rotation of buffer b done
    freed = [torch.cuda.Event() for _ in range(2)]  # last attention reading buffer b done
    counter = [0]
    mode = {"pipelined": False}

    def step(ev=None):
        pipelined = mode["pipelined"]
        b = counter[0] % 2 if pipelined else 0
        counter[0] += 1
        side = side_stream if pipelined else stream
        spp = C.c_void_p(side.cuda_stream)
        h = C.c_void_p()
        if pipelined:
            side.wait_event(freed[b])
        if ev: ev[0].record(side)
        _rk.check(lib.rk_mask_plan(C.byref(batch.c), C.byref(mp), H,
                                   C.c_void_p(wss[b].data_ptr()), C.c_size_t(wss[b].numel()),
                                   C.byref(h), spp), "rk_mask_plan")
        if ev: ev[1].record(side)
        if nq is not None:
            _rk.check(lib.rk_qk_norm_rope(C.byref(batch.c), C.byref(rp_step), C.c_float(1e-6),
                                          None, C.c_void_p(k.data_ptr()),
                                          C.c_void_p(krots[b].data_ptr()), dcode, H, d, H * d,
                                          d, H * d, d, spp), "rk_qk_norm_rope")
        else:
            _rk.check(lib.rk_time_rope(C.byref(batch.c), C.byref(rp_step),
                                       C.c_void_p(k.data_ptr()), C.c_void_p(krots[b].data_ptr()),
                                       dcode, H, d, H * d, d, H * d, d, spp), "rk_time_rope")
        if ev: ev[2].record(side)
        if pipelined:
            ready[b].record(side)
            stream.wait_event(ready[b])
        if ev: ev[3].record(stream)
        _rk.check(lib.rk_masked_attn_fwd(h, C.byref(attns[b]), sp), "rk_masked_attn_fwd")
        if ev: ev[4].record(stream)
        if pipelined:
            freed[b].record(stream)
        handles.append(h)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # warmup serially (timed, for the auto choice), then in the chosen mode
    _gc_before_warmup()
    torch.cuda.synchronize()
    tw = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - tw) * 1e3 / max(1, args.warmup)
    mode["pipelined"] = args.pipeline == "on" or (args.pipeline == "auto" and warm_ms > 1.0)
    pipelined = mode["pipelined"]
    if pipelined:
        for _ in range(2):
            step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with _gc_paused():
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # per-stage times: medians over the timed steps (attention: from the
    # point its inputs are ready to its end, on the stream it runs on)
    plan_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    rope_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    attn_ms = float(np.median([e[3].elapsed_time(e[4]) for e in evs]))
    attn_mean_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in evs]))
    # after the timed region: serial steps (one stream, nothing overlapping)
    # give each stage's own time, hence the planner's and the rotation's HBM
    # rates
    mode["pipelined"] = False
    n_serial = max(3, min(args.steps, 10))
    sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_serial)]
    for i in range(n_serial):
        step(sevs[i])
    torch.cuda.synchronize()
    for h in handles:
        lib.rk_plan_destroy(h)
    plan_ms_s = float(np.median([e[0].elapsed_time(e[1]) for e in sevs]))
    rope_ms_s = float(np.median([e[1].elapsed_time(e[2]) for e in sevs]))
    attn_ms_s = float(np.median([e[3].elapsed_time(e[4]) for e in sevs]))

    T = wl.total_tokens
    esz = 2 if wl.dtype == "bf16" else 4
    attn_alg_bytes = T * H * 4 * d * esz + T * 8            # Q, K, V read + O written, times
    n_rot = int((batch.seg_kind == _rk.RK_SEG_CANDIDATE).sum().item()) if args.candidates_only else T
    rope_alg_bytes = n_rot * H * 2 * d * esz + n_rot * 8 + wl.num_requests * 8
    nt = int(ref_plan.info.num_tiles)
    nnz_tiles = int(ref_plan.qtile_ptr()[-1].item()) if ref_plan.num_qtiles else 0
    # kind + time read, row descriptor written, class + count per tile, CSR index + class
    plan_alg_bytes = T * 9 + T * 8 + nt * 5 + nnz_tiles * 5
    achieved = flops / (attn_ms * 1e-3) / 1e12
    wname = wl.name + (" candidates-only" if args.candidates_only else "") + (
        " qk-norm" if args.qk_norm else "")
    traffic = _traffic_from_profile(wname)
    mfma_util = _mfma_util_from_profile(wname, attn_ms, achieved, flops)
    roof = _roofline(wl.dtype, flops, attn_alg_bytes, attn_ms, traffic)
    roof["mfma_util"] = mfma_util
    n_cand = wl.n_candidates
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded generator with the workload's shapes and time law)",
        "config": {"workload": wname,
                   "requests": wl.num_requests, "tokens": T, "heads": H,
                   "d_head": d, "visible_pairs_per_head": pairs, "candidates": n_cand,
                   "delay_s": wl.delay, "window": wl.window,
                   "static_bidirectional": wl.static_bidirectional},
        "pct_bf16_peak": round(100.0 * flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "candidates_per_s": round(n_cand / (ms_step * 1e-3), 1) if n_cand else None,
        "stage_ms": {"plan": round(plan_ms, 4), "rope_k": round(rope_ms, 4),
                     "attention": round(attn_ms, 4)},
        "pipelined": pipelined,
        "attention_mean_ms": round(attn_mean_ms, 4),
        # stage times of serial steps run after the timed region (each stage
        # alone on the GPU); the HBM rates are the algorithmic bytes over them
        "stage_ms_serial": {"plan": round(plan_ms_s, 4), "rope_k": round(rope_ms_s, 4),
                            "attention": round(attn_ms_s, 4)},
        "stage_hbm_gbs": {"plan": round(plan_alg_bytes / (plan_ms_s * 1e-3) / 1e9, 1),
                          "rope_k": round(rope_alg_bytes / (rope_ms_s * 1e-3) / 1e9, 1)},
        "stage_alg_bytes": {"plan": plan_alg_bytes, "rope_k": rope_alg_bytes},
        "tiles": {"full": stats["full_tiles"], "partial": stats["partial_tiles"],
                  "empty": stats["empty_tiles"]},
        "roofline": roof,
        # attention launches of this run in launch order: warmup steps, steps
        # that prime the pipelined mode, the timed steps, then the serial steps
        "launches": {"attention_before_timed": args.warmup + (2 if pipelined else 0),
                     "attention_timed": args.steps, "serial_after": n_serial},
        "cpu_baseline": None,
    }
    if args.candidates_only:
        # the attention stage holds the attention and, for split items, the merge
        out["split"] = {"work_entries": split_stats["work_entries"],
                        "split_items": split_stats["split_items"]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(wl, args.cpu_heads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
