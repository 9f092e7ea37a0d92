#!/usr/bin/env python3
"""Benchmark of the fused Multi-Token Attention forward on one MI355X.

One step = one fused forward (``mta_forward``, a single kernel launch) over the
T=4096 workload: B=2, T=4096, M=32, d=128, c_q=4, c_k=9, c_h=4, convolution after
softmax, head mixing before softmax, GroupNorm with gate 1/sqrt(12) (bf16 tensors,
fp32 accumulation). Inputs are seeded synthetic tensors already resident in HBM.

Printed: one JSON line with tokens/s (``value``), effective TFLOP/s and the fraction
of the bf16 MFMA peak, the roofline of the fused kernel (HIP events on its launch
stream), the library's plain causal attention and the default placement at the same
shape, both convolutions on both sides of softmax at the same shape, the unfused T^2
path, and the fp64 CPU oracle.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mta_inputs  # noqa: E402

METRIC = "MTA fwd tokens/sec + effective TFLOP/s (% bf16 MFMA peak), T=4096, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
HEADLINE = 4  # index of the T=4096 workload in mta_inputs.CONFIGS


def sides(placement) -> int:
    """Number of sides of softmax an operation acts on."""
    return {None: 0, "pre": 1, "post": 1, "both": 2}[placement]


def flops(cfg) -> int:
    """Algorithmic flops: causal pairs x (QK^T 2d + AV 2d + conv 2*c_q*c_k + mix 2*c_h),
    the convolution and mixing terms once per side they act on."""
    n_c = cfg.T * (cfg.T + 1) // 2
    per = 4 * cfg.d + sides(cfg.kq) * 2 * cfg.c_q * cfg.c_k + sides(cfg.mix) * 2 * cfg.c_h
    return cfg.B * cfg.M * n_c * per


def materialized_bytes(cfg) -> int:
    """Map traffic of the unfused chain (fp32 T x T maps) plus q, k, v, out."""
    maps = 1  # logits write
    maps += 2 * sides(cfg.mix) + 2 * sides(cfg.kq)  # read + write per step
    maps += 2  # softmax read + write
    maps += 1  # AV read
    elt = 2 if cfg.dtype == "bf16" else 4
    return cfg.B * cfg.M * cfg.T * cfg.T * 4 * maps + 4 * cfg.B * cfg.T * cfg.M * cfg.d * elt


def kernel_source_hash() -> str:
    """Hash of what the headline fused kernel is compiled from: its sources and the compiler
    flags of its translation unit."""
    from token_attention_amd import build as tab

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "token_attention_amd", "csrc")
    tu = "mta_fused_bf16_d128_postconv.hip"
    for name in ("mta_kmajor_impl.h", "mta_device.h", "mta_internal.h", tu):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    flags = list(tab.CFLAGS) + [f for suffix, fl in tab.EXTRA_FLAGS.items() if tu.endswith(suffix) for f in fl]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def device_clock_mhz(dev: int = 0):
    """Peak shader clock of the device in MHz (HIP attribute hipDeviceAttributeClockRate, in kHz),
    read through the HIP runtime already loaded in this process; None if it cannot be read."""
    import ctypes
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64.so" in ln}
        if not paths:
            return None
        hip = ctypes.CDLL(sorted(paths)[0])
        val = ctypes.c_int(0)
        HIP_DEVICE_ATTRIBUTE_CLOCK_RATE = 5
        if hip.hipDeviceGetAttribute(ctypes.byref(val), HIP_DEVICE_ATTRIBUTE_CLOCK_RATE, dev) != 0:
            return None
        return val.value / 1000.0
    except (OSError, AttributeError):
        return None


def measured_traffic():
    """HBM bytes per launch of the fused kernel from the committed counter summary,
    or None when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "fused_variant_T4096_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def gpu_inputs(cfg, torch):
    inp = mta_inputs.make_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(inp[n]).to("cuda").to(dt).contiguous() for n in ("q", "k", "v")}
    for n in ("theta", "w", "gamma", "beta"):
        d[n] = torch.from_numpy(np.ascontiguousarray(inp[n], np.float32)).to("cuda")
    d["lam"] = inp["lam"]
    return inp, d


def clock_warmup(fn, torch, seconds=0.5):
    """Bring the GPU to its steady clock before any timed region: about `seconds` of back-to-back
    calls of fn, the plain causal attention kernel on the workload's tensors (not the layer).
    From a cold start the first ~30 launches of the 1 ms variant kernel ran up to 25 % slower
    while the clock ramped up; a matrix-product load left it ~4 % slow, an attention load ~1 %."""
    torch.cuda.synchronize()
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    return time.time() - t0


def time_launches(fn, steps, warmup, torch):
    """Average ms per call, HIP events recorded on the current stream (the launch stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def training_step_record(ta, torch, wcfg, wd, steps):
    """mta_forward_train and mta_backward_fused on one workload's device tensors, each timed on its
    own (ms per call); the output gradient is a seeded N(0,1) tensor in the input dtype."""
    wkw = dict(c_q=wcfg.c_q, c_k=wcfg.c_k, c_h=wcfg.c_h, kq=wcfg.kq, mix=wcfg.mix, gn=wcfg.gn)
    need = ta.backward_fused_workspace_bytes(wcfg.B, wcfg.T, wcfg.M, wcfg.d, **wkw)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(wd["q"])
    lse = torch.empty((wcfg.B, wcfg.T, wcfg.M), dtype=torch.float32, device="cuda")
    opre = torch.empty(wd["q"].shape, dtype=torch.float32, device="cuda") if wcfg.gn else None
    gen = torch.Generator(device="cuda").manual_seed(7)
    dout = torch.randn(wd["q"].shape, generator=gen, device="cuda").to(wd["q"].dtype)
    args = (wd["q"], wd["k"], wd["v"], wd["theta"], wd["w"], wd["gamma"], wd["beta"], wd["lam"])

    def fwd():
        ta.forward_train(*args, out=out, lse=lse, out_pre_gn=opre, **wkw)

    def bwd():
        ta.backward_fused(*args, dout=dout, lse=lse, out_pre_gn=opre, workspace=ws, **wkw)
    ms_f = time_launches(fwd, max(2, steps // 2), 1, torch)
    ms_b = time_launches(bwd, max(2, steps // 4), 1, torch)
    return {"forward_train_ms": ms_f, "backward_fused_ms": ms_b, "train_step_ms": ms_f + ms_b,
            "train_tokens_per_s": wcfg.B * wcfg.T / ((ms_f + ms_b) * 1e-3), "workspace_gib": need / 2 ** 30}


def launch_spread(fn, reps, torch):
    """Min and median ms of reps individually timed calls (an event pair around each)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[0], t[len(t) // 2]


def cpu_info() -> dict:
    """Host CPU as ``lscpu`` reports it (model name, sockets, physical cores, threads), with
    /proc/cpuinfo's model name when lscpu is not available."""
    import subprocess
    info = {}
    try:
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in txt.splitlines():
            key, _, val = line.partition(":")
            info[key.strip()] = val.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    model = info.get("Model name")
    if not model:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass

    def num(key):
        try:
            return int(info.get(key, ""))
        except ValueError:
            return None
    sockets, per_socket, tpc = num("Socket(s)"), num("Core(s) per socket"), num("Thread(s) per core")
    return {"cpu_model": model or "unknown",
            "physical_cores": sockets * per_socket if sockets and per_socket else None,
            "threads_per_core": tpc, "logical_cpus": num("CPU(s)") or os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_baseline(cfg, inp, n_rows: int):
    """The fp64 oracle on the host cores: every row of the workload (n_rows <= 0), or a seeded
    sample of n_rows query rows of batch 0."""
    from oracle import oracle  # the CPU baseline leg is the only product-side user of the oracle

    c1 = cfg.replace(B=1)
    if n_rows > 0:
        rng = np.random.default_rng(2024)
        rows = np.sort(rng.choice(cfg.T, size=min(n_rows, cfg.T), replace=False)).astype(np.int32)
        batches = [0]
    else:
        rows, batches = None, list(range(cfg.B))
    t0 = time.perf_counter()
    for b in batches:
        sub = dict(inp, **{n: inp[n][b:b + 1] for n in ("q", "k", "v")})
        oracle.forward_cfg(c1, sub, rows=rows)
    dt = time.perf_counter() - t0
    n_tok = len(batches) * (cfg.T if rows is None else len(rows))
    what = (f"the whole workload ({cfg.B} x {cfg.T} query rows, all {cfg.M} heads)" if rows is None else
            f"{len(rows)} seeded random query rows of batch 0, all {cfg.M} heads, T={cfg.T}")
    rec = {
        "value": n_tok / dt,
        "unit": "tokens/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"{what} (fp64 C++ oracle, OpenMP); {dt:.1f} s",
    }
    rec.update(cpu_info())
    return rec


def cpu_single_thread():
    """The fp64 oracle on one host thread, for scale: the tiny fp32 workload in full and a
    seeded 64-row sample of the 880M-slice workload (batch 0, all heads)."""
    from oracle import oracle  # the CPU baseline leg is the only product-side user of the oracle

    rec = {}
    for name, idx, n_rows in (("tiny_fp32", 0, 0), ("slice880m_bf16", 1, 64)):
        cfg = mta_inputs.config(idx)
        inp = mta_inputs.make_inputs(cfg)
        c1 = cfg.replace(B=1)
        sub_inp = dict(inp, **{n: inp[n][:1] for n in ("q", "k", "v")})
        rows = None
        if n_rows:
            rng = np.random.default_rng(2025)
            rows = np.sort(rng.choice(cfg.T, size=n_rows, replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        oracle.forward_cfg(c1, sub_inp, rows=rows, n_threads=1)
        dt = time.perf_counter() - t0
        n_tok = cfg.T if rows is None else len(rows)
        rec[name] = {"tokens_per_s": n_tok / dt, "seconds": dt,
                     "sample": "every row of batch 0" if rows is None else f"{n_rows} seeded rows of batch 0"}
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle rows for cpu_baseline (0: the whole workload)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-materialized", action="store_true")
    ap.add_argument("--only", choices=["fused", "plain", "default", "both", "materialized", "backward",
                                       "backward_fused", "decode", "cpu"],
                    default=None,
                    help="run one path only (for counter collection); prints its timing")
    ap.add_argument("--workload", type=int, default=HEADLINE,
                    help="index of the workload in mta_inputs.CONFIGS for --only runs (profiling)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of this many MiB (calibrates HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1 (multi-GPU runs "
                                   "are not implemented; the layer would shard by batch and head group "
                                   "without communication)"}))
        sys.exit(2)

    if args.only == "cpu":
        # the fp64 oracle alone on the host cores: the workload of --workload, every row
        # (--cpu-rows 0) or a seeded sample of rows of batch 0
        cfg = mta_inputs.config(args.workload)
        inp = mta_inputs.make_inputs(cfg)
        print(json.dumps({"only": "cpu", "workload": cfg.name, **cpu_baseline(cfg, inp, args.cpu_rows)}))
        return

    import torch
    import token_attention_amd as ta

    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    ta.lib()  # fail loudly if the HIP library is missing
    if args.workload != HEADLINE and not args.only:
        print(json.dumps({"error": "--workload selects a profiling workload and needs --only"}))
        sys.exit(2)
    cfg = mta_inputs.config(args.workload)
    inp, d = gpu_inputs(cfg, torch)
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    out = torch.empty_like(d["q"])
    tokens = cfg.B * cfg.T
    n_c = cfg.T * (cfg.T + 1) // 2

    def fused():
        ta.forward(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], d["lam"], out=out, **kw)

    def plain():
        ta.attention_plain(d["q"], d["k"], d["v"], out=out)

    warm_s = clock_warmup(plain, torch)

    dflt = cfg.replace(kq="pre", mix="post")
    kw2 = dict(kw, kq="pre", mix="post")

    def fused_default():
        ta.forward(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], d["lam"], out=out, **kw2)

    # both convolutions on both sides of softmax, same shape (own seeded inputs)
    both_cfg = mta_inputs.config("both_sides_bf16")
    both_d = {}

    def fused_both():
        if not both_d:
            both_d.update(gpu_inputs(both_cfg, torch)[1])
        b = both_d
        ta.forward(b["q"], b["k"], b["v"], b["theta"], b["w"], b["gamma"], b["beta"], b["lam"], out=out,
                   c_q=both_cfg.c_q, c_k=both_cfg.c_k, c_h=both_cfg.c_h, kq=both_cfg.kq, mix=both_cfg.mix,
                   gn=both_cfg.gn)

    def both_record(ms_both, ms_plain):
        tf = flops(both_cfg) / (ms_both * 1e-3) / 1e12
        return {"placement": "convolution and mixing before and after softmax, c_q=4 c_k=9 c_h=4, GroupNorm",
                "ms": ms_both, "tokens_per_s": tokens / (ms_both * 1e-3), "tflops": tf,
                "pct_bf16_peak": 100.0 * tf / PEAK_BF16_TFLOPS,
                "mta_slowdown_vs_plain": ms_both / ms_plain if ms_plain else None}

    def plain_record(ms_plain, ms):
        return {"ms": ms_plain, "tflops": cfg.B * cfg.M * n_c * 4 * cfg.d / (ms_plain * 1e-3) / 1e12,
                "mta_slowdown": ms / ms_plain if ms else None}

    def default_record(ms_dflt, ms_plain):
        tf = flops(dflt) / (ms_dflt * 1e-3) / 1e12
        return {"ms": ms_dflt, "tokens_per_s": tokens / (ms_dflt * 1e-3), "tflops": tf,
                "pct_bf16_peak": 100.0 * tf / PEAK_BF16_TFLOPS,
                "mta_slowdown_vs_plain": ms_dflt / ms_plain if ms_plain else None}

    def materialized_record(ms):
        ws = torch.empty(ta.materialized_workspace_bytes(cfg.B, cfg.T, cfg.M), dtype=torch.uint8, device="cuda")

        def mat():
            ta.forward_materialized(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"],
                                    d["lam"], out=out, workspace=ws, **kw)
        ms_mat = time_launches(mat, max(2, args.steps // 4), 1, torch)
        mb = materialized_bytes(cfg)
        rec = {"ms": ms_mat, "tokens_per_s": tokens / (ms_mat * 1e-3), "bytes": mb,
               "gbs": mb / (ms_mat * 1e-3) / 1e9, "frac_hbm_peak": mb / (ms_mat * 1e-3) / 1e9 / PEAK_HBM_GBS,
               "workspace_gib": ws.numel() / 2 ** 30, "fused_speedup": ms_mat / ms if ms else None}
        del ws
        return rec

    def backward_record(ms_fwd_mat):
        """The gradients of the layer at this workload (mta_backward_materialized), one call per step."""
        kwb = dict(kw)
        need = ta.backward_workspace_bytes(cfg.B, cfg.T, cfg.M, cfg.d, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h,
                                           kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        gen = torch.Generator(device="cuda").manual_seed(7)
        dout = torch.randn(d["q"].shape, generator=gen, device="cuda").to(d["q"].dtype)

        def bwd():
            ta.backward_materialized(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], d["lam"],
                                     dout=dout, workspace=ws, **kwb)
        ms_b = time_launches(bwd, max(2, args.steps // 4), 1, torch)
        rec = {"ms": ms_b, "tokens_per_s": tokens / (ms_b * 1e-3), "workspace_gib": need / 2 ** 30,
               "vs_materialized_forward": ms_b / ms_fwd_mat if ms_fwd_mat else None}
        del ws
        return rec

    def fused_backward_record(ms_fwd):
        """A training step's layer work at this workload: mta_forward_train, then
        mta_backward_fused (no T x T map in memory), each timed on its own."""
        kwb = dict(kw)
        need = ta.backward_fused_workspace_bytes(cfg.B, cfg.T, cfg.M, cfg.d, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h,
                                                 kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        lse = torch.empty((cfg.B, cfg.T, cfg.M), dtype=torch.float32, device="cuda")
        opre = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda") if cfg.gn else None
        gen = torch.Generator(device="cuda").manual_seed(7)
        dout = torch.randn(d["q"].shape, generator=gen, device="cuda").to(d["q"].dtype)

        def fwd_train():
            ta.forward_train(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], d["lam"], out=out,
                             lse=lse, out_pre_gn=opre, **kwb)

        def bwd():
            ta.backward_fused(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], d["lam"],
                              dout=dout, lse=lse, out_pre_gn=opre, workspace=ws, **kwb)
        ms_f = time_launches(fwd_train, max(2, args.steps // 2), 1, torch)
        ms_b = time_launches(bwd, max(2, args.steps // 4), 1, torch)
        kept = lse.numel() * 4 + (opre.numel() * 4 if opre is not None else 0)
        rec = {"ms": ms_b, "forward_train_ms": ms_f, "train_step_ms": ms_f + ms_b,
               "train_tokens_per_s": tokens / ((ms_f + ms_b) * 1e-3),
               "workspace_gib": need / 2 ** 30, "kept_from_forward_gib": kept / 2 ** 30,
               "vs_fused_forward": ms_b / ms_fwd if ms_fwd else None}
        del ws, lse, opre
        return rec

    if args.only == "backward":
        print(json.dumps({"only": "backward", "workload": cfg.name, **backward_record(None)}))
        return
    if args.only == "backward_fused":
        print(json.dumps({"only": "backward_fused", "workload": cfg.name, **fused_backward_record(None)}))
        return
    if args.only == "decode":
        # one decode step (the last row of every sequence) with the key range split over workgroups
        rb = cfg.T - 1
        need = ta.rows_split_workspace_bytes(cfg.B, cfg.T, cfg.M, cfg.d, row_begin=rb, **kw)
        ws_dec = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

        def decode():
            ta.forward_rows_split(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], d["lam"],
                                  row_begin=rb, out=out, workspace=ws_dec, **kw)
        ms_dec = time_launches(decode, args.steps, args.warmup, torch)
        print(json.dumps({"only": "decode", "workload": cfg.name, "row_begin": rb, "ms": ms_dec}))
        return
    if args.only:
        fn = {"fused": fused, "plain": plain, "default": fused_default, "both": fused_both}.get(args.only)
        if fn is not None:
            ms_only = time_launches(fn, args.steps, args.warmup, torch)
            print(json.dumps({"only": args.only, "workload": cfg.name, "ms": ms_only}))
        else:
            print(json.dumps({"only": args.only, "workload": cfg.name, **materialized_record(None)}))
        return

    ms = time_launches(fused, args.steps, args.warmup, torch)
    ms_min, ms_med = launch_spread(fused, args.steps, torch)
    F = flops(cfg)
    tflops = F / (ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_launch_min": ms_min,
        "ms_launch_median": ms_med,
        "clock_warmup_s": warm_s,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v rounded to bf16; theta = delta + N(0,0.05); w = I + N(0,0.05))",
        "config": {
            "workload": "variant_bf16: B=2 T=4096 M=32 d=128 c_q=4 c_k=9 c_h=4, key-query conv after softmax, "
                        "head mixing before softmax, GroupNorm + gate 1/sqrt(12)",
            "global_batch": cfg.B, "seq_len": cfg.T, "parallelism": "single GPU",
        },
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "flops_per_step": F,
        "roofline": {
            "bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
        },
    }
    ms_plain = time_launches(plain, args.steps, args.warmup, torch)
    result["plain_attention"] = plain_record(ms_plain, ms)
    result["default_placement_same_shape"] = default_record(
        time_launches(fused_default, args.steps, args.warmup, torch), ms_plain)
    result["default_placement_same_shape"]["training_step"] = training_step_record(ta, torch, dflt, d, args.steps)
    if cfg.T == both_cfg.T and cfg.B == both_cfg.B and cfg.M == both_cfg.M and cfg.d == both_cfg.d:
        result["both_sides_same_shape"] = both_record(time_launches(fused_both, args.steps, args.warmup, torch),
                                                      ms_plain)
        result["both_sides_same_shape"]["training_step"] = training_step_record(ta, torch, both_cfg, both_d,
                                                                                args.steps)
        both_d.clear()
    # a suffix of rows against all keys: one decode step (the last row of every sequence) and
    # a 512-row prefill chunk, both at the headline placement
    # (mta_forward_rows: row tiles only; mta_forward_rows_split: key range split over workgroups)
    rows_rec = {}
    for name, rb in (("decode_step", cfg.T - 1), ("prefill_chunk_512", cfg.T - 512)):
        def part(rb=rb):
            ta.forward_rows(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], d["lam"],
                            row_begin=rb, out=out, **kw)
        ms_rows = time_launches(part, args.steps, args.warmup, torch)
        rows_rec[name] = {"row_begin": rb, "ms": ms_rows, "tokens_per_s": cfg.B * (cfg.T - rb) / (ms_rows * 1e-3)}
        need = ta.rows_split_workspace_bytes(cfg.B, cfg.T, cfg.M, cfg.d, row_begin=rb, **kw)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

        def part_split(rb=rb, ws=ws):
            ta.forward_rows_split(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], d["lam"],
                                  row_begin=rb, out=out, workspace=ws, **kw)
        ms_split = time_launches(part_split, args.steps, args.warmup, torch)
        rows_rec[name + "_split"] = {"row_begin": rb, "ms": ms_split,
                                     "tokens_per_s": cfg.B * (cfg.T - rb) / (ms_split * 1e-3)}
        if name == "decode_step":
            # the same step captured once in a HIP graph and replayed, as a serving loop would;
            # a capture error is recorded instead of ending the benchmark
            try:
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    part_split()
                torch.cuda.current_stream().wait_stream(side)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    part_split()
                ms_graph = time_launches(graph.replay, args.steps, args.warmup, torch)
                rows_rec[name + "_split_graph"] = {"row_begin": rb, "ms": ms_graph,
                                                   "tokens_per_s": cfg.B * (cfg.T - rb) / (ms_graph * 1e-3)}
                del graph
            except RuntimeError as err:
                torch.cuda.synchronize()
                rows_rec[name + "_split_graph"] = {"row_begin": rb, "error": str(err)[:200]}
    result["rows_forward"] = rows_rec
    # The cost of the exact fallback: with q and k scaled by 6 (logit standard deviation 36) a key
    # late in a row exceeds the maximum of the row's first key tile by far more than 64 in log2
    # units, so the row sum against that fixed reference passes 2^64 and essentially every
    # workgroup repeats its statistics pass exactly (a pass for the row maxima, then the sums).
    q6 = (d["q"].float() * 6.0).to(d["q"].dtype)
    k6 = (d["k"].float() * 6.0).to(d["k"].dtype)

    def fused_fallback():
        ta.forward(q6, k6, d["v"], d["theta"], d["w"], d["gamma"], d["beta"], d["lam"], out=out, **kw)
    ms_fb = time_launches(fused_fallback, args.steps, args.warmup, torch)
    result["exact_fallback_every_workgroup"] = {"ms": ms_fb, "vs_headline": ms_fb / ms,
                                                "inputs": "headline workload with q and k scaled by 6"}
    del q6, k6
    # the other bf16 workloads at their full shapes: the fused layer, and the library's plain
    # causal attention at the same shape (the degenerate workload's kernels are identities, so
    # its ratio is the overhead of the convolution and mixing machinery itself)
    result["workloads"] = {}
    for idx in (1, 2, 3):
        wcfg = mta_inputs.config(idx)
        _, wd = gpu_inputs(wcfg, torch)
        wout = torch.empty_like(wd["q"])
        wkw = dict(c_q=wcfg.c_q, c_k=wcfg.c_k, c_h=wcfg.c_h, kq=wcfg.kq, mix=wcfg.mix, gn=wcfg.gn)

        def wfused(wd=wd, wout=wout, wkw=wkw):
            ta.forward(wd["q"], wd["k"], wd["v"], wd["theta"], wd["w"], wd["gamma"], wd["beta"], wd["lam"], out=wout,
                       **wkw)

        def wplain(wd=wd, wout=wout):
            ta.attention_plain(wd["q"], wd["k"], wd["v"], out=wout)
        ms_w = time_launches(wfused, args.steps, args.warmup, torch)
        ms_p = time_launches(wplain, args.steps, args.warmup, torch)
        wn_c = wcfg.T * (wcfg.T + 1) // 2
        tf = flops(wcfg) / (ms_w * 1e-3) / 1e12
        result["workloads"][wcfg.name] = {
            "shape": f"B={wcfg.B} T={wcfg.T} M={wcfg.M} d={wcfg.d} c_q={wcfg.c_q} c_k={wcfg.c_k} c_h={wcfg.c_h}, "
                     f"conv {wcfg.kq} softmax, mixing {wcfg.mix} softmax, GroupNorm {'on' if wcfg.gn else 'off'}",
            "ms": ms_w, "tokens_per_s": wcfg.B * wcfg.T / (ms_w * 1e-3), "tflops": tf,
            "pct_bf16_peak": 100.0 * tf / PEAK_BF16_TFLOPS, "flops_per_call": flops(wcfg),
            "plain_ms": ms_p, "plain_tflops": wcfg.B * wcfg.M * wn_c * 4 * wcfg.d / (ms_p * 1e-3) / 1e12,
            "mta_slowdown_vs_plain": ms_w / ms_p,
            "training_step": training_step_record(ta, torch, wcfg, wd, args.steps)}
        del wd, wout
    result["backward_fused"] = fused_backward_record(ms)
    if not args.no_materialized:
        result["materialized"] = materialized_record(ms)
        result["backward_materialized"] = backward_record(result["materialized"]["ms"])
    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "clock_mhz": device_clock_mhz(), "gcn_arch": getattr(props, "gcnArchName", "")}
    result["cpu_baseline"] = None if args.no_cpu else cpu_baseline(cfg, inp, args.cpu_rows)
    if not args.no_cpu:
        result["cpu_baseline"]["single_thread"] = cpu_single_thread()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
