#!/usr/bin/env python3
"""Throughput of the fused attention forward pass on one MI355X.

A step is one pass of the whole hot path over the training-shape workload
(B=4, H=16, N=2048, d=128, bf16): the non-causal and the causal forward, the
two cases that workload lists.  Inputs are seeded synthetic tensors resident
in HBM before timing starts.  Prints ONE JSON line:

  value        metric TFLOPS of the whole step: (4 B H N^2 d  +  half that for
               the causal case) / time per step
  roofline     the dominant kernel (the non-causal launch) against the bf16
               dense MFMA peak, timed with HIP events on its own stream
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same workload,
               on this host's cores

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --config C --case I     (another workload, same format;
                                                the fp8 workload's step is the
                                                three block quantisations, Q and K
                                                rotated, then the fp8 attention;
                                                the quantiser is reported apart)
       python bench.py --bwd                   (the backward pass of the same
                                                workload instead: dQ, dK, dV from
                                                the forward's O and logsumexp;
                                                flops 2.5x the forward's: five
                                                N x N x d products instead of two)
       python bench.py --profile-launches K    (only K non-causal launches; for
                                                rocprofv3 runs)
       python bench.py --copy-calib            (one 1 GiB device copy: the HBM
                                                byte-counter calibration kernel)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "fwd_bf16_d128_B4H16N2048_noncausal_pmc.md")
KERNEL_SOURCES = [os.path.join(ROOT, "io_aware_exact_05_amd", "csrc", f)
                  for f in ("fa_fwd.hip", "fa_fwd_pipe.hip", "fa_device.h", "fa_kernels.h")]


def kernel_source_sha() -> str:
    """First 16 hex digits of the sha256 of the kernel sources with comments
    and blank lines removed (edits to comments keep the measured kernel)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            txt = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in txt.splitlines())
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None
    when it is missing or was taken on a different kernel source."""
    try:
        txt = open(PROFILE_SUMMARY).read()
    except OSError:
        return None
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_b.group(1))


def kernel_name(w) -> str:
    """The kernel the library dispatches for workload w (for labels only)."""
    if w.dtype == "e4m3":
        return "fwd_fp8"
    if w.dtype == "f32":
        return "fwd_f32"
    if w.d == 128:  # every fp16 / bf16 launch at d = 128
        return "fwd_pipe"
    # rows per workgroup and workgroups per CU of the one-wave-per-SIMD kernel
    if w.d in (64, 128) and w.causal and (w.N + 511) // 512 * w.B * w.H >= 2 * 256:
        return "fwd_wide (long causal)"
    rows, per_cu = {(64, 0): (512, 1), (64, 1): (128, 3), (128, 0): (512, 1), (128, 1): (128, 3),
                    (256, 0): (256, 1), (256, 1): (256, 1)}.get((w.d, w.causal), (0, 0))
    if rows and (not w.causal or (w.N + rows - 1) // rows * w.B * w.H > per_cu * 256):
        return "fwd_wide"
    return "fwd_mfma16"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--case", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU-baseline budget; the sample is sized to about this")
    ap.add_argument("--profile-launches", type=int, default=0)
    ap.add_argument("--bwd", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="time attention over a key/value cache (decoding shapes)")
    ap.add_argument("--copy-calib", action="store_true")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); "
              "every (batch, head) is independent, so N GPUs would each run B*H/N heads "
              "with no communication — see the sharding paragraph of the design notes.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from io_aware_exact_05_amd import fa, inputs

    torch.cuda.init()
    dev = torch.device("cuda:0")

    if args.copy_calib:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": n, "copy_calib_bytes_written": n}))
        return

    if args.decode:
        return bench_decode(args, np, torch, fa, inputs, dev)

    # the fp8 configuration is one case; its head-dimension and causal
    # variants run only when named with --case
    pool = inputs.WORKLOADS + inputs.FP8_VARIANTS
    cases = [w for w in pool if w.config_id == args.config
             and (w.case_id == args.case if args.case is not None
                  else (w.config_id != 5 or w.case_id == 0))]
    if not cases:
        sys.exit(f"no workload config={args.config} case={args.case}")
    fp8 = cases[0].dtype == "e4m3"
    stream = torch.cuda.current_stream()

    # Each entry of `parts` is one launch of the step: (name, workload or None
    # for a quantiser launch, callable).  Every buffer is allocated here.
    data, parts = [], []
    multi_d = len({w.d for w in cases}) > 1
    for w in cases:
        q, k, v = inputs.workload_inputs(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        data.append((w, (q, k, v)))
        if args.bwd:
            if w.dtype not in ("bf16", "f16"):
                sys.exit("the backward pass takes bf16 or f16 workloads")
            o = torch.empty_like(qd)
            fa.fa_fwd(qd, kd, vd, o, lse, bool(w.causal), w.scale, stream)
            do = inputs.upstream_grad((w.B, w.H, w.N, w.d), w.dtype, w.config_id).to(dev)
            dq_, dk_, dv_ = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
            ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
            name = ("causal" if w.causal else "noncausal") + (f"_d{w.d}" if multi_d else "")
            parts.append((name, w,
                          lambda w=w, t=(qd, kd, vd, o, do, lse, dq_, dk_, dv_, ws):
                          fa.fa_bwd(*t, bool(w.causal), w.scale, stream)))
            continue
        if not fp8:
            o = torch.empty_like(qd)
            name = ("causal" if w.causal else "noncausal") + (f"_d{w.d}" if multi_d else "")
            parts.append((name, w,
                          lambda w=w, t=(qd, kd, vd, o, lse):
                          fa.fa_fwd(*t, bool(w.causal), w.scale, stream)))
            continue
        signs = inputs.rotation_signs(w.d, seed=0).to(dev)
        nblk = (w.N + 127) // 128
        q8, k8, v8 = (torch.empty(qd.shape, dtype=torch.uint8, device=dev) for _ in range(3))
        dq, dk, dv = (torch.empty((w.B, w.H, nblk), device=dev) for _ in range(3))
        o = torch.empty(qd.shape, dtype=torch.bfloat16, device=dev)
        for nm, x, x8, ds, rot in (("quantize_q", qd, q8, dq, 1), ("quantize_k", kd, k8, dk, 1),
                                   ("quantize_v", vd, v8, dv, 0)):
            parts.append((nm, None, lambda t=(x, x8, ds, rot):
                          fa.fa_quantize_e4m3(t[0], t[1], t[2], t[3], signs if t[3] else None,
                                              stream)))
        parts.append(("attention_fp8", w, lambda w=w, t=(q8, k8, v8, dq, dk, dv, o, lse):
                      fa.fa_fwd_fp8(*t, bool(w.causal), w.scale, stream)))

    def launch(i):
        parts[i][2]()

    if args.profile_launches:
        if fp8:
            for i in range(len(parts) - 1):
                launch(i)
        att = [i for i, pt in enumerate(parts) if pt[1] is not None][0]
        for _ in range(args.profile_launches):
            launch(att)
        torch.cuda.synchronize()
        print(json.dumps({"profile_launches": args.profile_launches, "workload": cases[0].label()}))
        return

    for _ in range(args.warmup):
        for i in range(len(parts)):
            launch(i)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record(stream)
        for i in range(len(parts)):
            launch(i)
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # algorithmic flops of one launch: the forward's 2 products, the backward's 5
    fmul = 2.5 if args.bwd else 1.0
    ms_step = (t1 - t0) * 1e3 / K
    per_part_ms = [[ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K)] for i in range(len(parts))]
    cold_ms = cold_runs(torch, dev, stream, parts, launch)
    step_flops = sum(w.flops for w, _ in data) * fmul
    value = step_flops / (ms_step * 1e-3) / 1e12
    dtype = cases[0].dtype
    peak = PEAK_TFLOPS[dtype]

    case_rep = {}
    for i, (nm, w, _) in enumerate(parts):
        t = np.array(per_part_ms[i])
        rep_i = {"ms_median": round(float(np.median(t)), 5), "ms_min": round(float(t.min()), 5),
                 "ms_p90": round(float(np.percentile(t, 90)), 5), "ms_cold": round(cold_ms[i], 5)}
        if w is not None:
            tf = fmul * w.flops / (np.median(t) * 1e-3) / 1e12
            rep_i.update(tflops=round(tf, 2), pct_of_peak=round(100 * tf / peak, 2))
        else:  # quantiser: 4 bytes read and 1 written per element, plus the descales
            w0 = cases[0]
            nbytes = 5.0 * w0.B * w0.H * w0.N * w0.d + 4.0 * w0.B * w0.H * ((w0.N + 127) // 128)
            rep_i.update(hbm_gbs=round(nbytes / (np.median(t) * 1e-3) / 1e9, 1),
                         pct_of_hbm_peak=round(100 * nbytes / (np.median(t) * 1e-3) / 1e9
                                               / HBM_PEAK_GBS, 2))
        case_rep[nm] = rep_i
    if fp8:
        t_att = float(np.median(per_part_ms[-1]))
        case_rep["attention_only_tflops"] = round(step_flops / (t_att * 1e-3) / 1e12, 2)

    # dominant kernel: the attention launch with the largest average launch time
    avg = [float(np.mean(t)) if parts[i][1] is not None else -1.0
           for i, t in enumerate(per_part_ms)]
    dom = int(np.argmax(avg))
    wd = parts[dom][1]
    achieved = fmul * wd.flops / (avg[dom] * 1e-3) / 1e12
    traffic = measured_traffic() if (wd.config_id, wd.case_id) == (2, 0) and not args.bwd else None
    kname = "bwd_dq+bwd_dkdv" if args.bwd else kernel_name(wd)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": f"{kname} {wd.label()}", "avg_launch_ms": round(avg[dom], 5)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_bwd(data, args.cpu_seconds) if args.bwd else \
            cpu_baseline(data, args.cpu_seconds)

    label = ", ".join(("causal" if w.causal else "noncausal") for w, _ in data)
    w0 = cases[0]
    out = {
        "metric": ("attention bwd TFLOPS (10*B*H*N^2*d, halved if causal) and % of MFMA peak, 1 GPU"
                   if args.bwd else
                   "attention fwd TFLOPS (4*B*H*N^2*d, halved if causal) and % of MFMA peak, 1 GPU"),
        "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "pct_of_peak": round(100 * value / peak, 2),
        "config": {"workload": f"{w0.name} ({label})", "B": w0.B, "H": w0.H, "N": w0.N,
                   "d": w0.d, "causal": [w.causal for w, _ in data], "dtype": dtype,
                   "step_flops": step_flops,
                   **({"step": "quantise Q, K (rotated), V; fp8 attention"} if fp8 else {}),
                   **({"step": "backward: dQ, dK, dV from O, logsumexp and dO"} if args.bwd else {})},
        "cases": case_rep,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_decode(args, np, torch, fa, inputs, dev):
    """One step = one fa_fwd_kvcache call per decoding shape (every cache byte
    read once).  The pass is bound by HBM: the roofline is algorithmic bytes
    (Q, K, V read, O and the logsumexp written) over the launch time of the
    call (its partial kernel and, when the cache is cut, the merge kernel)."""
    stream = torch.cuda.current_stream()
    cases = [w for w in inputs.DECODE_WORKLOADS if args.case is None or w.case_id == args.case]
    if not cases:
        sys.exit(f"no decoding workload case={args.case}")
    parts, data = [], []
    for w in cases:
        q, k, v = inputs.decode_inputs(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        nb = fa.kvcache_workspace_bytes(w.B, w.H, w.Hkv, w.Nq, w.Nkv, w.d)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        data.append((w, (q, k, v)))
        parts.append((w, lambda w=w, t=(qd, kd, vd, o, lse, ws):
                      fa.fa_fwd_kvcache(*t, bool(w.causal), w.scale, stream)))
    if args.profile_launches:
        for _ in range(args.profile_launches):
            for _, f in parts:
                f()
        torch.cuda.synchronize()
        print(json.dumps({"profile_launches": args.profile_launches,
                          "workload": [w.label() for w in cases]}))
        return
    for _ in range(args.warmup):
        for _, f in parts:
            f()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record(stream)
        for i, (_, f) in enumerate(parts):
            f()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    step_bytes = sum(w.hbm_bytes for w in cases)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    per = [[ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K)] for i in range(len(parts))]
    case_rep = {}
    for i, (w, _) in enumerate(parts):
        t = np.array(per[i])
        gbs = w.hbm_bytes / (np.median(t) * 1e-3) / 1e9
        case_rep[f"case{w.case_id}"] = {
            "shape": w.label(), "ms_median": round(float(np.median(t)), 5),
            "ms_min": round(float(t.min()), 5), "ms_p90": round(float(np.percentile(t, 90)), 5),
            "hbm_gbs": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "tflops": round(w.flops / (np.median(t) * 1e-3) / 1e12, 2)}
    avg = [float(np.mean(t)) for t in per]
    dom = int(np.argmax(avg))
    wd = parts[dom][0]
    achieved = wd.hbm_bytes / (avg[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": f"decode_partial+decode_merge {wd.label()}",
                "avg_launch_ms": round(avg[dom], 5)}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nbytes, t = 0.0, time.perf_counter()
        for w, (q, k, v) in data:
            oracle.attention_kvcache(q, k, v, w.causal, w.scale)
            nbytes += w.hbm_bytes
        dt = time.perf_counter() - t
        cpu = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": _blas_threads(),
               "kind": "oracle", "seconds": round(dt, 2), "cpu_model": cpu_model(),
               "sample": "every head of every decoding shape of the step, fp64 numpy "
                         "(one matrix-vector product per head)"}
    w0 = cases[0]
    out = {
        "metric": "attention over a key/value cache: algorithmic HBM GB/s, 1 GPU",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w0.dtype, "data": "synthetic",
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "config": {"workload": w0.name, "shapes": [w.label() for w in cases],
                   "step_bytes": step_bytes},
        "cases": case_rep, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cold_runs(torch, dev, stream, parts, launch):
    """Diagnostic, outside the timed steps: each launch once more right after
    writing 512 MiB of other memory, so that its inputs are no longer held in
    the L2 caches or the Infinity Cache.  Returns one time (ms) per launch."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = []
    for i in range(len(parts)):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch(i)
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del flush
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    """Threads of numpy's BLAS, which runs the oracle's matrix products."""
    try:
        from threadpoolctl import threadpool_info
        return max([p["num_threads"] for p in threadpool_info() if p["user_api"] == "blas"],
                   default=1)
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline(data, budget_s):
    """fp64 oracle on whole heads of the same workload, sized to ~budget_s."""
    import numpy as np
    import oracle

    lib = oracle.load()
    threads = oracle.num_threads(lib)
    # pilot: one head of each case to estimate the rate
    t_head = 0.0
    for w, (q, k, v) in data:
        q1, k1, v1 = (x[:1, :1].double().numpy() for x in (q, k, v))
        t = time.perf_counter()
        oracle.attention(q1, k1, v1, w.causal, w.scale, lib=lib)
        t_head += time.perf_counter() - t
    n_heads = data[0][0].B * data[0][0].H
    take = int(max(1, min(n_heads, budget_s // max(t_head, 1e-6))))
    sample = []
    for w, (q, k, v) in data:
        b_ = take // w.H
        rem = take % w.H
        if b_:
            sample.append((w, tuple(x[:b_].double().numpy() for x in (q, k, v))))
        if rem:
            sample.append((w, tuple(x[b_:b_ + 1, :rem].double().numpy() for x in (q, k, v))))
    # When the whole step is shorter than half the budget, the sample is run
    # again (same inputs) until about half the budget has passed, so that the
    # rate is timed over several seconds.
    flops, passes = 0.0, 0
    t = time.perf_counter()
    while True:
        for w, (qq, kk, vv) in sample:
            oracle.attention(qq, kk, vv, w.causal, w.scale, lib=lib)
        flops += sum(w.flops for w, _ in data) * take / n_heads
        passes += 1
        if take < n_heads or passes >= 20 or time.perf_counter() - t >= budget_s / 2:
            break
    dt = time.perf_counter() - t
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOPS", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2), "cpu_model": cpu_model(),
            "sample": f"{take} of {n_heads} heads (all {data[0][0].N} rows each) of every case "
                      f"of the step, fp64, OpenMP over query rows; {passes} pass(es)"}


def cpu_baseline_bwd(data, budget_s):
    """fp64 backward oracle on whole heads of the same workload, sized to ~budget_s."""
    import oracle
    from io_aware_exact_05_amd import inputs

    t_head = 0.0
    for w, (q, k, v) in data:
        do = inputs.upstream_grad((1, 1, w.N, w.d), w.dtype, w.config_id)
        t = time.perf_counter()
        oracle.attention_bwd(q[:1, :1], k[:1, :1], v[:1, :1], do, w.causal, w.scale)
        t_head += time.perf_counter() - t
    n_heads = data[0][0].B * data[0][0].H
    take = int(max(1, min(n_heads, budget_s // max(t_head, 1e-6))))
    flops = 0.0
    t = time.perf_counter()
    for w, (q, k, v) in data:
        do = inputs.upstream_grad((w.B, w.H, w.N, w.d), w.dtype, w.config_id)
        b_, rem = take // w.H, take % w.H
        sl = [(slice(0, b_), slice(None))] if b_ else []
        if rem:
            sl.append((slice(b_, b_ + 1), slice(0, rem)))
        for bs, hs in sl:
            oracle.attention_bwd(q[bs, hs], k[bs, hs], v[bs, hs], do[bs, hs], w.causal, w.scale)
        flops += 2.5 * w.flops * take / n_heads
    dt = time.perf_counter() - t
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOPS", "cores": _blas_threads(),
            "kind": "oracle", "seconds": round(dt, 2), "cpu_model": cpu_model(),
            "sample": f"{take} of {n_heads} heads (all {data[0][0].N} rows each) of every case "
                      f"of the step, fp64 numpy (BLAS threads for the matrix products)"}


if __name__ == "__main__":
    main()
