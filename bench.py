#!/usr/bin/env python3
"""Benchmark of the SLA2 inference forward on one MI355X.

One step = one sla2_forward call over the whole workload (router, quantise, linear
branch, sparse branch, combine) with inputs resident in HBM. Prints ONE JSON line:
value = full-attention-equivalent TFLOPS (4 B H N^2 d per call / time), ms_per_step =
ms per call, plus the roofline of the dominant kernel (HIP events recorded by the
library around each of its kernels) and the CPU oracle timed on a bounded sample.

Default workload: Wan2.1-1.3B-480P-shaped latents, B=1 H=12 N=32768 (21x30x52 tokens
padded) d=128, 3% of key blocks kept (97% sparsity). Inputs are seeded synthetic
stand-ins for the model's Q/K/V (see block_sparse_linear_pool_amd/workloads.py).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

METRIC = "SLA2 fwd ms/call + full-attn-equiv TFLOPS, N=32768 H=12 d=128 @97%"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan13b_480p_N32768")
    ap.add_argument("--keep", type=float, default=None, help="kept fraction (default: workload's)")
    ap.add_argument("--cpu-heads", type=int, default=2,
                    help="fewest heads in the CPU-oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU-oracle sample takes heads 0, 1, ... until at least this long")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--traffic", default=None,
                    help="JSON with the measured HBM bytes per launch of the dominant kernel "
                         "(default: profiles/<kernel>_traffic_<workload>.json when present)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run plain device copies of a known size (the calibration "
                         "workload for the FETCH_SIZE / WRITE_SIZE counters), then exit")
    ap.add_argument("--op", choices=("forward", "router_soft", "sla1", "backward", "fit_alpha",
                                     "router_grad"),
                    default="forward",
                    help="forward (default): the inference forward; router_soft: the SoftTop-k "
                         "router (training-time step 1); sla1: the earlier SLA mix O = O_s + "
                         "O_l Wo with the heuristic router (comparison workload); backward: "
                         "the gradients dQ, dK, dV, dalpha for the router's mask; fit_alpha: "
                         "the stage-1 alpha fit against full attention; router_grad: the "
                         "stage-1 router gradient (straight-through SoftTop-k) against full "
                         "attention; each prints its own JSON line")
    ap.add_argument("--tau", type=float, default=0.1, help="SoftTop-k temperature (router_soft)")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


HERE = os.path.dirname(os.path.abspath(__file__))
COPY_PROBE_BYTES = 256 * 1024 * 1024


def kernel_source_hash(kernel):
    """sha256 of the sources a kernel is built from: a stored traffic figure is void once
    they change."""
    import hashlib
    files = {"attn": ["sparse.hip"], "kv_prep": ["linear.hip"], "linear_total": ["linear.hip"]}
    if kernel.startswith("bwd_") or kernel in ("key_lists", "key_plan", "dh_total", "dk_center"):
        files[kernel] = ["backward.hip"]
    files = files.get(kernel, ["router.hip"]) + ["sla2_common.h"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, "block_sparse_linear_pool_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(args, kernel, w, keep):
    """HBM bytes per launch of `kernel` from its rocprofv3 counter record under profiles/
    (FETCH_SIZE and WRITE_SIZE runs, scaled by a copy of known size), or None when there is
    none for this workload or the kernel's sources have changed since it was taken."""
    tpath = args.traffic or os.path.join(HERE, "profiles", f"{kernel}_traffic_{w.name}.json")
    if not os.path.exists(tpath):
        return None
    with open(tpath) as f:
        tr = json.load(f)
    if (tr.get("kernel") == kernel and tr.get("workload") == w.name and tr.get("keep_frac") == keep
            and tr.get("source_sha256") == kernel_source_hash(kernel)):
        return tr.get("bytes_per_launch")
    return None


def copy_probe():
    """Ten device-to-device copies of COPY_PROBE_BYTES (read that many, write that many)."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "copies": 10}), flush=True)


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def timed_heads(args, w, work):
    """Run work(h) for heads 0, 1, ... of batch 0 (starting over after the last head) until at
    least args.cpu_seconds have passed and at least args.cpu_heads heads were done; returns
    (the heads done, in order, with repeats; seconds)."""
    t0 = time.perf_counter()
    done = []
    while len(done) < args.cpu_heads or time.perf_counter() - t0 < args.cpu_seconds:
        h = len(done) % w.H
        work(h)
        done.append(h)
    return done, time.perf_counter() - t0


def heads_text(heads, w):
    """'heads 0-6 of 12', or 'heads 0-11 of 12 (30 head passes)' when the sample went round."""
    top = min(len(heads), w.H) - 1
    text = f"heads 0-{top} of {w.H}"
    return text + (f" ({len(heads)} head passes)" if len(heads) > w.H else "")


def cpu_baseline(args, w, q, k, v, wq, wk, alpha, keep, acc):
    """Time the fp64 oracle (as it stands) on the first heads of batch 0."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import sla2 as oracle

    cores = min(16, len(os.sched_getaffinity(0)))
    with threadpool_limits(limits=cores):
        heads, dt = timed_heads(args, w, lambda h: oracle.forward_head(
            q[0, h].astype(np.float64), k[0, h].astype(np.float64), v[0, h].astype(np.float64),
            wq[h], wk[h], alpha[h], keep, quant=True))
    flops = 4.0 * w.N * w.N * w.d * len(heads)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOPS (full-attention-equivalent)",
        "cores": cores,
        "kind": "oracle",
        "sample": f"batch 0, {heads_text(heads, w)} ({len(heads)}/{w.B * w.H} of one "
                  f"call), fp64 numpy oracle with quantisation, {dt:.1f} s; "
                  f"ms/call extrapolated {dt * 1e3 * w.B * w.H / len(heads):.0f}",
        "cpu": platform.processor() or platform.machine(),
    }


def run_router_soft(args, w, q, k, wq, wk, keep):
    """Times sla2_router_soft (SoftTop-k router) like the forward: W warm-up calls, K timed
    back-to-back calls, then K calls with the library's events around its four kernels."""
    import numpy as np
    import torch

    from block_sparse_linear_pool_amd import accounting as acc
    from block_sparse_linear_pool_amd import sla2

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    gq, gk = (torch.from_numpy(a).to(dev, dt) for a in (q, k))
    gwq, gwk = (torch.from_numpy(a).to(dev) for a in (wq, wk))
    soft = torch.empty((w.B, w.H, w.n_qb, w.n_kb), dtype=torch.float32, device=dev)
    ws = sla2.workspace_for(gq, "router_soft")
    kb = sla2.sla2_blocks_kept(w.n_kb, keep)
    prob = acc.Problem(w.B, w.H, w.N, kb, in_bytes=2 if dt == torch.bfloat16 else 4)

    def step(events=None):
        sla2.sla2_router_soft(gq, gk, gwq, gwk, keep, args.tau, workspace=ws, out=soft,
                              events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    names = acc.KERNELS_SOFT_ROUTER
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    per = np.zeros(len(names))
    for _ in range(args.steps):
        step(evs)
        torch.cuda.synchronize()
        per += [evs[i].elapsed_time(evs[i + 1]) for i in range(len(names))]
    per /= args.steps
    kernels = {}
    for n, t in zip(names, per):
        fl, by = acc.kernel_flops(prob, n), acc.kernel_bytes(prob, n)
        kernels[n] = {"ms": round(float(t), 5),
                      "tflops": round(fl / (t * 1e-3) / 1e12, 2) if fl else None,
                      "gbs": round(by / (t * 1e-3) / 1e9, 1) if by else None}
        log(args, f"[bench]   {n:11s} {t * 1e3:9.1f} us  {kernels[n]}")
    dom = names[int(np.argmax(per))]
    t_dom = float(np.max(per)) * 1e-3
    if acc.kernel_bound(dom) == "mfma_fp32":
        achieved = acc.kernel_flops(prob, dom) / t_dom / 1e12
        peak, unit, bound = acc.MI355X_PEAK["mfma_fp32_tflops"], "TFLOP/s", "mfma"
    else:
        achieved = acc.kernel_bytes(prob, dom) / t_dom / 1e9
        peak, unit, bound = acc.MI355X_PEAK["hbm_gbs"], "GB/s", "hbm"
    rows = w.B * w.H * w.n_qb
    result = {
        "metric": "SLA2 SoftTop-k router rows/s (training-time step 1), N=32768 H=12 d=128 @97%",
        "value": round(rows / (ms * 1e-3), 1),
        "unit": "query-block rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "input_dtype": w.dtype, "keep_frac": keep, "kb": kb, "tau": args.tau},
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": None,
                     "avg_launch_ms": round(t_dom * 1e3, 5)},
        "kernels": kernels,
    }
    if not args.no_cpu:
        from threadpoolctl import threadpool_limits

        from oracle import sla2 as oracle
        cores = min(16, len(os.sched_getaffinity(0)))

        def one_head(h):
            K = k[0, h].astype(np.float64)
            mu, mu32 = oracle.colmean(K)
            _, P = oracle.router_scores(oracle.block_mean(q[0, h].astype(np.float64), 128),
                                        oracle.block_mean(oracle.smooth_k(K, mu32), 64),
                                        wq[h], wk[h])
            oracle.soft_topk(P, kb, args.tau)
        with threadpool_limits(limits=cores):
            heads, dt_cpu = timed_heads(args, w, one_head)
        result["cpu_baseline"] = {
            "value": round(len(heads) * w.n_qb / dt_cpu, 1), "unit": "query-block rows/s",
            "cores": cores, "kind": "oracle",
            "sample": f"batch 0, {heads_text(heads, w)}: the oracle's router up to "
                      f"P_c and its fp64-bisection SoftTop-k, {dt_cpu:.2f} s"}
    print(json.dumps(result), flush=True)


def run_sla1(args, w, q, k, v, keep):
    """Times sla2_forward_sla1 (the earlier SLA mix, a comparison workload) like the forward."""
    import numpy as np
    import torch

    from block_sparse_linear_pool_amd import accounting as acc
    from block_sparse_linear_pool_amd import sla2

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    gq, gk, gv = (torch.from_numpy(a).to(dev, dt) for a in (q, k, v))
    rng = np.random.default_rng([w.seed, 99])
    wo = torch.from_numpy(rng.normal(0.0, 1.0 / np.sqrt(w.d), (w.H, w.d, w.d)).astype(np.float32)).to(dev)
    out = torch.empty(gq.shape, dtype=torch.float32, device=dev)
    ol = torch.empty_like(out)
    ws = sla2.workspace_for(gq, "forward_sla1", keep)
    kb = sla2.sla2_blocks_kept(w.n_kb, keep)
    prob = acc.Problem(w.B, w.H, w.N, kb, in_bytes=2 if dt == torch.bfloat16 else 4)

    def step(events=None):
        sla2.sla2_forward_sla1(gq, gk, gv, wo, keep, out=out, o_l=ol, workspace=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    names = acc.KERNELS_SLA1
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(sla2.MAX_STAGES + 1)]
    per = np.zeros(len(names))
    for _ in range(args.steps):
        step(evs)
        torch.cuda.synchronize()
        per += [evs[i].elapsed_time(evs[i + 1]) for i in range(len(names))]
    per /= args.steps
    kernels = {}
    for n, t in zip(names, per):
        fl, by = acc.kernel_flops(prob, n), acc.kernel_bytes(prob, n)
        kernels[n] = {"ms": round(float(t), 5),
                      "tflops": round(fl / (t * 1e-3) / 1e12, 2) if fl else None,
                      "gbs": round(by / (t * 1e-3) / 1e9, 1) if by else None}
        log(args, f"[bench]   {n:13s} {t * 1e3:9.1f} us  {kernels[n]}")
    dom = names[int(np.argmax(per))]
    t_dom = float(np.max(per)) * 1e-3
    if acc.kernel_bound(dom) == "mfma":
        achieved = acc.kernel_flops(prob, dom) / t_dom / 1e12
        peak, unit, bound = acc.MI355X_PEAK["mfma_i8_fp8_tflops"], "TFLOP/s", "mfma"
    else:
        achieved = acc.kernel_bytes(prob, dom) / t_dom / 1e9
        peak, unit, bound = acc.MI355X_PEAK["hbm_gbs"], "GB/s", "hbm"
    full = acc.full_attention_flops(prob)
    result = {
        "metric": "Earlier SLA mix (comparison) fwd full-attn-equiv TFLOPS, N=32768 H=12 d=128 @97%",
        "value": round(full / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOPS (full-attention-equivalent)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8+fp8",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "input_dtype": w.dtype, "keep_frac": keep, "kb": kb},
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": None,
                     "avg_launch_ms": round(t_dom * 1e3, 5)},
        "kernels": kernels,
    }
    if not args.no_cpu:
        from threadpoolctl import threadpool_limits

        from oracle import sla2 as oracle
        cores = min(16, len(os.sched_getaffinity(0)))
        wo_h = wo.cpu().numpy()
        with threadpool_limits(limits=cores):
            heads, dt_cpu = timed_heads(args, w, lambda h: oracle.forward_head_sla1(
                q[0, h].astype(np.float64), k[0, h].astype(np.float64),
                v[0, h].astype(np.float64), wo_h[h], keep))
        result["cpu_baseline"] = {
            "value": round(4.0 * w.N * w.N * w.d * len(heads) / dt_cpu / 1e12, 4),
            "unit": "TFLOPS (full-attention-equivalent)", "cores": cores, "kind": "oracle",
            "sample": f"batch 0, {heads_text(heads, w)}, fp64 oracle, {dt_cpu:.1f} s"}
    print(json.dumps(result), flush=True)


def run_backward(args, w, q, k, v, wq, wk, alpha, keep):
    """Times sla2_backward (dQ, dK, dV, dalpha for a fixed mask: the router's on these inputs,
    computed once before the timed region, as the forward would hand it over)."""
    import numpy as np
    import torch

    from block_sparse_linear_pool_amd import accounting as acc
    from block_sparse_linear_pool_amd import sla2
    from block_sparse_linear_pool_amd import workloads as W

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    gq, gk, gv = (torch.from_numpy(a).to(dev, dt) for a in (q, k, v))
    ga = torch.from_numpy(alpha).to(dev)
    dO_h = W.grad_out(w.seed, q.shape)
    gdo = torch.from_numpy(dO_h).to(dev)
    ws = sla2.workspace_for(gq, "backward")   # also serves the router call (a smaller plan)
    _, mask, _ = sla2.sla2_router(gq, gk, torch.from_numpy(wq).to(dev),
                                  torch.from_numpy(wk).to(dev), keep, workspace=ws)
    out = (torch.empty(gq.shape, dtype=torch.float32, device=dev),
           torch.empty(gq.shape, dtype=torch.float32, device=dev),
           torch.empty(gq.shape, dtype=torch.float32, device=dev),
           torch.empty((w.B, w.H, w.n_qb), dtype=torch.float32, device=dev))
    kb = sla2.sla2_blocks_kept(w.n_kb, keep)
    # how the library splits the key lists: at most C query blocks per key block in bwd_kv,
    # C = max(16, ceil(2 P / nkb)) per head (P kept pairs), the rest in bwd_kv_extra
    tj = mask.to(torch.int32).sum(dim=2).cpu().numpy().reshape(w.B * w.H, w.n_kb)
    main_pairs = 0
    for row in tj:
        C = max(16, -(-2 * int(row.sum()) // w.n_kb))
        main_pairs += int(np.minimum(row, C).sum())
    prob = acc.Problem(w.B, w.H, w.N, kb, in_bytes=2 if dt == torch.bfloat16 else 4,
                       kv_main_pairs=main_pairs)

    def step(events=None):
        sla2.sla2_backward(gq, gk, gv, mask, ga, gdo, out=out, workspace=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(args, f"[bench] backward {ms:.4f} ms/call")
    names = acc.KERNELS_BACKWARD
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(sla2.BACKWARD_STAGES + 1)]
    per = np.zeros(len(names))
    for _ in range(args.steps):
        step(evs)
        torch.cuda.synchronize()
        per += [evs[i].elapsed_time(evs[i + 1]) for i in range(len(names))]
    per /= args.steps
    kernels = {}
    for n, t in zip(names, per):
        fl, by = acc.kernel_flops(prob, n), acc.kernel_bytes(prob, n)
        kernels[n] = {"ms": round(float(t), 5),
                      "tflops": round(fl / (t * 1e-3) / 1e12, 2) if fl else None,
                      "gbs": round(by / (t * 1e-3) / 1e9, 1) if by else None}
        log(args, f"[bench]   {n:13s} {t * 1e3:9.1f} us  {kernels[n]}")
    dom = names[int(np.argmax(per))]
    t_dom = float(np.max(per)) * 1e-3
    if acc.kernel_bound(dom) == "mfma_bf16":
        achieved = acc.kernel_flops(prob, dom) / t_dom / 1e12
        peak, unit, bound = acc.MI355X_PEAK["mfma_bf16_tflops"], "TFLOP/s", "mfma"
    else:
        achieved = acc.kernel_bytes(prob, dom) / t_dom / 1e9
        peak, unit, bound = acc.MI355X_PEAK["hbm_gbs"], "GB/s", "hbm"
    full = acc.full_attention_backward_flops(prob)
    result = {
        "metric": "SLA2 backward full-attn-bwd-equiv TFLOPS, N=32768 H=12 d=128 @97%",
        "value": round(full / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOPS (full-attention-backward-equivalent, 10 B H N^2 d per call)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "input_dtype": w.dtype, "keep_frac": keep, "kb": kb,
                   "kept_pairs": prob.pairs, "kv_main_pairs": main_pairs},
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": stored_traffic(args, dom, w, keep),
                     "avg_launch_ms": round(t_dom * 1e3, 5)},
        "kernels": kernels,
    }
    if not args.no_cpu:
        from threadpoolctl import threadpool_limits

        from oracle import sla2_backward as oracle_bw
        cores = min(16, len(os.sched_getaffinity(0)))
        mask_h = mask.cpu().numpy()
        with threadpool_limits(limits=cores):
            heads, dt_cpu = timed_heads(args, w, lambda h: oracle_bw.backward(
                q[0, h], k[0, h], v[0, h], mask_h[0, h], alpha[h], dO_h[0, h]))
        result["cpu_baseline"] = {
            "value": round(10.0 * w.N * w.N * w.d * len(heads) / dt_cpu / 1e12, 4),
            "unit": "TFLOPS (full-attention-backward-equivalent)", "cores": cores,
            "kind": "oracle",
            "sample": f"batch 0, {heads_text(heads, w)}, fp64 oracle backward, "
                      f"{dt_cpu:.1f} s"}
    print(json.dumps(result), flush=True)


def run_fit_alpha(args, w, q, k, v, wq, wk, keep):
    """Times sla2_fit_alpha on the taps of this workload: O_full from sla2_forward with every
    block kept, O_s and O_l from sla2_forward with the router (both computed once, before the
    timed region)."""
    import numpy as np
    import torch

    from block_sparse_linear_pool_amd import sla2

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    gq, gk, gv = (torch.from_numpy(a).to(dev, dt) for a in (q, k, v))
    eye = torch.eye(w.d, device=dev).expand(w.H, w.d, w.d).contiguous()
    ones = torch.ones((w.H, w.n_qb), device=dev)
    ws = sla2.workspace_for(gq, "forward", 1.0)
    o_full = sla2.sla2_forward(gq, gk, gv, eye, eye, ones, 1.0, workspace=ws)
    _, taps = sla2.sla2_forward(gq, gk, gv, torch.from_numpy(wq).to(dev),
                                torch.from_numpy(wk).to(dev), ones, keep, taps=("O_s", "O_l"),
                                workspace=ws)
    o_s, o_l = taps["O_s"], taps["O_l"]
    alpha = torch.empty((w.H, w.n_qb), device=dev)
    del ws, gq, gk, gv
    for _ in range(args.warmup):
        sla2.sla2_fit_alpha(o_full, o_s, o_l, out=alpha)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        sla2.sla2_fit_alpha(o_full, o_s, o_l, out=alpha)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    E = w.B * w.H * w.N * w.d
    nbytes = 3 * E * 4 + w.H * w.n_qb * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    a = alpha.cpu().numpy()
    result = {
        "metric": "SLA2 stage-1 alpha fit GB/s, N=32768 H=12 d=128 @97%",
        "value": round(gbs, 1), "unit": "GB/s (three fp32 [B,H,N,d] tensors read)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "input_dtype": w.dtype, "keep_frac": keep,
                   "alpha_mean": round(float(a.mean()), 4),
                   "alpha_range": [round(float(a.min()), 4), round(float(a.max()), 4)]},
        "roofline": {"kernel": "fit_alpha", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": 8000.0, "unit": "GB/s", "frac": round(gbs / 8000.0, 4),
                     "traffic": None, "avg_launch_ms": round(ms, 5)},
    }
    if not args.no_cpu:
        from threadpoolctl import threadpool_limits

        from oracle import sla2_fit as oracle_fit
        cores = min(16, len(os.sched_getaffinity(0)))
        heads = list(range(min(4, w.H)))
        f, s_, l_ = (t[:, heads].cpu().numpy() for t in (o_full, o_s, o_l))
        with threadpool_limits(limits=cores):
            t0 = time.perf_counter()
            reps = 0
            while time.perf_counter() - t0 < 10.0:
                oracle_fit.fit_alpha(f, s_, l_)
                reps += 1
            dt_cpu = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(3 * f.size * 4 * reps / dt_cpu / 1e9, 2), "unit": "GB/s",
            "cores": cores, "kind": "oracle",
            "sample": f"batch 0, heads {heads[0]}-{heads[-1]} of {w.H}, fp64 oracle fit, "
                      f"{reps} repetitions in {dt_cpu:.1f} s"}
    print(json.dumps(result), flush=True)


def run_router_grad(args, w, gq, gk, gv, gwq, gwk, ga, keep):
    """Times sla2_router_grad (the whole call: router, unquantised forward, the dense pass over
    every block pair, the router's chain) against O_full = the library's unquantised forward
    with every block kept (dense softmax attention), computed once before the timed region."""
    import torch

    from block_sparse_linear_pool_amd import accounting as acc
    from block_sparse_linear_pool_amd import sla2

    dev = gq.device
    eye = torch.eye(w.d, device=dev).expand(w.H, w.d, w.d).contiguous()
    ones = torch.ones((w.H, w.n_qb), device=dev)
    o_full = sla2.sla2_forward(gq, gk, gv, eye, eye, ones, 1.0, quant="none")
    ws = sla2.workspace_for(gq, "router_grad", keep)
    for _ in range(args.warmup):
        res = sla2.sla2_router_grad(gq, gk, gv, gwq, gwk, ga, keep, o_full, tau=args.tau,
                                    workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        res = sla2.sla2_router_grad(gq, gk, gv, gwq, gwk, ga, keep, o_full, tau=args.tau,
                                    workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    kb = sla2.sla2_blocks_kept(w.n_kb, keep)
    prob = acc.Problem(w.B, w.H, w.N, kb, in_bytes=2 if w.dtype == "bf16" else 4)
    fl = acc.kernel_flops(prob, "mask_grad")
    tf = fl / (ms * 1e-3) / 1e12
    loss = res[0].cpu().numpy()
    result = {
        "metric": "SLA2 stage-1 router gradient ms/call, N=32768 H=12 d=128 @97%",
        "value": round(ms, 4), "unit": "ms per call", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16+fp32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "input_dtype": w.dtype, "keep_frac": keep, "kb": kb, "tau": args.tau,
                   "dense_pass_tflop_per_call": round(fl / 1e12, 3),
                   "loss_mean_per_head": float(loss.mean())},
        "roofline": {"kernel": "whole call (dense pass FLOPs)", "bound": "mfma_f16",
                     "achieved": round(tf, 2), "peak": acc.MI355X_PEAK["mfma_bf16_tflops"],
                     "unit": "TFLOP/s", "frac": round(tf / acc.MI355X_PEAK["mfma_bf16_tflops"], 4),
                     "traffic": None, "avg_launch_ms": round(ms, 5)},
    }
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the forward shards by (batch, head); see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_linear_pool_amd import accounting as acc
    from block_sparse_linear_pool_amd import sla2
    from block_sparse_linear_pool_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    sla2.lib()                                   # fail loudly if the library is missing
    w = W.WORKLOADS[args.workload]
    keep = args.keep if args.keep is not None else w.keep_frac[-1]
    log(args, f"[bench] generating {w.name} B={w.B} H={w.H} N={w.N} keep={keep}")
    t0 = time.time()
    q, k, v = W.generate(w)
    wq, wk, alpha = W.weights(w)
    log(args, f"[bench] inputs ready in {time.time() - t0:.1f} s")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    gq, gk, gv = (torch.from_numpy(a).to(dev, dt) for a in (q, k, v))
    gwq, gwk, ga = (torch.from_numpy(a).to(dev) for a in (wq, wk, alpha))
    out = torch.empty(gq.shape, dtype=torch.float32, device=dev)
    ws = sla2.workspace_for(gq, "forward", keep)
    kb = sla2.sla2_blocks_kept(w.n_kb, keep)
    prob = acc.Problem(w.B, w.H, w.N, kb, in_bytes=2 if dt == torch.bfloat16 else 4)
    if args.op == "router_soft":
        del gv, out
        run_router_soft(args, w, q, k, wq, wk, keep)
        return
    if args.op == "sla1":
        del gv, out
        run_sla1(args, w, q, k, v, keep)
        return
    if args.op == "backward":
        del gq, gk, gv, out, ws
        run_backward(args, w, q, k, v, wq, wk, alpha, keep)
        return
    if args.op == "fit_alpha":
        del gq, gk, gv, out, ws
        run_fit_alpha(args, w, q, k, v, wq, wk, keep)
        return
    if args.op == "router_grad":
        del out, ws
        run_router_grad(args, w, gq, gk, gv, gwq, gwk, ga, keep)
        return

    def step(events=None):
        sla2.sla2_forward(gq, gk, gv, gwq, gwk, ga, keep, out=out, workspace=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # ---- timed region: exactly `steps` calls between synchronisations
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    log(args, f"[bench] {ms:.3f} ms/call (events), {t_wall * 1e3 / args.steps:.3f} ms/call (wall)")

    # ---- per-kernel durations: the library records events around each kernel
    names = acc.KERNELS_FORWARD
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(sla2.MAX_STAGES + 1)]
    per = np.zeros(len(names))
    for _ in range(args.steps):
        step(evs)
        torch.cuda.synchronize()
        per += [evs[i].elapsed_time(evs[i + 1]) for i in range(len(names))]
    per /= args.steps
    kernels = {}
    for n, t in zip(names, per):
        fl, by = acc.kernel_flops(prob, n), acc.kernel_bytes(prob, n)
        kernels[n] = {"ms": round(float(t), 5),
                      "tflops": round(fl / (t * 1e-3) / 1e12, 2) if fl else None,
                      "gbs": round(by / (t * 1e-3) / 1e9, 1) if by else None}
        log(args, f"[bench]   {n:13s} {t * 1e3:9.1f} us  {kernels[n]}")
    dom = names[int(np.argmax(per))]
    t_dom = float(per[int(np.argmax(per))]) * 1e-3
    if acc.kernel_bound(dom) == "mfma":
        achieved = acc.kernel_flops(prob, dom) / t_dom / 1e12
        peak, unit = acc.MI355X_PEAK["mfma_i8_fp8_tflops"], "TFLOP/s"
    else:
        achieved = acc.kernel_bytes(prob, dom) / t_dom / 1e9
        peak, unit = acc.MI355X_PEAK["hbm_gbs"], "GB/s"
    traffic = stored_traffic(args, dom, w, keep)
    roofline = {"kernel": dom, "bound": acc.kernel_bound(dom), "achieved": round(achieved, 2),
                "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": traffic, "avg_launch_ms": round(t_dom * 1e3, 5),
                "whole_call_frac": round(acc.whole_call_frac(prob, ms * 1e-3), 4),
                "whole_call_min_bytes": round(acc.call_min_bytes(prob))}

    full = acc.full_attention_flops(prob)
    result = {
        "metric": METRIC,
        "value": round(full / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOPS (full-attention-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp8",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "input_dtype": w.dtype, "keep_frac": keep, "kb": kb, "n_key_blocks": w.n_kb,
                   "sparsity": round(prob.sparsity, 4),
                   "full_attn_tflop_per_call": round(full / 1e12, 3),
                   "sparse_tflop_per_call": round(acc.sparse_flops(prob) / 1e12, 4)},
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_cpu:
        log(args, f"[bench] timing the CPU oracle on {args.cpu_heads} heads")
        result["cpu_baseline"] = cpu_baseline(args, w, q, k, v, wq, wk, alpha, keep, acc)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
