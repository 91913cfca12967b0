"""Benchmark of one Muon optimizer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload ladder24] [--gpus 1]

A step is the whole hot path over every 2-D matrix of the workload: momentum update +
bf16 cast, Frobenius normalisation, k quintic Newton–Schulz iterations (SYRK, SYRK+poly,
GEMM+axpy per iteration), and the float32 apply with decoupled weight decay — all in
libmuon's HIP kernels, with inputs resident in HBM.  W untimed steps run first (the first
eagerly, the rest as replays of the captured step graph); then K graph replays are timed
between device synchronisations.  Prints one JSON line.

  value        effective NS TFLOP/s over the whole step: conventional Newton–Schulz FLOPs
               (4 m^2 n + 2 m^3 per iteration and matrix) / step time
  roofline     the kernel that takes the most time, from HIP events recorded around each
               of its launches on its own stream during K further steps launched kernel
               by kernel (a graph replay hides its kernels from events): algorithmic
               FLOPs (or bytes) per launch / mean launch time, against MI355X's published
               peak (bf16 dense MFMA 2.5 PFLOP/s; HBM 8 TB/s)
  cpu_baseline the float64 CPU oracle (test infrastructure, untuned) on a bounded sample
               of the same workload, extrapolated per bucket; also a parity check of the
               sampled matrices' first step
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

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
DEFAULT_WORKLOAD = "ladder24"
METRIC = "batched Newton–Schulz TFLOP/s (% bf16 MFMA peak) + Muon step ms per shape mix"
KERNEL_SOURCES = ["ns_gemm.hip", "ns_small.hip", "elementwise.hip", "api.hip", "kernels.h", "device_common.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "muon_newton_schulz_momentum_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = data.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--max-workspace-gib", type=float, default=-1.0,
                    help="workspace cap in GiB (0: none; default: none if it fits next to the inputs, "
                         "else 8 GiB chunks)")
    ap.add_argument("--pipeline", type=int, choices=(0, 1), default=1,
                    help="1: the two-stream step (side-stream elementwise kernels beside the NS products)")
    ap.add_argument("--adamw-elements", type=int, default=0,
                    help="also update one AdamW parameter of this many float32 elements (an embedding "
                         "table) inside every step")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "the Muon step here runs on one GPU only; --gpus must be 1 "
                                   "(no path across several GPUs is implemented)"}))
        return 2
    if args.steps < 1 or args.warmup < 1:
        print(json.dumps({"error": "--steps and --warmup must be >= 1"}))
        return 2

    import numpy as np
    import torch

    from muon_newton_schulz_momentum_amd import binding as L
    from muon_newton_schulz_momentum_amd import harness, workloads as wl

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    torch.cuda.set_device(0)
    w = wl.get(args.workload)
    t0 = time.time()
    params = harness.make_params(w, device="cuda")
    adamw_cfg = None
    if args.adamw_elements > 0:
        n_el = args.adamw_elements
        gen = torch.Generator(device="cuda")
        gen.manual_seed(wl.seed_of(w.cid, len(w.params), 9))
        emb = harness.ParamTensors(torch.randn(n_el, generator=gen, device="cuda") * 0.02,
                                   torch.zeros(n_el, device="cuda"),
                                   torch.randn(n_el, generator=gen, device="cuda") * 1e-3,
                                   exp_avg_sq=torch.zeros(n_el, device="cuda"))
        params.append(emb)
        adamw_cfg = harness.Plan.adamw_config(3e-4, 0.9, 0.95, 1e-8, 0.1, 1)
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    # bounded oracle sample: first, middle and last matrix of every canonical bucket
    buckets = {}
    for i, p in enumerate(w.params):
        if p.is_matrix:
            buckets.setdefault(tuple(sorted(p.shape)), []).append(i)
    sample = {}
    for key, idx in buckets.items():
        pick = sorted({idx[0], idx[len(idx) // 2], idx[-1]})
        sample[key] = pick
    snap = {}
    if not args.no_cpu_baseline:
        for idx in sample.values():
            for i in idx:
                snap[i] = tuple(t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else
                                t.detach().cpu().numpy() for t in (params[i].weight, params[i].momentum, params[i].grad))

    # Workspace: the whole plan if it fits in the memory the inputs leave, otherwise
    # chunks that share one region of a few GiB (the moe_slice workload: 261 GB of inputs).
    cap = 0
    if args.max_workspace_gib >= 0:
        cap = int(args.max_workspace_gib * (1 << 30))
    else:
        probe = harness.Plan(params, bind=False)
        need = probe.workspace_bytes
        probe.close()
        free, _ = torch.cuda.mem_get_info()
        if need > free - (4 << 30):
            cap = 8 << 30
    plan = harness.Plan(params, max_workspace_bytes=cap,
                        flags=L.MUON_PLAN_PIPELINE if args.pipeline else 0)
    stream = torch.cuda.current_stream()
    kw = dict(a=w.a, b=w.b, c=w.c, steps=w.steps, eps=w.eps, adamw=adamw_cfg)

    def step(pipeline):
        plan.step_ex(w.beta, w.lr, w.wd, pipeline=pipeline, **kw)

    # first warm-up step (eager, in the timed configuration): its outputs are the sampled
    # parity check
    step(bool(args.pipeline))
    torch.cuda.synchronize()
    first = {}
    for i in snap:
        first[i] = (plan.output_oriented(i).float().cpu().numpy().astype(np.float64),
                    params[i].momentum.cpu().numpy(), params[i].weight.cpu().numpy())

    # the step as one graph; the remaining warm-up steps are replays of it
    graph = plan.capture_ex(w.beta, w.lr, w.wd, pipeline=bool(args.pipeline), **kw)
    for _ in range(args.warmup - 1):
        graph.launch(stream)
    torch.cuda.synchronize()

    # ---- timed region: K graph replays, between device synchronisations ---------------
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        graph.launch(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    replay_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    graph_nodes = graph.nodes
    graph.close()

    # ---- kernel timing: K more steps launched eagerly in the timed configuration, each
    # kernel between a HIP event pair on its own launch stream (with --pipeline 1 the
    # side-stream kernels run beside the products, as in the replays, and are reported
    # under their own names) -------------------------------------------------------------
    launches_per_step = plan.n_chunks * (4 + 3 * w.steps) + 1
    plan.timing_enable(launches_per_step * args.steps + 16)
    torch.cuda.synchronize()
    t_eager = time.perf_counter()
    for _ in range(args.steps):
        step(bool(args.pipeline))
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t_eager) * 1e3 / args.steps

    kernels = {}
    for k in range(L.MUON_KERNEL_COUNT):
        ms, n, work = plan.timing_read(k)
        if n == 0:
            continue
        name = L.muon_kernel_name(k).decode()
        mfma = k in (L.MUON_KERNEL_SYRK, L.MUON_KERNEL_SYRK_POLY, L.MUON_KERNEL_GEMM_AXPY, L.MUON_KERNEL_NS_SMALL)
        rate = work / (ms * 1e-3) / (1e12 if mfma else 1e9)
        peak = PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS
        kernels[name] = {
            "ms_per_step": ms / args.steps, "launches_per_step": n / args.steps,
            "mean_launch_ms": ms / n, "work_per_launch": work / n,
            "achieved": rate, "unit": "TFLOP/s" if mfma else "GB/s", "frac": rate / peak,
            "bound": "mfma" if mfma else "hbm",
        }
    plan.timing_enable(0)

    # ---- per-bucket NS rates: each chunk's momentum, then its Newton-Schulz alone between
    # two events (one stream; the chunks' times are summed per bucket) ------------------
    per_bucket = {}
    for ch in range(plan.n_chunks):
        info = plan.chunk_info(ch)
        plan.momentum_update(w.beta, chunk=ch, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        plan.ns_batched(w.a, w.b, w.c, w.steps, w.eps, chunk=ch, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        b = per_bucket.setdefault(info.bucket, {"m": info.m, "n": info.n, "matrices": 0, "chunks": 0, "ms": 0.0,
                                                "alg": 0.0, "conv": 0.0, "fused_small": bool(info.fused_small)})
        b["matrices"] += info.count
        b["chunks"] += 1
        b["ms"] += e0.elapsed_time(e1)
        b["alg"] += info.flops_algorithmic * w.steps
        b["conv"] += info.flops_conventional * w.steps
    buckets_out = []
    for b in sorted(per_bucket.values(), key=lambda v: -v["ms"]):
        m, n = b["m"], b["n"]
        ai = (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n) / (6 * m * n + 8 * m * m)   # FLOP/B per iteration
        roof = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3)                              # TFLOP/s
        alg_rate = b["alg"] / (b["ms"] * 1e-3) / 1e12
        buckets_out.append({
            "m": m, "n": n, "matrices": b["matrices"], "chunks": b["chunks"], "fused_small": b["fused_small"],
            "ns_ms": round(b["ms"], 4),
            "effective_tflops_conventional": round(b["conv"] / (b["ms"] * 1e-3) / 1e12, 2),
            "algorithmic_tflops": round(alg_rate, 2),
            "algorithmic_frac_of_peak": round(alg_rate / PEAK_BF16_TFLOPS, 4),
            "roof_tflops": round(roof, 1), "bound": "mfma" if roof >= PEAK_BF16_TFLOPS else "hbm",
            "frac_of_own_roof": round(alg_rate / roof, 4),
        })

    # ---- a plain device-to-device copy, for scale next to the elementwise kernels -------
    cp_n = (1 << 30) // 4
    cp_src = torch.ones(cp_n, dtype=torch.float32, device="cuda")
    cp_dst = torch.empty_like(cp_src)
    cp_ms = []
    for _ in range(6):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        cp_dst.copy_(cp_src)
        c1.record(stream)
        torch.cuda.synchronize()
        cp_ms.append(c0.elapsed_time(c1))
    copy_gbs = 2 * (1 << 30) / (sorted(cp_ms[1:])[2] * 1e-3) / 1e9
    del cp_src, cp_dst
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    roofline = {
        "kernel": dom, "bound": dk["bound"], "achieved": round(dk["achieved"], 2),
        "peak": PEAK_BF16_TFLOPS if dk["bound"] == "mfma" else PEAK_HBM_GBS, "unit": dk["unit"],
        "frac": round(dk["frac"], 4), "traffic": load_traffic(dom, w.key),
        "work_per_launch": dk["work_per_launch"], "mean_launch_ms": dk["mean_launch_ms"],
        "measured_over": f"{args.steps} eager steps in the timed configuration, launched kernel by kernel right "
                         f"after the timed graph replays (HIP events on each kernel's own stream)",
    }

    conv, alg = w.ns_flops()
    ns_ms = sum(kernels[k]["ms_per_step"] for k in ("syrk", "syrk_poly", "gemm_axpy", "normalize", "norm_finalize",
                                                    "ns_small")
                if k in kernels)
    value = conv / (ms_per_step * 1e-3) / 1e12

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- CPU oracle: timing on the sample, and parity of the sampled first step -------
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        from oracle import muon_oracle as orc
        per_bucket = {}
        worst, bitwise_ok = 0.0, True
        for key, idx in sample.items():
            times = []
            for i in idx:
                W0, M0, G0 = snap[i]
                t1 = time.perf_counter()
                ref = orc.muon_step_ref(W0, M0, G0, beta=w.beta, a=w.a, b=w.b, c=w.c, steps=w.steps,
                                        eps=w.eps, lr=w.lr, wd=w.wd)
                times.append(time.perf_counter() - t1)
                O_gpu, M_gpu, W_gpu = first[i]
                worst = max(worst, float(np.linalg.norm(O_gpu - ref["O"]) / np.linalg.norm(ref["O"])))
                bitwise_ok &= bool(np.array_equal(M_gpu, ref["M"]))
                bitwise_ok &= bool(np.array_equal(W_gpu, orc.apply_update(W0, O_gpu, w.lr, w.wd)))
            per_bucket[key] = float(np.median(times))
        oracle_step_s = sum(per_bucket[k] * len(buckets[k]) for k in buckets)
        n_sample = sum(len(v) for v in sample.values())
        cpu = {
            "value": round(conv / oracle_step_s / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{n_sample} matrices (first, middle, last of each of {len(buckets)} buckets), "
                      f"one full float64 step each; step time extrapolated as sum over buckets of "
                      f"count x median per-matrix time = {oracle_step_s:.1f} s",
            "ms_per_step": oracle_step_s * 1e3,
        }
        parity = {"sampled_matrices": n_sample, "ns_worst_rel_frobenius": worst, "ns_tolerance": 1e-2,
                  "momentum_and_apply_bitwise": bitwise_ok, "ok": bool(worst <= 1e-2 and bitwise_ok)}

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, sigma) draws on the GPU; no dataset, no trained weights)",
        "config": {
            "workload": w.key, "description": w.description,
            "matrices": len(w.matrices), "buckets": plan.n_buckets, "chunks": plan.n_chunks,
            "workspace_gib": round(plan.workspace_bytes / (1 << 30), 3),
            "ns_iterations": w.steps, "coefficients": [w.a, w.b, w.c], "beta": w.beta,
            "lr": w.lr, "wd": w.wd, "parallelism": "single GPU",
            "streams": "two (pipeline)" if args.pipeline else "one",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "graph": {
            "nodes": graph_nodes, "replay_ms_median": round(replay_ms[len(replay_ms) // 2], 4),
            "replay_ms_min": round(replay_ms[0], 4),
            "eager_ms_per_step": round(eager_ms, 4),
        },
        "ns": {
            "ms_per_step": round(ns_ms, 4),
            "effective_tflops_conventional": round(conv / (ns_ms * 1e-3) / 1e12, 2),
            "algorithmic_tflops": round(alg / (ns_ms * 1e-3) / 1e12, 2),
            "algorithmic_frac_of_peak": round(alg / (ns_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "conventional_flops_per_step": conv, "algorithmic_flops_per_step": alg,
        },
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "buckets": buckets_out,
        "device_copy_gbs": round(copy_gbs, 1),
        "parity": parity,
        "input_generation_s": round(gen_s, 2),
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out))
    plan.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
