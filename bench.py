"""Benchmark of one Muon optimizer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload moe_slice] [--gpus 1]

A step is the whole hot path over every 2-D matrix of the workload: momentum update +
bf16 cast, Frobenius normalisation, k quintic Newton–Schulz iterations (SYRK, SYRK+poly,
GEMM+axpy per iteration), and the float32 apply with decoupled weight decay — all in
libmuon's HIP kernels, with inputs resident in HBM.  W untimed steps run first (the first
eagerly, the rest as replays of the captured step graph); then K graph replays are timed
between device synchronisations.  Prints one JSON line.

The default workload is the largest one that fits one GPU: the mixed-shape optimizer
step of a 4-layer MoE slice (6,184 matrices in 8 shape buckets, 261 GB of weights,
momenta and bf16 gradients resident in HBM).  After it, each of the other full-size
workloads (MoE expert bucket, full-width share, ladder rung) is stepped the same way
with fewer replays and reported under "other_workloads" (--others none to skip).

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
DEFAULT_WORKLOAD = "moe_slice"
OTHER_WORKLOADS = ("moe_bucket", "full_width", "ladder24")
METRIC = "batched Newton–Schulz TFLOP/s (% bf16 MFMA peak) + Muon step ms per shape mix"
KERNEL_SOURCES = ["ns_gemm.hip", "ns_small.hip", "elementwise.hip", "api.hip", "kernels.h", "device_common.h"]


def log(msg: str) -> None:
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "muon_newton_schulz_momentum_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it is current, and a note
    saying where the figure comes from or why there is none."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        why = ("its FETCH_SIZE pass ended in a crash of the profiler's host process and is not re-run; "
               "moe_bucket's summary covers the same (1024, 4096) expert chunks") if workload == "moe_slice" \
            else "no counter summary was taken for this workload"
        return None, f"no profiles/traffic_{workload}.json: {why}"
    with open(path) as fh:
        data = json.load(fh)
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None, f"profiles/traffic_{workload}.json was taken with other kernel sources"
    k = data.get("kernels", {}).get(kernel)
    if k is None:
        return None, f"profiles/traffic_{workload}.json has no {kernel} entry"
    return k.get("hbm_bytes_per_launch"), f"profiles/traffic_{workload}.json (FETCH_SIZE and WRITE_SIZE, calibrated)"


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


# float64 FLOP/s of the oracle on a host of about 16 threads (measured), used only to size
# its sample so that the CPU leg takes about ORACLE_BUDGET_S seconds
ORACLE_RATE = 0.3e12
ORACLE_BUDGET_S = 20.0
ORACLE_MAX_PER_BUCKET = 16


def oracle_sample(w):
    """Matrices the CPU oracle runs, per canonical bucket.

    Every bucket gets its first matrix; a bucket of many matrices also its last one and,
    with per-expert gradient scales, the matrices of the experts with the smallest and the
    largest scale.  Then the cheapest buckets are filled up (evenly spaced matrices, at
    most 16 per bucket) while the estimated oracle time stays within the budget: small
    buckets are run whole, the giant expert bucket gets 16 matrices, the large-m buckets
    one or two.  A bucket whose single matrix would take the oracle longer than the whole
    budget (8704 x 8704) is left out.  Returns ({bucket: [indices]}, {bucket: [all indices]}).
    """
    from muon_newton_schulz_momentum_amd import workloads as wl

    buckets = {}
    for i, p in enumerate(w.params):
        if p.is_matrix:
            buckets.setdefault(tuple(sorted(p.shape)), []).append(i)

    def cost(key):
        m, n = key
        return w.steps * (4.0 * m * m * n + 2.0 * m ** 3) / ORACLE_RATE

    pick = {}
    for key, idx in buckets.items():
        if cost(key) > ORACLE_BUDGET_S:
            continue                  # timed by the measured rate of the others (see run_workload)
        sel = {idx[0]}
        if len(idx) > ORACLE_MAX_PER_BUCKET:
            sel.add(idx[-1])
            if w.scale_groups:
                grouped = [i for i in idx if w.params[i].group >= 0]
                if grouped:
                    sc = {i: wl.group_scale(w.cid, w.params[i].group) for i in grouped}
                    sel.add(min(grouped, key=lambda i: sc[i]))
                    sel.add(max(grouped, key=lambda i: sc[i]))
        pick[key] = sel
    total = sum(cost(k) * len(v) for k, v in pick.items())
    for key in sorted(pick, key=cost):
        idx = buckets[key]
        want = min(len(idx), ORACLE_MAX_PER_BUCKET)
        for r in range(want):
            if len(pick[key]) >= want or total + cost(key) > ORACLE_BUDGET_S:
                break
            i = idx[(r * (len(idx) - 1)) // max(want - 1, 1)]
            if i not in pick[key]:
                pick[key].add(i)
                total += cost(key)
    return {k: sorted(v) for k, v in pick.items()}, buckets


def run_workload(key, args, steps, warmup, cpu_leg, detail):
    """One workload: inputs, plan, timed graph replays; with `detail` also per-kernel and
    per-bucket rates, the device copy rate and (with `cpu_leg`) the oracle leg."""
    import gc

    import numpy as np
    import torch

    from muon_newton_schulz_momentum_amd import binding as L
    from muon_newton_schulz_momentum_amd import harness, workloads as wl

    w = wl.get(key)
    log(f"{key}: generating inputs")
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    t0 = time.time()
    params = harness.make_params(w, device="cuda")
    adamw_cfg = None
    if detail and args.adamw_elements > 0:
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

    sample, buckets = oracle_sample(w)
    snap = {}
    if cpu_leg:
        for idx in sample.values():
            for i in idx:
                snap[i] = tuple(t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else
                                t.detach().cpu().numpy() for t in (params[i].weight, params[i].momentum, params[i].grad))

    # Workspace: the whole plan if it fits in the memory the inputs leave, otherwise
    # chunks in capped regions (the moe_slice workload: 261 GB of inputs).  16 GiB when it
    # leaves 4 GiB free (25 chunks for moe_slice; measured 0.3-0.65 % faster per step than 12
    # and 8 GiB, whose chunks are smaller), else 8 GiB.
    cap = 0
    if args.max_workspace_gib >= 0:
        cap = int(args.max_workspace_gib * (1 << 30))
    else:
        probe = harness.Plan(params, bind=False)
        need = probe.workspace_bytes
        probe.close()
        free, _ = torch.cuda.mem_get_info()
        if need > free - (4 << 30):
            cap = (16 << 30) if free - (16 << 30) >= (4 << 30) else (8 << 30)
    plan = harness.Plan(params, max_workspace_bytes=cap,
                        flags=L.MUON_PLAN_PIPELINE if args.pipeline else 0)
    stream = torch.cuda.current_stream()
    kw = dict(a=w.a, b=w.b, c=w.c, steps=w.steps, eps=w.eps, adamw=adamw_cfg)

    def step(pipeline):
        plan.step_ex(w.beta, w.lr, w.wd, pipeline=pipeline, **kw)

    log(f"{key}: {plan.n_chunks} chunks, workspace {plan.workspace_bytes / (1 << 30):.2f} GiB; warm-up")
    # first warm-up step: its outputs are the sampled parity check.  It runs eagerly in the
    # timed configuration when every chunk has a region of its own; when chunks share
    # workspace regions (moe_slice under its cap) a later chunk overwrites an earlier one's
    # output, so the step then runs chunk by chunk and each chunk's sampled outputs are
    # read before the next one starts (the same kernels; the two-stream step is bitwise
    # equal to it, which the GPU tests check)
    first = {}

    def grab(indices):
        for i in indices:
            first[i] = (plan.output_oriented(i).float().cpu().numpy().astype(np.float64),
                        params[i].momentum.cpu().numpy(), params[i].weight.cpu().numpy())

    shared = plan.n_chunks > 0 and bool(plan.chunk_info(0).shared_region)
    if snap and shared:
        by_chunk = {}
        for i in snap:
            by_chunk.setdefault(plan.param_info(i).chunk, []).append(i)
        for ch in range(plan.n_chunks):
            plan.step_ex(w.beta, w.lr, w.wd, chunk=ch, **kw)
            torch.cuda.synchronize()
            grab(by_chunk.get(ch, []))
    else:
        step(bool(args.pipeline))
        torch.cuda.synchronize()
        grab(snap)

    # the step as one graph; the remaining warm-up steps are replays of it
    graph = plan.capture_ex(w.beta, w.lr, w.wd, pipeline=bool(args.pipeline), **kw)
    for _ in range(warmup - 1):
        graph.launch(stream)
    torch.cuda.synchronize()

    log(f"{key}: timing {steps} graph replays")
    # ---- timed region: K graph replays, between device synchronisations ---------------
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        graph.launch(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / steps
    replay_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    graph_nodes = graph.nodes
    graph.close()

    conv, alg = w.ns_flops()
    value = conv / (ms_per_step * 1e-3) / 1e12
    rec = {
        "workload": w.key, "description": w.description,
        "matrices": len(w.matrices), "buckets": plan.n_buckets, "chunks": plan.n_chunks,
        "workspace_gib": round(plan.workspace_bytes / (1 << 30), 3),
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
        "effective_tflops_conventional": round(value, 3),
        "algorithmic_tflops_over_step": round(alg / (ms_per_step * 1e-3) / 1e12, 3),
        "algorithmic_frac_of_peak_over_step": round(alg / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "graph": {"nodes": graph_nodes, "replay_ms_median": round(replay_ms[len(replay_ms) // 2], 4),
                  "replay_ms_min": round(replay_ms[0], 4)},
        "input_generation_s": round(gen_s, 2),
        "conventional_flops_per_step": conv, "algorithmic_flops_per_step": alg,
        "_w": w,
    }

    # ---- kernel timing: K more steps launched eagerly in the timed configuration, each
    # kernel between a HIP event pair on its own launch stream (with --pipeline 1 the
    # side-stream kernels run beside the products, as in the replays, and are reported
    # under their own names) -------------------------------------------------------------
    log(f"{key}: {ms_per_step:.3f} ms per step; per-kernel timing")
    launches_per_step = plan.n_chunks * (4 + 3 * w.steps) + 1
    plan.timing_enable(launches_per_step * steps + 16)
    torch.cuda.synchronize()
    t_eager = time.perf_counter()
    for _ in range(steps):
        step(bool(args.pipeline))
    torch.cuda.synchronize()
    rec["graph"]["eager_ms_per_step"] = round((time.perf_counter() - t_eager) * 1e3 / steps, 4)

    kernels = {}
    for k in range(L.MUON_KERNEL_COUNT):
        ms, n, work = plan.timing_read(k)
        if n == 0:
            continue
        name = L.muon_kernel_name(k).decode()
        mfma = k in (L.MUON_KERNEL_SYRK, L.MUON_KERNEL_SYRK_POLY, L.MUON_KERNEL_GEMM_AXPY, L.MUON_KERNEL_NS_SMALL,
                     getattr(L, "MUON_KERNEL_NS_GROUPED", -1))
        rate = work / (ms * 1e-3) / (1e12 if mfma else 1e9)
        peak = PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS
        kernels[name] = {
            "ms_per_step": ms / steps, "launches_per_step": n / steps,
            "mean_launch_ms": ms / n, "work_per_launch": work / n,
            "achieved": rate, "unit": "TFLOP/s" if mfma else "GB/s", "frac": rate / peak,
            "bound": "mfma" if mfma else "hbm",
        }
    plan.timing_enable(0)
    rec["kernels"] = {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                      for k, v in kernels.items()}
    ns_ms = sum(kernels[k]["ms_per_step"] for k in ("syrk", "syrk_poly", "gemm_axpy", "normalize", "norm_finalize",
                                                    "ns_small", "ns_grouped")
                if k in kernels)
    rec["ns"] = {
        "ms_per_step": round(ns_ms, 4),
        "effective_tflops_conventional": round(conv / (ns_ms * 1e-3) / 1e12, 2),
        "algorithmic_tflops": round(alg / (ns_ms * 1e-3) / 1e12, 2),
        "algorithmic_frac_of_peak": round(alg / (ns_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    traffic, traffic_src = load_traffic(dom, w.key)
    rec["roofline"] = {
        "kernel": dom, "bound": dk["bound"], "achieved": round(dk["achieved"], 2),
        "peak": PEAK_BF16_TFLOPS if dk["bound"] == "mfma" else PEAK_HBM_GBS, "unit": dk["unit"],
        "frac": round(dk["frac"], 4), "traffic": traffic, "traffic_source": traffic_src,
        "work_per_launch": dk["work_per_launch"], "mean_launch_ms": dk["mean_launch_ms"],
        "measured_over": f"{steps} eager steps in the timed configuration, launched kernel by kernel right "
                         f"after the timed graph replays (HIP events on each kernel's own stream)",
    }

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
    rec["buckets_ns_one_stream"] = buckets_out
    if not detail:
        plan.close()
        return rec

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
    rec["device_copy_gbs"] = round(2 * (1 << 30) / (sorted(cp_ms[1:])[2] * 1e-3) / 1e9, 1)
    del cp_src, cp_dst

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    plan.close()
    del params, plan

    # ---- CPU oracle: timing on the sample, and parity of the sampled first step -------
    rec["cpu_baseline"] = None
    rec["parity"] = None
    if cpu_leg:
        log(f"{key}: CPU oracle on {sum(len(v) for v in sample.values())} sampled matrices")
        from oracle import muon_oracle as orc
        per_matrix = {}
        worst, bitwise_ok = 0.0, True
        t_cpu = time.perf_counter()
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
            per_matrix[key] = float(np.median(times))
        cpu_s = time.perf_counter() - t_cpu

        def conv_of(k):
            return w.steps * (4.0 * k[0] * k[0] * k[1] + 2.0 * k[0] ** 3)
        # buckets left out of the sample: per-matrix time at the sampled buckets' FLOP rate
        rate = sum(conv_of(k) * len(sample[k]) for k in sample) / max(cpu_s, 1e-9)
        unsampled = [k for k in buckets if k not in sample]
        for k in unsampled:
            per_matrix[k] = conv_of(k) / rate
        oracle_step_s = sum(per_matrix[k] * len(buckets[k]) for k in buckets)
        n_sample = sum(len(v) for v in sample.values())
        desc = ", ".join(f"{len(sample.get(k, []))} of {len(buckets[k])} ({k[0]}x{k[1]})" for k in buckets)
        if unsampled:
            desc += (f"; {', '.join(f'{k[0]}x{k[1]}' for k in unsampled)} timed at the sampled buckets' "
                     f"rate ({rate / 1e12:.3f} TFLOP/s conventional)")
        rec["cpu_baseline"] = {
            "value": round(conv / oracle_step_s / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{n_sample} matrices, one full float64 step each (momentum, normalise, {w.steps} NS "
                      f"iterations, apply), {cpu_s:.1f} s of CPU time: {desc}; per bucket the first matrix, "
                      f"for large buckets also the last and the extreme per-expert gradient scales, then "
                      f"evenly spaced matrices within a {ORACLE_BUDGET_S:.0f} s estimate. Step time "
                      f"extrapolated as the sum over buckets of count x median per-matrix time = "
                      f"{oracle_step_s:.1f} s",
            "ms_per_step": oracle_step_s * 1e3,
        }
        rec["parity"] = {"sampled_matrices": n_sample, "ns_worst_rel_frobenius": worst, "ns_tolerance": 1e-2,
                         "momentum_and_apply_bitwise": bitwise_ok, "ok": bool(worst <= 1e-2 and bitwise_ok)}
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--others", default=",".join(OTHER_WORKLOADS),
                    help="comma-separated workloads also stepped after the headline one and reported under "
                         "other_workloads ('none' to skip)")
    ap.add_argument("--others-steps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--max-workspace-gib", type=float, default=-1.0,
                    help="workspace cap in GiB (0: none; default: none if it fits next to the inputs, "
                         "else 16 GiB, or 8 GiB when memory is short)")
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
    if args.steps < 1 or args.warmup < 1 or args.others_steps < 1:
        print(json.dumps({"error": "--steps, --warmup and --others-steps must be >= 1"}))
        return 2

    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    torch.cuda.set_device(0)

    rec = run_workload(args.workload, args, args.steps, args.warmup, not args.no_cpu_baseline, True)
    others = []
    if args.others and args.others != "none":
        for key in args.others.split(","):
            if key == args.workload:
                continue
            o = run_workload(key, args, args.others_steps, 2, False, False)
            o.pop("_w")
            others.append(o)
    w = rec.pop("_w")

    out = {
        "metric": METRIC,
        "value": rec["effective_tflops_conventional"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, sigma) draws on the GPU; no dataset, no trained weights)",
        "config": {
            "workload": w.key, "description": w.description,
            "matrices": rec["matrices"], "buckets": rec["buckets"], "chunks": rec["chunks"],
            "workspace_gib": rec["workspace_gib"],
            "ns_iterations": w.steps, "coefficients": [w.a, w.b, w.c], "beta": w.beta,
            "lr": w.lr, "wd": w.wd, "parallelism": "single GPU",
            "streams": "two (pipeline)" if args.pipeline else "one",
        },
        "roofline": rec["roofline"],
        "cpu_baseline": rec["cpu_baseline"],
        "graph": rec["graph"],
        "ns": dict(rec["ns"], conventional_flops_per_step=rec["conventional_flops_per_step"],
                   algorithmic_flops_per_step=rec["algorithmic_flops_per_step"]),
        "algorithmic_frac_of_peak_over_step": rec["algorithmic_frac_of_peak_over_step"],
        "kernels": rec["kernels"],
        "buckets": rec["buckets_ns_one_stream"],
        "device_copy_gbs": rec["device_copy_gbs"],
        "parity": rec["parity"],
        "input_generation_s": rec["input_generation_s"],
        "other_workloads": others,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
