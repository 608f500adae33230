#!/usr/bin/env python3
"""Throughput of one SignMuon worker step on one MI355X.

A step is one worker's momentum EMA with per-matrix norms, Newton-Schulz
(5 iterations, bf16 MFMA operands / fp32 accumulation; fp32 for the 256 x 256
workload), sign + 1-bit pack (written by the last product's epilogue where the
matrix allows it), then the majority vote over the M workers' packed buffers
resident on the GPU and the update W <- W - eta * vote.  The headline workload
is one 4096 x 14336 bf16 matrix (Llama-3-8B MLP shape), 1% heavy columns,
M = 7 workers.

The headline times the shipped calls (SignMuonStep: muon_momentum,
ns_orthogonalize, vote_and_update) with HIP events between them.  The same step
driven through the stage calls (ns_gram / ns_poly / ns_apply, the kernels
ns_orthogonalize launches) gives per-kernel times and the roofline.  Then the
full step of the four other workloads, the elementwise kernels with cold
caches (the pack and vote GB/s reported at the top level), the extra rows, and
the CPU oracle timed on the host.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload 4] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

METRIC = "Muon steps/sec + NS MFMA TFLOP/s (% bf16 peak) at 4096×14336; pack/vote GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "matrix_aware_optimizer_amd", "csrc")
KERNEL_SOURCES = ["common.h", "gemm.h", "ns.hip", "elementwise.hip"]
TRAFFIC_RECORDS = os.path.join(ROOT, "profiles", "signmuon_step_{shape}_hbm_traffic.md")


def kernel_sources_digest() -> str:
    """First 16 hex digits of the sha256 of the kernel sources, in a fixed order."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, rows: int, cols: int):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter summary.

    The summary holds one ``record:`` line per kernel with the calibrated
    FETCH_SIZE and WRITE_SIZE bytes and the digest of the kernel sources it
    was taken with.  Returns None when there is no record or the sources
    have changed since."""
    path = TRAFFIC_RECORDS.format(shape=f"{rows}x{cols}")
    if not os.path.exists(path):
        return None
    digest = kernel_sources_digest()
    for line in open(path):
        if not line.startswith("record:"):
            continue
        fields = dict(kv.split("=", 1) for kv in line.split()[1:])
        if fields.get("kernel") == kernel and fields.get("sources") == digest:
            return {"bytes": int(fields["fetch_bytes"]) + int(fields["write_bytes"]),
                    "fetch_bytes": int(fields["fetch_bytes"]),
                    "write_bytes": int(fields["write_bytes"]),
                    "source": os.path.relpath(path, ROOT)}
    return None


MFMA_RECORDS = os.path.join(ROOT, "profiles", "signmuon_step_{shape}_mfma_counters.md")


def recorded_mfma(kernel: str, rows: int, cols: int):
    """MFMA busy fraction, sustained clock and L2 hit rate of ``kernel`` from the
    committed rocprofv3 counter summary (``record:`` lines), or None when there is
    none for the current kernel sources."""
    path = MFMA_RECORDS.format(shape=f"{rows}x{cols}")
    if not os.path.exists(path):
        return None
    digest = kernel_sources_digest()
    for line in open(path):
        if not line.startswith("record:"):
            continue
        fields = dict(kv.split("=", 1) for kv in line.split()[1:])
        if fields.get("kernel") == kernel and fields.get("sources") == digest:
            out = {k: float(v) for k, v in fields.items() if k not in ("kernel", "sources")}
            out["source"] = os.path.relpath(path, ROOT)
            return out
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--config-steps", type=int, default=10,
                    help="timed steps of each of the other workloads (the 7168 x 18432 one: half)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused-tail", action="store_true",
                    help="run majority_vote and apply_update as two calls instead of vote_and_update")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip every measurement after the headline step "
                         "(profiling runs then trace the step's kernels only)")
    ap.add_argument("--extras", default="stages,configs,cold,int8,reorth,dion,library",
                    help="comma list of measurements after the headline step: "
                         "stages (the same step as stage calls, with HIP events between kernels: "
                         "per-kernel times and the roofline), configs (the full step of the other "
                         "workloads), cold (elementwise kernels with cold caches), int8 (int8 SUM "
                         "exchange), reorth (re-orthogonalised update), dion (Dion step), "
                         "library (vendor GEMM library on the same shapes)")
    ap.add_argument("--repeat-kernel", default=None,
                    help="profiling aid: after the run, launch one stage N more times "
                         "(gram|poly|apply|copy:N)")
    return ap.parse_args()


def ns_flops(s: int, l: int, c_nonzero: bool):
    """Algorithmic flops of one iteration: symmetric Gram, symmetric A*A, B*X."""
    gram = s * (s + 1) * l
    poly = s * s * (s + 1) if c_nonzero else 0
    apply = 2 * s * s * l
    return gram, poly, apply


def ns_work(wl):
    """(algorithmic flops, algorithmic HBM bytes if every intermediate streams
    through memory) of the Newton-Schulz iteration over all of the workload's
    matrices.  Bytes per iteration: X read by the Gram, A written and read, B
    written and read, X read and X' written by the product, in the operand type."""
    es = 2 if wl.precision == "bf16" else 4
    flops = nbytes = 0
    for r, c in wl.shapes:
        s, l = min(r, c), max(r, c)
        g, p, a = ns_flops(s, l, wl.coeffs[2] != 0.0)
        flops += wl.ns_steps * (g + p + a)
        sq = 4 * s * s if wl.coeffs[2] != 0.0 else 2 * s * s
        nbytes += wl.ns_steps * es * (3 * s * l + sq)
    return flops, nbytes


ES = {"bf16": 2, "f32": 4}


def elementwise_bytes(wl):
    """Algorithmic bytes of the HBM-bound stages of one step (whole parameter set)."""
    n = wl.numel
    nwords = (n + 63) // 64
    out = {"momentum": n * (2 * ES[wl.m_dtype] + ES[wl.g_dtype]),
           "pack": n * ES[wl.precision] + nwords * 8,
           "vote": (wl.workers + 1) * nwords * 8}
    if wl.w_dtype is not None:
        out["update"] = 2 * n * ES[wl.w_dtype] + nwords * 8
        out["vote_update"] = 2 * n * ES[wl.w_dtype] + wl.workers * nwords * 8
    return out


class Events:
    """HIP events on the current stream (the one every call here runs on).

    ``mark(name)`` records an event after a named call (the step's timeline, gaps
    between kernels included).  ``kernel(name)`` hands a pair of events to the
    library for the next kernel it launches (muon_time_next_launch): they are
    recorded by that launch at the kernel's own start and end, so their interval is
    the kernel's duration, the figure rocprofv3's kernel trace also reports."""

    def __init__(self, torch, mao=None):
        self.torch = torch
        self.mao = mao
        self.marks = []
        self.kernels = []

    def mark(self, name):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.marks.append((name, ev))

    def kernel(self, name):
        e0, e1 = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()            # creates the HIP events; the launch records them again
        self.mao.time_next_launch(e0, e1)
        self.kernels.append((name, e0, e1))


def per_kernel_ms(events_list):
    """{name: [ms per launch]} from the launch-bound event pairs, and launches per step."""
    per, counts = {}, {}
    for ev in events_list:
        for name, e0, e1 in ev.kernels:
            per.setdefault(name, []).append(e0.elapsed_time(e1))
            counts[name] = counts.get(name, 0) + 1
    return per, {k: v / len(events_list) for k, v in counts.items()}


def per_call_ms(events_list):
    """{name: [ms per step]} summed over the calls of that name in each step, plus
    {name: launches per step}."""
    per, counts = {}, {}
    for ev in events_list:
        prev = ev.marks[0][1]
        step = {}
        for name, e in ev.marks[1:]:
            step[name] = step.get(name, 0.0) + prev.elapsed_time(e)
            counts[name] = counts.get(name, 0) + 1
            prev = e
        for k, v in step.items():
            per.setdefault(k, []).append(v)
    return per, {k: v / len(events_list) for k, v in counts.items()}


def make_inputs(torch, wl, dev):
    """W0, M0 and worker 0's G on the device, from the seeded host generators."""
    from workloads import gen_G, gen_M0, gen_W0

    def dev_tensor(arr, dt):
        if dt == "bf16":
            return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(arr).to(dev)

    W0 = gen_W0(wl)
    return {"W": None if W0 is None else dev_tensor(W0, wl.w_dtype),
            "M0": dev_tensor(gen_M0(wl), wl.m_dtype),
            "G0": dev_tensor(gen_G(wl, 0, 0), wl.g_dtype),
            "G": lambda k: dev_tensor(gen_G(wl, k, 0), wl.g_dtype)}


def product_step(mao, torch, wl, dev, steps, warmup, fuse_tail=True):
    """Time the shipped step: SignMuonStep's calls for worker 0 (muon_momentum, then
    ns_orthogonalize writing the packed signs, plus sign_pack where the signs are not
    fused), then the vote over the M resident buffers and the update
    (vote_and_update), HIP events between the calls.  The other M - 1 workers' packed
    signs are made once beforehand by the same calls on their own gradients."""
    t0 = time.time()
    inp = make_inputs(torch, wl, dev)
    step = mao.SignMuonStep(wl.shapes, m_dtype=wl.m_dtype, precision=wl.precision,
                            coeffs=wl.coeffs, ns_steps=wl.ns_steps, beta=wl.beta, alpha=wl.alpha,
                            eta=wl.eta, device=dev)
    bits = step.new_bits(wl.workers)
    for k in range(1, wl.workers):
        Mk = inp["M0"].clone()
        Gk = inp["G"](k)
        step.worker(Mk, Gk, bits[k])
        del Mk, Gk
    M, G, W = inp["M0"].clone(), inp["G0"], inp["W"]
    gen_s = time.time() - t0
    vote = torch.zeros(step.nwords, dtype=torch.int64, device=dev)

    def one(ev=None):
        mark = ev.mark if ev is not None else (lambda name: None)
        kern = ev.kernel if ev is not None else (lambda name: None)
        mark("start")
        kern("momentum")
        step.momentum(M, G)
        mark("momentum")
        if step.signs_per_matrix:
            step.orthogonalize(M, bits[0])
            mark("ns")
        else:
            step.orthogonalize(M)
            mark("ns")
            kern("pack")
            step.pack(bits[0])
            mark("pack")
        if W is not None and wl.workers > 0:
            if fuse_tail:
                kern("vote_update")
                step.vote_update(W, bits, fused=True)
                mark("vote_update")
            else:
                step.vote_update(W, bits, vote_out=vote)
                mark("vote_and_update_unfused")

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    step.check()                 # a split product that gave up would make the timing meaningless
    evs = []
    t_start = time.perf_counter()
    for _ in range(steps):
        ev = Events(torch, mao)
        one(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step.check()
    per, launches = per_call_ms(evs)
    med = {k: float(np.median(v)) for k, v in per.items()}
    kper, _ = per_kernel_ms(evs)
    kmed = {k: float(np.median(v)) for k, v in kper.items()}
    step_ev = [ev.marks[0][1].elapsed_time(ev.marks[-1][1]) for ev in evs]
    ms = wall * 1e3 / steps
    flops, ns_bytes = ns_work(wl)
    eb = elementwise_bytes(wl)
    peak = PEAK_BF16_TFLOPS if wl.precision == "bf16" else PEAK_F32_TFLOPS
    ns_ms = med["ns"]
    tf = flops / (ns_ms * 1e-3) / 1e12
    hbm_floor_ms = ns_bytes / (PEAK_HBM_GBS * 1e9) * 1e3
    mfma_floor_ms = flops / (peak * 1e12) * 1e3
    out = {"workload": wl.name, "matrices": len(wl.shapes), "workers": wl.workers,
           "steps": steps, "ms_per_step": ms, "steps_per_s": 1e3 / ms,
           "event_ms_per_step": float(np.median(step_ev)),
           "calls_ms": med,
           "ns": {"ms": ns_ms, "TFLOP/s": tf, "frac_peak": tf / peak,
                  "peak": "bf16 MFMA" if wl.precision == "bf16" else "fp32 MFMA",
                  "orthogonalizations_per_s": len(wl.shapes) / (ns_ms * 1e-3),
                  "algorithmic_flops": flops,
                  # both floors: the MFMA one, and the HBM one if X, A and B all
                  # streamed through memory between the products
                  "mfma_floor_ms": mfma_floor_ms, "hbm_floor_ms": hbm_floor_ms,
                  "frac_of_floor": max(mfma_floor_ms, hbm_floor_ms) / ns_ms},
           "input_generation_s": gen_s}
    # elementwise kernels: the kernel's own duration (launch-bound events); the
    # momentum call also runs the short per-matrix reduction of the norms
    gb = {k: eb[k] / (kmed[k] * 1e-3) / 1e9 for k in ("momentum", "pack", "vote_update") if k in kmed}
    out["elementwise"] = {k: {"ms": kmed[k], "GB/s": v, "frac_hbm": v / PEAK_HBM_GBS, "call_ms": med[k]}
                          for k, v in gb.items()}
    out["_objects"] = {"step": step, "M": M, "G": G, "W": W, "bits": bits, "vote": vote}
    return out


def stage_sequence(mao, torch, wl, dev, objs, steps, warmup):
    """The headline step with Newton-Schulz driven through the stage calls (ns_gram,
    ns_poly, ns_apply, and ns_apply_signs for the last product: the kernels and
    arguments ns_orthogonalize launches, bit-identical by test), with HIP events
    between every kernel on the stream they run on: per-kernel times of the timed
    steps and the roofline of the dominant kernel."""
    rows, cols = wl.shapes[0]
    s, l = min(rows, cols), max(rows, cols)
    prec = wl.precision
    a, b, c = wl.coeffs
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[prec]
    step, M, G, W, bits = objs["step"], objs["M"], objs["G"], objs["W"], objs["bits"]
    X = [torch.empty((1, s, l), dtype=tdt, device=dev) for _ in range(2)]
    Xlo = torch.empty((1, s, l), dtype=tdt, device=dev)
    A = torch.empty((1, s, s), dtype=tdt, device=dev)
    B = torch.empty((1, s, s), dtype=tdt, device=dev)
    stage_ws = mao.new_stage_workspace(s, l, 1, prec, dev)
    fold = prec == "bf16" and wl.m_dtype == "bf16"
    kres = mao.ns_residual_iterations(rows, cols, a, b, c, wl.ns_steps, prec)

    def one(ev=None):
        mark = ev.mark if ev is not None else (lambda name: None)
        kern = ev.kernel if ev is not None else (lambda name: None)
        mark("start")
        kern("momentum")
        step.momentum(M, G)
        mark("momentum")
        if not fold:
            kern("normalize")
            mao.ns_normalize(M.view(1, rows, cols), step.sumsq, X[0], prec)
            mark("normalize")
        cur = 0
        for it in range(wl.ns_steps):
            Xc, ss = (M.view(1, rows, cols), step.sumsq) if fold and it == 0 else (X[cur], None)
            lo_in = Xlo if 1 <= it <= kres else None
            lo_out = Xlo if it < kres and it + 1 < wl.ns_steps else None
            kern("gram")
            mao.ns_gram(Xc, A, prec, sumsq=ss, workspace=stage_ws)
            mark("gram")
            if c != 0.0:
                kern("poly")
                mao.ns_poly(A, B, b, c, prec, workspace=stage_ws)
                mark("poly")
            Bm, alpha = (B, 1.0) if c != 0.0 else (A, b)
            if it + 1 == wl.ns_steps:
                kern("apply_signs")
                mao.ns_apply_signs(Bm, Xc, None, bits[0], a, alpha, prec, sumsq=ss, workspace=stage_ws,
                                   X_lo=lo_in)
                mark("apply_signs")
            else:
                # the products that also read or write the residual of X are timed apart
                kern("apply" if lo_in is None and lo_out is None else "apply_residual")
                mao.ns_apply(Bm, Xc, X[1 - cur], a, alpha, prec, sumsq=ss, workspace=stage_ws,
                             X_lo=lo_in, Xout_lo=lo_out)
                mark("apply")
            cur = 1 - cur
        kern("vote_update")
        step.vote_update(W, bits, fused=True)
        mark("vote_update")

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    evs = []
    t_start = time.perf_counter()
    for _ in range(steps):
        ev = Events(torch, mao)
        one(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    mao.ns_workspace_status(stage_ws)
    per, launches = per_kernel_ms(evs)
    # per launch: the kernel's own duration, averaged over the timed steps' launches
    avg = {k: float(np.mean(v)) for k, v in per.items()}
    total = {k: avg[k] * launches[k] for k in avg}
    gram_f, poly_f, apply_f = ns_flops(s, l, c != 0.0)
    peak = PEAK_BF16_TFLOPS if prec == "bf16" else PEAK_F32_TFLOPS
    eb = elementwise_bytes(wl)
    kernels = {}
    for k, fl in (("gram", gram_f), ("poly", poly_f), ("apply", apply_f), ("apply_residual", apply_f),
                  ("apply_signs", apply_f)):
        if k in avg:
            tf = fl / (avg[k] * 1e-3) / 1e12
            kernels[k] = {"ms": avg[k], "TFLOP/s": tf, "frac_peak": tf / peak, "launches_per_step": launches[k]}
    for k in ("momentum", "vote_update"):
        gbs = eb[k] / (avg[k] * 1e-3) / 1e9
        kernels[k] = {"ms": avg[k], "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS, "launches_per_step": launches[k]}
    if "normalize" in avg:
        gbs = wl.numel * (ES[wl.m_dtype] + ES[prec]) / (avg["normalize"] * 1e-3) / 1e9
        kernels["normalize"] = {"ms": avg["normalize"], "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}
    ns_ms = sum(total[k] for k in ("normalize", "gram", "poly", "apply", "apply_residual", "apply_signs")
                if k in total)
    flops, _ = ns_work(wl)
    return {"ms_per_step": wall * 1e3 / steps, "ns_kernel_ms": ns_ms,
            "ns_kernel_TFLOP/s": flops / (ns_ms * 1e-3) / 1e12, "residual_iterations": kres,
            "kernels": kernels, "total_ms": total,
            "_buffers": {"X": X, "A": A, "B": B, "stage_ws": stage_ws}}


def roofline_of(kernels, total, rows, cols, wl):
    """Roofline of the kernel function with the most time per step (from the stage
    sequence).  The B X product is one kernel whatever its epilogue writes (the
    direction, its residual, or only the packed signs), so its launches are taken
    together, as rocprofv3 averages them under one kernel name."""
    groups = {"apply": ("apply", "apply_residual", "apply_signs"), "gram": ("gram",), "poly": ("poly",),
              "momentum": ("momentum",), "vote_update": ("vote_update",), "normalize": ("normalize",)}
    tot = {g: sum(total.get(k, 0.0) for k in ks) for g, ks in groups.items()}
    dominant = max(tot, key=tot.get)
    launches = sum(kernels[k]["launches_per_step"] for k in groups[dominant] if k in kernels)
    ms = tot[dominant] / launches
    peak = PEAK_BF16_TFLOPS if wl.precision == "bf16" else PEAK_F32_TFLOPS
    counters = recorded_traffic(dominant, rows, cols)
    s, l = min(rows, cols), max(rows, cols)
    fl = dict(zip(("gram", "poly", "apply"), ns_flops(s, l, wl.coeffs[2] != 0.0)))
    if dominant in fl:
        ach = fl[dominant] / (ms * 1e-3) / 1e12
        roof = {"kernel": dominant, "bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                "frac": ach / peak, "traffic": None if counters is None else counters["bytes"],
                "per_launch_flops": fl[dominant], "avg_launch_ms": ms, "launches_per_step": launches}
    else:
        nb = elementwise_bytes(wl)[dominant]
        ach = nb / (ms * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "traffic": None if counters is None else counters["bytes"],
                "per_launch_bytes": nb, "avg_launch_ms": ms, "launches_per_step": launches}
    roof["timing"] = "HIP events recorded by each launch at the kernel's start and end"
    if counters is not None:
        roof["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"
        roof["traffic_detail"] = counters
    util = recorded_mfma(dominant, rows, cols)
    if util is not None:
        roof["mfma_counters"] = util
    return roof


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the exchange of packed signs between GPUs "
                                   "is not built, so only --gpus 1 is measured"}))
        sys.exit(2)

    import torch

    import matrix_aware_optimizer_amd as mao
    from workloads import WORKLOADS

    dev = torch.device("cuda", 0)
    wl = WORKLOADS[args.workload]
    extras = set() if args.no_extras else {e.strip() for e in args.extras.split(",") if e.strip()}

    head = product_step(mao, torch, wl, dev, args.steps, args.warmup, fuse_tail=not args.unfused_tail)
    objs = head.pop("_objects")
    rows, cols = wl.shapes[0]
    peak = PEAK_BF16_TFLOPS if wl.precision == "bf16" else PEAK_F32_TFLOPS
    result = {
        "metric": METRIC,
        "value": head["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.precision,
        "data": "synthetic",
        "config": {"workload": wl.name, "shapes": sorted(set(wl.shapes)), "matrices": len(wl.shapes),
                   "workers": wl.workers, "ns_steps": wl.ns_steps, "coeffs": list(wl.coeffs),
                   "beta": wl.beta, "eta": wl.eta, "momentum_dtype": wl.m_dtype,
                   "weight_dtype": wl.w_dtype, "path": "SignMuonStep (product calls)"},
        "ns_tflops": head["ns"]["TFLOP/s"],
        "ns_frac_bf16_peak": head["ns"]["TFLOP/s"] / PEAK_BF16_TFLOPS,
        "orthogonalizations_per_s": head["ns"]["orthogonalizations_per_s"],
        "step": head,
    }
    single = len(wl.shapes) == 1 and rows <= cols and rows % mao.MUON_NS_PAD == 0 \
        and cols % mao.MUON_NS_PAD == 0 and wl.w_dtype is not None
    stages = None
    if "stages" in extras and single:
        stages = stage_sequence(mao, torch, wl, dev, objs, args.steps, args.warmup)
        bufs = stages.pop("_buffers")
        result["stage_sequence"] = stages
        result["kernels"] = stages["kernels"]
        result["roofline"] = roofline_of(stages["kernels"], stages["total_ms"], rows, cols, wl)
    else:
        # no per-kernel events: the whole orthogonalisation against the MFMA peak
        result["roofline"] = {"kernel": "ns_orthogonalize (all launches)", "bound": "mfma",
                              "achieved": head["ns"]["TFLOP/s"], "peak": peak, "unit": "TFLOP/s",
                              "frac": head["ns"]["frac_peak"], "traffic": None}

    if "cold" in extras:
        cold = cold_elementwise(mao, torch, wl, objs, dev)
        result["kernels_cold"] = cold
        result["pack_gbs"] = cold["pack"]["GB/s"]
        result["vote_gbs"] = cold["vote"]["GB/s"]
    if "configs" in extras:
        cfgs = {}
        del objs
        for cfg in (1, 2, 3, 4, 5):
            if cfg == args.workload:
                continue
            other = WORKLOADS[cfg]
            n_steps = max(2, args.config_steps // (2 if cfg == 5 else 1))
            r = product_step(mao, torch, other, dev, n_steps, 2)
            r.pop("_objects")
            cfgs[other.name] = r
            torch.cuda.empty_cache()
        cfgs[wl.name] = {k: v for k, v in head.items()}
        result["configs"] = cfgs
        objs = None
    if "int8" in extras and stages is not None:
        result["int8_exchange"] = int8_exchange(mao, torch, bufs["X"][0], wl, wl.numel,
                                                mao.packed_words(wl.numel), dev)
    if "reorth" in extras and single:
        vote = torch.zeros(mao.packed_words(wl.numel), dtype=torch.int64, device=dev)
        W = make_inputs(torch, wl, dev)["W"]
        bits = torch.randint(-2 ** 62, 2 ** 62, (1, vote.numel()), dtype=torch.int64, device=dev)
        mao.majority_vote(bits, vote)
        result["reorthogonalized_update"] = reorth_update(mao, torch, wl, W, vote, dev)
    if "dion" in extras:
        result["dion"] = dion_bench(mao, torch, dev)
    if "library" in extras and stages is not None and wl.precision == "bf16":
        avg = {k: v["ms"] for k, v in stages["kernels"].items()}
        result["library_reference"] = library_reference(torch, avg, min(rows, cols), max(rows, cols), dev)

    if args.repeat_kernel and stages is not None:
        name, _, cnt = args.repeat_kernel.partition(":")
        cnt = int(cnt or 10)
        a, b, c = wl.coeffs
        X, A, B, stage_ws = bufs["X"], bufs["A"], bufs["B"], bufs["stage_ws"]
        for _ in range(cnt):
            if name == "gram":
                mao.ns_gram(X[0], A, wl.precision, workspace=stage_ws)
            elif name == "poly":
                mao.ns_poly(A, B, b, c, wl.precision, workspace=stage_ws)
            elif name == "apply":
                mao.ns_apply(B, X[0], X[1], a, 1.0, wl.precision, workspace=stage_ws)
            elif name == "copy":
                X[1].copy_(X[0])
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
        result["cpu_baseline"]["other_workloads"] = cpu_baseline_configs()
    print(json.dumps(result), flush=True)


def cold_elementwise(mao, torch, wl, objs, dev, reps=5):
    """The HBM-bound kernels with cold caches: before each timed call a 1 GiB buffer
    is read (a sum over it), which replaces the 256 MB Infinity Cache's contents with
    clean lines, so every operand comes from HBM and no write-back of someone else's
    data is charged to the kernel.  The kernel's duration comes from HIP events its
    launch records at its start and end (on the stream it runs on); the median of
    ``reps`` calls.  The momentum call's short norm reduction is not in the timed
    kernel."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)        # 1 GiB
    step, M, G, W, bits, vote = (objs[k] for k in ("step", "M", "G", "W", "bits", "vote"))
    U = step.U
    U.copy_(M.to(U.dtype))                  # a direction-like operand for the standalone pack
    eb = elementwise_bytes(wl)
    calls = {
        "momentum": (lambda: step.momentum(M, G), eb["momentum"]),
        "pack": (lambda: mao.sign_pack(U, bits[0]), eb["pack"]),
        "vote": (lambda: mao.majority_vote(bits, vote), eb["vote"]),
    }
    if W is not None:
        calls["update"] = (lambda: mao.apply_update(W, vote, wl.eta), eb["update"])
        calls["vote_update"] = (lambda: mao.vote_and_update(W, bits, wl.eta), eb["vote_update"])
    # reference: a device-to-device copy moving as many bytes as the vote, and as the
    # pack (half read, half written); its kernel is the runtime's, so only the call
    # bracket is timed here and its own duration is read from the kernel trace
    refs = {}
    for name in ("vote", "pack"):
        half = eb[name] // 2
        src, dst = torch.empty(half, dtype=torch.uint8, device=dev), torch.empty(half, dtype=torch.uint8, device=dev)
        refs["copy_like_" + name] = ((lambda d=dst, s_=src: d.copy_(s_)), eb[name])
    out = {}
    for name, (fn, nbytes) in calls.items():
        fn()
        times, calls_ms = [], []
        for _ in range(reps):
            flush.sum()
            ev = Events(torch, mao)
            ev.mark("start")
            ev.kernel(name)
            fn()
            ev.mark("end")
            torch.cuda.synchronize()
            times.append(ev.kernels[0][1].elapsed_time(ev.kernels[0][2]))
            calls_ms.append(ev.marks[0][1].elapsed_time(ev.marks[1][1]))
        ms = float(np.median(times))
        gbs = nbytes / (ms * 1e-3) / 1e9
        # call_ms: events around the host call, dispatch gaps included
        out[name] = {"ms": ms, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
                     "call_ms": float(np.median(calls_ms))}
    for name, (fn, nbytes) in refs.items():
        fn()
        calls_ms = []
        for _ in range(reps):
            flush.sum()
            ev = Events(torch, mao)
            ev.mark("start")
            fn()
            ev.mark("end")
            torch.cuda.synchronize()
            calls_ms.append(ev.marks[0][1].elapsed_time(ev.marks[1][1]))
        out[name] = {"bytes": nbytes, "call_ms": float(np.median(calls_ms))}
    del flush, refs
    return out


def kernel_and_call_ms(mao, torch, fn, reps):
    """(median kernel ms, ms per call) of a call that launches one kernel: the
    kernel's own start and end events (muon_time_next_launch) for each of `reps`
    calls, and HIP events around the `reps` calls back to back (launch gaps
    included)."""
    pairs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()            # creates the HIP events; the launch records them again
        mao.time_next_launch(e0, e1)
        fn()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    kernel = float(np.median([a.elapsed_time(b) for a, b in pairs]))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return kernel, start.elapsed_time(end) / reps


def int8_exchange(mao, torch, U, wl, n, nwords, dev, reps=10):
    """The int8 exchange format next to the 1-bit one: sign_int8 of one direction,
    sum_int8 over the M resident int8 buffers, threshold_pack of the sum; each
    kernel timed with HIP events on the stream it runs on.  Not part of the step."""
    M = wl.workers
    S = torch.empty((M, n), dtype=torch.int8, device=dev)
    for k in range(M):
        mao.sign_int8(U, S[k])
    total = torch.empty(n, dtype=torch.int8, device=dev)
    vote = torch.zeros(nwords, dtype=torch.int64, device=dev)
    es = 2 if U.dtype == torch.bfloat16 else 4
    calls = {
        "sign_int8": (lambda: mao.sign_int8(U, S[0]), n * (es + 1)),
        "sum_int8": (lambda: mao.sum_int8(S, total), n * (M + 1)),
        "threshold_pack": (lambda: mao.threshold_pack(total, vote), n + nwords * 8),
    }
    out = {}
    for name, (fn, nbytes) in calls.items():
        fn()
        ms, call_ms = kernel_and_call_ms(mao, torch, fn, reps)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS, "call_ms": call_ms}
    out["payload_bytes_per_worker"] = {"fp32": 4 * n, "int8": n, "packed_bits": nwords * 8}
    return out


def reorth_update(mao, torch, wl, W, vote, dev, reps=3):
    """The optional local re-orthogonalisation of the vote: unpack_signs, Newton-Schulz
    of the +-1 matrix, apply_update_dense; timed as a whole and kernel by kernel
    (HIP events on the stream the kernels run on).  Not part of the step."""
    step = mao.SignMuonStep(wl.shapes, m_dtype=wl.precision, precision=wl.precision,
                            coeffs=wl.coeffs, ns_steps=wl.ns_steps, beta=wl.beta, alpha=wl.alpha,
                            eta=wl.eta, device=dev)
    Wc = W.clone()
    step.reorthogonalized_update(Wc, vote)          # allocates its buffers
    torch.cuda.synchronize()

    def timed(fn):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps

    n = step.numel
    es_u = step.U.element_size()
    es_w = W.element_size()
    whole = timed(lambda: step.reorthogonalized_update(Wc, vote))
    unpack, unpack_call = kernel_and_call_ms(mao, torch, lambda: mao.unpack_signs(vote, step._sbar), 10)
    dense, dense_call = kernel_and_call_ms(mao, torch, lambda: mao.apply_update_dense(Wc, step.U, wl.eta), 10)
    gbs_u = (n * es_u + n / 8) / (unpack * 1e-3) / 1e9
    gbs_d = (n * (2 * es_w + es_u)) / (dense * 1e-3) / 1e9
    return {"ms": whole,
            "unpack_signs": {"ms": unpack, "GB/s": gbs_u, "frac_hbm": gbs_u / PEAK_HBM_GBS, "call_ms": unpack_call},
            "apply_update_dense": {"ms": dense, "GB/s": gbs_d, "frac_hbm": gbs_d / PEAK_HBM_GBS,
                                   "call_ms": dense_call}}


def dion_bench(mao, torch, dev, reps=5):
    """One Dion step on the d = 768 layer set (48 fp32 matrices, one batched call per
    shape) at ranks d/4, d/8, d/16; HIP events on the stream it runs on.  Algorithmic
    flops per matrix: B Q, B^T P, P R^T, P Q^T (2mnr each) and two Cholesky-QR
    passes (Gram and P L^-T, 2mr^2 each)."""
    from workloads import DION_WORKLOADS, gen_dion
    out = {}
    for rank in (192, 96, 48):
        wl = DION_WORKLOADS[rank]
        inp = gen_dion(wl)
        offs, qoffs = wl.offsets, wl.q_offsets
        M = torch.zeros(wl.numel, dtype=torch.float32, device=dev)
        G = torch.from_numpy(inp["G"]).to(dev)
        X = torch.from_numpy(inp["W0"]).to(dev)
        Q = torch.from_numpy(inp["Q0"]).to(dev)
        probs = [(M[offs[j]:offs[j + 1]].view(r, c), G[offs[j]:offs[j + 1]].view(r, c),
                  X[offs[j]:offs[j + 1]].view(r, c), Q[qoffs[j]:qoffs[j + 1]].view(c, rank))
                 for j, (r, c) in enumerate(wl.shapes)]
        ws = torch.empty(mao.dion_workspace_bytes(probs, rank), dtype=torch.uint8, device=dev)
        mao.dion_step(probs, rank, wl.mu, wl.eta, ws)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            mao.dion_step(probs, rank, wl.mu, wl.eta, ws)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        flops = sum(8 * r * c * rank + 8 * r * rank * rank for r, c in wl.shapes)
        tf = flops / (ms * 1e-3) / 1e12
        out[f"rank_{rank}"] = {"ms": ms, "TFLOP/s": tf, "frac_fp32_peak": tf / PEAK_F32_TFLOPS,
                               "workload": wl.name}
    return out


def library_reference(torch, avg, s, l, dev, reps=10):
    """Context only, not on the product path: the vendor GEMM library (hipBLASLt,
    reached through torch.matmul on contiguous bf16 operands) timed on the shapes
    of the Newton-Schulz products, beside this library's own kernels from the
    timed steps.  The library computes the Gram in full (dense flops), the
    kernels here its lower triangle."""
    g = torch.Generator(device=dev).manual_seed(7)
    X = torch.randn(s, l, device=dev, generator=g).to(torch.bfloat16)
    Xt = X.t().contiguous()
    Bm = torch.randn(s, s, device=dev, generator=g).to(torch.bfloat16)
    out_sl = torch.empty(s, l, device=dev, dtype=torch.bfloat16)
    out_ss = torch.empty(s, s, device=dev, dtype=torch.bfloat16)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    apply_ms = timed(lambda: torch.addmm(X, Bm, X, beta=3.4445, alpha=1.0, out=out_sl))
    gram_ms = timed(lambda: torch.matmul(X, Xt, out=out_ss))
    poly_ms = timed(lambda: torch.addmm(Bm, Bm, Bm, beta=-4.775, alpha=2.0315, out=out_ss))
    dense_apply, dense_gram, dense_poly = 2.0 * s * s * l, 2.0 * s * s * l, 2.0 * s ** 3
    out = {"library": "hipBLASLt via torch.matmul/addmm (bf16, fp32 accumulation)",
           "apply_aX_plus_BX": {"library_ms": apply_ms, "library_TFLOP/s": dense_apply / apply_ms / 1e9},
           "gram_dense_XXt": {"library_ms": gram_ms, "library_TFLOP/s": dense_gram / gram_ms / 1e9},
           "poly_bA_plus_cAA": {"library_ms": poly_ms, "library_TFLOP/s": dense_poly / poly_ms / 1e9}}
    # the apply with no residual, else the one that also reads and writes the bf16
    # residual of X (more bytes than the library's aX + BX moves)
    apply_kind = "apply" if "apply" in avg else "apply_residual"
    for key, ours in (("apply_aX_plus_BX", apply_kind), ("gram_dense_XXt", "gram"), ("poly_bA_plus_cAA", "poly")):
        if ours in avg:
            out[key]["this_library_ms"] = avg[ours]
            out[key]["this_library_kernel"] = ours
            out[key]["speedup_vs_library"] = out[key]["library_ms"] / avg[ours]
    return out


def _numpy_f32_step(wl, W0, M0, G, others):
    """The same worker step in numpy float32 (the CPU baseline comparable in
    precision to the GPU's fp32 accumulation; not the oracle): EMA, Frobenius
    scaling, the iteration on the short side, sign and packing (numpy.packbits,
    little bit order), the vote over the M packed buffers and the update."""
    rows, cols = wl.shapes[0]
    a, b, c = (np.float32(x) for x in wl.coeffs)
    to32 = (lambda x, dt: (x.astype(np.uint32) << 16).view(np.float32) if dt == "bf16" else x)
    Mn = np.float32(wl.beta) * to32(M0, wl.m_dtype) + np.float32(wl.alpha) * to32(G, wl.g_dtype)
    X = Mn.reshape(rows, cols)
    X = (X.T if rows > cols else X) / np.float32(np.sqrt(np.sum(Mn.astype(np.float64) ** 2)))
    X = np.ascontiguousarray(X, dtype=np.float32)
    for _ in range(wl.ns_steps):
        A = X @ X.T
        Bm = b * A + c * (A @ A)
        X = a * X + Bm @ X
    U = X.T if rows > cols else X
    mine = np.packbits(~(U.ravel() < 0), bitorder="little")
    buffers = np.stack([mine] + [others] * (wl.workers - 1))
    counts = np.unpackbits(buffers, axis=1, bitorder="little")[:, :wl.numel].sum(0, dtype=np.int32)
    vote = 2 * counts >= wl.workers
    return to32(W0, wl.w_dtype) - np.float32(wl.eta) * np.where(vote, np.float32(1), np.float32(-1))


def _numpy_f32_set_step(wl, W0, M0, G):
    """_numpy_f32_step over a set of matrices (each on its short side), for the
    per-workload CPU timings."""
    a, b, c = (np.float32(x) for x in wl.coeffs)
    to32 = (lambda x, dt: (x.astype(np.uint32) << 16).view(np.float32) if dt == "bf16" else x)
    Mn = np.float32(wl.beta) * to32(M0, wl.m_dtype) + np.float32(wl.alpha) * to32(G, wl.g_dtype)
    U = np.empty_like(Mn)
    offs = wl.offsets
    for j, (rows, cols) in enumerate(wl.shapes):
        X = Mn[offs[j]:offs[j + 1]].reshape(rows, cols)
        X = np.ascontiguousarray((X.T if rows > cols else X) / np.float32(np.sqrt(np.sum(X.astype(np.float64) ** 2))))
        for _ in range(wl.ns_steps):
            A = X @ X.T
            Bm = b * A + c * (A @ A)
            X = a * X + Bm @ X
        U[offs[j]:offs[j + 1]] = (X.T if rows > cols else X).ravel()
    mine = np.packbits(~(U < 0), bitorder="little")
    if W0 is None:
        return mine
    counts = np.unpackbits(np.stack([mine] * wl.workers), axis=1, bitorder="little")[:, :wl.numel].sum(0, dtype=np.int32)
    vote = 2 * counts >= wl.workers
    return to32(W0, wl.w_dtype) - np.float32(wl.eta) * np.where(vote, np.float32(1), np.float32(-1))


def _oracle_set_step(wl, W0, M0, G):
    """One worker step of the fp64 oracle over a workload's matrix set: momentum,
    Newton-Schulz of every matrix, sign and packing, then (workloads with
    weights) the vote over M copies of the worker's bits and the update."""
    import oracle.muon_oracle as O
    Mn = O.momentum(M0, wl.m_dtype, G, wl.g_dtype, wl.beta, wl.alpha)
    U = O.worker_direction(Mn, wl.m_dtype, wl.shapes, wl.offsets, *wl.coeffs, wl.ns_steps)
    words = O.sign_pack(U)
    if W0 is not None:
        O.apply_update(W0, wl.w_dtype, O.majority_vote(np.stack([words] * wl.workers), wl.numel), wl.eta)


def cpu_baseline_configs(samples=((1, 1), (2, 4), (3, 4))):
    """fp64 oracle and numpy fp32 worker steps on a bounded sample of the
    smaller workloads: (workload, k) times one worker step over the set's first k
    matrices (the GPT-2-small set's first layer, four of the 128 1024^2
    matrices), each measured once, reported per orthogonalisation so that it
    compares with the GPU's orthogonalisations per second on the whole set.  The
    7168x18432 step takes minutes on the host and is not timed."""
    import dataclasses
    from workloads import WORKLOADS, gen_G, gen_M0, gen_W0
    out = {}
    for cfg, k in samples:
        full = WORKLOADS[cfg]
        wl = dataclasses.replace(full, shapes=full.shapes[:k])
        W0, M0, G = gen_W0(wl), gen_M0(wl), gen_G(wl, 0, 0)
        t0 = time.perf_counter()
        _oracle_set_step(wl, W0, M0, G)
        t_oracle = time.perf_counter() - t0
        t1 = time.perf_counter()
        _numpy_f32_set_step(wl, W0, M0, G)
        t_f32 = time.perf_counter() - t1
        out[full.name] = {"sample": f"one worker step over the first {k} of the set's {len(full.shapes)} matrices",
                          "oracle_seconds": t_oracle, "oracle_orthogonalizations_per_s": k / t_oracle,
                          "numpy_f32_seconds": t_f32, "numpy_f32_orthogonalizations_per_s": k / t_f32}
    return out


def cpu_baseline(wl):
    """The fp64 oracle on the host cores, one whole worker step on the headline
    workload, measured (nothing extrapolated): momentum, Newton-Schulz with all its
    iterations, sign and packing, the vote over M packed buffers (worker 0's and M - 1
    copies of it: the vote costs the same whatever the bits), the update.  Beside it
    the same step in numpy float32 (not the oracle)."""
    import oracle.muon_oracle as O
    from workloads import gen_G, gen_M0, gen_W0

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    rows, cols = wl.shapes[0]
    W0, M0, G = gen_W0(wl), gen_M0(wl), gen_G(wl, 0, 0)
    t0 = time.perf_counter()
    Mn = O.momentum(M0, wl.m_dtype, G, wl.g_dtype, wl.beta, wl.alpha)
    U = O.newton_schulz(O.decode(Mn, wl.m_dtype).reshape(rows, cols), *wl.coeffs, wl.ns_steps)
    words = O.sign_pack(U.ravel())
    vote = O.majority_vote(np.stack([words] * wl.workers), wl.numel)
    O.apply_update(W0, wl.w_dtype, vote, wl.eta)
    t_oracle = time.perf_counter() - t0
    t1 = time.perf_counter()
    _numpy_f32_step(wl, W0, M0, G, np.packbits(np.ones(wl.numel, bool), bitorder="little"))
    t_f32 = time.perf_counter() - t1
    return {"value": 1.0 / t_oracle, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"one whole fp64 oracle worker step on the full {rows}x{cols} workload "
                      f"({wl.ns_steps} Newton-Schulz iterations, {wl.workers}-way vote over copies of "
                      f"worker 0's bits, update): {t_oracle:.2f} s measured",
            "numpy_f32": {"value": 1.0 / t_f32, "unit": "steps/s", "seconds": t_f32,
                          "sample": "the same step in numpy float32 (not the oracle)"},
            "cpu": platform.processor() or platform.machine(),
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


if __name__ == "__main__":
    main()
