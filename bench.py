#!/usr/bin/env python3
"""Throughput of one SignMuon worker step on one MI355X.

A step is one worker's momentum EMA with per-matrix norms, Newton-Schulz
(5 quintic iterations, bf16 MFMA / fp32 accumulation), sign + 1-bit pack
(written by the last product's epilogue),
then the majority vote over the M workers' packed buffers resident on the GPU
and the update W <- W - eta * vote.  Default workload: one 4096 x 14336 bf16
matrix (Llama-3-8B MLP shape), 1% heavy columns, M = 7 workers.

Prints one JSON line.  The timed region records HIP events on the stream
the kernels run on between every library call, so per-kernel times come from
the same steps as the headline number.

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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused-pack", action="store_true",
                    help="pack the signs with sign_pack after the last product instead of in it")
    ap.add_argument("--unfused-tail", action="store_true",
                    help="run majority_vote and apply_update as two calls instead of vote_and_update")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra measurements after the timed steps "
                         "(profiling runs then trace the step's kernels only)")
    ap.add_argument("--extras", default="cold,int8,reorth,dion,library,configs",
                    help="comma list of extra measurements to run after the timed steps: "
                         "cold (elementwise kernels with cold caches), int8 (int8 SUM exchange), "
                         "reorth (re-orthogonalised update), dion (Dion step), "
                         "library (vendor GEMM library on the same shapes), "
                         "configs (ns_orthogonalize on the other workloads' matrix sets)")
    ap.add_argument("--repeat-kernel", default=None,
                    help="profiling aid: after the run, launch one stage N more times "
                         "(gram|poly|apply|momentum|pack|vote|update|copy:N)")
    return ap.parse_args()


def ns_flops(s: int, l: int, c_nonzero: bool):
    """Algorithmic flops of one iteration: symmetric Gram, symmetric A*A, B*X."""
    gram = s * (s + 1) * l
    poly = s * s * (s + 1) if c_nonzero else 0
    apply = 2 * s * s * l
    return gram, poly, apply


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the step has no multi-GPU path; use --gpus 1"}))
        sys.exit(2)

    import torch

    import matrix_aware_optimizer_amd as mao
    from workloads import WORKLOADS, gen_G, gen_M0, gen_W0

    wl = WORKLOADS[args.workload]
    if len(set(wl.shapes)) != 1 or len(wl.shapes) != 1:
        # the instrumented step below drives the stage kernels of one matrix shape
        raise SystemExit("bench.py times single-matrix workloads (4 or 5); others are parity cases")
    rows, cols = wl.shapes[0]
    s, l = min(rows, cols), max(rows, cols)
    if rows > cols or s % mao.MUON_NS_PAD or l % mao.MUON_NS_PAD:
        raise SystemExit("bench workload must be wide and pad-free")
    dev = torch.device("cuda", 0)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    prec = wl.precision
    a, b, c = wl.coeffs

    def dev_tensor(arr, dt):
        if dt == "bf16":
            return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(arr).to(dev)

    t0 = time.time()
    W = dev_tensor(gen_W0(wl), wl.w_dtype)
    M0 = gen_M0(wl)
    Ms = [dev_tensor(M0, wl.m_dtype) for _ in range(wl.workers)]
    Gs = [dev_tensor(gen_G(wl, k, 0), wl.g_dtype) for k in range(wl.workers)]
    gen_s = time.time() - t0

    n = wl.numel
    nwords = mao.packed_words(n)
    offsets = torch.tensor([0, n], dtype=torch.int64, device=dev)
    sumsq = torch.zeros(1, dtype=torch.float32, device=dev)
    mom_ws = torch.empty(mao.muon_momentum_workspace_bytes(n, 1), dtype=torch.uint8, device=dev)
    X = [torch.empty((s, l), dtype=tdt[prec], device=dev) for _ in range(2)]
    A = torch.empty((s, s), dtype=tdt[prec], device=dev)
    B = torch.empty((s, s), dtype=tdt[prec], device=dev)
    # split scratch of the stage calls (zeroed once; every call leaves its counters at zero)
    stage_ws = mao.new_stage_workspace(s, l, 1, prec, dev)
    fold = prec == "bf16" and wl.m_dtype == "bf16"      # wide and pad-free: checked above
    fuse_signs = prec == "bf16" and wl.ns_steps > 0 and not args.unfused_pack
    fuse_tail = not args.unfused_tail
    bits = torch.zeros((wl.workers, nwords), dtype=torch.int64, device=dev)
    vote = torch.zeros(nwords, dtype=torch.int64, device=dev)

    def worker(k, ev=None):
        """a1-a6 for worker k; with `ev`, record an event after every call."""
        mark = (lambda name: ev.append((name, torch.cuda.Event(enable_timing=True))) or
                ev[-1][1].record()) if ev is not None else (lambda name: None)
        mark("start")
        mao.muon_momentum(Ms[k], Gs[k], wl.beta, wl.alpha, offsets, sumsq, mom_ws)
        mark("momentum")
        if not fold:
            mao.ns_normalize(Ms[k].view(rows, cols), sumsq, X[0], prec)
            mark("normalize")
        cur = 0
        for it in range(wl.ns_steps):
            # a bf16 wide pad-free momentum is read as is by the first iteration,
            # whose products fold in the Frobenius scaling (as ns_orthogonalize does)
            Xc, ss = (Ms[k].view(1, rows, cols), sumsq) if fold and it == 0 else (X[cur], None)
            mao.ns_gram(Xc, A, prec, sumsq=ss, workspace=stage_ws)
            mark("gram")
            if c != 0.0:
                mao.ns_poly(A, B, b, c, prec, workspace=stage_ws)
                mark("poly")
            Bm, alpha = (B, 1.0) if c != 0.0 else (A, b)
            if fuse_signs and it + 1 == wl.ns_steps:
                # the last product packs the signs of its values (nothing else of
                # the direction is needed by the vote)
                mao.ns_apply_signs(Bm, Xc, None, bits[k], a, alpha, prec, sumsq=ss, workspace=stage_ws)
                mark("apply_signs")
            else:
                mao.ns_apply(Bm, Xc, X[1 - cur], a, alpha, prec, sumsq=ss, workspace=stage_ws)
                mark("apply")
            cur = 1 - cur
        if not fuse_signs or wl.ns_steps == 0:
            mao.sign_pack(X[cur], bits[k])
            mark("pack")

    def tail(ev=None):
        def mark(name):
            if ev is not None:
                ev.append((name, torch.cuda.Event(enable_timing=True)))
                ev[-1][1].record()
        if fuse_tail:
            # a7 + a8 in one pass: the vote is never written (nothing else reads it)
            mao.vote_and_update(W, bits, wl.eta)
            mark("vote_update")
        else:
            mao.majority_vote(bits, vote)
            mark("vote")
            mao.apply_update(W, vote, wl.eta)
            mark("update")

    # the other workers' packed signs, resident on the GPU (what an all-gather would deliver)
    for k in range(1, wl.workers):
        worker(k)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        worker(0)
        tail()
    torch.cuda.synchronize()

    cur_final = wl.ns_steps % 2          # X buffer holding the final direction
    events = []
    t_start = time.perf_counter()
    for _ in range(args.steps):
        ev = []
        worker(0, ev)
        tail(ev)
        events.append(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    # per-kernel times from the events of the timed steps
    per = {}
    step_ms = []
    for ev in events:
        prev = ev[0][1]
        for name, e in ev[1:]:
            per.setdefault(name, []).append(prev.elapsed_time(e))
            prev = e
        step_ms.append(ev[0][1].elapsed_time(ev[-1][1]))
    launches = {k: len(v) / args.steps for k, v in per.items()}
    avg = {k: float(np.mean(v)) for k, v in per.items()}            # ms per launch
    total = {k: avg[k] * launches[k] for k in avg}                  # ms per step

    ms_per_step = wall * 1e3 / args.steps
    gram_f, poly_f, apply_f = ns_flops(s, l, c != 0.0)
    ns_ms = sum(total[k] for k in ("normalize", "gram", "poly", "apply", "apply_signs") if k in total)
    ns_flop = wl.ns_steps * (gram_f + poly_f + apply_f)
    peak = PEAK_BF16_TFLOPS if prec == "bf16" else PEAK_F32_TFLOPS
    ns_tflops = ns_flop / (ns_ms * 1e-3) / 1e12

    es = {"bf16": 2, "f32": 4}
    bytes_momentum = n * (2 * es[wl.m_dtype] + es[wl.g_dtype])
    bytes_pack = n * es[prec] + nwords * 8
    bytes_vote = (wl.workers + 1) * nwords * 8
    bytes_update = 2 * n * es[wl.w_dtype] + nwords * 8

    def gbs(nbytes, key):
        return nbytes / (avg[key] * 1e-3) / 1e9

    kernels = {
        "momentum": {"ms": avg["momentum"], "GB/s": gbs(bytes_momentum, "momentum")},
        "gram": {"ms": avg["gram"], "TFLOP/s": gram_f / (avg["gram"] * 1e-3) / 1e12},
        "apply": {"ms": avg["apply"], "TFLOP/s": apply_f / (avg["apply"] * 1e-3) / 1e12},
    }

    def standalone(fn, reps=20):
        """Average time of `reps` back-to-back calls (after 3 untimed), for a
        kernel the step runs fused into another."""
        for _ in range(3):
            fn()
        t0_, t1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0_.record()
        for _ in range(reps):
            fn()
        t1_.record()
        torch.cuda.synchronize()
        return t0_.elapsed_time(t1_) / reps

    bytes_vote_update = 2 * n * es[wl.w_dtype] + wl.workers * nwords * 8
    if "vote_update" in avg:
        kernels["vote_update"] = {"ms": avg["vote_update"], "GB/s": gbs(bytes_vote_update, "vote_update")}
    for key, fn, nb in (("vote", lambda: mao.majority_vote(bits, vote), bytes_vote),
                        ("update", lambda: mao.apply_update(W, vote, wl.eta), bytes_update)):
        if key in avg:
            kernels[key] = {"ms": avg[key], "GB/s": gbs(nb, key)}
        else:
            # fused into vote_and_update in the step; timed on its own here
            avg[key] = standalone(fn)
            launches[key] = 0.0
            kernels[key] = {"ms": avg[key], "GB/s": gbs(nb, key), "fused_in_step": True}
    if "normalize" in avg:
        kernels["normalize"] = {"ms": avg["normalize"],
                                "GB/s": gbs(n * (es[wl.m_dtype] + es[prec]), "normalize")}
    if "poly" in avg:
        kernels["poly"] = {"ms": avg["poly"], "TFLOP/s": poly_f / (avg["poly"] * 1e-3) / 1e12}
    if "apply_signs" in avg:
        kernels["apply_signs"] = {"ms": avg["apply_signs"],
                                  "TFLOP/s": apply_f / (avg["apply_signs"] * 1e-3) / 1e12}
    if "pack" in avg:
        kernels["pack"] = {"ms": avg["pack"], "GB/s": gbs(bytes_pack, "pack")}
    else:
        # fused into the last product in the step; the standalone kernel (the
        # path of tall or fp32 problems) is timed here on the same buffers
        avg["pack"] = standalone(lambda: mao.sign_pack(X[0], bits[0]))
        launches["pack"] = 0.0
        kernels["pack"] = {"ms": avg["pack"], "GB/s": gbs(bytes_pack, "pack"), "fused_in_step": True}
    for k in kernels:
        kernels[k]["launches_per_step"] = launches[k]
        if "GB/s" in kernels[k]:
            kernels[k]["frac_hbm"] = kernels[k]["GB/s"] / PEAK_HBM_GBS
        else:
            kernels[k]["frac_peak"] = kernels[k]["TFLOP/s"] / peak

    dominant = max(total, key=total.get)
    counters = recorded_traffic({"pack": "sign_pack", "vote": "majority_vote"}.get(dominant, dominant),
                                rows, cols)
    traffic = None if counters is None else counters["bytes"]
    dom_flops = {"gram": gram_f, "poly": poly_f, "apply": apply_f}.get(dominant)
    if dom_flops is not None:
        ach = dom_flops / (avg[dominant] * 1e-3) / 1e12
        roofline = {"kernel": dominant, "bound": "mfma", "achieved": ach, "peak": peak,
                    "unit": "TFLOP/s", "frac": ach / peak, "traffic": traffic,
                    "per_launch_flops": dom_flops, "avg_launch_ms": avg[dominant]}
    else:
        nb = {"momentum": bytes_momentum, "pack": bytes_pack, "vote": bytes_vote,
              "update": bytes_update, "vote_update": bytes_vote_update}[dominant]
        ach = gbs(nb, dominant)
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": traffic,
                    "per_launch_bytes": nb, "avg_launch_ms": avg[dominant]}

    if counters is not None:
        roofline["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"
        roofline["traffic_detail"] = counters

    result = {
        "metric": METRIC,
        "value": 1e3 / ms_per_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prec,
        "data": "synthetic",
        "config": {"workload": wl.name, "shape": [rows, cols], "workers": wl.workers,
                   "ns_steps": wl.ns_steps, "coeffs": list(wl.coeffs), "beta": wl.beta,
                   "eta": wl.eta, "momentum_dtype": wl.m_dtype, "weight_dtype": wl.w_dtype},
        "ns_tflops": ns_tflops,
        "ns_frac_bf16_peak": ns_tflops / peak,
        "orthogonalizations_per_s": 1e3 / ns_ms,
        "pack_gbs": kernels["pack"]["GB/s"],
        "vote_gbs": kernels["vote"]["GB/s"],
        "event_ms_per_step": float(np.median(step_ms)),
        "kernels": kernels,
        "roofline": roofline,
        "input_generation_s": gen_s,
    }
    extras = set() if args.no_extras else {e.strip() for e in args.extras.split(",") if e.strip()}
    if "cold" in extras:
        result["kernels_cold"] = cold_elementwise(mao, torch, wl, Ms[0], Gs[0], W, X[cur_final], bits, vote,
                                                  offsets, sumsq, mom_ws, dev)
    if "int8" in extras:
        result["int8_exchange"] = int8_exchange(mao, torch, X[cur_final], wl, n, nwords, dev)
    if "reorth" in extras:
        result["reorthogonalized_update"] = reorth_update(mao, torch, wl, W, vote, dev)
    if "dion" in extras:
        result["dion"] = dion_bench(mao, torch, dev)
    if "configs" in extras:
        result["ns_configs"] = ns_configs(mao, torch, dev)
    if "library" in extras and prec == "bf16":
        result["library_reference"] = library_reference(torch, avg, s, l, dev)

    if args.repeat_kernel:
        name, _, cnt = args.repeat_kernel.partition(":")
        cnt = int(cnt or 10)
        for _ in range(cnt):
            if name == "gram":
                mao.ns_gram(X[0], A, prec, workspace=stage_ws)
            elif name == "poly":
                mao.ns_poly(A, B, b, c, prec, workspace=stage_ws)
            elif name == "apply":
                mao.ns_apply(B, X[0], X[1], a, 1.0, prec, workspace=stage_ws)
            elif name == "copy":
                X[1].copy_(X[0])
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


def cold_elementwise(mao, torch, wl, M, G, W, U, bits, vote, offsets, sumsq, mom_ws, dev, reps=5):
    """The HBM-bound kernels with cold caches: before each timed call a 1 GiB buffer
    is read (a sum over it), which replaces the 256 MB Infinity Cache's contents with
    clean lines, so every operand comes from HBM and no write-back of someone else's
    data is charged to the kernel.  HIP events bracket the call alone, on the stream
    it runs on."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)        # 1 GiB
    n, nwords = wl.numel, mao.packed_words(wl.numel)
    es = {"bf16": 2, "f32": 4}
    calls = {
        "momentum": (lambda: mao.muon_momentum(M, G, wl.beta, wl.alpha, offsets, sumsq, mom_ws),
                     n * (2 * es[wl.m_dtype] + es[wl.g_dtype])),
        "pack": (lambda: mao.sign_pack(U, bits[0]), n * es[wl.precision] + nwords * 8),
        "vote": (lambda: mao.majority_vote(bits, vote), (wl.workers + 1) * nwords * 8),
        "update": (lambda: mao.apply_update(W, vote, wl.eta), 2 * n * es[wl.w_dtype] + nwords * 8),
        "vote_update": (lambda: mao.vote_and_update(W, bits, wl.eta),
                        2 * n * es[wl.w_dtype] + wl.workers * nwords * 8),
    }
    out = {}
    for name, (fn, nbytes) in calls.items():
        times = []
        for _ in range(reps):
            flush.sum()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            fn()
            end.record()
            torch.cuda.synchronize()
            times.append(start.elapsed_time(end))
        ms = float(np.median(times))
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}
    del flush
    return out


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
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}
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
    unpack = timed(lambda: mao.unpack_signs(vote, step._sbar))
    dense = timed(lambda: mao.apply_update_dense(Wc, step.U, wl.eta))
    gbs_u = (n * es_u + n / 8) / (unpack * 1e-3) / 1e9
    gbs_d = (n * (2 * es_w + es_u)) / (dense * 1e-3) / 1e9
    return {"ms": whole,
            "unpack_signs": {"ms": unpack, "GB/s": gbs_u, "frac_hbm": gbs_u / PEAK_HBM_GBS},
            "apply_update_dense": {"ms": dense, "GB/s": gbs_d, "frac_hbm": gbs_d / PEAK_HBM_GBS}}


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


def ns_configs(mao, torch, dev, reps=5):
    """ns_orthogonalize alone on the other workloads' matrix sets, as one call per
    set (the library batches equal shapes): the GPT-2-small layer set (48
    matrices, 4 shapes), 128 batched 1024 x 1024, and 7168 x 18432 (fp32 momentum),
    5 quintic steps.  The per-matrix sums of squares are passed in, as the
    optimizer step passes muon_momentum's (computed once here, before timing).
    Seeded normal inputs; HIP events on the stream the call runs on."""
    from workloads import WORKLOADS
    out = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    for cfg in (2, 3, 5):
        wl = WORKLOADS[cfg]
        offs = wl.offsets
        M = torch.randn(wl.numel, generator=gen, device=dev).to(tdt[wl.m_dtype])
        U = torch.empty(wl.numel, dtype=tdt[wl.precision], device=dev)
        offs_d = torch.from_numpy(offs).to(dev)
        sums = torch.zeros(len(wl.shapes), dtype=torch.float32, device=dev)
        mws = torch.empty(mao.muon_momentum_workspace_bytes(wl.numel, len(wl.shapes)), dtype=torch.uint8,
                          device=dev)
        # beta = 1, alpha = 0 leaves M as it is and writes its sums of squares
        mao.muon_momentum(M, M, 1.0, 0.0, offs_d, sums, mws)
        probs = [(M[offs[j]:offs[j + 1]].view(r, c), U[offs[j]:offs[j + 1]].view(r, c), sums[j:j + 1])
                 for j, (r, c) in enumerate(wl.shapes)]
        ws = torch.empty(max(mao.ns_workspace_bytes(probs, wl.precision), 1), dtype=torch.uint8, device=dev)
        a, b, c = wl.coeffs
        mao.ns_orthogonalize(probs, a, b, c, wl.ns_steps, wl.precision, ws)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            mao.ns_orthogonalize(probs, a, b, c, wl.ns_steps, wl.precision, ws)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        flops = 0
        for r, cc in wl.shapes:
            g_, p_, ap_ = ns_flops(min(r, cc), max(r, cc), c != 0.0)
            flops += wl.ns_steps * (g_ + p_ + ap_)
        tf = flops / (ms * 1e-3) / 1e12
        out[wl.name] = {"workload": wl.name, "matrices": len(wl.shapes), "ms_per_call": ms,
                          "orthogonalizations_per_s": len(wl.shapes) / (ms * 1e-3),
                          "TFLOP/s": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS}
        del M, U, ws
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
    for key, ours in (("apply_aX_plus_BX", "apply"), ("gram_dense_XXt", "gram"), ("poly_bA_plus_cAA", "poly")):
        if ours in avg:
            out[key]["this_library_ms"] = avg[ours]
            out[key]["speedup_vs_library"] = out[key]["library_ms"] / avg[ours]
    return out


def cpu_baseline(wl):
    """The fp64 oracle on the host cores: the elementwise stages on the whole matrix
    and one of the Newton-Schulz iterations, scaled to a full worker step."""
    import oracle.muon_oracle as O
    from workloads import gen_G, gen_M0, gen_W0

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    rows, cols = wl.shapes[0]
    W0, M0, G = gen_W0(wl), gen_M0(wl), gen_G(wl, 0, 0)
    a, b, c = wl.coeffs
    t0 = time.perf_counter()
    Mn = O.momentum(M0, wl.m_dtype, G, wl.g_dtype, wl.beta, wl.alpha)
    Mf = O.decode(Mn, wl.m_dtype).reshape(rows, cols)
    X = O.frobenius_normalize(Mf)
    X = X.T if rows > cols else X
    t_elem0 = time.perf_counter() - t0
    t1 = time.perf_counter()
    X1 = O.ns_iterate(X, a, b, c, 1)
    t_iter = time.perf_counter() - t1
    t2 = time.perf_counter()
    words = O.sign_pack(X1)
    packed = np.stack([words] * wl.workers)
    vote = O.majority_vote(packed, wl.numel)
    O.apply_update(W0, wl.w_dtype, vote, wl.eta)
    t_elem1 = time.perf_counter() - t2
    est = t_elem0 + t_elem1 + wl.ns_steps * t_iter
    return {"value": 1.0 / est, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle on the full {rows}x{cols} matrix: momentum, norm, sign/pack, "
                      f"{wl.workers}-way vote, update, and 1 of {wl.ns_steps} Newton-Schulz "
                      f"iterations (timed {t_iter:.2f} s), step time = elementwise + "
                      f"{wl.ns_steps} x iteration = {est:.2f} s",
            "cpu": platform.processor() or platform.machine()}


if __name__ == "__main__":
    main()
