#!/usr/bin/env python3
"""Benchmark of the SwiGLU MLP training step on one MI355X.

One step = the whole hot path over one batch: forward GEMM-1 + SwiGLU
epilogue, down GEMM, fused dgrad + SwiGLU-backward, dW_down, dx, dW1, run as
the product runs it (swiglu_mlp_fwd then swiglu_mlp_bwd on resident inputs);
ms_per_step, fwd_ms and bwd_ms time it.  A second loop launches the same six
GEMMs one by one through the single-step calls so that each kernel is timed
with HIP events on the stream it runs on.

Printed: one JSON line.  `value` is the fused dgrad kernel's throughput
(2*M*Dout*I FLOPs per launch / its mean event-timed duration) in TFLOP/s.  Extra fields: per-kernel times, the
paired fused-vs-unfused A/B comparison of the dgrad segment (random
interleave, medians, 3% tie rule, as the drop-h report times its variants),
the roofline of the fused kernel and the CPU oracle timed on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload target]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import random
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SOURCES = ["bwd_gemm_epilogue_amd/csrc/gemm_core.hpp", "bwd_gemm_epilogue_amd/csrc/swiglu_mlp.hip",
                  "bwd_gemm_epilogue_amd/csrc/swiglu_math.hpp", "bwd_gemm_epilogue_amd/csrc/skinny.hpp"]


def code_text(src: str) -> str:
    """Source text without comments and whitespace runs: the digest below
    changes with the code, not with its comments."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (profiles/<name>_traffic.json), if it was taken on the current kernel
    source; else None."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def measured_mfma(name: str):
    """MFMA busy and clock of a kernel from a committed rocprofv3 counter
    pass (profiles/<name>_mfma.json), if it was taken on the current kernel
    source; else None."""
    p = os.path.join(ROOT, "profiles", f"{name}_mfma.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest():
        return None
    return {k: t[k] for k in ("mfma_busy_pct", "clock_ghz", "pct_of_peak_at_2p4ghz")}


def fused_dgrad_bytes(M, I, Dout, experts=1):
    """Algorithmic HBM bytes of one fused dgrad launch, every tensor once in
    bf16: it reads dy [M,Dout], W_down ([I,Dout] per expert) and preact
    [M,2I], and writes grad_preact [M,2I] and h [M,I]."""
    return 2 * (M * Dout + experts * I * Dout + M * 2 * I + M * 2 * I + M * I)


def forward_bytes(M, D, I, Dout):
    """Algorithmic HBM bytes of one forward: reads x [M,D], W1 [D,2I] and
    W_down [I,Dout], writes preact [M,2I] and y [M,Dout]; the transient h
    [M,I] is written once and read once."""
    return 2 * (M * D + D * 2 * I + I * Dout + M * 2 * I + M * Dout + 2 * M * I)


def paired_samples(variants, rounds, stream, seed):
    """The drop-h report's protocol: `rounds` rounds, each running every
    variant once in a random order, timed with HIP events on `stream`.
    variants: {name: fn(events)}, where fn records events[0] .. events[k] on
    `stream` around its parts; returns {name: [[ms of part 0, ...], ...]}."""
    import torch
    rnd = random.Random(seed)
    out = {n: [] for n in variants}
    for _ in range(rounds):
        order = list(variants.items())
        rnd.shuffle(order)
        for name, fn in order:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            n = fn(ev)
            ev[n].synchronize()
            out[name].append([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    return out


def paired_summary(a, b, tag_a, tag_b):
    """Medians of two paired sample lists (one part each), the median paired
    relative delta (a - b) / b, and the 3% tie rule."""
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    delta = float(np.median((a - b) / b))
    return {f"{tag_a}_ms_median": round(float(np.median(a)), 4), f"{tag_b}_ms_median": round(float(np.median(b)), 4),
            "paired_delta": round(delta, 4),
            "verdict": "tie" if abs(delta) < 0.03 else (f"{tag_a} faster" if delta < 0 else f"{tag_b} faster")}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="target")
    ap.add_argument("--ab-pairs", type=int, default=40)
    ap.add_argument("--stack-layers", type=int, default=4, help="blocks in the stacked workload (0: skip)")
    ap.add_argument("--stack-iters", type=int, default=5)
    ap.add_argument("--other-workloads", type=int, default=1,
                    help="also time the fused dgrad at the small and Llama-like shapes and the decode forward (0: skip)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (1 GiB read, 1 GiB written), "
                         "the reference for scaling HBM byte counters")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bwd_gemm_epilogue_amd as sw
    from workload import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        return copy_calibration()
    from workload import MOE_WORKLOADS
    if args.workload in MOE_WORKLOADS:
        return bench_moe(args, MOE_WORKLOADS[args.workload])
    w = WORKLOADS[args.workload]
    if w.fwd_only:
        return bench_decode(args, w)
    M, D, I, Dout = w.M, w.D, w.I, w.Dout
    dev = torch.device("cuda:0")

    def to_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    xb, W1b, Wdb, dyb = make_inputs(w)
    x, W1, Wd, dy = (to_dev(a) for a in (xb, W1b, Wdb, dyb))
    print(f"[bench] inputs for {w.name} {M}x{D}x{I}x{Dout} ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    bf = torch.bfloat16
    preact = torch.empty((M, 2 * I), dtype=bf, device=dev)
    h_fwd = torch.empty((M, I), dtype=bf, device=dev)
    y = torch.empty((M, Dout), dtype=bf, device=dev)
    gp = torch.empty((M, 2 * I), dtype=bf, device=dev)
    h_bwd = torch.empty((M, I), dtype=bf, device=dev)
    dout = torch.empty((M, I), dtype=bf, device=dev)
    dx = torch.empty((M, D), dtype=bf, device=dev)
    dW1 = torch.empty((D, 2 * I), dtype=bf, device=dev)
    dWd = torch.empty((I, Dout), dtype=bf, device=dev)

    names = ["fwd_gemm1_swiglu", "fwd_down", "bwd_dgrad_fused", "bwd_dw_down", "bwd_dx", "bwd_dw1"]
    calls = [
        lambda: sw.swiglu_fwd_gemm1(x, W1, preact, h_fwd),
        lambda: sw.swiglu_fwd_down(h_fwd, Wd, y),
        lambda: sw.swiglu_bwd_dgrad_fused(dy, Wd, preact, gp, h_bwd),
        lambda: sw.swiglu_bwd_dw_down(h_bwd, dy, dWd),
        lambda: sw.swiglu_bwd_dx(gp, W1, dx),
        lambda: sw.swiglu_bwd_dw1(x, gp, dW1),
    ]
    flops = {
        "fwd_gemm1_swiglu": 4 * M * D * I, "fwd_down": 2 * M * I * Dout, "bwd_dgrad_fused": 2 * M * Dout * I,
        "bwd_dw_down": 2 * M * I * Dout, "bwd_dx": 4 * M * D * I, "bwd_dw1": 4 * M * D * I,
    }
    stream = torch.cuda.current_stream(dev)

    def step(evs=None):
        for k, c in enumerate(calls):
            if evs is not None:
                evs[k].record(stream)
            c()
        if evs is not None:
            evs[len(calls)].record(stream)

    # ---- the step: the whole-step calls of the product path
    # (swiglu_mlp_fwd, swiglu_mlp_bwd, whose plain-store GEMMs split their
    # last partly filled round of tiles) on resident inputs ----
    wsf = torch.empty(max(1, sw.swiglu_mlp_fwd_workspace(M, D, I, Dout)), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(1, sw.swiglu_mlp_bwd_workspace(M, D, I, Dout)), dtype=torch.uint8, device=dev)

    def whole(evs=None):
        if evs is not None:
            evs[0].record(stream)
        sw.swiglu_mlp_fwd(x, W1, Wd, preact, y, wsf)
        if evs is not None:
            evs[1].record(stream)
        sw.swiglu_mlp_bwd(x, W1, Wd, preact, dy, dx, dW1, dWd, wsb)
        if evs is not None:
            evs[2].record(stream)

    for _ in range(args.warmup):
        whole()
    torch.cuda.synchronize()
    wevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        whole(wevs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in wevs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in wevs]))
    step_ms = [e[0].elapsed_time(e[2]) for e in wevs]

    # ---- the same six GEMMs launched one by one through the single-step
    # calls (one launch each, no split tail), timed per kernel; B1's time
    # here is the headline value ----
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evsets = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(evsets[k])
    torch.cuda.synchronize()
    per = {n: [] for n in names}
    for evs in evsets:
        for k, n in enumerate(names):
            per[n].append(evs[k].elapsed_time(evs[k + 1]))
    ms = {n: float(np.mean(v)) for n, v in per.items()}
    b1_ms = ms["bwd_dgrad_fused"]
    b1_tflops = flops["bwd_dgrad_fused"] / (b1_ms * 1e-3) / 1e12
    total_flops = sum(flops.values())
    single_step_ms = float(np.mean([evs[0].elapsed_time(evs[-1]) for evs in evsets]))

    # ---- paired A/B (the drop-h report's protocol: randomly interleaved
    # rounds, medians, paired delta, < 3% a tie): fused dgrad segment vs
    # dgrad GEMM + elementwise; the save-h path's fused dgrad (grad_preact
    # only) vs the drop-h one; the residual epilogues vs the plain GEMMs ----
    def timed(fn):
        def run(ev):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            return 1
        return run

    ab = save_h_ab = residual = library_gemm = None
    if args.ab_pairs > 0:
        def seg_unfused():
            sw.swiglu_bwd_dgrad_plain(dy, Wd, dout)
            sw.swiglu_bwd_elementwise(preact, dout, gp, h_bwd)

        variants = {
            "fused": timed(lambda: sw.swiglu_bwd_dgrad_fused(dy, Wd, preact, gp, h_bwd)),
            "unfused": timed(seg_unfused),
            "fused_gp_only": timed(lambda: sw.swiglu_bwd_dgrad_fused_gp(dy, Wd, preact, gp)),
            # context, not the product: this library's plain dgrad GEMM (U1)
            # against the platform's library GEMM (torch.matmul, hipBLASLt)
            # computing the same product dout = dy . W_down^T
            "plain_gemm": timed(lambda: sw.swiglu_bwd_dgrad_plain(dy, Wd, dout)),
            "torch_matmul": timed(lambda: torch.matmul(dy, Wd.t(), out=dout)),
        }
        if D == Dout:
            y_res = torch.empty((M, D), dtype=bf, device=dev)
            dx_res = torch.empty((M, D), dtype=bf, device=dev)
            variants.update({
                "down": timed(lambda: sw.swiglu_fwd_down(h_fwd, Wd, y)),
                "down_residual": timed(lambda: sw.swiglu_fwd_down_residual(h_fwd, Wd, x, y_res)),
                "dx": timed(lambda: sw.swiglu_bwd_dx(gp, W1, dx)),
                "dx_residual": timed(lambda: sw.swiglu_bwd_dx_residual(gp, W1, dy, dx_res)),
            })
        for fn in variants.values():
            fn([torch.cuda.Event(enable_timing=True) for _ in range(2)])
        torch.cuda.synchronize()
        smp = paired_samples(variants, args.ab_pairs, stream, seed=1234)
        one = {n: [v[0] for v in smp[n]] for n in smp}
        ab = {"pairs": args.ab_pairs, **paired_summary(one["fused"], one["unfused"], "fused", "unfused"),
              "dout_hbm_bytes_avoided": 2 * M * I * 2}
        lib = paired_summary(one["plain_gemm"], one["torch_matmul"], "plain_gemm", "torch_matmul")
        fl_d = flops["bwd_dgrad_fused"]
        library_gemm = {"pairs": args.ab_pairs, "what": "dout = dy . W_down^T, bf16 out, no epilogue",
                        "plain_gemm_ms": lib["plain_gemm_ms_median"], "torch_matmul_ms": lib["torch_matmul_ms_median"],
                        "paired_delta_plain_vs_torch": lib["paired_delta"],
                        "plain_gemm_tflops": round(fl_d / (lib["plain_gemm_ms_median"] * 1e-3) / 1e12, 2),
                        "torch_matmul_tflops": round(fl_d / (lib["torch_matmul_ms_median"] * 1e-3) / 1e12, 2),
                        "fused_ms_same_rounds": round(float(np.median(one["fused"])), 4)}
        gp_only = paired_summary(one["fused_gp_only"], one["fused"], "gp_only", "fused")
        save_h_ab = {"pairs": args.ab_pairs,
                  "bwd_dgrad_gp_ms": gp_only["gp_only_ms_median"],
                  "bwd_dgrad_fused_ms_same_pairs": gp_only["fused_ms_median"],
                  "paired_delta_gp_only_vs_fused": gp_only["paired_delta"], "verdict": gp_only["verdict"],
                  "bwd_dgrad_gp_tflops": round(flops["bwd_dgrad_fused"] / (gp_only["gp_only_ms_median"] * 1e-3) / 1e12, 2),
                  "activation_bytes_after_fwd": {"drop_h": 2 * M * 2 * I, "save_h": 2 * M * 2 * I + 2 * M * I},
                  "h_bytes_not_written_in_bwd": 2 * M * I}
        if D == Dout:
            r_down = paired_summary(one["down_residual"], one["down"], "residual", "plain")
            r_dx = paired_summary(one["dx_residual"], one["dx"], "residual", "plain")
            residual = {"pairs": args.ab_pairs,
                        "fwd_down_ms": r_down["plain_ms_median"], "fwd_down_residual_ms": r_down["residual_ms_median"],
                        "fwd_down_paired_delta": r_down["paired_delta"],
                        "bwd_dx_ms": r_dx["plain_ms_median"], "bwd_dx_residual_ms": r_dx["residual_ms_median"],
                        "bwd_dx_paired_delta": r_dx["paired_delta"],
                        "epilogue_add_ms": round(r_down["residual_ms_median"] - r_down["plain_ms_median"]
                                                 + r_dx["residual_ms_median"] - r_dx["plain_ms_median"], 4),
                        "separate_add_hbm_bytes_avoided": 2 * 3 * M * D * 2,
                        "separate_add_ms_at_hbm_peak": round(2 * 3 * M * D * 2 / (PEAK_HBM_GBS * 1e9) * 1e3, 4)}

    # ---- one MLP block, drop-h against save-h (the drop-h report's table:
    # the normal MLPBlock keeps h, drop-h recomputes it), through the
    # autograd functions: fwd, bwd and full ms in randomly interleaved
    # rounds, and the memory each keeps after the forward and at its peak ----
    block = block_compare(sw, x, W1, Wd, dy, args.ab_pairs, stream) if args.ab_pairs > 0 else None

    # ---- stack of blocks (the drop-h report's 4-layer stack): forward,
    # backward and full ms through the autograd functions, after-forward and
    # peak allocated MiB above the inputs, drop-h vs save-h in alternation.
    # Layers 1..L-1 hold copies of layer 0's weight values (the same seeded
    # distribution; one more target-shape weight set costs ~20 s of CPU).
    stack = None
    if D == Dout and args.stack_layers > 0:
        L = args.stack_layers
        layers = [(W1.clone().requires_grad_(True), Wd.clone().requires_grad_(True)) for _ in range(L)]
        xs = x.clone().requires_grad_(True)
        res = {False: [], True: []}
        mem = {}
        # pass 0 measures memory from an emptied allocator cache (allocations
        # then land in fresh segments, as in a fresh process) and is not timed;
        # the timed passes run with a warm cache
        for it in range(1 + args.stack_iters):
            for save_h in (False, True):
                for W in (xs, *[w for pair in layers for w in pair]):
                    W.grad = None
                torch.cuda.synchronize()
                if it == 0:
                    torch.cuda.empty_cache()
                base = torch.cuda.memory_allocated()
                torch.cuda.reset_peak_memory_stats()
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record()
                out = sw.swiglu_mlp_stack(xs, layers, save_h=save_h)
                e[1].record()
                torch.cuda.synchronize()
                after = torch.cuda.memory_allocated() - base
                out.backward(dy)
                e[2].record()
                torch.cuda.synchronize()
                peak = torch.cuda.max_memory_allocated() - base
                del out
                if it > 0:
                    res[save_h].append((e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])))
                else:
                    mem[save_h] = (after, peak)
        stack = {"layers": L, "iters": args.stack_iters}
        for save_h, tag in ((False, "drop_h"), (True, "save_h")):
            f = float(np.median([a for a, _ in res[save_h]]))
            b = float(np.median([b for _, b in res[save_h]]))
            stack[tag] = {"fwd_ms": round(f, 4), "bwd_ms": round(b, 4), "full_ms": round(f + b, 4),
                          "after_fwd_MiB": round(mem[save_h][0] / 2**20, 3), "peak_MiB": round(mem[save_h][1] / 2**20, 3)}
        stack["after_fwd_saving_MiB"] = round((mem[True][0] - mem[False][0]) / 2**20, 3)
        stack["after_fwd_saving_expected_MiB"] = round(L * M * I * 2 / 2**20, 3)
        # the saved tensors' own bytes (the allocator's figure adds the slack
        # of blocks it does not split)
        stack["saved_tensor_MiB"] = {"drop_h": round(L * (M * 2 * I * 2 + M * D * 2) / 2**20, 3),
                                     "save_h": round(L * (M * 2 * I * 2 + M * D * 2 + M * I * 2) / 2**20, 3)}
        del layers, xs

    # ---- roofline of the fused dgrad kernel ----
    roofline = {"kernel": "bwd_dgrad_fused", "bound": "mfma", "achieved": round(b1_tflops, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(b1_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(f"dgrad_fused_{w.name}"),
                "counters": measured_mfma(f"dgrad_fused_{w.name}"),
                "algorithmic_flops_per_launch": flops["bwd_dgrad_fused"],
                "algorithmic_bytes_per_launch": fused_dgrad_bytes(M, I, Dout)}

    cpu = cpu_baseline(w, xb, W1b, Wdb, dyb, args.cpu_seconds) if args.cpu_seconds > 0 else None
    cpu_step = cpu_baseline_step(WORKLOADS["small"], args.cpu_seconds) if args.cpu_seconds > 0 else None

    # ---- the other workloads of the measurement plan, in the same run: the
    # fused dgrad at the small and Llama-like shapes (MFMA roofline) and the
    # decode-shaped forward (HBM roofline) ----
    other = None
    if args.other_workloads:
        del preact, h_fwd, y, gp, h_bwd, dout, dx, dW1, dWd, wsf, wsb
        torch.cuda.empty_cache()
        other = {"dgrad_fused": {n: b1_at(WORKLOADS[n], max(args.steps, 10)) for n in ("small", "llama")}}
        torch.cuda.empty_cache()
        other["decode_forward"] = decode_measure(WORKLOADS["decode"], max(args.steps, 20), args.warmup)

    out = {
        "metric": "fused dout-GEMM+SwiGLU-bwd TFLOP/s (% MFMA peak); MLP fwd+bwd ms",
        "value": round(b1_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} SwiGLU MLP fwd+bwd", "M": M, "D": D, "I": I, "Dout": Dout,
                   "global_batch": M, "parallelism": "single GPU"},
        "pct_of_mfma_peak": round(100 * b1_tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "full_ms_median": round(float(np.median(step_ms)), 4),
        "single_step_calls_ms": round(single_step_ms, 4),
        "step_tflops": round(total_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "kernels": {n: {"ms": round(ms[n], 4), "tflops": round(flops[n] / (ms[n] * 1e-3) / 1e12, 2)} for n in names},
        "ab_fused_vs_unfused": ab,
        "save_h_variant": save_h_ab,
        "residual_block": residual,
        "library_gemm_context": library_gemm,
        "block_drop_h_vs_save_h": block,
        "stack": stack,
        "roofline": roofline,
        "other_workloads": other,
        "cpu_baseline": cpu,
        "cpu_baseline_step": cpu_step,
        "kernel_source_digest": source_digest(),
    }
    print(json.dumps(out), flush=True)


def block_compare(sw, x, W1, Wd, dy, rounds, stream):
    """One MLP block through the autograd functions, drop-h
    (SwiGLUMLPFunction: saves {x, W1, W_down, preact}) against save-h
    (SwiGLUMLPSaveHFunction: also keeps h), as the drop-h report compares
    them: fwd, bwd and full (fwd + bwd of one sample) ms in `rounds`
    randomly interleaved rounds with medians and paired deltas, and the
    allocated MiB above the inputs after the forward and at the peak of
    fwd + bwd, each taken once from an emptied allocator cache."""
    import torch
    xs, W1r, Wdr = (t.clone().requires_grad_(True) for t in (x, W1, Wd))
    fns = {"drop_h": sw.swiglu_mlp, "save_h": sw.swiglu_mlp_save_h}
    mem = {}
    for name, fn in fns.items():
        for t in (xs, W1r, Wdr):
            t.grad = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        out = fn(xs, W1r, Wdr)
        torch.cuda.synchronize()
        after = torch.cuda.memory_allocated() - base
        out.backward(dy)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        del out
        mem[name] = (after, peak)

    def runner(fn):
        def run(ev):
            for t in (xs, W1r, Wdr):
                t.grad = None
            ev[0].record(stream)
            out = fn(xs, W1r, Wdr)
            ev[1].record(stream)
            out.backward(dy)
            ev[2].record(stream)
            return 2
        return run

    variants = {n: runner(f) for n, f in fns.items()}
    for v in variants.values():
        v([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    torch.cuda.synchronize()
    smp = paired_samples(variants, rounds, stream, seed=4321)
    res = {"pairs": rounds}
    for part, idx in (("fwd", 0), ("bwd", 1), ("full", None)):
        a = [v[idx] if idx is not None else v[0] + v[1] for v in smp["drop_h"]]
        b = [v[idx] if idx is not None else v[0] + v[1] for v in smp["save_h"]]
        res[part] = paired_summary(a, b, "drop_h", "save_h")
    for name, (after, peak) in mem.items():
        res[f"{name}_after_fwd_MiB"] = round(after / 2**20, 3)
        res[f"{name}_peak_MiB"] = round(peak / 2**20, 3)
    res["after_fwd_saving_MiB"] = round((mem["save_h"][0] - mem["drop_h"][0]) / 2**20, 3)
    del xs, W1r, Wdr
    return res


def _threads():
    """Threads the oracle's numpy runs on: its BLAS pool (the matrix
    products are nearly all of the oracle's time; its elementwise work is
    single-threaded numpy)."""
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def _host():
    return {"host_cpu_count": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "blas_threads": _threads()}


def cpu_baseline(w, xb, W1b, Wdb, dyb, budget_s):
    """The fp64 oracle of the fused dgrad step (dout = dy.W_down^T and the
    SwiGLU backward) on a sample of token rows, scaled to TFLOP/s."""
    import oracle
    from workload import bf16_bits_to_f64
    Wd = bf16_bits_to_f64(Wdb)
    W1 = bf16_bits_to_f64(W1b)

    def run(rows):
        r = np.arange(rows)
        pre = bf16_bits_to_f64(xb[r]) @ W1            # setup: the saved preact of those rows
        dyr = bf16_bits_to_f64(dyb[r])
        t = time.perf_counter()
        dout = dyr @ Wd.T
        oracle.swiglu_bwd_elementwise(pre, dout)
        return time.perf_counter() - t

    rows = min(64, w.M)
    dt = run(rows)
    rows = int(min(w.M, max(rows, rows * budget_s / max(dt, 1e-3))))
    dt = run(rows)
    passes = 1
    if rows == w.M:
        # the whole workload fits the budget: repeat it until the budget is spent
        while dt < budget_s:
            dt += run(rows)
            passes += 1
    fl = 2 * rows * w.Dout * w.I * passes
    what = (f"all {rows} token rows, {passes} passes" if rows == w.M else
            f"the first {rows} of {w.M} token rows")
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "sample": f"fused dgrad step (dout GEMM + SwiGLU backward) of {what}, fp64 numpy, {dt:.1f}s",
            **_host()}


def cpu_baseline_step(w, budget_s):
    """The fp64 oracle of the whole step (forward and backward) at a workload
    the oracle finishes in seconds, repeated until the time budget is spent;
    TFLOP/s of the step's GEMMs (6 M D I + 6 M I Dout per step)."""
    import oracle
    from workload import bf16_bits_to_f64, make_inputs
    x, W1, Wd, dy = (bf16_bits_to_f64(a) for a in make_inputs(w))
    t = time.perf_counter()
    passes = 0
    while True:
        oracle.backward(x, W1, Wd, dy)
        passes += 1
        dt = time.perf_counter() - t
        if dt >= budget_s / 2 or passes >= 50:
            break
    fl = (6 * w.M * w.D * w.I + 6 * w.M * w.I * w.Dout) * passes
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "ms_per_step": round(dt * 1e3 / passes, 1),
            "sample": f"whole fwd+bwd step of the {w.name} workload ({w.M}x{w.D}x{w.I}x{w.Dout}), "
                      f"{passes} passes, fp64 numpy, {dt:.1f}s", **_host()}


def copy_calibration():
    """A plain elementwise copy (bf16 -> fp16 conversion, one read and one
    write of 2 B per element) over 512 Mi elements: 1 GiB read, 1 GiB
    written.  Profiling its FETCH_SIZE / WRITE_SIZE gives the factor that
    turns those counters into bytes on this machine."""
    import torch
    n = 512 * 1024 * 1024
    src = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty(n, dtype=torch.float16, device="cuda")
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"elements": n, "read_bytes": 2 * n, "write_bytes": 2 * n}}), flush=True)


def decode_measure(w, steps, warmup):
    """Decode-shaped forward (GEMM-1 + SwiGLU epilogue, down GEMM): HBM GB/s
    of algorithmic bytes per launch of swiglu_mlp_fwd, mean HIP-event time.
    Weights are rotated over three copies (1.06 GB at 16 x 4096 x 14336,
    more than the 256 MB last-level cache), so every launch streams them from
    HBM."""
    import torch
    import bwd_gemm_epilogue_amd as sw
    from workload import make_inputs
    M, D, I, Dout = w.M, w.D, w.I, w.Dout
    dev = torch.device("cuda:0")

    def to_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    xb, W1b, Wdb, _ = make_inputs(w)
    x = to_dev(xb)
    copies = 3
    W1s = [to_dev(W1b) for _ in range(copies)]
    Wds = [to_dev(Wdb) for _ in range(copies)]
    preact = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, Dout), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(sw.swiglu_mlp_fwd_workspace(M, D, I, Dout), dtype=torch.uint8, device=dev)
    for k in range(warmup):
        sw.swiglu_mlp_fwd(x, W1s[k % copies], Wds[k % copies], preact, y, ws)
    rot = [0]

    def one_fwd():
        sw.swiglu_mlp_fwd(x, W1s[rot[0] % copies], Wds[rot[0] % copies], preact, y, ws)
        rot[0] += 1
    warm_up(one_fwd)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for k in range(steps):
        evs[k].record(stream)
        sw.swiglu_mlp_fwd(x, W1s[k % copies], Wds[k % copies], preact, y, ws)
    evs[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([evs[k].elapsed_time(evs[k + 1]) for k in range(steps)]))
    nbytes = forward_bytes(M, D, I, Dout)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"fwd_us": round(ms * 1e3, 2), "wall_ms_per_step": round(wall * 1e3 / steps, 4),
            "gbs": round(gbs, 1), "config": {"workload": f"{w.name} SwiGLU MLP forward", "M": M, "D": D, "I": I,
                                            "Dout": Dout, "weight_copies_rotated": copies},
            "roofline": {"kernel": "swiglu_mlp_fwd", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(f"forward_{w.name}"), "algorithmic_bytes_per_launch": nbytes}}


def bench_decode(args, w):
    d = decode_measure(w, args.steps, args.warmup)
    out = {
        "metric": "decode-shaped SwiGLU MLP forward HBM GB/s", "value": d["gbs"], "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": d["wall_ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": d["config"], "roofline": d["roofline"], "fwd_us": d["fwd_us"],
    }
    print(json.dumps(out), flush=True)


def warm_up(fn, min_ms=300.0):
    """Run fn until at least min_ms of wall time has passed (checked every 8
    calls, synchronised).  The first tens of milliseconds of launches after
    fresh buffers run slow (the Llama-like fused dgrad: 0.73 ms per launch in
    the first 20, then 0.62 ms), so a fixed small count of warm-up launches
    would leak that into the timed ones."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return n


def b1_at(w, iters, warmup=3):
    """The fused dgrad kernel at another workload's shape: preact from the
    workload's own x and W1 (GEMM-1 on the GPU), then `iters` launches timed
    with HIP events; mean ms, TFLOP/s and the fraction of the bf16 peak."""
    import torch
    import bwd_gemm_epilogue_amd as sw
    from workload import make_inputs
    dev = torch.device("cuda:0")

    def to_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    xb, W1b, Wdb, dyb = make_inputs(w)
    x, W1, Wd, dy = (to_dev(a) for a in (xb, W1b, Wdb, dyb))
    preact, _ = sw.swiglu_fwd_gemm1(x, W1)
    del x, W1
    gp = torch.empty((w.M, 2 * w.I), dtype=torch.bfloat16, device=dev)
    h = torch.empty((w.M, w.I), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        sw.swiglu_bwd_dgrad_fused(dy, Wd, preact, gp, h)
    warm_up(lambda: sw.swiglu_bwd_dgrad_fused(dy, Wd, preact, gp, h))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    for k in range(iters):
        ev[k].record(stream)
        sw.swiglu_bwd_dgrad_fused(dy, Wd, preact, gp, h)
    ev[-1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([ev[k].elapsed_time(ev[k + 1]) for k in range(iters)]))
    tf = 2 * w.M * w.Dout * w.I / (ms * 1e-3) / 1e12
    return {"M": w.M, "D": w.D, "I": w.I, "Dout": w.Dout, "ms": round(ms, 4), "tflops": round(tf, 2),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "algorithmic_bytes_per_launch": fused_dgrad_bytes(w.M, w.I, w.Dout)}


def bench_moe(args, w):
    """Mixture-of-experts block (expert MLPs over expert-packed rows): the
    grouped fused dgrad's TFLOP/s (one launch for all experts), the whole
    block's forward and backward, and paired A/B of the grouped launches
    against the same work as one dense launch per expert."""
    import torch
    import bwd_gemm_epilogue_amd as sw
    from workload import make_moe_inputs
    dev = torch.device("cuda:0")

    def to_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    xb, W1b, Wdb, dyb, offb = make_moe_inputs(w, weight_sets=2)
    x, W1, Wd, dy = (to_dev(a) for a in (xb, W1b, Wdb, dyb))
    off = torch.from_numpy(offb).to(dev)
    M, D, I, Dout, E = int(offb[-1]), w.D, w.I, w.Dout, w.experts
    counts = np.diff(offb)
    print(f"[bench] moe inputs {M}x{D}x{I}x{Dout}, {E} experts (rows {counts.min()}..{counts.max()}) "
          f"ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    bf = torch.bfloat16
    preact = torch.empty((M, 2 * I), dtype=bf, device=dev)
    y = torch.empty((M, Dout), dtype=bf, device=dev)
    dx = torch.empty((M, D), dtype=bf, device=dev)
    dW1 = torch.empty((E, D, 2 * I), dtype=bf, device=dev)
    dWd = torch.empty((E, I, Dout), dtype=bf, device=dev)
    gp = torch.empty((M, 2 * I), dtype=bf, device=dev)
    h = torch.empty((M, I), dtype=bf, device=dev)
    wsf = torch.empty(max(1, sw.swiglu_moe_fwd_workspace(M, D, I, Dout, E)), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(1, sw.swiglu_moe_bwd_workspace(M, D, I, Dout, E)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sl = [(int(offb[e]), int(offb[e + 1])) for e in range(E)]

    def fwd():
        sw.swiglu_moe_fwd(x, W1, Wd, off, preact, y, wsf)

    def bwd():
        sw.swiglu_moe_bwd(x, W1, Wd, off, preact, dy, dx, dW1, dWd, wsb)

    def b1_grouped():
        sw.swiglu_moe_bwd_dgrad_fused(dy, Wd, off, preact, gp, h)

    def b1_per_expert():
        for e, (a, b) in enumerate(sl):
            sw.swiglu_bwd_dgrad_fused(dy[a:b], Wd[e], preact[a:b], gp[a:b], h[a:b])

    def step_per_expert():
        for e, (a, b) in enumerate(sl):
            sw.swiglu_mlp_fwd(x[a:b], W1[e], Wd[e], preact[a:b], y[a:b])
        for e, (a, b) in enumerate(sl):
            sw.swiglu_mlp_bwd(x[a:b], W1[e], Wd[e], preact[a:b], dy[a:b], dx[a:b], dW1[e], dWd[e])

    for _ in range(args.warmup):
        fwd(); bwd(); b1_grouped()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t1 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record(stream)
        fwd()
        ev[k][1].record(stream)
        bwd()
        ev[k][2].record(stream)
        b1_grouped()
        ev[k][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    b1_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    b1_flops = 2 * M * Dout * I
    b1_tflops = b1_flops / (b1_ms * 1e-3) / 1e12
    step_flops = 3 * (4 * M * D * I + 2 * M * I * Dout)  # forward 4MDI + 2MIDout, backward twice that

    # paired A/B: grouped launches against one dense launch per expert
    def pairs(fa, fb, n):
        ta, tb = [], []
        e3 = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for _ in range(n):
            e3[0].record(stream); fa(); e3[1].record(stream); fb(); e3[2].record(stream)
            torch.cuda.synchronize()
            ta.append(e3[0].elapsed_time(e3[1])); tb.append(e3[1].elapsed_time(e3[2]))
        return float(np.median(ta)), float(np.median(tb))

    g_b1, d_b1 = pairs(b1_grouped, b1_per_expert, 10)
    g_st, d_st = pairs(lambda: (fwd(), bwd()), step_per_expert, 6)
    cpu = cpu_baseline_moe(w, xb, W1b, Wdb, dyb, offb, args.cpu_seconds) if args.cpu_seconds > 0 else None
    out = {
        "metric": "grouped fused dout-GEMM+SwiGLU-bwd TFLOP/s over all experts; MoE block fwd+bwd ms",
        "value": round(b1_tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name} mixture-of-experts SwiGLU block fwd+bwd", "routed_rows": M, "D": D,
                   "I": I, "Dout": Dout, "experts": E, "top_k": w.top_k, "tokens": w.tokens,
                   "rows_per_expert_min_max": [int(counts.min()), int(counts.max())],
                   "distinct_expert_weight_sets": 2},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "step_tflops": round(step_flops / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2),
        "ab_grouped_vs_per_expert": {
            "dgrad_fused_grouped_ms": round(g_b1, 4), "dgrad_fused_per_expert_ms": round(d_b1, 4),
            "step_grouped_ms": round(g_st, 4), "step_per_expert_ms": round(d_st, 4),
            "launches_grouped": 6, "launches_per_expert": 6 * E},
        "roofline": {"kernel": "grouped bwd_dgrad_fused", "bound": "mfma", "achieved": round(b1_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(b1_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(f"dgrad_fused_{w.name}"),
                     "algorithmic_flops_per_launch": b1_flops,
                     "algorithmic_bytes_per_launch": fused_dgrad_bytes(M, I, Dout, experts=E)},
        "cpu_baseline": cpu,
        "kernel_source_digest": source_digest(),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_moe(w, xb, W1b, Wdb, dyb, offb, budget_s):
    """The fp64 oracle of the fused dgrad step, expert by expert, over the
    first experts' rows until the time budget is spent, scaled to TFLOP/s."""
    import oracle
    from workload import bf16_bits_to_f64
    t_total, rows, experts = 0.0, 0, 0
    for e in range(w.experts):
        a, b = int(offb[e]), int(offb[e + 1])
        if a == b:
            continue
        pre = bf16_bits_to_f64(xb[a:b]) @ bf16_bits_to_f64(W1b[e])     # setup: the saved preact
        dyr, Wd = bf16_bits_to_f64(dyb[a:b]), bf16_bits_to_f64(Wdb[e])
        t = time.perf_counter()
        oracle.swiglu_bwd_elementwise(pre, dyr @ Wd.T)
        t_total += time.perf_counter() - t
        rows += b - a
        experts += 1
        if t_total > budget_s:
            break
    fl = 2 * rows * w.Dout * w.I
    return {"value": round(fl / t_total / 1e12, 5), "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "sample": f"fused dgrad step of the first {experts} experts ({rows} of {int(offb[-1])} routed rows), "
                      f"fp64 numpy, {t_total:.1f}s", **_host()}


if __name__ == "__main__":
    main()
