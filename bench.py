#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

One step = one fa_fwd call (the whole forward: Q load, K/V staging, QK^T, masks, online
softmax, PV, epilogue) over one batch of synthetic inputs already resident in HBM.

Headline workload: the pages' benchmark shape, B=4 H=4 Nq=Nk=4096 d=64 fp32 non-causal
(page "Add Fused Multi-Head Attention example"). The same JSON line carries every other
workload (the bf16 d=128 causal/non-causal pair, the long causal bf16 run and the ragged
fp16 run), each with its TFLOP/s, fraction of the dtype's dense MFMA peak and kernel time,
a short-sequence HBM sweep (GB/s) and the fp64 CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--quick]
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

# MI355X published dense peaks (no sparsity), TFLOP/s, and HBM3E bandwidth, GB/s.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# the forward kernels' source: the kernel file and the device headers it includes
KERNEL_SRC = [os.path.join(ROOT, "exact_attention_58_amd", "csrc", f)
              for f in ("fa_fwd_kernels.hip", "fa_device.h", "fa_internal.h")]

# HBM traffic per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per
# dispatch, scaled by the factor a plain copy kernel of known size reads on the same
# counters), keyed by workload, valid only for the kernel source whose sha256 prefix is
# recorded. Filled in from the committed profiles; a source change makes it stale (null).
TRAFFIC = {
    # profiles/fwd32_pages_f32.txt: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0
    "pages_f32": {"bytes": 67564207, "kernel_sha": "5f7e9dbfce818502"},
    # profiles/fwd32_tiny_causal_f32.txt: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0
    "tiny_causal_f32": {"bytes": 882616, "kernel_sha": "5f7e9dbfce818502"},
    # profiles/fwd16_pp_d128_bf16.txt: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0
    "d128_bf16": {"bytes": 269676802, "kernel_sha": "5f7e9dbfce818502"},
    # profiles/fwd16_pp_d128_bf16_causal.txt: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0
    "d128_bf16_causal": {"bytes": 354087341, "kernel_sha": "5f7e9dbfce818502"},
    # profiles/fwd16_pp_long_causal_bf16.txt: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0
    "long_causal_bf16": {"bytes": 78337608, "kernel_sha": "5f7e9dbfce818502"},
    # profiles/fwd16_split_ragged_f16.txt: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0
    "ragged_f16": {"bytes": 37128163, "kernel_sha": "5f7e9dbfce818502"},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Untimed warm-up floor. The host prepares each workload's inputs while the GPU idles, and
# an idle MI355X needs tens of milliseconds of work before its clock is back up: after 5
# warm-up launches the first timed runs measured 7-15% slow (d128 bf16 causal 331 vs
# 287 us per launch). Every timed section therefore runs its own calls untimed for the
# requested warm-up steps and at least WARM_MS of GPU time.
WARM_MS = 100.0


def warm_up(torch, call, steps, stream) -> int:
    """Runs call() untimed: `steps` times, and on until WARM_MS of GPU time has passed
    (estimated from the first call). Returns the number of calls made."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    call()
    e1.record(stream)
    torch.cuda.synchronize()
    per_ms = max(e0.elapsed_time(e1), 1e-3)
    n = max(steps - 1, int(WARM_MS / per_ms))
    for _ in range(n):
        call()
    torch.cuda.synchronize()
    return n + 1


def kernel_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def launch_stats(torch, call, n, stream):
    """n more launches, each between its own pair of HIP events on the launch stream; returns
    the median, mean and 10th/90th percentiles of the launch durations (ms)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    pick = lambda f: t[min(n - 1, int(round(f * (n - 1))))]
    return {"launches": n, "median_ms": round(pick(0.5), 5), "mean_ms": round(sum(t) / n, 5),
            "p10_ms": round(pick(0.1), 5), "p90_ms": round(pick(0.9), 5)}


def per_launch_count(w, steps) -> int:
    """Launches timed one by one: at least 30, and at least 200 for workloads under a GFLOP."""
    return max(steps, 200 if w.flops < 1e9 else 30)


def time_workload(fa, torch, w, steps, warmup, inputs=None, keep_outputs=False):
    """Runs `steps` back-to-back fa_fwd calls on torch's current stream, after warm_up, then
    per_launch_count() more calls timed one by one.

    Returns (wall ms per step, average launch duration in ms from HIP events recorded on the
    launch stream around the timed region, warm-up calls made, per-launch statistics, and the
    outputs (o, lse) on the host when keep_outputs)."""
    from exact_attention_58_amd.workloads import make_inputs
    dev = torch.device("cuda:0")
    if inputs is None:
        q, k, v = (t.to(dev) for t in make_inputs(w))
    else:
        q, k, v = inputs
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    call = lambda: fa.fa_fwd(q, k, v, o, lse, w.softmax_scale, w.causal, stream)
    n_warm = warm_up(torch, call, warmup, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev_ms = e0.elapsed_time(e1) / steps
    stats = launch_stats(torch, call, per_launch_count(w, steps), stream)
    outs = (o.cpu(), lse.cpu()) if keep_outputs else None
    del o, lse
    return wall_ms, ev_ms, n_warm, stats, outs


def time_backward(fa, torch, w, steps, warmup):
    """Times fa_bwd (row terms, dK/dV, dQ kernels) on the workload's inputs and a seeded
    upstream gradient, after one forward for O and L; returns ms per call (HIP events on
    the launch stream) and the number of untimed warm-up calls before the timed ones."""
    from exact_attention_58_amd.workloads import make_inputs, make_random
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_inputs(w))
    do = make_random(tuple(q.shape), w.dtype, w.seed + 100).to(dev)
    o, lse = fa.attention(q, k, v, scale=w.softmax_scale, causal=w.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    n_warm = warm_up(torch, lambda: fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, w.softmax_scale,
                                              w.causal, stream), warmup, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, delta, w.softmax_scale, w.causal, stream)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    del q, k, v, do, o, lse, dq, dk, dv, delta
    return ms, n_warm


def time_varlen(fa, torch, causal, steps, warmup):
    """Packed batch of 16 bf16 sequences (lengths seeded uniform in [512, 4096], same for
    queries and keys), H=16, d=128, through fa_fwd_varlen. FLOP: the sum over sequences of
    4*H*n*n*d, halved for causal. Returns (description, ms per call, TFLOP/s)."""
    from exact_attention_58_amd.workloads import make_lengths, make_random, offsets
    dev = torch.device("cuda:0")
    H, d = 16, 128
    lens = make_lengths(16, 512, 4096, seed=77)
    T = sum(lens)
    q, k, v = (make_random((H, T, d), "bf16", 700 + i).to(dev) for i in range(3))
    cu = offsets(lens).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    scale = 1.0 / d ** 0.5
    stream = torch.cuda.current_stream(dev)
    call = lambda: fa.fa_fwd_varlen(q, k, v, o, lse, cu, cu, max(lens), max(lens), scale, causal, stream)
    warm_up(torch, call, warmup, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    flops = sum(4.0 * H * n * n * d for n in lens) / (2 if causal else 1)
    desc = f"16 sequences, lengths {min(lens)}..{max(lens)} (total {T}), H={H} d={d} bf16"
    del q, k, v, o, lse
    return desc, ms, flops / (ms * 1e-3) / 1e12


def tune_table(fa, torch, steps):
    """fa_tune_fwd on a few problems off the headline set: the built-in tile choice and the
    tuned one, each timed over `steps` launches with HIP events in two alternating rounds,
    keeping each one's faster round (the record is cleared after)."""
    from exact_attention_58_amd.workloads import Workload, make_inputs
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    probs = [Workload("tune_d128_N1024", 16, 16, 1024, 1024, 128, "bf16", False, seed=31),
             Workload("tune_d64_N2048_causal", 2, 8, 2048, 2048, 64, "bf16", True, seed=32),
             Workload("tune_d96_ragged", 2, 12, 1000, 3001, 96, "f16", False, seed=33, std=0.5),
             Workload("tune_d128_N8192_causal", 1, 16, 8192, 8192, 128, "bf16", True, seed=34)]
    out = []
    stream = torch.cuda.current_stream(dev)
    for w in probs:
        q, k, v = (t.to(dev) for t in make_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        rule = fa.fa_select_config(w.dtype, w.B, w.H, w.Nq, w.Nk, w.d, w.causal, num_cus=cus)
        rule = {x: rule[x] for x in ("Br", "Bc", "waves")}
        best = fa.fa_tune_fwd(q, k, v, o, lse, w.softmax_scale, w.causal, reps=max(3, steps // 5))
        times = {}
        for _ in range(2):
            for name, cfg in (("built_in", rule), ("tuned", best)):
                warm_up(torch, lambda: fa.fa_fwd_config(q, k, v, o, lse, w.softmax_scale, w.causal, cfg, stream),
                        2, stream)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(steps):
                    fa.fa_fwd_config(q, k, v, o, lse, w.softmax_scale, w.causal, cfg, stream)
                e1.record(stream)
                torch.cuda.synchronize(dev)
                times[name] = min(times.get(name, float("inf")), e0.elapsed_time(e1) / steps)
        out.append({"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                    "dtype": w.dtype, "causal": w.causal, "built_in": rule, "tuned": best,
                    "built_in_ms": round(times["built_in"], 4), "tuned_ms": round(times["tuned"], 4),
                    "tuned_tflops": round(w.flops / (times["tuned"] * 1e-3) / 1e12, 1)})
        del q, k, v, o, lse
    fa.fa_tune_clear()
    return out


def roofline_for(w, ev_ms, sha):
    achieved = w.flops / (ev_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    tr = TRAFFIC.get(w.name)
    traffic = tr["bytes"] if tr and tr.get("kernel_sha") == sha else None
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic}


def hbm_sweep(fa, torch, steps):
    """Short sequences (HBM-bound): bf16 d=128 non-causal, N in {128, 256, 512}, three
    rotating input sets larger than the 256 MB Infinity Cache; GB/s = algorithmic bytes / t."""
    from exact_attention_58_amd.workloads import Workload, make_random
    dev = torch.device("cuda:0")
    out = []
    for N, B, H in ((128, 64, 128), (256, 32, 128), (512, 16, 128)):
        w = Workload(f"short_N{N}", B, H, N, N, 128, "bf16", False, seed=100 + N)
        sets = []
        for s in range(3):
            q = make_random((B, H, N, 128), "bf16", 1000 * N + 3 * s).to(dev)
            k = make_random((B, H, N, 128), "bf16", 1000 * N + 3 * s + 1).to(dev)
            v = make_random((B, H, N, 128), "bf16", 1000 * N + 3 * s + 2).to(dev)
            o = torch.empty_like(q)
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
            sets.append((q, k, v, o, lse))
        stream = torch.cuda.current_stream(dev)
        rot = [0]

        def call():
            fa.fa_fwd(*sets[rot[0] % 3], w.softmax_scale, False, stream)
            rot[0] += 1
        warm_up(torch, call, 3, stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        n = max(3, steps)
        e0.record(stream)
        for i in range(n):
            fa.fa_fwd(*sets[i % 3], w.softmax_scale, False, stream)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1) / n
        gbs = w.io_bytes / (ms * 1e-3) / 1e9
        out.append({"N": N, "B": B, "H": H, "d": 128, "ms": round(ms, 4), "GB_per_s": round(gbs, 1),
                    "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                    "tflops": round(w.flops / (ms * 1e-3) / 1e12, 1)})
        del sets
    # attainable yardstick: a 2 GiB device-to-device copy
    a = torch.empty(2 ** 30, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    warm_up(torch, lambda: b.copy_(a), 1, torch.cuda.current_stream(dev))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / 5
    copy_gbs = 2 * a.numel() * 2 / (ms * 1e-3) / 1e9
    del a, b
    return out, round(copy_gbs, 1)


def oracle_leg(w, outs):
    """CPU-baseline leg: the fp64 oracle as it stands, on the host cores, over every row of the
    workload (outside every timed region). Reports its wall time and rate, and the max-abs
    error of the GPU's O and L (the launch the benchmark timed) with where it occurs."""
    import numpy as np

    import oracle
    from exact_attention_58_amd.workloads import make_inputs
    q, k, v = make_inputs(w)
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.attention_fwd(q.double(), k.double(), v.double(), w.softmax_scale, w.causal,
                                        threads=threads)
    dt = time.perf_counter() - t0
    rep = {"rows": w.B * w.H * w.Nq, "wall_s": round(dt, 2), "cores": threads,
           "tflops": round(w.flops / dt / 1e12, 5)}
    if outs is not None:
        o, lse = outs
        do = np.abs(o.double().numpy() - o_ref)
        dl = np.abs(lse.double().numpy() - l_ref)
        io, il = np.unravel_index(np.argmax(do), do.shape), np.unravel_index(np.argmax(dl), dl.shape)
        tol_o = 1e-4 if w.dtype == "f32" else 2e-2
        rep.update({"max_abs_err_O": float(do[io]), "at_O_bhic": [int(x) for x in io],
                    "ref_O_there": round(float(o_ref[io]), 4),
                    "max_abs_err_L": float(dl[il]), "at_L_bhi": [int(x) for x in il],
                    "tol_O": tol_o, "tol_L": 1e-3,
                    "within_tol": bool(do[io] <= tol_o and dl[il] <= 1e-3)})
    return rep


def cpu_baseline(w, rep):
    """The headline's CPU baseline line from its oracle leg (all rows of the workload)."""
    return {"value": rep["tflops"], "unit": "TFLOP/s", "cores": rep["cores"], "kind": "oracle",
            "sample": f"all {rep['rows']} query rows of {w.name} (the whole workload), "
                      f"{rep['wall_s']:.1f} s wall on {rep['cores']} threads, fp64"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="pages_f32")
    ap.add_argument("--shape", default=None, metavar="B,H,Nq,Nk,d,dtype,causal",
                    help="time this shape instead of a named workload (seeded N(0,1) inputs; implies --quick), "
                         "e.g. 4,16,4096,4096,32,bf16,0")
    ap.add_argument("--quick", action="store_true", help="headline only: no other workloads, sweep or CPU baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--backward", action="store_true",
                    help="only time fa_bwd on the workload (warm-up calls, then the timed calls; "
                         "prints one JSON line): the command the backward profiles run")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the forward is measured on a single MI355X "
              "(multi-GPU sharding is not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_58_amd as fa
    from exact_attention_58_amd.workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy * 2 ** 20
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return
    fa.ensure_built()
    fa.lib()
    sha = kernel_sha()
    props = torch.cuda.get_device_properties(0)

    w = WORKLOADS[args.workload]
    if args.shape:
        from exact_attention_58_amd.workloads import Workload
        B_, H_, Nq_, Nk_, d_, dt_, c_ = args.shape.split(",")
        w = Workload(f"shape_{B_}x{H_}x{Nq_}x{Nk_}x{d_}_{dt_}{'_causal' if int(c_) else ''}", int(B_), int(H_),
                     int(Nq_), int(Nk_), int(d_), dt_, bool(int(c_)), seed=11)
        args.quick = True
    if args.backward:
        ms, n_warm = time_backward(fa, torch, w, args.steps, args.warmup)
        tf = 2.5 * w.flops / (ms * 1e-3) / 1e12
        log(f"  {w.name} backward: calls {n_warm}..{n_warm + args.steps - 1} of fa_bwd are the timed region "
            f"({n_warm} warm-up calls before them), {ms:.4f} ms per call, {tf:.1f} TFLOP/s")
        print(json.dumps({"metric": "attention bwd TFLOP/s (FLOP = 2.5 x the forward's)", "workload": w.name,
                          "value": round(tf, 2), "unit": "TFLOP/s", "ms_per_call": round(ms, 4),
                          "steps": args.steps, "warmup": args.warmup, "dtype": w.dtype,
                          "pct_of_peak": round(100 * tf / PEAK_TFLOPS[w.dtype], 2)}), flush=True)
        return
    with_oracle = not args.quick and not args.no_cpu
    log(f"headline {w.name}: {args.warmup} warmup + {args.steps} timed steps")
    torch.cuda.synchronize()
    wall_ms, ev_ms, n_warm, stats, outs = time_workload(fa, torch, w, args.steps, args.warmup,
                                                        keep_outputs=with_oracle)
    tflops = w.flops / (wall_ms * 1e-3) / 1e12
    log(f"  {w.name}: dispatches {n_warm}..{n_warm + args.steps - 1} of its kernel are the timed region; "
        f"{wall_ms:.3f} ms/step wall, {ev_ms:.4f} ms/launch (events), {tflops:.1f} TFLOP/s; "
        f"one by one: median {stats['median_ms']} ms over {stats['launches']}")
    outputs = {w.name: outs}

    also = []
    sweep, copy_gbs, tuned = None, None, None
    if not args.quick:
        for name, ow in WORKLOADS.items():
            if name == w.name:
                continue
            steps = max(5, min(args.steps, 200 if ow.flops < 1e9 else args.steps))
            wm, em, _, st, oo = time_workload(fa, torch, ow, steps, args.warmup, keep_outputs=with_oracle)
            outputs[name] = oo
            r = roofline_for(ow, em, sha)
            also.append({"workload": name, "B": ow.B, "H": ow.H, "Nq": ow.Nq, "Nk": ow.Nk, "d": ow.d,
                         "dtype": ow.dtype, "causal": ow.causal, "steps": steps, "ms_per_step": round(wm, 4),
                         "tflops": round(ow.flops / (wm * 1e-3) / 1e12, 2), "kernel_ms_mean": round(em, 5),
                         "per_launch": st,
                         "tflops_at_median": round(ow.flops / (st["median_ms"] * 1e-3) / 1e12, 2),
                         "roofline": r})
            log(f"  {name}: {wm:.4f} ms/step, {r['achieved']} TFLOP/s kernel, {100 * r['frac']:.1f}% of "
                f"{ow.dtype} peak; median {st['median_ms']} ms over {st['launches']} launches")
        # backward (FLOP convention: 2.5 x the forward's, i.e. five products of the forward's
        # size; this implementation recomputes S and dP in both tile kernels)
        for name in ("d128_bf16", "d128_bf16_causal", "long_causal_bf16", "pages_f32"):
            ow = WORKLOADS[name]
            ms, _ = time_backward(fa, torch, ow, max(5, min(args.steps, 20)), 2)
            tf = 2.5 * ow.flops / (ms * 1e-3) / 1e12
            peak = PEAK_TFLOPS[ow.dtype]
            also.append({"workload": f"{name} backward", "B": ow.B, "H": ow.H, "Nq": ow.Nq, "Nk": ow.Nk,
                         "d": ow.d, "dtype": ow.dtype, "causal": ow.causal, "ms_per_step": round(ms, 4),
                         "tflops": round(tf, 2),
                         "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak,
                                      "unit": "TFLOP/s", "frac": round(tf / peak, 4), "traffic": None}})
            log(f"  {name} backward: {ms:.3f} ms, {tf:.1f} TFLOP/s ({100 * tf / peak:.1f}% of {ow.dtype} peak)")
        # packed sequences of different lengths in one launch
        for causal in (False, True):
            desc, ms, tf = time_varlen(fa, torch, causal, max(5, min(args.steps, 20)), 2)
            peak = PEAK_TFLOPS["bf16"]
            name = f"varlen_bf16{'_causal' if causal else ''}"
            also.append({"workload": name, "shape": desc, "dtype": "bf16", "causal": causal,
                         "ms_per_step": round(ms, 4), "tflops": round(tf, 2),
                         "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak,
                                      "unit": "TFLOP/s", "frac": round(tf / peak, 4), "traffic": None}})
            log(f"  {name} ({desc}): {ms:.3f} ms, {tf:.1f} TFLOP/s ({100 * tf / peak:.1f}% of bf16 peak)")
        tuned = tune_table(fa, torch, max(5, min(args.steps, 20)))
        for t in tuned:
            log(f"  {t['workload']}: built-in {t['built_in']} {t['built_in_ms']} ms, tuned {t['tuned']} "
                f"{t['tuned_ms']} ms ({t['tuned_tflops']} TFLOP/s)")
        sweep, copy_gbs = hbm_sweep(fa, torch, args.steps)
        for s in sweep:
            log(f"  short N={s['N']}: {s['GB_per_s']} GB/s ({100 * s['hbm_frac']:.1f}% of 8 TB/s)")
        log(f"  2 GiB device copy: {copy_gbs} GB/s")

    cpu, head_oracle = None, None
    if with_oracle:
        # CPU-baseline leg: the oracle over every row of every workload, outside the timed
        # regions; its time is the baseline, its comparison the error report per workload
        for name, oo in outputs.items():
            rep = oracle_leg(WORKLOADS[name], oo)
            log(f"  oracle {name}: {rep}")
            if name == w.name:
                cpu = cpu_baseline(w, rep)
                head_oracle = rep
            else:
                next(a for a in also if a["workload"] == name)["oracle"] = rep
        del outputs

    line = {
        "metric": "attention fwd TFLOP/s and % of MI355X dtype peak (B4 H4 N4096 d64/d128)",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "warmup_note": f"untimed: the requested warm-up steps, extended to at least {WARM_MS:.0f} ms of GPU work (clock settle)",
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) q, k, v (torch CPU generator, rounded to the dtype), resident in HBM",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d} {w.dtype} "
                               f"{'causal' if w.causal else 'non-causal'} scale={w.softmax_scale:.6g}",
                   "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal,
                   "global_batch": w.B, "seq_len": w.Nq, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * tflops / PEAK_TFLOPS[w.dtype], 2),
        "kernel_ms_mean": round(ev_ms, 5),
        "per_launch": stats,
        "roofline": roofline_for(w, ev_ms, sha),
        "cpu_baseline": cpu,
        "oracle": head_oracle,
        "also": also,
        "hbm_sweep": {"runs": sweep, "device_copy_GB_per_s": copy_gbs} if sweep else None,
        "autotune": tuned,
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "kernel_sha": sha,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
