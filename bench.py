#!/usr/bin/env python3
"""Benchmark of skip-softmax block-sparse attention on one MI355X.

One step = one split-KV decode step at 32K context (Llama-3.1-8B-like layer:
B=1, Hq=32, Hkv=8, d=128, N=32768, Bc=128, lambda=1e-3, 16 splits) followed by
the log-sum-exp combine, on seeded synthetic heavy-tailed inputs.  The KV cache
is rotated over identical copies, about 2 GiB in all (eight times the 256 MB
Infinity Cache), so every step reads from HBM whatever cache policy the
kernels' loads carry.

Printed: one JSON line whose `value` is the decode step's algorithmic HBM
throughput (GB/s: all of K, the kept V blocks, q, the split partials and the
decision bytes, divided by the step time), plus the decode split kernel's
roofline (its algorithmic bytes per launch over its average launch duration
from HIP events on the launch stream), the 32K causal prefill's executed
TFLOP/s at lambda in {1e-4, 1e-3, 1e-2} and the dense (lambda = 0) reference,
block sparsity, the MLA decode kernel at 32K context (128 heads, 576-column latent
cache) against its HBM and MFMA rooflines, and the FP64 oracle timed on this host
as a CPU baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode µs & HBM GB/s at 32K; prefill TFLOP/s at 32K; block sparsity %"


# Counter-measured HBM bytes per launch live in the committed profile records
# (profiles/*.md, a "key: value" block).  A record counts only while the
# kernel's sources hash to the value it was taken with.
KERNEL_SOURCES = {
    "decode_split_kernel": ["decode.hip", "device_common.h", "tile_copy.h", "kernels.h"],
    "prefill_kernel": ["prefill.hip", "device_common.h", "tile_copy.h", "kernels.h"],
}


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "block_sparse_attention_flash_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (copy-calibrated), or None if stale or absent."""
    import glob
    want = source_hash(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        rec = {}
        with open(path, encoding="utf-8") as fh:
            for line in fh:
                line = line.strip()
                if ":" in line and " " not in line.split(":", 1)[0]:
                    k, v = line.split(":", 1)
                    rec[k] = v.strip()
        if rec.get("kernel") == kernel and rec.get("workload") == workload and "traffic_bytes_per_launch" in rec:
            return int(rec["traffic_bytes_per_launch"]) if rec.get("source_sha256_16") == want else None
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=None,
                   help="KV copies rotated to defeat the Infinity Cache (default: enough for 2 GiB)")
    p.add_argument("--prefill-reps", type=int, default=5, help="launches per prefill timing trial")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-mla", action="store_true")
    p.add_argument("--all-configs", action="store_true",
                   help="(the default) also time every other workload configuration (prefill_1k_tiny, "
                        "decode_128k_b16, decode_mqa_16k besides the two 32K ones) and two ragged batches: time, "
                        "fraction of the roofline, block sparsity")
    p.add_argument("--no-other-configs", action="store_true",
                   help="skip the other workload configurations and the ragged batches")
    p.add_argument("--no-length-sweep-timing", action="store_true",
                   help="skip the decode and prefill timing of the 128K length-sweep sequences at lambda = a/L")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--profile-target", choices=["decode", "decode_mqa", "decode_dense", "decode_ceiling",
                                                 "decode_sweep128", "prefill", "prefill_sweep128", "copy"],
                   default=None,
                   help="run only one kernel a few times (for hardware-counter collection) and exit")
    p.add_argument("--profile-lambda", type=float, default=None,
                   help="lambda for --profile-target decode / decode_mqa / prefill (default: the workload's) and "
                        "decode_sweep128 / prefill_sweep128 (default 0)")
    p.add_argument("--profile-launches", type=int, default=10)
    p.add_argument("--length-sweep", action="store_true",
                   help="instead of the bench: sparsity drift over 4K-128K context and the lambda = a/L calibration")
    p.add_argument("--speedup-curve", action="store_true",
                   help="instead of the bench: decode (128K) and causal prefill (32K-128K) kernel speed-up against "
                        "block sparsity 0-90%%, lambda read off each sequence's own margins")
    return p.parse_args()


COPY_BYTES = 512 << 20  # plain device-to-device copy used to calibrate byte counters
ROTATE_BYTES = 2 << 30  # KV bytes a timed loop rotates through: 8x the 256 MB Infinity Cache


def kv_copies(args, footprint):
    """Copies of a KV cache of `footprint` bytes to rotate: --copies if given, else enough for ROTATE_BYTES.
    Fewer would let the Infinity Cache serve part of each pass, and how much depends on the loads'
    cache policy (non-temporal lines are not kept), so an A/B of policies would time the cache."""
    if args.copies:
        return max(1, args.copies)
    return max(1, int(np.ceil(ROTATE_BYTES / footprint)))


def interleaved_trials(torch, stream, fns, reps, warm=1):
    """(median, min, max) time in ms of each of fns over TRIALS rounds; every round runs each fn reps
    times in turn, so clock and thermal drift during a run weigh on every point alike (timed one after
    another, the first points ran up to 6% slower while the clocks ramped)."""
    for fn in fns:
        for _ in range(warm):
            fn()
    torch.cuda.synchronize()
    ts = [[] for _ in fns]
    for _ in range(TRIALS):
        for i, fn in enumerate(fns):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for _ in range(reps):
                fn()
            s1.record(stream)
            torch.cuda.synchronize()
            ts[i].append(s0.elapsed_time(s1) / reps)
    return [(float(np.median(t)), min(t), max(t)) for t in ts]
TRIALS = 7  # repeated kernel-only timing trials (median reported)


def profile_target(args, lib, torch, W):
    """Launch one kernel --profile-launches times on the bench workload (no timing, no JSON)."""
    n = args.profile_launches
    if args.profile_target == "copy":
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(n):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copy: %d launches of %d bytes read + %d bytes written" % (n, COPY_BYTES, COPY_BYTES))
        return
    if args.profile_target in ("decode_dense", "decode_ceiling"):
        w = W.CONFIGS["decode_32k"]
        c0 = {k: dev(v) for k, v in W.generate(w).items()}
        copies = [c0] + [{k: v.clone() for k, v in c0.items()}
                         for _ in range(kv_copies(args, 2 * c0["k"].nbytes) - 1)]
        B, Hq, N, d, Bc, S = w.B, w.Hq, w.T, w.d, w.Bc, w.num_splits
        o_part = torch.empty((B, Hq, S, d), dtype=torch.float32, device="cuda")
        lse_part = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        for i in range(n):
            c = copies[i % len(copies)]
            if args.profile_target == "decode_dense":
                st = lib.blasst_decode_dense(P(c["q"]), P(c["k"]), P(c["v"]), P(o_part), P(lse_part), B, Hq, N, d, w.G,
                                             Bc, S, sp)
            else:
                st = lib.blasst_decode_load_ceiling(P(c["k"]), P(c["v"]), B, w.Hkv, N, d, Bc, S, sp)
            assert st == 0
        torch.cuda.synchronize()
        print("%s on %s: %d launches; K + V bytes per launch %d" % (args.profile_target, w.name, n,
                                                                  2 * B * w.Hkv * N * d * 2))
        return
    if args.profile_target in ("decode", "decode_mqa", "decode_sweep128"):
        if args.profile_target == "decode_sweep128":
            w = W.sweep_workload("decode", W.SWEEP_LENGTHS[-1], "evaluation").with_(num_splits=SWEEP128_SPLITS)
            w = w.with_(lambdas=(args.profile_lambda or 0.0,))
        else:
            w = W.CONFIGS["decode_32k" if args.profile_target == "decode" else "decode_mqa_16k"]
            if args.profile_lambda is not None:
                w = w.with_(lambdas=(args.profile_lambda,))
        c0 = {k: dev(v) for k, v in W.generate(w).items()}
        ncopies = 1 if args.profile_target == "decode_sweep128" else kv_copies(args, 2 * c0["k"].nbytes)
        copies = [c0] + [{k: v.clone() for k, v in c0.items()} for _ in range(ncopies - 1)]
        B, Hq, N, d, Bc, S = w.B, w.Hq, w.T, w.d, w.Bc, w.num_splits
        nk = -(-N // Bc)
        o_part = torch.empty((B, Hq, S, d), dtype=torch.float32, device="cuda")
        lse_part = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device="cuda")
        vskip = torch.empty((B, w.Hkv, nk), dtype=torch.uint8, device="cuda")
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        for i in range(n):
            c = copies[i % len(copies)]
            assert lib.blasst_decode(P(c["q"]), P(c["k"]), P(c["v"]), P(o_part), P(lse_part), P(skip), P(vskip),
                                     B, Hq, N, d, w.G, Bc, ctypes.c_double(w.lambdas[0]), 1, S, sp) == 0
        torch.cuda.synchronize()
        by = decode_bytes(w, vskip.cpu().numpy())
        print("%s at lambda %g: %d launches, algorithmic bytes per launch %d (read %d, written %d); "
              "V-load sparsity %.4f" % (w.name, w.lambdas[0], n, by["split"], by["k"] + by["v_kept"] + B * Hq * d * 2,
                                       by["split"] - by["k"] - by["v_kept"] - B * Hq * d * 2,
                                       float(vskip.cpu().numpy().mean())))
        return
    if args.profile_target == "prefill_sweep128":
        w = W.sweep_workload("prefill", W.SWEEP_LENGTHS[-1], "evaluation")
        lam = args.profile_lambda or 0.0
    else:
        w = W.CONFIGS["prefill_32k"]
        lam = 1e-3 if args.profile_lambda is None else args.profile_lambda
    x = {k: dev(v) for k, v in W.generate(w).items()}
    B, Hq, T, d, Bc = w.B, w.Hq, w.T, w.d, w.Bc
    nq = -(-T // Bc)
    o = torch.empty((B, Hq, T, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, nq, nq), dtype=torch.uint8, device="cuda")
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    for _ in range(n):
        assert lib.blasst_prefill(P(x["q"]), P(x["k"]), P(x["v"]), P(o), P(lse), P(mask), B, Hq, T, d, w.G, Bc,
                                  ctypes.c_double(lam), 1, sp) == 0
    torch.cuda.synchronize()
    visited = B * Hq * nq * (nq + 1) // 2
    print("%s: %d launches at lambda=%g, block sparsity %.4f" % (w.name, n, lam,
                                                                 float((mask == 1).sum().item()) / visited))


SWEEP_LAMBDAS = tuple(float(x) for x in np.geomspace(1e-5, 0.9, 50))  # candidate thresholds
DECODE_SWEEP_LAMBDAS = (0.0, 1e-3, 1e-2, 1e-1, 0.5)  # decode_32k inputs, split kernel against the dense one
SWEEP128_SPLITS = 4  # splits of the timed 128K length-sweep decode
SWEEP_FIXED = (1e-3, 3e-3)
SWEEP_TARGETS = (0.5, 0.7)


def sweep_margins(kind, L, split, W, bsa, B=None, num_splits=None):
    """GPU decision margins of one length-sweep batch (flattened) and the margin kernel's time."""
    import torch
    w = W.sweep_workload(kind, L, split, B)
    if num_splits is not None:
        w = w.with_(num_splits=num_splits)
    x = W.generate(w, parts=("q", "k"))
    q, k = dev(x["q"]), dev(x["k"])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    if kind == "decode":
        m, _ = bsa.decode_margins(q, k, w.num_splits, Bc=w.Bc)
    else:
        m = bsa.prefill_margins(q, k, Bc=w.Bc, causal=True)
    e1.record()
    torch.cuda.synchronize()
    return m.cpu().numpy().ravel(), e0.elapsed_time(e1)


def length_sweep(kind, lengths, calib_lengths, W, bsa, B=None, log=None):
    """Sparsity at fixed lambda over context lengths (the drift), then the one-pass calibration of
    lambda = alpha * exp(beta * S) / L on the calibration sequences and its sparsity on other sequences."""
    from block_sparse_attention_flash_amd import policy
    cal, ev, ms = {}, {}, {}
    for L in lengths:
        if L in calib_lengths:
            cal[L], _ = sweep_margins(kind, L, "calibration", W, bsa, B)
        ev[L], ms[L] = sweep_margins(kind, L, "evaluation", W, bsa, B)
        if log:
            log("%s L=%d: %d decisions, margin kernel %.3f ms" % (kind, L, np.count_nonzero(~np.isnan(ev[L])), ms[L]))
    a, s = policy.calibration_points([cal[L] for L in calib_lengths], list(calib_lengths), SWEEP_LAMBDAS)
    alpha, beta = policy.fit_exponential(a, s)
    out = {"lengths": list(lengths), "calibration_lengths": list(calib_lengths),
           "margin_kernel_ms": [round(ms[L], 3) for L in lengths],
           "fixed_lambda": {str(lam): [round(float(policy.sparsity_at(ev[L], [lam])[0]), 4) for L in lengths]
                            for lam in SWEEP_FIXED},
           "fit": {"alpha": alpha, "beta": beta, "points": int(len(a))}, "calibrated": {}}
    for S in SWEEP_TARGETS:
        lams = [policy.lambda_for(S, L, alpha, beta) for L in lengths]
        sp = [float(policy.sparsity_at(ev[L], [lam])[0]) for L, lam in zip(lengths, lams)]
        out["calibrated"][str(S)] = {"a": alpha * float(np.exp(beta * S)), "lambda": lams,
                                     "sparsity": [round(v, 4) for v in sp],
                                     "mean_abs_dev": round(float(np.mean(np.abs(np.asarray(sp) - S))), 4),
                                     "spread": round(max(sp) - min(sp), 4)}
    return out


def dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def decode_bytes(w, vskip: np.ndarray):
    """Algorithmic bytes of one split-kernel launch and of one combine launch."""
    B, Hq, Hkv, N, d, Bc, S = w.B, w.Hq, w.Hkv, w.T, w.d, w.Bc, w.num_splits
    nk = -(-N // Bc)
    rows_per_block = np.minimum(Bc, N - np.arange(nk) * Bc)
    kept_rows = int(((vskip == 0) * rows_per_block[None, None, :]).sum())
    k_bytes = B * Hkv * N * d * 2
    v_bytes = kept_rows * d * 2
    q_bytes = B * Hq * d * 2
    part_bytes = B * Hq * S * (d + 1) * 4
    mask_bytes = B * Hq * nk + B * Hkv * nk
    split = k_bytes + v_bytes + q_bytes + part_bytes + mask_bytes
    combine = part_bytes + B * Hq * (d + 1) * 4
    return dict(split=split, combine=combine, k=k_bytes, v_kept=v_bytes, v_dense=B * Hkv * N * d * 2)


def bench_decode(args, lib, torch, W):
    w = W.CONFIGS["decode_32k"]
    lam = w.lambdas[0]
    x = W.generate(w)
    copies = [{k: dev(v) for k, v in x.items()} for _ in range(kv_copies(args, 2 * x["k"].nbytes))]
    B, Hq, N, d, Bc, S = w.B, w.Hq, w.T, w.d, w.Bc, w.num_splits
    nk = -(-N // Bc)
    f32 = dict(dtype=torch.float32, device="cuda")
    o_part = torch.empty((B, Hq, S, d), **f32)
    lse_part = torch.empty((B, Hq, S), **f32)
    o = torch.empty((B, Hq, d), **f32)
    lse = torch.empty((B, Hq), **f32)
    skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device="cuda")
    vskip = torch.empty((B, w.Hkv, nk), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def split_args(c, lam_):
        return (P(c["q"]), P(c["k"]), P(c["v"]), P(o_part), P(lse_part), P(skip), P(vskip),
                B, Hq, N, d, w.G, Bc, ctypes.c_double(lam_), 1, S, sp)

    comb = (P(o_part), P(lse_part), P(o), P(lse), B, Hq, d, S, sp)
    sargs = [split_args(c, lam) for c in copies]
    dense_args = [split_args(c, 0.0) for c in copies]
    decode_fn, combine_fn = lib.blasst_decode, lib.blasst_decode_combine

    def check(st):
        if st != 0:
            raise RuntimeError("libblasst call failed with status %d" % st)

    for s in range(args.warmup):
        check(decode_fn(*sargs[s % len(sargs)]))
        check(combine_fn(*comb))
    torch.cuda.synchronize()

    # timed region: K steps (split + combine), HIP events on the launch stream at both ends
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        check(decode_fn(*sargs[s % len(sargs)]))
        check(combine_fn(*comb))
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = start.elapsed_time(stop) / args.steps

    # the split kernel alone: TRIALS trials of K back-to-back launches, each
    # between one pair of events on the launch stream; the median trial is used
    trials = []
    for _ in range(TRIALS):
        torch.cuda.synchronize()
        start.record(stream)
        for s in range(args.steps):
            check(decode_fn(*sargs[s % len(sargs)]))
        stop.record(stream)
        torch.cuda.synchronize()
        trials.append(start.elapsed_time(stop) / args.steps)
    split_ms = float(np.median(trials))

    def step_time(fn_args):
        """Time of one step (kernel + combine) over K back-to-back steps, after W warm-up steps."""
        for s in range(args.warmup):
            fn_args(s)
            check(combine_fn(*comb))
        torch.cuda.synchronize()
        start.record(stream)
        for s in range(args.steps):
            fn_args(s)
            check(combine_fn(*comb))
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    # the same kernel at lambda = 0 (nothing skipped; the test and the decision bytes still run)
    lambda0_step_ms = step_time(lambda s: check(decode_fn(*dense_args[s % len(dense_args)])))
    # the dense kernel (blasst_decode_dense: one pass over K and V, no decision)
    ref_args = [(P(c["q"]), P(c["k"]), P(c["v"]), P(o_part), P(lse_part), B, Hq, N, d, w.G, Bc, S, sp) for c in copies]
    ref_fn = lambda s: check(lib.blasst_decode_dense(*ref_args[s % len(ref_args)]))  # noqa: E731
    dense_step_ms = step_time(ref_fn)
    reps = max(args.steps, 50)
    # the split kernel's loads alone at lambda = 0 (blasst_decode_load_ceiling): the floor its bytes and
    # its access pattern set on this part
    ceil_args = [(P(c["k"]), P(c["v"]), B, w.Hkv, N, d, Bc, S, sp) for c in copies]

    # decisions of the timed configuration (identical on every copy)
    check(decode_fn(*sargs[0]))
    torch.cuda.synchronize()
    sk, vsk = skip.cpu().numpy(), vskip.cpu().numpy()
    by = decode_bytes(w, vsk)

    def rotating(launch):
        """A callable launching launch(i) with i = 0, 1, 2, ... (the KV copies rotate with i)."""
        it = [0]

        def f():
            launch(it[0])
            it[0] += 1
        return f

    # lambda sweep on the same inputs: each lambda once for its decisions, then the dense kernel, the
    # load ceiling and every lambda timed in turns (reps launches per case and round)
    dense_by = decode_bytes(w, np.zeros_like(vsk))
    fns = [rotating(ref_fn), rotating(lambda s: check(lib.blasst_decode_load_ceiling(*ceil_args[s % len(ceil_args)])))]
    stats = []
    for lam_ in DECODE_SWEEP_LAMBDAS:
        la = [split_args(c, lam_) for c in copies]
        check(decode_fn(*la[0]))
        torch.cuda.synchronize()
        stats.append((skip.cpu().numpy(), vskip.cpu().numpy()))
        fns.append(rotating(lambda s, la=la: check(decode_fn(*la[s % len(la)]))))
    times = interleaved_trials(torch, stream, fns, reps, warm=4)
    dense_kernel_ms, load_ceiling_ms = times[0], times[1]
    sweep = []
    for lam_, (sk_, vsk_), ms in zip(DECODE_SWEEP_LAMBDAS, stats, times[2:]):
        by_ = decode_bytes(w, vsk_)
        sweep.append(dict(
            lam=lam_, split_kernel_us=round(ms[0] * 1e3, 3), split_kernel_us_min=round(ms[1] * 1e3, 3),
            split_kernel_us_max=round(ms[2] * 1e3, 3), block_sparsity=round(float(sk_.mean()), 5),
            vload_sparsity=round(float(vsk_.mean()), 5), bytes_per_launch=by_["split"],
            GBs=round(by_["split"] / (ms[0] * 1e-3) / 1e9, 1),
            frac_of_hbm_peak=round(by_["split"] / (ms[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            speedup_vs_dense_kernel=round(dense_kernel_ms[0] / ms[0], 4),
            bytes_ratio_dense_over_this=round(dense_by["split"] / by_["split"], 4)))
    l0 = next(r for r in sweep if r["lam"] == 0.0)["split_kernel_us"]
    for r in sweep:
        r["speedup_vs_lambda0"] = round(l0 / r["split_kernel_us"], 4)
    return dict(w=w, x=x, step_ms=step_ms, split_ms=split_ms, split_trials_ms=trials, lambda0_step_ms=lambda0_step_ms,
                dense_step_ms=dense_step_ms, dense_kernel_ms=dense_kernel_ms, load_ceiling_ms=load_ceiling_ms,
                wall=wall, bytes=by, kv_copies_rotated=len(copies),
                block_sparsity=float(sk.mean()), vload_sparsity=float(vsk.mean()), lambda_sweep=sweep)


def bench_prefill(args, lib, torch, W):
    w = W.CONFIGS["prefill_32k"]
    x = {k: dev(v) for k, v in W.generate(w).items()}
    B, Hq, T, d, Bc = w.B, w.Hq, w.T, w.d, w.Bc
    nq = -(-T // Bc)
    o = torch.empty((B, Hq, T, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, nq, nq), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    out = {}
    visited = B * Hq * nq * (nq + 1) // 2
    tile_flops = 2.0 * Bc * Bc * d
    sp = ctypes.c_void_p(stream.cuda_stream)

    def check(st):
        assert st == 0

    # each lambda once for its mask and its error against the lambda = 0 output (untimed), then every
    # lambda and the kernel without the skip test timed in turns, prefill_reps launches per round
    lams = (0.0,) + tuple(w.lambdas)
    o0 = lse0 = None
    fns = []
    for lam in lams:
        a = (P(x["q"]), P(x["k"]), P(x["v"]), P(o), P(lse), P(mask), B, Hq, T, d, w.G, Bc,
             ctypes.c_double(lam), 1, sp)
        check(lib.blasst_prefill(*a))
        torch.cuda.synchronize()
        fns.append(lambda a=a: check(lib.blasst_prefill(*a)))
        skipped = int((mask == 1).sum().item())
        out["%g" % lam] = dict(block_sparsity=round(skipped / visited, 5),
                               executed_tflop=round((2 * visited - skipped) * tile_flops / 1e12, 4))
        # the skip's error against the dense (lambda = 0) output of the same kernel
        if o0 is None:
            o0, lse0 = o.clone(), lse.clone()
        else:
            diff = (o - o0).view(-1, d)
            rel = diff.norm(dim=1) / o0.view(-1, d).norm(dim=1).clamp_min(1e-30)
            out["%g" % lam]["error_vs_dense"] = dict(
                o_max_abs=float(diff.abs().max().item()), row_rel_l2_max=float(rel.max().item()),
                row_rel_l2_mean=float(rel.mean().item()), lse_max_abs=float((lse - lse0).abs().max().item()),
                rows_changed=round(float((rel > 0).float().mean().item()), 5))
            del diff, rel
    del o0, lse0
    # the kernel built without the skip test (blasst_prefill_dense): what the test costs at 0% sparsity
    nt_a = (P(x["q"]), P(x["k"]), P(x["v"]), P(o), P(lse), B, Hq, T, d, w.G, Bc, 1, sp)
    fns.append(lambda: check(lib.blasst_prefill_dense(*nt_a)))
    times = interleaved_trials(torch, stream, fns, args.prefill_reps, warm=2)
    for lam, (ms, ms_min, ms_max) in zip(lams, times):
        v = out["%g" % lam]
        tflops = v["executed_tflop"] * 1e12 / (ms * 1e-3) / 1e12
        v.update(ms=round(ms, 4), ms_min=round(ms_min, 4), ms_max=round(ms_max, 4),
                 tflops_executed=round(tflops, 2), frac_of_mfma_peak=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4))
    dense = out["0"]["ms"]
    for k, v in out.items():
        v["speedup_vs_lambda0"] = round(dense / v["ms"], 4)
    ref_ms = times[-1][0]
    no_test = dict(ms=round(ref_ms, 4), tflops=round(2 * visited * tile_flops / (ref_ms * 1e-3) / 1e12, 2),
                   lambda0_speed_vs_no_test=round(ref_ms / dense, 4))
    return dict(workload=w.name, B=B, Hq=Hq, Hkv=w.Hkv, d=d, T=T, Bc=Bc, by_lambda=out, no_skip_test=no_test,
                hbm_traffic_bytes_per_launch=measured_traffic("prefill_kernel", w.name))


def bench_config(name, args, lib, torch, W):
    """One workload configuration at its own lambda: a decode step (split + combine) or a prefill launch,
    median of TRIALS trials, with the roofline fraction on the work done and the block sparsity."""
    w = W.CONFIGS[name]
    lam = w.lambdas[0]
    x = W.generate(w)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    f32 = dict(dtype=torch.float32, device="cuda")
    B, Hq, T, d, Bc = w.B, w.Hq, w.T, w.d, w.Bc
    nk = -(-T // Bc)

    def trials(fns, reps):
        for f in fns[:2]:
            f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(TRIALS):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for i in range(reps):
                fns[i % len(fns)]()
            s1.record(stream)
            torch.cuda.synchronize()
            ts.append(s0.elapsed_time(s1) / reps)
        return float(np.median(ts)), min(ts), max(ts)

    def ok(st):
        if st != 0:
            raise RuntimeError("libblasst call failed with status %d" % st)

    if w.kind == "prefill":
        xd = {k: dev(v) for k, v in x.items()}
        o = torch.empty((B, Hq, T, d), **f32)
        lse = torch.empty((B, Hq, T), **f32)
        mask = torch.empty((B, Hq, nk, nk), dtype=torch.uint8, device="cuda")
        a = (P(xd["q"]), P(xd["k"]), P(xd["v"]), P(o), P(lse), P(mask), B, Hq, T, d, w.G, Bc, ctypes.c_double(lam), 1, sp)
        ms, lo, hi = trials([lambda: ok(lib.blasst_prefill(*a))], max(args.prefill_reps, 20))
        m = mask.cpu().numpy()
        visited = B * Hq * nk * (nk + 1) // 2
        skipped = int((m == 1).sum())
        flops = (2 * visited - skipped) * 2.0 * Bc * Bc * d
        tf = flops / (ms * 1e-3) / 1e12
        return dict(kind="prefill", lam=lam, ms=round(ms, 4), ms_min=round(lo, 4), ms_max=round(hi, 4),
                    tflops_executed=round(tf, 2), frac_of_mfma_peak=round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                    block_sparsity=round(skipped / visited, 5))
    S = w.num_splits
    footprint = 2 * x["k"].nbytes
    ncopy = kv_copies(args, footprint)
    xs = [{k: dev(v) for k, v in x.items()} for _ in range(ncopy)]
    del x
    o_part = torch.empty((B, Hq, S, d), **f32)
    lse_part = torch.empty((B, Hq, S), **f32)
    o = torch.empty((B, Hq, d), **f32)
    lse = torch.empty((B, Hq), **f32)
    skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device="cuda")
    vskip = torch.empty((B, w.Hkv, nk), dtype=torch.uint8, device="cuda")
    comb = (P(o_part), P(lse_part), P(o), P(lse), B, Hq, d, S, sp)
    sargs = [(P(c["q"]), P(c["k"]), P(c["v"]), P(o_part), P(lse_part), P(skip), P(vskip), B, Hq, T, d, w.G, Bc,
              ctypes.c_double(lam), 1, S, sp) for c in xs]

    def step(a):
        return lambda: (ok(lib.blasst_decode(*a)), ok(lib.blasst_decode_combine(*comb)))

    def split(a):
        return lambda: ok(lib.blasst_decode(*a))

    reps = 200 if footprint < 1e9 else 20
    step_ms, _, _ = trials([step(a) for a in sargs], reps)
    split_ms, lo, hi = trials([split(a) for a in sargs], reps)
    ok(lib.blasst_decode(*sargs[0]))
    torch.cuda.synchronize()
    sk, vsk = skip.cpu().numpy(), vskip.cpu().numpy()
    by = decode_bytes(w, vsk)
    gbs = by["split"] / (split_ms * 1e-3) / 1e9
    return dict(kind="decode", lam=lam, step_us=round(step_ms * 1e3, 2), split_kernel_us=round(split_ms * 1e3, 2),
                split_kernel_us_min=round(lo * 1e3, 2), split_kernel_us_max=round(hi * 1e3, 2),
                split_GBs=round(gbs, 1), frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
                step_GBs=round((by["split"] + by["combine"]) / (step_ms * 1e-3) / 1e9, 1),
                bytes_per_split_launch=by["split"], kv_copies_rotated=ncopy,
                block_sparsity=round(float(sk.mean()), 5), vload_sparsity=round(float(vsk.mean()), 5))


def bench_ragged(args, lib, torch, W):
    """Ragged batches through blasst_decode_ragged / blasst_prefill_ragged: a decode serving batch of 16
    sequences with 1K-32K contexts in a 32K-capacity cache (the GPU test's recipe), and a causal prefill
    of four sequences of 16K, 9K, 4K and 1.5K rows in a 16K-capacity buffer.  Work is counted over each
    sequence's own length: the K rows and kept V rows of its context (decode), the visited and kept tiles
    of its causal range (prefill)."""
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    f32 = dict(dtype=torch.float32, device="cuda")

    def ok(st):
        if st != 0:
            raise RuntimeError("libblasst call failed with status %d" % st)

    def trials(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(TRIALS):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for _ in range(reps):
                fn()
            s1.record(stream)
            torch.cuda.synchronize()
            ts.append(s0.elapsed_time(s1) / reps)
        return float(np.median(ts)), min(ts), max(ts)

    # ---- decode serving batch
    rng = np.random.default_rng(7)
    lens = [int(v) for v in rng.integers(1024, 32769, size=16)]
    lens[3] = 32768
    w = W.Workload("decode_ragged_serving", "decode", B=16, Hq=32, Hkv=8, d=128, T=32768, Bc=128,
                   lambdas=(1e-3,), hot_rate=0.01, seed=707, window=512, num_splits=16)
    B, Hq, Hkv, N, d, Bc, S, lam = w.B, w.Hq, w.Hkv, w.T, w.d, w.Bc, w.num_splits, w.lambdas[0]
    nk = -(-N // Bc)
    xd = {k: dev(v) for k, v in W.generate(w).items()}
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o_part = torch.empty((B, Hq, S, d), **f32)
    lse_part = torch.empty((B, Hq, S), **f32)
    o = torch.empty((B, Hq, d), **f32)
    lse = torch.empty((B, Hq), **f32)
    skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device="cuda")
    vskip = torch.empty((B, Hkv, nk), dtype=torch.uint8, device="cuda")
    sa = (P(xd["q"]), P(xd["k"]), P(xd["v"]), P(o_part), P(lse_part), P(skip), P(vskip), P(lens_d), B, Hq, N, d,
          Hq // Hkv, Bc, ctypes.c_double(lam), S, sp)
    ca = (P(o_part), P(lse_part), P(o), P(lse), B, Hq, d, S, sp)
    split_ms, lo, hi = trials(lambda: ok(lib.blasst_decode_ragged(*sa)), 50)
    step_ms, _, _ = trials(lambda: (ok(lib.blasst_decode_ragged(*sa)), ok(lib.blasst_decode_combine(*ca))), 50)
    vsk = vskip.cpu().numpy()
    kept_rows = 0
    for b, L in enumerate(lens):
        rows = np.minimum(Bc, L - np.arange(-(-L // Bc)) * Bc)
        kept_rows += int(((vsk[b, :, :len(rows)] == 0) * rows[None, :]).sum())
    split_bytes = (Hkv * sum(lens) * d * 2 + kept_rows * d * 2 + B * Hq * d * 2 + B * Hq * S * (d + 1) * 4
                   + (B * Hq + B * Hkv) * nk)
    comb_bytes = B * Hq * S * (d + 1) * 4 + B * Hq * (d + 1) * 4
    gbs = split_bytes / (split_ms * 1e-3) / 1e9
    dec = dict(lens=lens, capacity=N, B=B, Hq=Hq, Hkv=Hkv, d=d, Bc=Bc, num_splits=S, lam=lam,
               split_kernel_us=round(split_ms * 1e3, 2), split_kernel_us_min=round(lo * 1e3, 2),
               split_kernel_us_max=round(hi * 1e3, 2), step_us=round(step_ms * 1e3, 2),
               bytes_per_split_launch=split_bytes, split_GBs=round(gbs, 1),
               frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
               step_GBs=round((split_bytes + comb_bytes) / (step_ms * 1e-3) / 1e9, 1),
               vload_sparsity=round(1.0 - kept_rows / (Hkv * sum(lens)), 5))
    del xd
    torch.cuda.empty_cache()

    # ---- causal prefill, four sequences
    plens = [16384, 9000, 4000, 1500]
    w = W.Workload("prefill_ragged", "prefill", B=4, Hq=32, Hkv=8, d=128, T=16384, Bc=128, lambdas=(1e-3,),
                   hot_rate=0.01, seed=708)
    B, Hq, T, d, Bc, lam = w.B, w.Hq, w.T, w.d, w.Bc, w.lambdas[0]
    nq = -(-T // Bc)
    xd = {k: dev(v) for k, v in W.generate(w).items()}
    lens_d = torch.tensor(plens, dtype=torch.int32, device="cuda")
    o = torch.empty((B, Hq, T, d), **f32)
    lse = torch.empty((B, Hq, T), **f32)
    mask = torch.empty((B, Hq, nq, nq), dtype=torch.uint8, device="cuda")
    pa = (P(xd["q"]), P(xd["k"]), P(xd["v"]), P(o), P(lse), P(mask), P(lens_d), B, Hq, T, d, Hq // w.Hkv, Bc,
          ctypes.c_double(lam), 1, sp)
    ms, lo, hi = trials(lambda: ok(lib.blasst_prefill_ragged(*pa)), 5)
    m = mask.cpu().numpy()
    visited, skipped = int((m != 2).sum()), int((m == 1).sum())
    flops = (2 * visited - skipped) * 2.0 * Bc * Bc * d
    tf = flops / (ms * 1e-3) / 1e12
    pre = dict(lens=plens, capacity=T, B=B, Hq=Hq, Hkv=w.Hkv, d=d, Bc=Bc, lam=lam, ms=round(ms, 4),
               ms_min=round(lo, 4), ms_max=round(hi, 4), tflops_executed=round(tf, 2),
               frac_of_mfma_peak=round(tf / MFMA_BF16_PEAK_TFLOPS, 4), block_sparsity=round(skipped / visited, 5))
    del xd
    torch.cuda.empty_cache()
    return {"decode_serving_batch": dec, "prefill_causal": pre}


def calibrate_decode_policy(W, bsa, B=None, num_splits=1):
    """lambda = a/L for decode, fitted on the calibration sequences of the length-sweep family
    (4K-64K, GPU margins at num_splits splits): returns (alpha, beta, number of points).  A split
    restarts the running max, so the margins -- and the lambda a target sparsity needs -- depend
    on the split count; the fit is taken at the count the kernel then runs with."""
    from block_sparse_attention_flash_amd import policy
    lengths = W.SWEEP_LENGTHS[:5]
    margins = [sweep_margins("decode", L, "calibration", W, bsa, B, num_splits)[0] for L in lengths]
    a, s = policy.calibration_points(margins, list(lengths), SWEEP_LAMBDAS)
    alpha, beta = policy.fit_exponential(a, s)
    return alpha, beta, int(len(a))


def bench_decode_length_sweep(args, lib, torch, W, bsa):
    """What a decode skip buys where skipping is common: the length-sweep family's held-out 128K
    sequences (B = 4, Hq = 32, Hkv = 8, d = 128), split 4 ways (128 units: the two-workgroups-per-split
    layout fills the GPU), timed through the split kernel at lambda = a/L for 50% and 70% target
    sparsity (a fitted on the 4K-64K calibration sequences' margins at the same split count) and at
    fixed lambdas, against lambda = 0 and the dense kernel.  The split kernel reads all of K and the kept
    V blocks, so the bytes predict the speed-up: 1 / (1 - vload * V / (K + V))."""
    from block_sparse_attention_flash_amd import policy
    alpha, beta, npts = calibrate_decode_policy(W, bsa, num_splits=SWEEP128_SPLITS)
    L = W.SWEEP_LENGTHS[-1]
    w = W.sweep_workload("decode", L, "evaluation").with_(num_splits=SWEEP128_SPLITS)
    x = {k: dev(v) for k, v in W.generate(w).items()}
    B, Hq, N, d, Bc, S = w.B, w.Hq, w.T, w.d, w.Bc, w.num_splits
    nk = -(-N // Bc)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    o_part = torch.empty((B, Hq, S, d), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device="cuda")
    vskip = torch.empty((B, w.Hkv, nk), dtype=torch.uint8, device="cuda")

    def ok(st):
        if st != 0:
            raise RuntimeError("libblasst call failed with status %d" % st)

    dense_a = (P(x["q"]), P(x["k"]), P(x["v"]), P(o_part), P(lse_part), B, Hq, N, d, w.G, Bc, S, sp)
    targets = {"a/L, 50%": policy.lambda_for(0.5, L, alpha, beta), "a/L, 70%": policy.lambda_for(0.7, L, alpha, beta)}
    # sparsity-matched points: lambda read off these sequences' own margins (block sparsity 50%, and the
    # 73.2% at which the blog quotes its decode speed-up)
    own, _ = bsa.decode_margins(x["q"], x["k"], S, Bc=Bc)
    matched = {"matched 50%": policy.lambda_at_sparsity(own, 0.5),
               "matched 73.2%": policy.lambda_at_sparsity(own, 0.732)}
    del own
    points = [("lambda = 0", 0.0), ("fixed 1e-3", 1e-3), ("fixed 3e-3", 3e-3)] + list(targets.items()) + \
        list(matched.items())
    dense_bytes = decode_bytes(w, np.zeros((B, w.Hkv, nk), np.uint8))["split"]
    stats, fns = [], []
    for label, lam in points:
        a = (P(x["q"]), P(x["k"]), P(x["v"]), P(o_part), P(lse_part), P(skip), P(vskip), B, Hq, N, d, w.G, Bc,
             ctypes.c_double(lam), 1, S, sp)
        ok(lib.blasst_decode(*a))
        torch.cuda.synchronize()
        stats.append((skip.cpu().numpy(), vskip.cpu().numpy()))
        fns.append(lambda a=a: ok(lib.blasst_decode(*a)))
    times = interleaved_trials(torch, stream, [lambda: ok(lib.blasst_decode_dense(*dense_a))] + fns, 20, warm=3)
    dense_ms = times[0]
    rows = []
    for (label, lam), (sk, vsk), ms in zip(points, stats, times[1:]):
        by = decode_bytes(w, vsk)["split"]
        rows.append(dict(point=label, lam=lam, split_kernel_us=round(ms[0] * 1e3, 2),
                         split_kernel_us_min=round(ms[1] * 1e3, 2), split_kernel_us_max=round(ms[2] * 1e3, 2),
                         block_sparsity=round(float(sk.mean()), 4), vload_sparsity=round(float(vsk.mean()), 4),
                         bytes_per_launch=by, GBs=round(by / (ms[0] * 1e-3) / 1e9, 1),
                         frac_of_hbm_peak=round(by / (ms[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         speedup_vs_dense_kernel=round(dense_ms[0] / ms[0], 4),
                         bytes_ratio_dense_over_this=round(dense_bytes / by, 4)))
    l0 = rows[0]["split_kernel_us"]
    for r in rows:
        r["speedup_vs_lambda0"] = round(l0 / r["split_kernel_us"], 4)
    del x
    torch.cuda.empty_cache()
    return dict(workload=w.name, B=B, Hq=Hq, Hkv=w.Hkv, d=d, context=N, Bc=Bc, num_splits=S,
                policy={"alpha": alpha, "beta": beta, "points": npts, "calibration_lengths": list(W.SWEEP_LENGTHS[:5]),
                        "calibration_splits": SWEEP128_SPLITS},
                dense_kernel_us=round(dense_ms[0] * 1e3, 2), by_lambda=rows)


def bench_prefill_length_sweep(args, lib, torch, W, bsa):
    """What a prefill skip buys where skipping is common: the length-sweep family's held-out 128K causal
    sequence (B = 1, Hq = 32, Hkv = 8, d = 128, Bc = 128) through blasst_prefill at lambda = a/L for 50% and
    70% target sparsity (a fitted on the prefill margins of the 4K-64K calibration sequences) and at fixed
    lambdas, against lambda = 0 and the kernel built without the skip test.  A skipped tile still costs
    its S = Q K^T product and row maxima; only the exponentials and P V are saved, so at block sparsity s
    the executed FLOPs fall to (1 - s/2) of the dense count."""
    from block_sparse_attention_flash_amd import policy
    lengths = W.SWEEP_LENGTHS[:5]
    margins = [sweep_margins("prefill", L, "calibration", W, bsa)[0] for L in lengths]
    a_pts, s_pts = policy.calibration_points(margins, list(lengths), SWEEP_LAMBDAS)
    alpha, beta = policy.fit_exponential(a_pts, s_pts)
    del margins
    L = W.SWEEP_LENGTHS[-1]
    w = W.sweep_workload("prefill", L, "evaluation")
    x = {k: dev(v) for k, v in W.generate(w).items()}
    B, Hq, T, d, Bc = w.B, w.Hq, w.T, w.d, w.Bc
    nq = -(-T // Bc)
    o = torch.empty((B, Hq, T, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    mask = torch.empty((B, Hq, nq, nq), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    visited = B * Hq * nq * (nq + 1) // 2
    tile_flops = 2.0 * Bc * Bc * d

    def ok(st):
        if st != 0:
            raise RuntimeError("libblasst call failed with status %d" % st)

    no_test_a = (P(x["q"]), P(x["k"]), P(x["v"]), P(o), P(lse), B, Hq, T, d, w.G, Bc, 1, sp)
    targets = {"a/L, 50%": policy.lambda_for(0.5, L, alpha, beta), "a/L, 70%": policy.lambda_for(0.7, L, alpha, beta)}
    # sparsity-matched points: lambda read off this sequence's own margins (block sparsity 50%, and the
    # 71.9% at which the blog quotes its prefill speed-up)
    own = bsa.prefill_margins(x["q"], x["k"], Bc=Bc, causal=True)
    matched = {"matched 50%": policy.lambda_at_sparsity(own, 0.5),
               "matched 71.9%": policy.lambda_at_sparsity(own, 0.719)}
    del own
    points = [("lambda = 0", 0.0), ("fixed 1e-3", 1e-3), ("fixed 3e-3", 3e-3)] + list(targets.items()) + \
        list(matched.items())
    skips, fns = [], []
    for label, lam in points:
        a = (P(x["q"]), P(x["k"]), P(x["v"]), P(o), P(lse), P(mask), B, Hq, T, d, w.G, Bc,
             ctypes.c_double(lam), 1, sp)
        ok(lib.blasst_prefill(*a))
        torch.cuda.synchronize()
        skips.append(int((mask == 1).sum().item()))
        fns.append(lambda a=a: ok(lib.blasst_prefill(*a)))
    times = interleaved_trials(torch, stream, [lambda: ok(lib.blasst_prefill_dense(*no_test_a))] + fns, 2)
    no_test_ms = times[0]
    rows = []
    for (label, lam), skipped, ms in zip(points, skips, times[1:]):
        kept = visited - skipped
        flops = (visited + kept) * tile_flops
        rows.append(dict(point=label, lam=lam, ms=round(ms[0], 3), ms_min=round(ms[1], 3), ms_max=round(ms[2], 3),
                         block_sparsity=round(skipped / visited, 4),
                         executed_tflop=round(flops / 1e12, 2),
                         tflops_executed=round(flops / (ms[0] * 1e-3) / 1e12, 1),
                         frac_of_mfma_peak=round(flops / (ms[0] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         speedup_vs_no_test_kernel=round(no_test_ms[0] / ms[0], 4),
                         flops_ratio_dense_over_this=round(2 * visited / (visited + kept), 4)))
    l0 = rows[0]["ms"]
    for r in rows:
        r["speedup_vs_lambda0"] = round(l0 / r["ms"], 4)
    del x, o, lse, mask
    torch.cuda.empty_cache()
    return dict(workload=w.name, B=B, Hq=Hq, Hkv=w.Hkv, d=d, context=T, Bc=Bc, causal=True,
                policy={"alpha": alpha, "beta": beta, "points": int(len(a_pts)), "calibration_lengths": list(lengths)},
                no_skip_test_kernel_ms=round(no_test_ms[0], 3), by_lambda=rows)


CURVE_TARGETS = (0.0, 0.25, 0.4, 0.5, 0.6, 0.7, 0.8, 0.9)  # block sparsities of the speed-up curve


def speedup_curve(args, lib, torch, W, bsa):
    """Kernel speed-up against block sparsity, the pages' kernel-speed figure re-measured on this GPU:
    the length-sweep family's evaluation sequences, decoded at 128K (B = 4, 32/8 heads, 4 splits,
    split kernel) and prefilled causally at 32K, 64K and 128K (B = 1, 32/8 heads).  For each target
    sparsity lambda is read off the sequence's own decision margins (policy.lambda_at_sparsity); each
    point gives the kernel time, the sparsity reached, the speed-up over lambda = 0 and the bound the
    skipped work sets (decode: HBM bytes, all of K always read; prefill: FLOPs, S = Q K^T always
    formed)."""
    from block_sparse_attention_flash_amd import policy
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def ok(st):
        if st != 0:
            raise RuntimeError("libblasst call failed with status %d" % st)

    def interleaved(fns, reps):
        return [t[0] for t in interleaved_trials(torch, stream, fns, reps, warm=0)]

    out = {}
    # ---- decode, 128K
    L = W.SWEEP_LENGTHS[-1]
    w = W.sweep_workload("decode", L, "evaluation").with_(num_splits=SWEEP128_SPLITS)
    x = {k: dev(v) for k, v in W.generate(w).items()}
    B, Hq, N, d, Bc, S = w.B, w.Hq, w.T, w.d, w.Bc, w.num_splits
    nk = -(-N // Bc)
    o_part = torch.empty((B, Hq, S, d), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device="cuda")
    vskip = torch.empty((B, w.Hkv, nk), dtype=torch.uint8, device="cuda")
    own, _ = bsa.decode_margins(x["q"], x["k"], S, Bc=Bc)
    dense_a = (P(x["q"]), P(x["k"]), P(x["v"]), P(o_part), P(lse_part), B, Hq, N, d, w.G, Bc, S, sp)
    rows, fns = [], []
    for target in CURVE_TARGETS:
        lam = policy.lambda_at_sparsity(own, target) if target > 0 else 0.0
        a = (P(x["q"]), P(x["k"]), P(x["v"]), P(o_part), P(lse_part), P(skip), P(vskip), B, Hq, N, d, w.G, Bc,
             ctypes.c_double(lam), 1, S, sp)
        ok(lib.blasst_decode(*a))
        torch.cuda.synchronize()
        rows.append(dict(target=target, lam=lam, block_sparsity=round(float(skip.float().mean().item()), 4),
                         vload_sparsity=round(float(vskip.float().mean().item()), 4),
                         bytes_per_launch=decode_bytes(w, vskip.cpu().numpy())["split"]))
        fns.append(lambda a=a: ok(lib.blasst_decode(*a)))
    times = interleaved([lambda: ok(lib.blasst_decode_dense(*dense_a))] + fns, 20)
    dense_us = 1e3 * times[0]
    for r, t in zip(rows, times[1:]):
        r["us"] = round(1e3 * t, 2)
    for r in rows:
        r["speedup_vs_lambda0"] = round(rows[0]["us"] / r["us"], 4)
        r["speedup_vs_dense_kernel"] = round(dense_us / r["us"], 4)
        r["bytes_bound"] = round(rows[0]["bytes_per_launch"] / r["bytes_per_launch"], 4)
    out["decode_%dk" % (L // 1024)] = dict(B=B, Hq=Hq, Hkv=w.Hkv, d=d, context=N, Bc=Bc, num_splits=S,
                                           dense_kernel_us=round(dense_us, 2), points=rows)
    del x, o_part, lse_part, skip, vskip, own
    torch.cuda.empty_cache()
    # ---- causal prefill, 32K / 64K / 128K
    for L in W.SWEEP_LENGTHS[3:]:
        w = W.sweep_workload("prefill", L, "evaluation")
        x = {k: dev(v) for k, v in W.generate(w).items()}
        B, Hq, T, d, Bc = w.B, w.Hq, w.T, w.d, w.Bc
        nq = -(-T // Bc)
        o = torch.empty((B, Hq, T, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
        mask = torch.empty((B, Hq, nq, nq), dtype=torch.uint8, device="cuda")
        own = bsa.prefill_margins(x["q"], x["k"], Bc=Bc, causal=True)
        visited = B * Hq * nq * (nq + 1) // 2
        reps = max(1, (131072 // T) ** 2 // 4)
        rows, fns = [], []
        for target in CURVE_TARGETS:
            lam = policy.lambda_at_sparsity(own, target) if target > 0 else 0.0
            a = (P(x["q"]), P(x["k"]), P(x["v"]), P(o), P(lse), P(mask), B, Hq, T, d, w.G, Bc,
                 ctypes.c_double(lam), 1, sp)
            ok(lib.blasst_prefill(*a))
            torch.cuda.synchronize()
            kept = visited - int((mask == 1).sum().item())
            rows.append(dict(target=target, lam=lam, block_sparsity=round(1 - kept / visited, 4),
                             flops_bound=round(2 * visited / (visited + kept), 4)))
            fns.append(lambda a=a: ok(lib.blasst_prefill(*a)))
        for r, t in zip(rows, interleaved(fns, reps)):
            r["ms"] = round(t, 3)
        for r in rows:
            r["speedup_vs_lambda0"] = round(rows[0]["ms"] / r["ms"], 4)
        out["prefill_%dk" % (L // 1024)] = dict(B=B, Hq=Hq, Hkv=w.Hkv, d=d, context=T, Bc=Bc, causal=True,
                                                points=rows)
        del x, o, lse, mask, own
        torch.cuda.empty_cache()
    return out


def bench_mla(args, lib, torch, W):
    """MLA decode split kernel at 32K context, with 64- and 32-token blocks: time, HBM bytes (the cache
    rows are read once), the executed FLOPs (S for every head and token; P V for the kept blocks of each
    head group) and the roofline bound by both HBM and MFMA."""
    w = W.MLA_CONFIGS["decode_mla_32k"]
    x = W.generate(w, parts=("q", "k"))
    q = dev(np.ascontiguousarray(x["q"][:, :, 0]))
    kvs = [dev(np.ascontiguousarray(x["k"][:, 0]))]
    kvs += [kvs[0].clone() for _ in range(kv_copies(args, kvs[0].nbytes) - 1)]
    del x
    B, Hq, N, dqk, dv, S = w.B, w.Hq, w.T, w.d, w.dv, w.num_splits
    stream = torch.cuda.current_stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    o_part = torch.empty((B, Hq, S, dv), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    hg = 64 if Hq % 64 == 0 else 32
    # the unit whose P V product a block skips only when every head in it skips: a 16-head
    # tile in the 64-head pipeline, the whole 32-head workgroup in the 32-head kernel
    tile = 16 if hg == 64 else 32
    # every (block size, lambda) case is run once for its decisions, then all are timed
    # interleaved (20 launches per case and round, the cache copies rotated)
    cases, fns = [], []
    for Bc in (w.Bc, 32):
        nk = -(-N // Bc)
        skip = torch.empty((B, Hq, nk), dtype=torch.uint8, device="cuda")
        for lam in (0.0,) + tuple(w.lambdas):
            args_ = [(P(q), P(kv), P(o_part), P(lse_part), P(skip), B, Hq, N, dqk, dv, Bc,
                      ctypes.c_double(w.score_scale), ctypes.c_double(lam), S, ctypes.c_void_p(stream.cuda_stream))
                     for kv in kvs]
            assert lib.blasst_decode_mla(*args_[0]) == 0
            torch.cuda.synchronize()
            cases.append((Bc, lam, skip.cpu().numpy().astype(bool)))

            def fn(args_=args_):
                for i in range(20):
                    assert lib.blasst_decode_mla(*args_[i % len(args_)]) == 0
            fns.append(fn)
    times = interleaved_trials(torch, stream, fns, 1)
    by_block = {}
    for (Bc, lam, sk), (med, lo, hi) in zip(cases, times):
        nk = -(-N // Bc)
        us, us_lo, us_hi = med * 1e3 / 20, lo * 1e3 / 20, hi * 1e3 / 20
        tile_kept = ~sk.reshape(B, Hq // tile, tile, nk).all(axis=2)  # P V formed for the tile
        rows = np.minimum(Bc, N - Bc * np.arange(nk))                  # tokens per block
        s_flops = 2.0 * dqk * N * Hq * B
        pv_flops = 2.0 * dv * tile * float((tile_kept * rows).sum())
        by = B * N * dqk * 2 + B * Hq * dqk * 2 + B * Hq * S * (dv + 1) * 4 + B * Hq * nk
        out = by_block.setdefault("Bc%d" % Bc, dict(heads_per_workgroup=hg, pv_skip_unit_heads=tile,
                                                     by_lambda={}))["by_lambda"]
        out["%g" % lam] = dict(us=round(us, 2), us_min=round(us_lo, 2), us_max=round(us_hi, 2),
                               GBs=round(by / us / 1e3, 1), frac_of_hbm_peak=round(by / us / 1e3 / HBM_PEAK_GBS, 4),
                               tflops_executed=round((s_flops + pv_flops) / us / 1e6, 1),
                               block_sparsity=round(float(sk.mean()), 5),
                               pv_skipped_fraction=round(1.0 - float(tile_kept.mean()), 5))
    for blk in by_block.values():
        dense = blk["by_lambda"]["0"]["us"]
        for v in blk["by_lambda"].values():
            v["speedup_vs_lambda0"] = round(dense / v["us"], 4)
    by = B * N * dqk * 2
    return dict(workload=w.name, B=B, Hq=Hq, d_qk=dqk, d_v=dv, context=N, num_splits=S, kv_copies_rotated=len(kvs),
                by_block=by_block,
                hbm_roofline_us=round(by / (HBM_PEAK_GBS * 1e3), 2),
                mfma_roofline_us_dense=round(2.0 * (dqk + dv) * N * Hq * B / (MFMA_BF16_PEAK_TFLOPS * 1e6), 2))


def cpu_model():
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_threads():
    """Threads for the oracle: the host's CPU share for one GPU (OMP_NUM_THREADS where the job
    sets it), never more than the CPUs this process may run on."""
    affinity = len(os.sched_getaffinity(0))
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "16"))
    except ValueError:
        share = 16
    return max(1, min(share, affinity))


def cpu_baseline(args, dres):
    import oracle
    w = dres["w"]
    x = dres["x"]
    threads = oracle_threads()
    oracle.decode(x["q"], x["k"], x["v"], w.Bc, w.lambdas[0], w.num_splits, threads=threads)  # warm
    n, t0 = 0, time.perf_counter()
    while True:
        r = oracle.decode(x["q"], x["k"], x["v"], w.Bc, w.lambdas[0], w.num_splits, threads=threads)
        oracle.combine(r["o_part_full"], r["lse_part_full"])
        n += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    per = el / n
    by = decode_bytes(w, r["vskip_full"])
    gbs = (by["split"] + by["combine"]) / per / 1e9
    # one thread: one decode_32k step, and the 1K prefill (all heads)
    t1 = time.perf_counter()
    oracle.decode(x["q"], x["k"], x["v"], w.Bc, w.lambdas[0], w.num_splits, threads=1)
    one_decode = time.perf_counter() - t1
    import workloads as W
    wp = W.CONFIGS["prefill_1k_tiny"]
    xp = W.generate(wp)
    t1 = time.perf_counter()
    oracle.prefill(xp["q"], xp["k"], xp["v"], wp.Bc, wp.lambdas[0], threads=1)
    one_prefill = time.perf_counter() - t1
    return dict(value=round(gbs, 4), unit="GB/s", cores=threads, kind="oracle",
                sample="full decode_32k step (all 32 heads, 16 splits) + combine, repeated %d times in %.1f s; "
                       "%.1f ms per step; one task per (sequence, query head, split): %d tasks on %d threads"
                       % (n, el, per * 1e3, w.B * w.Hq * w.num_splits, threads),
                threads=threads, host_logical_cpus=os.cpu_count(), affinity_cpus=len(os.sched_getaffinity(0)),
                omp_num_threads_env=os.environ.get("OMP_NUM_THREADS"),
                cpu_model=cpu_model(),
                single_thread_s={"decode_32k_step": round(one_decode, 3), "prefill_1k_tiny": round(one_prefill, 3)})


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_attention_flash_amd as bsa
    import workloads as W
    torch.cuda.set_device(0)
    lib = bsa._load()
    if args.profile_target:
        profile_target(args, lib, torch, W)
        return
    if args.length_sweep:
        say = lambda msg: print(msg, file=sys.stderr, flush=True)  # noqa: E731
        rep = {"decode": length_sweep("decode", W.SWEEP_LENGTHS, W.SWEEP_LENGTHS[:5], W, bsa, log=say),
               "prefill": length_sweep("prefill", W.SWEEP_LENGTHS, W.SWEEP_LENGTHS[:5], W, bsa, log=say)}
        print(json.dumps({"length_sweep": rep}), flush=True)
        return
    if args.speedup_curve:
        print(json.dumps({"speedup_curve": speedup_curve(args, lib, torch, W, bsa)}), flush=True)
        return

    d = bench_decode(args, lib, torch, W)
    pre = None if args.no_prefill else bench_prefill(args, lib, torch, W)
    mla = None if args.no_mla else bench_mla(args, lib, torch, W)
    configs = None
    if not args.no_other_configs:
        configs = {}
        for name in ("prefill_1k_tiny", "decode_128k_b16", "decode_mqa_16k"):
            configs[name] = bench_config(name, args, lib, torch, W)
            torch.cuda.empty_cache()
        configs["ragged"] = bench_ragged(args, lib, torch, W)
    sweep128 = None if args.no_length_sweep_timing else bench_decode_length_sweep(args, lib, torch, W, bsa)
    psweep128 = None if args.no_length_sweep_timing else bench_prefill_length_sweep(args, lib, torch, W, bsa)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, d)

    by = d["bytes"]
    step_bytes = by["split"] + by["combine"]
    value = step_bytes / (d["step_ms"] * 1e-3) / 1e9
    achieved = by["split"] / (d["split_ms"] * 1e-3) / 1e9
    w = d["w"]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "kind": "split-KV decode + LSE combine", "B": w.B, "Hq": w.Hq,
                   "Hkv": w.Hkv, "d": w.d, "context": w.T, "Bc": w.Bc, "lambda": w.lambdas[0],
                   "num_splits": w.num_splits, "kv_copies_rotated": d["kv_copies_rotated"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode_split_kernel", w.name),
                     "kernel": "decode_split_kernel", "bytes_per_launch": by["split"],
                     "avg_launch_us": round(d["split_ms"] * 1e3, 3)},
        "decode": {"step_us": round(d["step_ms"] * 1e3, 3), "split_kernel_us": round(d["split_ms"] * 1e3, 3),
                   "split_kernel_trials_us": {"n": len(d["split_trials_ms"]),
                                              "min": round(min(d["split_trials_ms"]) * 1e3, 3),
                                              "median": round(d["split_ms"] * 1e3, 3),
                                              "max": round(max(d["split_trials_ms"]) * 1e3, 3)},
                   "lambda0_step_us": round(d["lambda0_step_ms"] * 1e3, 3),
                   "speedup_vs_lambda0": round(d["lambda0_step_ms"] / d["step_ms"], 4),
                   "dense_kernel_step_us": round(d["dense_step_ms"] * 1e3, 3),
                   "dense_kernel_us": round(d["dense_kernel_ms"][0] * 1e3, 3),
                   "load_ceiling_us": round(d["load_ceiling_ms"][0] * 1e3, 3),
                   "load_ceiling_GBs_on_kv_bytes": round((by["k"] + by["v_dense"]) / (d["load_ceiling_ms"][0] * 1e-3)
                                                          / 1e9, 1),
                   "split_kernel_over_load_ceiling": round(d["split_ms"] / d["load_ceiling_ms"][0], 4),
                   "speedup_vs_dense_kernel_step": round(d["dense_step_ms"] / d["step_ms"], 4),
                   "lambda0_speed_vs_dense_kernel_step": round(d["dense_step_ms"] / d["lambda0_step_ms"], 4),
                   "block_sparsity": round(d["block_sparsity"], 5), "vload_sparsity": round(d["vload_sparsity"], 5),
                   "bytes": by, "lambda_sweep": d["lambda_sweep"]},
        "prefill": pre,
        "mla_decode": mla,
        "other_configs": configs,
        "decode_length_sweep_128k": sweep128,
        "prefill_length_sweep_128k": psweep128,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
