#!/usr/bin/env python3
"""Benchmark of the gated delta rule chunked prefill forward on one MI355X.

Workload: one 32768-token sequence, 8 heads (one GPU's share of a 64-head layer under 8-way
tensor parallelism), d_k = d_v = 128, bf16 q/k/v/beta/o, fp32 g and state, chunk 64: the
single-sequence 32K prefill of "How to Speed Up GDN Kernels for Qwen Models", section "What it
adds up to".  Inputs are seeded synthetic values (gdn_inputs.py), resident in HBM before the
timed region.  Three input sets of the same shape rotate between steps so the 256 MB last-level
cache cannot serve a repeated working set.

A step is one forward (gdn_chunk_fwd: o and the final state) on the current stream.  The
on-device peaks are measured once the inputs are on the device, right before the timed forward
(which also brings the card to its sustained clock); then W warmup steps run, and exactly K steps are timed on that stream between device
synchronisations, with HIP events only between windows of 5 back-to-back steps.  ``value`` is
tokens per second at the median window's time per step (``ms_per_step``), in the headline mode
(the page's truncated-history split, section "Lever 1"); the exact mode is timed the same way and
reported beside it, so is the same forward with q and k L2-normalised inside the kernel (object
``qk_l2norm``), the forward on the pages' other workloads (object ``workloads``: the 8192-token
packed batch, the fork's 65536-token prefix and its 80 branches, the 65536-token training
batch), the training backward (object ``backward``) and the single-token decode step (object
``decode``).

``roofline``: the forward is bound by HBM bandwidth (about 176 flop per byte against the
MI355X's ~315 flop/byte ridge).  Algorithmic bytes per launch = 1030 B per (token, head)
(q, k, v, o in bf16, g in fp32, beta in bf16) + 64 KiB per (sequence, head) of final state.
``achieved`` = those bytes / the average launch duration over the whole timed region (one
launch per step; ``timing.mean_ms``); ``peak`` is the 8 TB/s HBM3E datasheet figure.
``traffic`` is the measured HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs
recorded in profiles/ (null when not measured for the current kernel).  ``roofline.median``
holds %HBM, %MFMA and the roofline fraction max(B / bandwidth, F / rate) / t at the median time
against the datasheet peaks, ``roofline.median_vs_measured_peaks`` the same against
``measured_peaks`` (the library's stream copy of 1 GiB and its loop of bf16 MFMAs, timed on this
GPU).  ``timing.host_call_us`` is the host's wall time for one call after a device
synchronisation (argument checks, segment planning, launches).

``cpu_baseline``: the fp64 token-recurrent oracle (plain C built with gcc -O2 -fopenmp, as for
the tests; OpenMP over (sequence, head) pairs) timed on this host on the same workload (8
(sequence, head) units, so at most 8 threads), and with one thread on two of the heads, scaled
to eight.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FLOP_PER_TH = 181_589        # chunked-form matrix products per (token, head), d = 128
BYTES_PER_TH = 4 * 256 + 4 + 2
BWD_BYTES_PER_TH = 7 * 256 + 2 * 4 + 2 * 2  # q k v dO dq dk dv (bf16), g dg (fp32), beta dbeta
STATE_BYTES = 128 * 128 * 4
PAGE_H200_MS = 0.31          # the page's FlashQLA figure for this workload (H200; context only)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_long32k.json")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bwd_train65k.json")
BWD_SOURCES = ("gdn_bwd_chain.hip", "gdn_bwd_grad.hip", "gdn_fwd_split.hip", "gdn_fwd_ws.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 200 timed steps (40 windows of 5, about 15 ms on the headline): the median window is then
    # taken over the card's sustained clock rather than a few milliseconds of it
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps before the timed ones (after the on-device peak "
                         "measurements, which bring the card to its sustained clock)")
    ap.add_argument("--sets", type=int, default=3, help="input sets rotated between steps")
    ap.add_argument("--mode", choices=["truncate", "exact", "both"], default="both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-l2norm", action="store_true",
                    help="skip the forward and backward timed with q/k L2 normalisation")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the on-device copy and bf16 matmul peak measurements")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training backward and the decode step timed beside the "
                         "forward")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the forward on the pages' other workloads")
    ap.add_argument("--only", choices=["truncate", "exact", "workloads", "backward",
                                       "backward_truncate", "decode"],
                    default=None,
                    help="profiling aid: run only this path (after the same warmup) and print its "
                         "object alone, not the benchmark line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device copies of MIB MiB each (reads and writes MIB MiB per "
                         "launch): the reference for scaling HBM traffic counters, then exit")
    return ap.parse_args()


def time_steps(gdn, torch, sets, mode, steps, warmup, qk_l2norm=False):
    outs = [torch.empty_like(s["v"]) for s in sets]
    hts = [torch.empty((1, 8, 128, 128), dtype=torch.float32, device="cuda") for _ in sets]
    cu_host = [0, sets[0]["q"].shape[0]]

    def step(i):
        s = sets[i % len(sets)]
        gdn.chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu_seqlens"], None,
                      mode=mode, cu_seqlens_host=cu_host, out=outs[i % len(sets)],
                      final_state=hts[i % len(sets)], qk_l2norm=qk_l2norm)

    return timed(torch, step, steps, warmup)


def timed(torch, step, steps, warmup, window=5):
    """Times ``step(i)``: ``warmup`` untimed calls, then exactly ``steps`` calls on the current
    stream between device synchronisations.  Events are recorded only between windows of
    ``window`` back-to-back calls (one before the first call, one after each window), so each
    window's calls run back to back as in a real sequence of calls.  ``mean_ms`` is the whole
    timed region over ``steps``; ``median_ms``, ``p10_ms`` and ``p90_ms`` are over the windows'
    per-call means."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    sizes = [min(window, steps - i) for i in range(0, steps, window)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sizes) + 1)]
    ev[0].record(stream)
    i = 0
    for w, n in enumerate(sizes):
        for _ in range(n):
            step(warmup + i)
            i += 1
        ev[w + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[w].elapsed_time(ev[w + 1]) / n for w, n in enumerate(sizes)])
    return {"mean_ms": ev[0].elapsed_time(ev[-1]) / steps, "median_ms": float(np.median(per)),
            "p10_ms": float(np.percentile(per, 10)), "p90_ms": float(np.percentile(per, 90)),
            "windows": len(sizes), "window_calls": window}


def host_call_us(torch, step, calls=20):
    """Host wall time of one call after a device synchronisation (argument checks, planning and
    kernel launches; the GPU work itself runs asynchronously): the median over ``calls``."""
    out = []
    for i in range(calls):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step(i)
        out.append((time.perf_counter() - t0) * 1e6)
    torch.cuda.synchronize()
    return float(np.median(out))


def measured_peaks(gdn, torch):
    """Peaks measured on this GPU, beside the datasheet ones: the HBM bandwidth of the library's
    stream-copy kernel on 1 GiB (read + write bytes over the time; torch's copy beside it) and the
    bf16 matrix-core rate of its register-resident MFMA loop (an 8192^3 torch.matmul beside it)."""
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t = timed(torch, lambda i: gdn.calib_copy(src, dst), 20, 3)
    hbm = 2 * n * 4 / (t["median_ms"] / 1e3) / 1e9
    assert torch.equal(dst[:: 1 << 16], src[:: 1 << 16])
    t = timed(torch, lambda i: dst.copy_(src), 20, 3)
    hbm_torch = 2 * n * 4 / (t["median_ms"] / 1e3) / 1e9
    del src, dst
    out = torch.empty(8 * 256 * 64, dtype=torch.float32, device="cuda")
    mfma = {}
    for w in (4, 8):
        flops = gdn.calib_mfma_bf16(out, w, 2000)
        t = timed(torch, lambda i: gdn.calib_mfma_bf16(out, w, 2000), 10, 2)
        mfma[w] = flops / (t["median_ms"] / 1e3) / 1e12
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    c = torch.empty(m, m, device="cuda", dtype=torch.bfloat16)
    t = timed(torch, lambda i: torch.matmul(a, b, out=c), 20, 3)
    gemm = 2 * m ** 3 / (t["median_ms"] / 1e3) / 1e12
    return {"hbm_GBps": hbm,
            "hbm_how": "gdn_calib_copy stream copy of 1 GiB (read + write), median of 20",
            "hbm_torch_copy_GBps": hbm_torch,
            "bf16_TFLOPs": max(mfma.values()),
            "bf16_how": "gdn_calib_mfma_bf16 (4 independent v_mfma_f32_32x32x16_bf16 chains per "
                        "wave, 4 and 8 waves per CU, the better), median of 10",
            "bf16_gemm_torch_TFLOPs": gemm}


def cpu_baseline(inp):
    import oracle

    cores = os.cpu_count() or 1
    units = 8  # one sequence x 8 heads
    threads = min(units, cores)
    args = [inp[x] for x in ("q", "k", "v", "g", "beta")]
    T = inp["q"].shape[0]
    t0 = time.perf_counter()
    oracle.fwd_recurrent(*args, inp["cu_seqlens"], nthreads=threads)
    dt = time.perf_counter() - t0
    t0 = time.perf_counter()  # one thread on two of the eight heads
    oracle.fwd_recurrent(*[np.ascontiguousarray(a[:, :2]) for a in args], inp["cu_seqlens"],
                         nthreads=1)
    dt1 = (time.perf_counter() - t0) * 4
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         "")
    except OSError:
        pass
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "build": "gcc -O2 -fopenmp (the oracle as built for the tests, not tuned)",
            "sample": f"full workload: 1 x {T} tokens x 8 heads, fp64 token recurrence, "
                      f"{dt:.2f} s wall on {threads} of {cores} host threads",
            "one_thread_tokens_per_s": T / dt1,
            "one_thread_sample": f"1 thread on heads 0-1 of the same input, {dt1 / 4:.2f} s, "
                                 "scaled to 8 heads",
            "nproc": cores, "cpu_model": model}


def copy_calibration(mib):
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "launches": 5}), flush=True)
    return 0


def main():
    args = parse()
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (--gpus {args.gpus} "
              "not supported; heads and documents shard across GPUs without communication).",
              file=sys.stderr)
        return 2
    if args.only:
        return only_path(args)
    import torch

    from gdn_inputs import workload
    import linear_attention_recurrence_prefill_amd as gdn

    gdn.load_library()
    inp = workload("long")
    T, H, D = inp["q"].shape
    tdt = torch.bfloat16

    def dev(x, dt=None):
        t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        return t.to(dt) if dt is not None else t

    base = {n: dev(inp[n], tdt) for n in ("q", "k", "v", "beta")}
    base["g"] = dev(inp["g"])
    base["cu_seqlens"] = dev(inp["cu_seqlens"])
    sets = [base]
    for j in range(1, args.sets):  # same values shifted along the sequence: distinct memory
        sets.append({n: (torch.roll(t, shifts=4096 * j, dims=0).contiguous()
                         if n != "cu_seqlens" else t) for n, t in base.items()})
    torch.cuda.synchronize()
    # the peak measurements run right before the timed forward (inputs already on the device), so
    # the card enters the timed region at its sustained clock rather than after an idle spell
    peaks = None if args.no_measured_peaks else measured_peaks(gdn, torch)

    results = {}
    modes = ["truncate", "exact"] if args.mode == "both" else [args.mode]
    for m in modes:
        results[m] = time_steps(gdn, torch, sets, m, args.steps, args.warmup)
    head = modes[0]
    r = results[head]
    ms = r["median_ms"]
    value = T / (ms / 1e3)
    bytes_launch = BYTES_PER_TH * T * H + STATE_BYTES * H
    flops_launch = FLOP_PER_TH * T * H
    achieved = bytes_launch / (r["mean_ms"] / 1e3) / 1e9  # over the average launch duration
    cu_host = [0, T]
    host_us = host_call_us(torch, lambda i: gdn.chunk_fwd(
        sets[0]["q"], sets[0]["k"], sets[0]["v"], sets[0]["g"], sets[0]["beta"],
        sets[0]["cu_seqlens"], None, mode=head, cu_seqlens_host=cu_host))
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        if rec.get("kernel_source_sha") == kernel_source_sha():
            traffic = rec.get("bytes_per_launch")
    line = {
        "metric": "GDN fwd tokens/s at 32K tok, 8 heads, d=128 bf16; % of MFMA/HBM roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        # the pages' FlashQLA time for this exact workload (H200): context, not a target
        "vs_baseline": value / (T / (PAGE_H200_MS / 1e3)),
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), g=-softplus(N(-3,1)), "
                "beta=sigmoid(N(0,1)))",
        "config": {"workload": "single-sequence prefill, 1 x 32768 tokens, H=8, d_k=d_v=128, "
                               "chunk 64, bf16 inputs, fp32 state",
                   "mode": head, "global_batch": 1, "seq_len": T, "heads": H,
                   "head_dim": D, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "mfma_frac": flops_launch / (r["mean_ms"] / 1e3) / 1e12
                     / BF16_MFMA_PEAK_TFLOPS,
                     "bytes_per_launch": bytes_launch, "flops_per_launch": flops_launch},
        "timing": dict(r, host_call_us=host_us),
        "context": {"page_h200_ms": PAGE_H200_MS,
                    "note": "the pages' FlashQLA time for this workload on an H200 (other "
                            "hardware, other kernels): context, not a baseline"},
    }
    line["roofline"].update(fractions(ms, bytes_launch, flops_launch, peaks))
    if peaks is not None:
        line["measured_peaks"] = peaks
    for m in modes[1:]:
        rm = results[m]
        line[f"{m}_mode"] = {"ms_per_step": rm["median_ms"],
                             "value": T / (rm["median_ms"] / 1e3),
                             "roofline_frac": bytes_launch / (rm["mean_ms"] / 1e3) / 1e9
                             / HBM_PEAK_GBS, "timing": rm,
                             **fractions(rm["median_ms"], bytes_launch, flops_launch, peaks)}
    if not args.no_l2norm:
        rn = time_steps(gdn, torch, sets, head, args.steps, args.warmup, qk_l2norm=True)
        line["qk_l2norm"] = {"mode": head, "ms_per_step": rn["median_ms"],
                             "value": T / (rn["median_ms"] / 1e3),
                             "roofline_frac": bytes_launch / (rn["mean_ms"] / 1e3) / 1e9
                             / HBM_PEAK_GBS, "timing": rn}
    del sets, base
    if not args.no_workloads:
        line["workloads"] = time_workloads(gdn, torch, args.steps, args.warmup)
    if not args.no_backward:
        line["backward"] = time_backward(gdn, torch, args.steps, args.warmup,
                                         with_l2norm=not args.no_l2norm)
        line["decode"] = time_decode(gdn, torch, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)
    return 0


def only_path(args):
    """One path alone, for profiling runs (rocprofv3 attributes every kernel of the run to it)."""
    import torch

    from gdn_inputs import workload
    import linear_attention_recurrence_prefill_amd as gdn

    gdn.load_library()
    out = {"only": args.only}
    if args.only in ("truncate", "exact"):
        inp = workload("long")
        base = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).cuda().to(torch.bfloat16)
                for n in ("q", "k", "v", "beta")}
        base["g"] = torch.from_numpy(inp["g"]).cuda()
        base["cu_seqlens"] = torch.from_numpy(inp["cu_seqlens"]).cuda()
        sets = [base] + [{n: (torch.roll(t, shifts=4096 * j, dims=0).contiguous()
                              if n != "cu_seqlens" else t) for n, t in base.items()}
                         for j in range(1, args.sets)]
        out["timing"] = time_steps(gdn, torch, sets, args.only, args.steps, args.warmup)
    elif args.only == "workloads":
        out["workloads"] = time_workloads(gdn, torch, args.steps, args.warmup)
    elif args.only == "backward":
        out["backward"] = time_backward(gdn, torch, args.steps, args.warmup, with_l2norm=False,
                                        with_truncate=False)
    elif args.only == "backward_truncate":
        out["backward"] = time_backward(gdn, torch, args.steps, args.warmup, with_l2norm=False,
                                        with_exact=False)
    else:
        out["decode"] = time_decode(gdn, torch, args.steps, args.warmup)
    print(json.dumps(out), flush=True)
    return 0


def synth(torch, lengths, H, D, seed, sets=1):
    """Seeded synthetic inputs drawn on the GPU with the recipe of gdn_inputs.py (q, k rows
    L2-normalised N(0, 1), v ~ N(0, 1), g = -softplus(N(-3, 1)) fp32, beta = sigmoid(N(0, 1)),
    bf16), ``sets`` independent draws over the same documents: timing inputs only (the parity
    tests draw theirs with numpy)."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    T = int(sum(lengths))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device="cuda")
    out = []
    for _ in range(sets):
        q = torch.nn.functional.normalize(torch.randn(T, H, D, device="cuda", generator=gen), dim=-1)
        k = torch.nn.functional.normalize(torch.randn(T, H, D, device="cuda", generator=gen), dim=-1)
        v = torch.randn(T, H, D, device="cuda", generator=gen)
        g = -torch.nn.functional.softplus(torch.randn(T, H, device="cuda", generator=gen) - 3.0)
        beta = torch.sigmoid(torch.randn(T, H, device="cuda", generator=gen))
        out.append({"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16),
                    "v": v.to(torch.bfloat16), "g": g.contiguous(),
                    "beta": beta.to(torch.bfloat16), "cu_seqlens": cu})
    return out


def time_workloads(gdn, torch, steps, warmup):
    """The exact forward on the pages' other workloads, timed like the headline (windows of
    back-to-back calls; tokens/s at the median; the HBM roofline fraction on the algorithmic
    bytes at the average launch time).  Algorithmic bytes: 1030 B per (token, head), plus 64 KiB
    per (sequence, head) for the final state and again for an initial state.  Input sets rotate
    where one set would fit in the 256 MB last-level cache."""
    from gdn_inputs import workload_shape

    res = {}

    def one(name, desc, lengths, H, sets, h0=None):
        N = len(lengths)
        T = int(sum(lengths))
        outs = [(torch.empty_like(s["v"]), torch.empty((N, H, 128, 128), device="cuda"))
                for s in sets]
        cu_host = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)

        def step(i):
            s = sets[i % len(sets)]
            o, ht = outs[i % len(sets)]
            gdn.chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu_seqlens"], h0,
                          mode="exact", cu_seqlens_host=cu_host, out=o, final_state=ht)

        r = timed(torch, step, steps, warmup)
        nbytes = BYTES_PER_TH * T * H + STATE_BYTES * H * N * (2 if h0 is not None else 1)
        nflops = FLOP_PER_TH * T * H
        res[name] = {"workload": desc, "mode": "exact", "tokens": T, "documents": N, "heads": H,
                     "input_sets": len(sets), "ms_per_step": r["median_ms"],
                     "tokens_per_s": T / (r["median_ms"] / 1e3),
                     "roofline": {"bound": "hbm", "bytes_per_launch": nbytes,
                                  "achieved_GBps": nbytes / (r["mean_ms"] / 1e3) / 1e9,
                                  "frac": nbytes / (r["mean_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                                  "mfma_frac": nflops / (r["mean_ms"] / 1e3) / 1e12
                                  / BF16_MFMA_PEAK_TFLOPS},
                     "timing": r}
        return outs[0]

    w = workload_shape("packed")
    sets = synth(torch, w["lengths"], w["H"], w["d"], 11, sets=4)
    one("packed_8k", "8192 tokens packed from U{256..2048}-token documents, H=8, d=128, bf16 "
        "(4 input sets rotated: one set is 72 MB)", w["lengths"], w["H"], sets)
    w = workload_shape("train")
    sets = synth(torch, w["lengths"], w["H"], w["d"], 12)
    one("train_65k_forward", "65536 tokens packed from U{4096..16384}-token documents, H=8, "
        "d=128, bf16 (the training batch's forward)", w["lengths"], w["H"], sets)
    w = workload_shape("fork")
    pre = synth(torch, [w["prefix_len"]], w["H"], w["d"], 13)
    _, ht = one("fork_prefix_64k", "fork prefix: 1 x 65536 tokens, H=16, d=128, bf16",
                [w["prefix_len"]], w["H"], pre)
    del pre
    shared = ht[0].contiguous()
    br = synth(torch, w["lengths"], w["H"], w["d"], 14)
    one("fork_branches", f"fork branches: {len(w['lengths'])} documents of U{{1024..4096}} "
        f"tokens ({sum(w['lengths'])} in all) packed, every one starting from the prefix's "
        "final state (broadcast), H=16, d=128, bf16", w["lengths"], w["H"], br, h0=shared)
    return res


def fractions(median_ms, nbytes, nflops, peaks):
    """The four figures of the roofline at the median time: %HBM = bytes / (t * peak bandwidth),
    %MFMA = flops / (t * peak bf16 rate), and the roofline fraction max(bytes / bandwidth,
    flops / rate) / t, against the datasheet peaks and (when measured) this GPU's."""
    t = median_ms / 1e3
    out = {"median": {"hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBS,
                      "mfma_frac": nflops / t / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                      "roofline_frac": max(nbytes / 1e9 / HBM_PEAK_GBS,
                                           nflops / 1e12 / BF16_MFMA_PEAK_TFLOPS) / t}}
    if peaks is not None:
        out["median_vs_measured_peaks"] = {
            "hbm_frac": nbytes / t / 1e9 / peaks["hbm_GBps"],
            "mfma_frac": nflops / t / 1e12 / peaks["bf16_TFLOPs"],
            "roofline_frac": max(nbytes / 1e9 / peaks["hbm_GBps"],
                                 nflops / 1e12 / peaks["bf16_TFLOPs"]) / t}
    return out


def time_decode(gdn, torch, steps, warmup, sets=6):
    """One decode step (gdn_decode_step) on the fork workload's serving shape: 80 sequences x
    16 heads, d = 128, bf16 inputs, fp32 states updated in place.  ``sets`` independent state
    sets (84 MB each) rotate between steps, so the working set (504 MB for six) exceeds the
    256 MB last-level cache and each step reads its states from HBM.  Algorithmic bytes per
    step: every state read and written once (2 x 64 KiB), q, k, v, o in bf16, g fp32, beta
    bf16."""
    B, H, D = 80, 16, 128
    gen = torch.Generator(device="cuda").manual_seed(7)
    data = []
    for _ in range(sets):
        q = torch.nn.functional.normalize(torch.randn(B, H, D, device="cuda", generator=gen),
                                          dim=-1).to(torch.bfloat16)
        k = torch.nn.functional.normalize(torch.randn(B, H, D, device="cuda", generator=gen),
                                          dim=-1).to(torch.bfloat16)
        v = torch.randn(B, H, D, device="cuda", generator=gen).to(torch.bfloat16)
        g = -torch.nn.functional.softplus(torch.randn(B, H, device="cuda", generator=gen) - 3.0)
        beta = torch.sigmoid(torch.randn(B, H, device="cuda", generator=gen)).to(torch.bfloat16)
        state = 0.1 * torch.randn(B, H, D, D, device="cuda", generator=gen)
        data.append((q, k, v, g, beta, state, torch.empty_like(v)))

    def step(i):
        q, k, v, g, beta, state, out = data[i % sets]
        gdn.decode_step(q, k, v, g, beta, state, out=out)

    r = timed(torch, step, steps, warmup)
    nbytes = B * H * (2 * D * D * 4 + 4 * D * 2 + 4 + 2)
    achieved = nbytes / (r["mean_ms"] / 1e3) / 1e9
    return {"workload": f"{B} sequences x {H} heads, d_k=d_v={D}, bf16 inputs, fp32 state "
                        f"({sets} state sets rotated, {sets * B * H * D * D * 4 / 1e6:.0f} MB)",
            "us_per_step": r["median_ms"] * 1e3, "tokens_per_s": B / (r["median_ms"] / 1e3),
            "timing": r,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "bytes_per_step": nbytes}}


def time_backward(gdn, torch, steps, warmup, with_l2norm=True, with_exact=True,
                  with_truncate=True):
    """The training step's backward (gdn_chunk_bwd: forward recompute, reverse chain, per-chunk
    gradients) on the packed 65536-token workload of 4096..16384-token documents, H = 8, d = 128,
    bf16, dO ~ N(0, 1), timed like the forward: the exact mode, and beside it the truncate mode.  Algorithmic bytes: q, k, v, dO read and dq, dk,
    dv written in bf16, g read and dg written in fp32, beta read and dbeta written in bf16."""
    from gdn_inputs import workload

    inp = workload("train")
    T, H, D = inp["q"].shape
    dev = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).cuda()
           for n in ("q", "k", "v", "beta", "dout")}
    for n in dev:
        dev[n] = dev[n].to(torch.bfloat16)
    g = torch.from_numpy(inp["g"]).cuda()
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    import ctypes

    from linear_attention_recurrence_prefill_amd.gdn import make_problem

    p = make_problem(T, len(inp["cu_seqlens"]) - 1, H, D, torch.bfloat16, "exact")
    cu_host = inp["cu_seqlens"]
    cu_arr = (ctypes.c_int32 * len(cu_host))(*[int(x) for x in cu_host])
    nbytes = ctypes.c_size_t(0)
    assert gdn.load_library().gdn_chunk_bwd_workspace_size(ctypes.byref(p), cu_arr,
                                                           ctypes.byref(nbytes)) == 0
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device="cuda")  # allocated once, outside

    def step(i):
        gdn.chunk_bwd(dev["q"], dev["k"], dev["v"], g, dev["beta"], cu, dev["dout"], workspace=ws,
                      cu_seqlens_host=cu_host)

    r = timed(torch, step, steps, warmup) if with_exact else None
    ms = r["median_ms"] if r else None
    rt = None
    if with_truncate:  # the truncate mode's backward (warmup windows instead of the extra passes)
        pt = make_problem(T, len(inp["cu_seqlens"]) - 1, H, D, torch.bfloat16, "truncate")
        assert gdn.load_library().gdn_chunk_bwd_workspace_size(ctypes.byref(pt), cu_arr,
                                                               ctypes.byref(nbytes)) == 0
        wst = torch.empty(nbytes.value, dtype=torch.uint8, device="cuda")
        rt = timed(torch, lambda i: gdn.chunk_bwd(dev["q"], dev["k"], dev["v"], g, dev["beta"], cu,
                                                  dev["dout"], workspace=wst, mode="truncate",
                                                  cu_seqlens_host=cu_host),
                   steps, warmup)
    rn = None
    if with_l2norm:  # the same backward with q and k normalised inside the kernels
        pn = make_problem(T, len(inp["cu_seqlens"]) - 1, H, D, torch.bfloat16, "exact",
                          qk_l2norm=True)
        assert gdn.load_library().gdn_chunk_bwd_workspace_size(ctypes.byref(pn), cu_arr,
                                                               ctypes.byref(nbytes)) == 0
        wsn = torch.empty(nbytes.value, dtype=torch.uint8, device="cuda")
        rn = timed(torch, lambda i: gdn.chunk_bwd(dev["q"], dev["k"], dev["v"], g, dev["beta"],
                                                  cu, dev["dout"], workspace=wsn, qk_l2norm=True,
                                                  cu_seqlens_host=cu_host),
                   steps, warmup)
    nbytes_alg = BWD_BYTES_PER_TH * T * H
    out = {"workload": f"packed {T} tokens ({len(inp['cu_seqlens']) - 1} documents of "
                       f"4096..16384), H={H}, d_k=d_v={D}, bf16, dO ~ N(0,1)",
           "qk_l2norm_ms_per_step": rn["median_ms"] if rn else None}
    if r:
        achieved = nbytes_alg / (r["mean_ms"] / 1e3) / 1e9
        traffic = None  # measured HBM bytes per call (rocprofv3), while the kernels are unchanged
        if os.path.exists(BWD_TRAFFIC_FILE):
            with open(BWD_TRAFFIC_FILE) as f:
                rec = json.load(f)
            if rec.get("kernel_source_sha") == kernel_source_sha(BWD_SOURCES):
                traffic = rec.get("bytes_per_call")
        out.update({"ms_per_step": ms, "tokens_per_s": T / (ms / 1e3), "timing": r,
                    "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                                 "bytes_per_step": nbytes_alg, "traffic": traffic}})
    if rt:
        out["truncate"] = {"ms_per_step": rt["median_ms"],
                           "tokens_per_s": T / (rt["median_ms"] / 1e3), "timing": rt,
                           "roofline_frac": nbytes_alg / (rt["median_ms"] / 1e3) / 1e9
                           / HBM_PEAK_GBS}
    return out


def kernel_source_sha(sources=("gdn_fwd_ws.hip",)):
    """Hash of the timed kernels' translation units (by default gdn_fwd_ws.hip) and the csrc
    headers they include, followed recursively, and of the compiler flags build.py gives them.
    Changes to other kernels leave it, and so the stored traffic figure, valid."""
    import hashlib

    from linear_attention_recurrence_prefill_amd import build as b

    csrc = b.CSRC
    seen, todo = [], list(sources)
    while todo:
        name = todo.pop(0)
        if name in seen or not os.path.exists(os.path.join(csrc, name)):
            continue
        seen.append(name)
        with open(os.path.join(csrc, name)) as f:
            todo += re.findall(r'^#include "([^"]+)"', f.read(), flags=re.M)
    h = hashlib.sha256()
    for name in sorted(seen):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    extra = (b.EXTRA_FLAGS.get(sources[0], []) if len(sources) == 1
             else [b.EXTRA_FLAGS.get(x, []) for x in sources])
    h.update(repr((b.HIP_FLAGS, extra)).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
