#!/usr/bin/env python3
"""Benchmark of the gated delta rule chunked prefill forward on one MI355X.

Workload: one 32768-token sequence, 8 heads (one GPU's share of a 64-head layer under 8-way
tensor parallelism), d_k = d_v = 128, bf16 q/k/v/beta/o, fp32 g and state, chunk 64: the
single-sequence 32K prefill of "How to Speed Up GDN Kernels for Qwen Models", section "What it
adds up to".  Inputs are seeded synthetic values (gdn_inputs.py), resident in HBM before the
timed region.  Three input sets of the same shape rotate between steps so the 256 MB last-level
cache cannot serve a repeated working set.

A step is one forward (gdn_chunk_fwd: o and the final state) on the current stream.  W warmup
steps run first; then exactly K steps are timed with HIP events on that stream, bracketed by
device synchronisations.  ``value`` is tokens per second of the headline mode (the page's
truncated-history split, section "Lever 1"); the exact mode is timed the same way and reported
beside it, and so is the training backward (gdn_chunk_bwd on the packed 65536-token workload of
the pages' training runs, object ``backward`` with its own HBM roofline fraction) and the
single-token decode step (object ``decode``).

``roofline``: the forward is bound by HBM bandwidth (about 176 flop per byte against the
MI355X's ~315 flop/byte ridge).  Algorithmic bytes per launch = 1030 B per (token, head)
(q, k, v, o in bf16, g in fp32, beta in bf16) + 64 KiB per (sequence, head) of final state.
``achieved`` = those bytes / the measured time per launch (one launch per step); ``peak`` is the
8 TB/s HBM3E datasheet figure.  ``traffic`` is the measured HBM bytes per launch from the
rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in profiles/ (null when not measured for the
current kernel).

``cpu_baseline``: the fp64 token-recurrent oracle (plain C, OpenMP over (sequence, head) pairs)
timed on this host on the same workload (8 (sequence, head) units, so at most 8 threads).
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


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=3, help="input sets rotated between steps")
    ap.add_argument("--mode", choices=["truncate", "exact", "both"], default="both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training backward timed beside the forward")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device copies of MIB MiB each (reads and writes MIB MiB per "
                         "launch): the reference for scaling HBM traffic counters, then exit")
    return ap.parse_args()


def time_steps(gdn, torch, sets, mode, steps, warmup):
    outs = [torch.empty_like(s["v"]) for s in sets]
    hts = [torch.empty((1, 8, 128, 128), dtype=torch.float32, device="cuda") for _ in sets]
    cu_host = [0, sets[0]["q"].shape[0]]

    def step(i):
        s = sets[i % len(sets)]
        gdn.chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu_seqlens"], None,
                      mode=mode, cu_seqlens_host=cu_host, out=outs[i % len(sets)],
                      final_state=hts[i % len(sets)])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


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
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"full workload: 1 x {T} tokens x 8 heads, fp64 token recurrence, "
                      f"{dt:.2f} s wall on {threads} of {cores} host threads"}


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

    results = {}
    modes = ["truncate", "exact"] if args.mode == "both" else [args.mode]
    for m in modes:
        ms = time_steps(gdn, torch, sets, m, args.steps, args.warmup)
        results[m] = ms
    head = modes[0]
    ms = results[head]
    value = T / (ms / 1e3)
    bytes_launch = BYTES_PER_TH * T * H + STATE_BYTES * H
    flops_launch = FLOP_PER_TH * T * H
    achieved = bytes_launch / (ms / 1e3) / 1e9
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
                     "mfma_frac": flops_launch / (ms / 1e3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                     "bytes_per_launch": bytes_launch, "flops_per_launch": flops_launch},
    }
    for m in modes[1:]:
        line[f"{m}_mode"] = {"ms_per_step": results[m], "value": T / (results[m] / 1e3),
                             "roofline_frac": bytes_launch / (results[m] / 1e3) / 1e9
                             / HBM_PEAK_GBS}
    if not args.no_backward:
        line["backward"] = time_backward(gdn, torch, args.steps, args.warmup)
        line["decode"] = time_decode(gdn, torch, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)
    return 0


def time_decode(gdn, torch, steps, warmup):
    """One decode step (gdn_decode_step) on the fork workload's serving shape: 80 sequences x
    16 heads, d = 128, bf16 inputs, fp32 states updated in place.  Algorithmic bytes per step:
    every state read and written once (2 x 64 KiB), q, k, v, o in bf16, g fp32, beta bf16."""
    B, H, D = 80, 16, 128
    gen = torch.Generator(device="cuda").manual_seed(7)
    q = torch.nn.functional.normalize(torch.randn(B, H, D, device="cuda", generator=gen), dim=-1)
    k = torch.nn.functional.normalize(torch.randn(B, H, D, device="cuda", generator=gen), dim=-1)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    v = torch.randn(B, H, D, device="cuda", generator=gen).to(torch.bfloat16)
    g = -torch.nn.functional.softplus(torch.randn(B, H, device="cuda", generator=gen) - 3.0)
    beta = torch.sigmoid(torch.randn(B, H, device="cuda", generator=gen)).to(torch.bfloat16)
    state = 0.1 * torch.randn(B, H, D, D, device="cuda", generator=gen)
    out = torch.empty_like(v)

    def step():
        gdn.decode_step(q, k, v, g, beta, state, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    nbytes = B * H * (2 * D * D * 4 + 4 * D * 2 + 4 + 2)
    achieved = nbytes / (ms / 1e3) / 1e9
    return {"workload": f"{B} sequences x {H} heads, d_k=d_v={D}, bf16 inputs, fp32 state",
            "us_per_step": ms * 1e3, "tokens_per_s": B / (ms / 1e3),
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "bytes_per_step": nbytes}}


def time_backward(gdn, torch, steps, warmup):
    """The training step's backward (gdn_chunk_bwd: forward recompute, reverse chain, per-chunk
    gradients) on the packed 65536-token workload of 4096..16384-token documents, H = 8, d = 128,
    bf16, dO ~ N(0, 1), timed like the forward.  Algorithmic bytes: q, k, v, dO read and dq, dk,
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
    nbytes = ctypes.c_size_t(0)
    assert gdn.load_library().gdn_chunk_bwd_workspace_size(ctypes.byref(p), ctypes.byref(nbytes)) == 0
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device="cuda")  # allocated once, outside

    def step():
        gdn.chunk_bwd(dev["q"], dev["k"], dev["v"], g, dev["beta"], cu, dev["dout"], workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    nbytes_alg = BWD_BYTES_PER_TH * T * H
    achieved = nbytes_alg / (ms / 1e3) / 1e9
    return {"workload": f"packed {T} tokens ({len(inp['cu_seqlens']) - 1} documents of "
                        f"4096..16384), H={H}, d_k=d_v={D}, bf16, dO ~ N(0,1)",
            "ms_per_step": ms, "tokens_per_s": T / (ms / 1e3),
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "bytes_per_step": nbytes_alg}}


def kernel_source_sha():
    """Hash of the timed kernel's translation unit (gdn_fwd_ws.hip and the csrc headers it
    includes, followed recursively) and of the compiler flags build.py gives it.  Changes to
    other kernels leave it, and so the stored traffic figure, valid."""
    import hashlib

    from linear_attention_recurrence_prefill_amd import build as b

    csrc = b.CSRC
    seen, todo = [], ["gdn_fwd_ws.hip"]
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
    h.update(repr((b.HIP_FLAGS, b.EXTRA_FLAGS.get("gdn_fwd_ws.hip", []))).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
