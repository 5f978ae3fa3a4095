#!/usr/bin/env python3
"""Throughput of the chunked SSD forward pass on one MI355X.

One step = one full forward pass of the layer (dt preprocessing and chunk
prefix sums, chunk states, state passing, chunk scan with the D skip) over one
batch of synthetic, already device-resident inputs.  Default workload: the
Mamba-2-2.7B-shaped layer, batch 4, seqlen 4096, 80 heads x P=64, N=128, one
B/C group, chunk 256, bf16 storage with fp32 accumulation.

Prints ONE JSON line: tokens/s for the whole step; the roofline of the dominant
kernel (algorithmic bytes per launch / its average duration from HIP events
recorded around every launch on the launch stream inside the timed region);
and the fp64 CPU oracle timed on a bounded sample of the same workload on this
host's cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--algo auto]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD fwd tokens/s and TFLOP/s (% MFMA peak), 2.7B-shaped layer, L=4096, 1 GPU"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA peaks
MAX_EVENTS = 8


def chunk_lengths(wl, inp):
    """Lengths of the chunks the kernels process (per batch row, or of the packed stream)."""
    L = inp.x.shape[1]
    Q = wl.chunk
    full, rem = divmod(L, Q)
    per_row = [Q] * full + ([rem] if rem else [])
    return per_row * inp.x.shape[0]


def model_flops(wl, inp):
    """Algorithmic FLOPs, causal pairs only, C B^T counted once per group:
    per chunk of q tokens G N q(q+1) + H P q(q+1) + 4 H q N P + 2 H N P."""
    H, P, N, G = wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    return float(sum(G * N * q * (q + 1) + H * P * q * (q + 1) + 4 * H * q * N * P + 2 * H * N * P
                     for q in chunk_lengths(wl, inp)))


def compulsory_bytes(wl, inp, with_final):
    """Inputs read once and outputs written once: x, y, B, C, dt, A, D, states in/out."""
    b, L, H, P = inp.x.shape
    G, N = wl.ngroups, wl.dstate
    e = 2 if wl.dtype == "bf16" else 4
    T = b * L
    nstate = (inp.nseqs if inp.initial_states is not None else 0) + (inp.nseqs if with_final else 0)
    return e * (2 * T * H * P + 2 * T * G * N + T * H) + 4 * 2 * H + 4 * H * N * P * nstate


def kernel_bytes(name, wl, inp, with_final):
    """Algorithmic bytes of one launch of each kernel of the chunked schedule:
    the data it must read and write once given its place in the schedule."""
    b, L, H, P = inp.x.shape
    G, N = wl.ngroups, wl.dstate
    e = 2 if wl.dtype == "bf16" else 4
    T = b * L
    nch = len(chunk_lengths(wl, inp))
    Q = wl.chunk
    per_chunk_f32 = 4 * H * nch * Q           # one fp32 value per (head, padded token)
    states = 4 * H * nch * N * P              # one fp32 state per (chunk, head)
    x = e * T * H * P
    bc = e * T * G * N
    if name == "dt_cumsum":
        return e * T * H + 2 * per_chunk_f32
    if name == "chunk_state":
        return x + bc + 2 * per_chunk_f32 + states
    if name == "state_passing":
        return 2 * states
    if name == "chunk_scan":
        return 2 * x + 2 * bc + 2 * per_chunk_f32 + states
    if name == "final_states":
        return 4 * H * N * P * inp.nseqs
    if name == "fused":
        return compulsory_bytes(wl, inp, with_final)
    return 0


def cpu_baseline(inp, budget_s):
    """Time the fp64 oracle on whole (sequence, head) streams of the workload until
    about budget_s of CPU work; report equivalent full-layer tokens/s."""
    import numpy as np

    import oracle

    lib = oracle.load()
    cores = oracle.num_threads(lib)
    H = inp.x.shape[2]
    S = inp.nseqs
    order = [(s, h) for h in range(H) for s in range(S)]
    lens = ([inp.x.shape[1]] * S if inp.cu_seqlens is None
            else list(np.diff(inp.cu_seqlens).astype(int)))
    done, tokens_heads, t_used = 0, 0, 0.0
    batch = max(cores, 1)
    while done < len(order) and t_used < budget_s:
        pairs = order[done:done + batch]
        t0 = time.perf_counter()
        oracle.ssd_ref(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.dt_bias,
                       inp.initial_states, inp.cu_seqlens, softplus=inp.softplus,
                       dt_min=inp.dt_min, dt_max=inp.dt_max, pairs=pairs, want_final=False,
                       lib=lib)
        t_used += time.perf_counter() - t0
        tokens_heads += sum(lens[s] for s, _ in pairs)
        done += len(pairs)
        if t_used > 0 and done < len(order):
            per_pair = t_used / done
            batch = max(cores, int((budget_s - t_used) / per_pair) // cores * cores)
    value = (tokens_heads / H) / t_used
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {len(order)} (sequence, head) streams, "
                      f"{tokens_heads} token-heads in {t_used:.1f} s, fp64 recurrence, "
                      f"OpenMP over streams"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mamba2_2p7b")
    ap.add_argument("--algo", default="auto", choices=["auto", "chunked", "fused"])
    ap.add_argument("--final-states", action="store_true", help="also return final states")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU work budget of the oracle baseline (0 disables it)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import ssd_scan_amd as ssd
    import ssd_synth

    wl = ssd_synth.workloads()[args.workload]
    inp = ssd_synth.make(args.workload)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    t = lambda a, d=tdt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(
        device=dev, dtype=d)
    x, dt, B, C = t(inp.x), t(inp.dt), t(inp.B), t(inp.C)
    A, D = t(inp.A, torch.float32), t(inp.D, torch.float32)
    init = t(inp.initial_states, torch.float32)
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to(dev)
    b, L, H, P = x.shape
    with_final = bool(args.final_states)
    y = torch.empty_like(x)
    fin = torch.empty((inp.nseqs, H, wl.dstate, P), dtype=torch.float32,
                      device=dev) if with_final else None
    prob = ssd.make_problem(b, L, H, P, wl.dstate, wl.ngroups, wl.chunk, bf16=wl.dtype == "bf16",
                            nseqs=0 if cu is None else inp.nseqs, softplus=True,
                            dt_min=inp.dt_min, dt_max=inp.dt_max, algo=args.algo)
    ws = torch.empty(max(ssd.workspace_size(prob), 1), dtype=torch.uint8, device=dev)
    lib = ssd.library()
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    ptr = lambda v: None if v is None else v.data_ptr()
    call_args = [ctypes.byref(prob), ptr(x), ptr(dt), ptr(A), ptr(B), ptr(C), ptr(D), None,
                 ptr(init), ptr(cu), ptr(y), ptr(fin), ptr(ws), ws.numel(), sptr]

    # events for every launch of every timed step (created by a first record)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(MAX_EVENTS)]
              for _ in range(args.steps)]
    for row in events:
        for ev in row:
            ev.record(stream)
    handles = [(ctypes.c_void_p * MAX_EVENTS)(*[ev.cuda_event for ev in row]) for row in events]
    names = [(ctypes.c_char_p * MAX_EVENTS)() for _ in range(args.steps)]
    counts = [ctypes.c_int(0) for _ in range(args.steps)]

    for _ in range(args.warmup):
        st = lib.ssd_fwd(*call_args)
        if st != 0:
            raise ssd.SsdError(st)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        st = lib.ssd_fwd_events(*call_args, handles[k], names[k], MAX_EVENTS,
                                ctypes.byref(counts[k]))
        if st != 0:
            raise ssd.SsdError(st)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = start.elapsed_time(end) / args.steps

    # per-kernel durations over the timed steps
    per_kernel = {}
    for k in range(args.steps):
        n = counts[k].value
        for i in range(n - 1):
            nm = names[k][i].decode()
            per_kernel.setdefault(nm, []).append(events[k][i].elapsed_time(events[k][i + 1]))
    kernel_ms = {nm: float(np.mean(v)) for nm, v in per_kernel.items()}
    dominant = max(kernel_ms, key=kernel_ms.get)
    kb = kernel_bytes(dominant, wl, inp, with_final)
    achieved = kb / (kernel_ms[dominant] * 1e-3) / 1e9

    tokens = b * L
    flops = model_flops(wl, inp)
    cbytes = compulsory_bytes(wl, inp, with_final)
    step_s = ms_per_step * 1e-3
    out = {
        "metric": METRIC,
        "value": tokens / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded, Mamba-2-shaped; see ssd_synth.py)",
        "config": {"workload": wl.name, "batch": b, "seqlen": L, "heads": H, "headdim": P,
                   "dstate": wl.dstate, "ngroups": wl.ngroups, "chunk": wl.chunk,
                   "final_states": with_final, "algo": args.algo},
        "tflops": flops / step_s / 1e12,
        "pct_mfma_peak": 100.0 * flops / step_s / 1e12 / MFMA_PEAK_TFLOPS[wl.dtype],
        "op_roofline_frac": (cbytes / (HBM_PEAK_GBS * 1e9)) / step_s,
        "kernel_ms": kernel_ms,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes": kb},
        "wall_s": t_wall,
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
